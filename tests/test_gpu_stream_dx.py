"""GPU parity of the streaming input gradient (small m, dX = dY deq(W) +
s U A with the packed weight read once) through the C ABI against the
oracles.

Exact checks: with dY holding one 1 per row at distinct columns (rows picked
across the weight, the last partial 16-row group included), dX row i is the
dequantized weight row exactly, in every weight format, through both the
unaligned (n % 8 != 0) and 16-byte dY paths, with and without the split over
rows.  Random inputs: dX, dA, dB within 2e-3 relative Frobenius error in
fp32 (fp32 accumulation of exact 16-bit products against float64), and the
streaming and GEMM paths within that bound of each other.
"""
import sys

import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import linear as olin
from oracle import nf4 as onf4

pytestmark = pytest.mark.gpu

REL_TOL = 2e-3
LV, MID = onf4.codebook()

# (name, fmt key for the binding, NF4 block, double quantization, fp16 compute)
FORMATS = [("nf4dq", "nf4", 64, True, False), ("nf4", "nf4", 64, False, False),
           ("b32dq", "nf4", 32, True, False), ("b32", "nf4", 32, False, False),
           ("b128dq", "nf4", 128, True, False), ("b128", "nf4", 128, False, False),
           ("u4_asym", "u4_asym", 64, False, False), ("q8_0", "q8_0", 64, False, False),
           ("f16", "nf4", 64, True, True)]
IDS = [f[0] for f in FORMATS]


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from qlora_fine_tuning_nf4_amd import binding
    binding.lib()
    return binding


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _t(bits, f16=False, dev="cuda"):
    dt = torch.float16 if f16 else torch.bfloat16
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(dt).to(dev)


def _rel(a, ref):
    ref = np.asarray(ref, dtype=np.float64)
    return np.linalg.norm(np.asarray(a, dtype=np.float64) - ref) / np.linalg.norm(ref)


def _same(got, ref, tag):
    got, ref = np.asarray(got), np.asarray(ref)
    bad = np.argwhere(got != ref)
    if bad.size:
        idx = [tuple(int(v) for v in b) for b in bad[:6]]
        raise AssertionError(f"{tag}: {len(bad)} mismatches, first {[(i, float(got[i]), float(ref[i])) for i in idx]}")


def _weight(n, k, seed, f16):
    if f16:
        return synth.normal_f16((n, k), 0.015, seed, outlier_rate=0.001, outlier_scale=20)
    return synth.normal_bf16((n, k), 0.015, seed, outlier_rate=0.001, outlier_scale=20)


def _quant(B, spec, w):
    name, key, block, dq, f16 = spec
    cb = B.device_codebook() if key == "nf4" else None
    if key == "nf4":
        return B.qlora_quantize(_t(w, f16), cb, double_quant=dq, block=block), cb
    return B.qlora_quantize(_t(w), None, fmt=B.FORMATS[key]), cb


def _oracle_wd_f32(spec, w):
    """The oracle's dequantized weight as fp32 values."""
    name, key, block, dq, f16 = spec
    if key == "u4_asym":
        c, s, z = F.u4_quantize(w)
        return onf4.bf16_to_f32(F.u4_dequantize(c, s, z).reshape(w.shape))
    if key == "q8_0":
        q, d16 = F.q8_quantize(w)
        return onf4.bf16_to_f32(F.q8_dequantize(q, d16).reshape(w.shape))
    if f16:
        c, q, st = onf4.quantize(w, MID, dtype="f16")
        return onf4.f16_to_f32(onf4.dequantize(c, q, st, LV, dtype="f16").reshape(w.shape))
    if dq:
        c, q, st = onf4.quantize(w, MID, block=block)
        return onf4.bf16_to_f32(onf4.dequantize(c, q, st, LV, block=block).reshape(w.shape))
    c, am = onf4.quantize_nodq(w, MID, block=block)
    return onf4.bf16_to_f32(onf4.dequantize_nodq(c, am, LV, block=block).reshape(w.shape))


def _picked_rows(n, m, seed):
    """m distinct rows of an n-row weight, the first and last included."""
    rows = {0, n - 1}
    rest = synth.rng(seed).permutation(n)
    for v in rest:
        if len(rows) >= m:
            break
        rows.add(int(v))
    return np.array(sorted(rows)[:m])


# n % 8 != 0 (element dY loads), a partial last 16-row group, one split or
# several, k not a multiple of 256 (block 128 needs k % 128 == 0)
@pytest.mark.parametrize("spec", FORMATS, ids=IDS)
@pytest.mark.parametrize("n,k,m", [(20, 384, 20), (300, 384, 32), (4096, 256, 17), (1000, 128, 5)])
def test_stream_dx_selects_rows_exactly(spec, n, k, m):
    B = _dev()
    f16 = spec[4]
    _say("stream dx rows", spec[0], n, k, m)
    w = _weight(n, k, 300 + n + k, f16)
    q, cb = _quant(B, spec, w)
    wd = _oracle_wd_f32(spec, w)
    rows = _picked_rows(n, m, n + m)
    dY = torch.zeros((m, n), dtype=torch.float32)
    dY[np.arange(m), rows] = 1.0
    dY = dY.to(torch.float16 if f16 else torch.bfloat16).cuda()
    dX, _, _ = B.qlora_linear_bwd(q, cb, None, dY, path="gemv")
    torch.cuda.synchronize()
    _same(dX.cpu().numpy(), wd[rows], (spec[0], n, k, m))


# (M, N, K, r): one 16-row tile and two (M > 16), a single split with the
# LoRA term added in the kernel (K = 32768: 512 k-blocks), many splits, the
# 7B shapes
CASES = [(1, 64, 64, 0), (3, 100, 192, 4), (16, 4096, 4096, 8), (17, 300, 320, 16),
         (32, 11008, 256, 8), (32, 4096, 11008, 8), (8, 257, 64, 0), (4, 200, 32768, 8),
         (2, 5000, 128, 0), (24, 11008, 4096, 8)]


@pytest.mark.parametrize("M,N,K,r", CASES)
def test_stream_dx_parity(M, N, K, r):
    B = _dev()
    _say("stream dx", M, N, K, r)
    s = 2.0
    seed = 7 * M + N + 3 * K + r
    X = synth.normal_bf16((M, K), 1.0, seed)
    W = synth.normal_bf16((N, K), 0.02, seed + 1)
    A = synth.normal_bf16((r, K), 0.01, seed + 2)
    Bm = synth.normal_bf16((N, r), 0.01, seed + 3)
    dY = synth.normal_bf16((M, N), 1.0, seed + 4)
    cb = B.device_codebook()
    q = B.qlora_quantize(_t(W), cb)
    Xd, Ad, Bd, dYd = _t(X), _t(A), _t(Bm), _t(dY)
    lo = (Xd, dYd, Ad, Bd, s) if r else (None, dYd)
    dXv, dAv, dBv = B.qlora_linear_bwd(q, cb, *lo, path="gemv")
    dXh, _, _ = B.qlora_linear_bwd(q, cb, *lo, dx_dtype=torch.bfloat16, path="gemv")
    dXg, _, _ = B.qlora_linear_bwd(q, cb, *lo, path="gemm")
    torch.cuda.synchronize()
    c, qs, st = onf4.quantize(W, MID)
    Wd = onf4.dequantize(c, qs, st, LV).reshape(W.shape)
    dXo, dAo, dBo = (olin.backward(Wd, X, dY, A, Bm, s) if r else olin.backward(Wd, X, dY))
    e = _rel(dXv.cpu().numpy(), dXo)
    _say(f"  rel_fro dX {e:.3e}")
    assert e <= REL_TOL
    # bf16 output: the fp32 result rounded once (within one bf16 ulp of it)
    hv = dXh.float().cpu().numpy().astype(np.float64)
    fv = dXv.cpu().numpy().astype(np.float64)
    ulp = np.spacing(np.abs(fv).astype(np.float32)).astype(np.float64) * 65536.0
    assert np.all(np.abs(hv - fv) <= ulp)
    assert _rel(dXg.cpu().numpy(), dXo) <= REL_TOL
    assert _rel(dXv.cpu().numpy(), dXg.cpu().numpy()) <= REL_TOL
    if r:
        assert _rel(dAv.cpu().numpy(), dAo) <= REL_TOL and _rel(dBv.cpu().numpy(), dBo) <= REL_TOL


def test_stream_dx_auto_path_and_limits():
    """AUTO takes the streaming kernel for m <= 32 (the results match a forced
    'gemv' call bit for bit), and a forced 'gemv' above that m is refused."""
    B = _dev()
    W = synth.normal_bf16((512, 1024), 0.02, 41)
    cb = B.device_codebook()
    q = B.qlora_quantize(_t(W), cb)
    dY = _t(synth.normal_bf16((32, 512), 1.0, 42))
    a, _, _ = B.qlora_linear_bwd(q, cb, None, dY)
    v, _, _ = B.qlora_linear_bwd(q, cb, None, dY, path="gemv")
    torch.cuda.synchronize()
    assert torch.equal(a, v)
    dY33 = _t(synth.normal_bf16((33, 512), 1.0, 43))
    with pytest.raises(B.QLoRAError, match="status 8"):
        B.qlora_linear_bwd(q, cb, None, dY33, path="gemv")


def test_stream_dx_deterministic():
    """The split partials are added in a fixed order: repeated calls agree bit
    for bit."""
    B = _dev()
    W = synth.normal_bf16((11008, 4096), 0.02, 51)
    cb = B.device_codebook()
    q = B.qlora_quantize(_t(W), cb)
    dY = _t(synth.normal_bf16((16, 11008), 1.0, 52))
    outs = [B.qlora_linear_bwd(q, cb, None, dY, path="gemv")[0] for _ in range(3)]
    torch.cuda.synchronize()
    assert all(torch.equal(outs[0], o) for o in outs[1:])


# (m, n, k, r): several 8-rank blocks (24, 64), a ragged last 16-row group, n
# not a multiple of 8 (U falls back to its own launch, T still formed in the
# forward's reduce), the 11008-wide contraction
RANK_ROW_CASES = [(32, 2048, 4096, 64), (5, 1024, 8192, 24), (16, 4104, 2048, 16),
                  (8, 1002, 4096, 8), (3, 4096, 11008, 8)]


@pytest.mark.parametrize("M,N,K,r", RANK_ROW_CASES)
def test_small_m_rank_rows_in_split_reduce(M, N, K, r):
    """Small-m forward and backward whose split reduces form the T and U rows
    themselves (www.lqnn.cn/news/228537 §3.2): Y, the saved T, dX, dA, dB
    against the oracle; a backward that recomputes T gives the same bytes as
    one given the forward's T; bf16 outputs within one bf16 ulp of fp32."""
    B = _dev()
    _say("rank rows", M, N, K, r)
    s = 2.0
    seed = 11 * M + N + 5 * K + r
    X = synth.normal_bf16((M, K), 1.0, seed)
    W = synth.normal_bf16((N, K), 0.02, seed + 1)
    A = synth.normal_bf16((r, K), 0.01, seed + 2)
    Bm = synth.normal_bf16((N, r), 0.01, seed + 3)
    dY = synth.normal_bf16((M, N), 1.0, seed + 4)
    cb = B.device_codebook()
    q = B.qlora_quantize(_t(W), cb)
    Xd, Ad, Bd, dYd = _t(X), _t(A), _t(Bm), _t(dY)
    Y, T = B.qlora_linear_fwd(q, cb, Xd, Ad, Bd, s)
    Yh, _ = B.qlora_linear_fwd(q, cb, Xd, Ad, Bd, s, y_dtype=torch.bfloat16)
    dX, dA, dB = B.qlora_linear_bwd(q, cb, Xd, dYd, Ad, Bd, s, T=T)
    dXr, dAr, dBr = B.qlora_linear_bwd(q, cb, Xd, dYd, Ad, Bd, s)   # T recomputed
    torch.cuda.synchronize()
    c, qs, st = onf4.quantize(W, MID)
    Wd = onf4.dequantize(c, qs, st, LV).reshape(W.shape)
    Yo, To = olin.forward(Wd, X, A, Bm, s)
    dXo, dAo, dBo = olin.backward(Wd, X, dY, A, Bm, s)
    errs = {"Y": _rel(Y.cpu().numpy(), Yo), "T": _rel(T.cpu().numpy(), To),
            "dX": _rel(dX.cpu().numpy(), dXo), "dA": _rel(dA.cpu().numpy(), dAo),
            "dB": _rel(dB.cpu().numpy(), dBo)}
    _say("  " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    assert max(errs.values()) <= REL_TOL, errs
    assert torch.equal(dX, dXr) and torch.equal(dA, dAr) and torch.equal(dB, dBr)
    hv = Yh.float().cpu().numpy().astype(np.float64)
    fv = Y.cpu().numpy().astype(np.float64)
    ulp = np.spacing(np.abs(fv).astype(np.float32)).astype(np.float64) * 65536.0
    assert np.all(np.abs(hv - fv) <= ulp)
