"""GPU parity of the alternate block formats (asymmetric uint4, Q8_0): the
HIP library through the C ABI against the format oracle.

Quantized codes and parameters, and the dequantized weight, must be
bit-exact; linear outputs are compared in fp32 by relative Frobenius error,
bound 2e-3 (the same bound as NF4: fp32 accumulation of exact bf16 products
against float64).
"""
import sys

import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import linear as olin
from oracle import merge as omerge
from oracle import nf4 as onf4

pytestmark = pytest.mark.gpu

REL_TOL = 2e-3
FMTS = ["u4_asym", "q8_0"]


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from qlora_fine_tuning_nf4_amd import binding
    binding.lib()
    return binding


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _t(bits, dev="cuda"):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def _bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _rel(a, ref):
    ref = np.asarray(ref, dtype=np.float64)
    num = np.linalg.norm(np.asarray(a, dtype=np.float64) - ref)
    den = np.linalg.norm(ref)
    return num / den if den > 0 else num


def _same(got, ref, tag):
    """Exact equality, reporting the first mismatches."""
    got, ref = np.asarray(got), np.asarray(ref)
    bad = np.argwhere(~((got == ref) | (np.isnan(got) & np.isnan(ref))))
    if bad.size:
        idx = [tuple(int(v) for v in b) for b in bad[:6]]
        detail = [(i, float(got[i]), float(ref[i])) for i in idx]
        raise AssertionError(f"{tag}: {len(bad)} mismatches, first {detail}")


def _fmt(B, name):
    return B.FORMATS[name]


def _quant(B, name, w_bits):
    """Device quantization of bf16 bits (n x k) in format `name`."""
    return B.qlora_quantize(_t(w_bits), None, fmt=_fmt(B, name))


def _oracle_wd(name, w_bits):
    if name == "u4_asym":
        c, s, z = F.u4_quantize(w_bits)
        return F.u4_dequantize(c, s, z).reshape(w_bits.shape)
    q, d16 = F.q8_quantize(w_bits)
    return F.q8_dequantize(q, d16).reshape(w_bits.shape)


def _weight(n, k, dist, seed):
    if dist == "normal":
        return synth.normal_bf16((n, k), 0.02, seed)
    if dist == "outlier":
        return synth.normal_bf16((n, k), 0.015, seed, outlier_rate=0.001, outlier_scale=20)
    if dist == "tiny":       # Q8_0 scales in the fp16 subnormal range
        return synth.normal_bf16((n, k), 2.0 ** -17, seed)
    w = synth.normal_bf16((n, k), 0.02, seed)
    flat = w.reshape(-1)
    nb = flat.size // 64
    flat[0:64] = 0                                          # zero unit
    if nb > 2:
        flat[64:128] = 0x3E80                               # all 0.25: one-sign block
    if nb > 3:
        flat[128:192] = 0xBF00                              # all -0.5
    if nb > 4:
        flat[192:224] = 0x8000                              # -0 half unit, then positives
        flat[224:256] = 0x3C00                              # 2^-7
    if nb > 5:
        flat[5 * 64] = 0xC2C8                               # -100: negative outlier
    return w


@pytest.mark.parametrize("name", FMTS)
@pytest.mark.parametrize("n,k,dist", [(1, 64, "normal"), (3, 128, "special"), (300, 64, "special"),
                                      (257, 11008, "outlier"), (1000, 4096, "normal"),
                                      (40, 320, "tiny")])
def test_quantize_bitexact(name, n, k, dist):
    """Codes and per-unit parameters in storage order, and the dense
    dequantization, bit for bit."""
    B = _dev()
    _say("quantize", name, n, k, dist)
    w = _weight(n, k, dist, n * 7 + k)
    q = _quant(B, name, w)
    torch.cuda.synchronize()
    if name == "u4_asym":
        c, s, z = F.u4_quantize(w)
        cs, ps = F.u4_to_storage(c, s, z, n, k)
        assert q.qscale is None
        assert np.array_equal(q.codes.cpu().numpy(), cs)
        assert np.array_equal(q.step.cpu().numpy().view(np.uint32), ps.reshape(-1).view(np.uint32))
    else:
        qq, d16 = F.q8_quantize(w)
        cs, ss = F.q8_to_storage(qq, d16, n, k)
        assert q.step is None
        assert np.array_equal(q.codes.cpu().numpy().view(np.int8), cs)
        assert np.array_equal(q.qscale.cpu().numpy().view(np.uint16), ss.reshape(-1).view(np.uint16))
    d = B.qlora_dequantize(q, None)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(d).reshape(-1), _oracle_wd(name, w).reshape(-1))


@pytest.mark.parametrize("name", FMTS)
@pytest.mark.parametrize("path", ["gemm", "gemv"])
def test_fused_identity_fwd(name, path):
    """X = identity rows: the fused forward returns deq(W)^T exactly."""
    B = _dev()
    n, k = 200, 512
    w = _weight(n, k, "special", 95)
    q = _quant(B, name, w)
    wd = onf4.bf16_to_f32(_oracle_wd(name, w))
    for r0 in (range(0, k, 32) if path == "gemv" else [0]):
        m = 32 if path == "gemv" else k
        eye = np.zeros((m, k), dtype=np.float32)
        eye[np.arange(m), r0 + np.arange(m)] = 1.0
        X = torch.from_numpy(eye).to(torch.bfloat16).cuda()
        Y, _ = B.qlora_linear_fwd(q, None, X, path=path)
        torch.cuda.synchronize()
        _same(Y.cpu().numpy(), wd[:, r0:r0 + m].T, (name, path, r0))


@pytest.mark.parametrize("name", FMTS)
@pytest.mark.parametrize("n,k", [(300, 384), (200, 384)])
def test_fused_identity_dx(name, n, k):
    """dY = identity: the fused backward returns deq(W) exactly (ragged last
    step and partial row group included)."""
    B = _dev()
    w = _weight(n, k, "outlier", 96 + n)
    q = _quant(B, name, w)
    wd = onf4.bf16_to_f32(_oracle_wd(name, w))
    dY = torch.eye(n, dtype=torch.float32).to(torch.bfloat16).cuda()
    dX, _, _ = B.qlora_linear_bwd(q, None, None, dY)
    torch.cuda.synchronize()
    _same(dX.cpu().numpy(), wd, (name, n, k))


def _inputs(M, N, K, r, seed):
    X = synth.normal_bf16((M, K), 1.0, seed)
    W = synth.normal_bf16((N, K), 0.02, seed + 1)
    A = synth.normal_bf16((r, K), 0.01, seed + 2)
    Bm = synth.normal_bf16((N, r), 0.01, seed + 3)
    dY = synth.normal_bf16((M, N), 1.0, seed + 4)
    return X, W, A, Bm, dY


@pytest.mark.parametrize("name", FMTS)
@pytest.mark.parametrize("M,N,K,r", [(130, 300, 512, 16), (257, 513, 640, 64), (33, 100, 192, 4),
                                     (4096, 3072, 3072, 64), (4096, 8192, 3072, 64),
                                     (4096, 3072, 8192, 64)])
def test_linear_parity(name, M, N, K, r):
    """Forward (GEMM, and the streaming path on the first 32 rows) and backward
    against the oracle; the 3.8B-style projections at seq 4096 with r = 64
    (alpha 128) compare 32 sampled rows of Y and dX and all of dA, dB."""
    B = _dev()
    _say("linear", name, M, N, K, r)
    s = 128.0 / 64 if r == 64 else 2.0
    X, W, A, Bm, dY = _inputs(M, N, K, r, seed=M + N * 3 + K + r)
    q = _quant(B, name, W)
    Xd, Ad, Bd, dYd = _t(X), _t(A), _t(Bm), _t(dY)
    Y, T = B.qlora_linear_fwd(q, None, Xd, Ad, Bd, s)
    dX, dA, dB = B.qlora_linear_bwd(q, None, Xd, dYd, Ad, Bd, s, T=T)
    Yv, _ = B.qlora_linear_fwd(q, None, Xd[:32], Ad, Bd, s, path="gemv")
    torch.cuda.synchronize()
    Wd = _oracle_wd(name, W)
    ms = np.arange(M) if M <= 512 else np.sort(synth.rng(8).choice(M, 32, replace=False))
    Yo, _ = olin.forward(Wd, X[ms], A, Bm, s)
    assert _rel(Y.cpu().numpy()[ms], Yo) <= REL_TOL
    Yvo, _ = olin.forward(Wd, X[:32], A, Bm, s)
    assert _rel(Yv.cpu().numpy(), Yvo) <= REL_TOL
    dXo = olin.backward(Wd, X[ms], dY[ms], A, Bm, s)[0]
    assert _rel(dX.cpu().numpy()[ms], dXo) <= REL_TOL
    xf, dyf = onf4.bf16_to_f32(X).astype(np.float64), onf4.bf16_to_f32(dY).astype(np.float64)
    af, bf = onf4.bf16_to_f32(A).astype(np.float64), onf4.bf16_to_f32(Bm).astype(np.float64)
    dAo = s * (dyf @ bf).T @ xf
    dBo = s * dyf.T @ (xf @ af.T)
    assert _rel(dA.cpu().numpy(), dAo) <= REL_TOL and _rel(dB.cpu().numpy(), dBo) <= REL_TOL


GROUP_SHAPES = [(3072, 3072, 64), (300, 320, 0), (8192, 3072, 64), (257, 8192, 8), (64, 64, 0)]


@pytest.mark.parametrize("name", FMTS)
@pytest.mark.parametrize("M", [1, 16, 32])
def test_grouped_forward(name, M):
    B = _dev()
    _say("grouped", name, M)
    jobs, ref = [], []
    for i, (N, K, r) in enumerate(GROUP_SHAPES):
        X, W, A, Bm, _ = _inputs(M, N, K, r, seed=500 + M + 17 * i)
        q = _quant(B, name, W)
        j = dict(w=q, X=_t(X), Y=torch.full((M, N), float("nan"), device="cuda"))
        if r:
            j.update(A=_t(A), B=_t(Bm), scaling=2.0, T=torch.full((M, r), float("nan"), device="cuda"))
        jobs.append(j)
        ref.append((W, X, A if r else None, Bm if r else None))
    g = B.qlora_group_init(jobs, M, y_dtype=torch.float32)
    B.qlora_linear_fwd_grouped(g, None)
    torch.cuda.synchronize()
    for j, (W, X, A, Bm) in zip(jobs, ref):
        Yo, _ = olin.forward(_oracle_wd(name, W), X, A, Bm, 2.0)
        assert _rel(j["Y"].cpu().numpy(), Yo) <= REL_TOL


# --------------------------------------------------------------------------- merge + requantize
_LV, _MID = onf4.codebook()


def _oracle_wd_any(name, w_bits):
    if name == "nf4":
        c, q, st = onf4.quantize(w_bits, _MID)
        return onf4.dequantize(c, q, st, _LV).reshape(w_bits.shape)
    return _oracle_wd(name, w_bits)


def _oracle_quant_storage(name, w_bits):
    """Expected device arrays of quantize(w) in format `name`, storage order:
    (codes bytes, second array bytes, third array bytes)."""
    n, k = w_bits.shape
    if name == "nf4":
        c, q, st = onf4.quantize(w_bits, _MID)
        cs, qs = onf4.to_storage(c, q, n, k)
        return cs, qs, st.view(np.uint8)
    if name == "u4_asym":
        c, sc, z = F.u4_quantize(w_bits)
        cs, ps = F.u4_to_storage(c, sc, z, n, k)
        return cs, None, ps.reshape(-1).view(np.uint8)
    qq, d16 = F.q8_quantize(w_bits)
    cs, ss = F.q8_to_storage(qq, d16, n, k)
    return cs.view(np.uint8), ss.reshape(-1).view(np.uint8), None


@pytest.mark.parametrize("src,dst,N,K,r", [("nf4", "nf4", 300, 512, 16), ("nf4", "q8_0", 257, 320, 8),
                                          ("q8_0", "nf4", 200, 384, 64), ("u4_asym", "u4_asym", 130, 256, 4),
                                          ("nf4", "nf4", 4096, 4096, 16)])
def test_merge_and_requantize(src, dst, N, K, r):
    """Merged bf16 weight bit-exact against the merge oracle, the requantized
    arrays bit-exact against the quantizer of the target format; the forward
    through the requantized merge is compared with the separate adapter."""
    B = _dev()
    _say("merge", src, dst, N, K, r)
    s = 2.0
    W = synth.normal_bf16((N, K), 0.02, N + K + r)
    A = synth.normal_bf16((r, K), 0.01, N + K + r + 1)
    Bm = synth.normal_bf16((N, r), 0.01, N + K + r + 2)
    cb = B.device_codebook()
    q = B.qlora_quantize(_t(W), cb if src == "nf4" else None, fmt=_fmt(B, src))
    out = B.NF4Weight.empty(N, K, "cuda", fmt=_fmt(B, dst))
    M, out = B.qlora_merge(q, cb, _t(A), _t(Bm), s, out=out)
    torch.cuda.synchronize()
    Wd = _oracle_wd_any(src, W)
    Mo = omerge.merged_weight(Wd, A, Bm, s)
    _same(_bits(M).astype(np.int64), Mo.astype(np.int64), ("merged", src, dst))
    cs, a2, a3 = _oracle_quant_storage(dst, Mo)
    assert np.array_equal(out.codes.cpu().numpy(), cs)
    if a2 is not None:
        assert np.array_equal(out.qscale.cpu().numpy(), a2)
    if a3 is not None:
        assert np.array_equal(out.step.cpu().numpy().view(np.uint8), a3)
    # what the merge costs against keeping the adapter separate (context)
    if N <= 512:
        X = synth.normal_bf16((64, K), 1.0, 9)
        Ysep, _ = olin.forward(Wd, X, A, Bm, s)
        Ymrg, _ = olin.forward(_oracle_wd_any(dst, Mo), X)      # deq(quant(merged)), the arrays above
        rel = _rel(Ymrg, Ysep)
        _say(f"  forward through the requantized merge vs separate adapter: rel {rel:.4f}")
        assert rel < 0.25
