"""GPU parity of the fp16 compute type (NF4, block 64, double quantization)
through the C ABI against the oracle: quantized arrays and the dequantized
fp16 weight bit-exact (subnormal outputs included), exact identity products
through every fused path, linear outputs within 2e-3 relative Frobenius error
in fp32, fp16 outputs within one fp16 ulp plus the accumulation bound, the
grouped forward, the split reductions and the merge bit-exact."""
import sys

import numpy as np
import pytest
import torch

import synth
from oracle import linear as olin
from oracle import merge as omerge
from oracle import nf4 as onf4

pytestmark = pytest.mark.gpu

REL_TOL = 2e-3
LV, MID = onf4.codebook()
F16 = "f16"


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from qlora_fine_tuning_nf4_amd import binding
    binding.lib()
    return binding


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _t(bits, dev="cuda"):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.float16).to(dev)


def _bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _rel(a, ref):
    ref = np.asarray(ref, dtype=np.float64)
    return np.linalg.norm(np.asarray(a, dtype=np.float64) - ref) / np.linalg.norm(ref)


def _same(got, ref, tag):
    got, ref = np.asarray(got), np.asarray(ref)
    bad = np.argwhere(got != ref)
    if bad.size:
        idx = [tuple(int(v) for v in b) for b in bad[:6]]
        raise AssertionError(f"{tag}: {len(bad)} mismatches, first {[(i, got[i], ref[i]) for i in idx]}")


def _oracle(w):
    c, q, st = onf4.quantize(w, MID, dtype=F16)
    return c, q, st, onf4.dequantize(c, q, st, LV, dtype=F16).reshape(w.shape)


def _weight(n, k, dist, seed):
    if dist == "normal":
        return synth.normal_f16((n, k), 0.02, seed)
    if dist == "outlier":
        return synth.normal_f16((n, k), 0.015, seed, outlier_rate=0.001, outlier_scale=20)
    if dist == "tiny":            # fp16 subnormal weights and dequantized values
        return synth.normal_f16((n, k), 3e-6, seed)
    w = synth.normal_f16((n, k), 0.02, seed)
    flat = w.reshape(-1)
    flat[0:128] = 0                                        # zero blocks
    flat[128:192] = 0x3400                                  # 0.25 run
    flat[200] = 0xD640                                      # -100
    flat[300] = 0x7BFF                                      # 65504: the largest fp16
    return w


def _inputs(M, N, K, r, seed, wsig=0.02):
    X = synth.normal_f16((M, K), 1.0, seed)
    W = synth.normal_f16((N, K), wsig, seed + 1)
    A = synth.normal_f16((r, K), 0.01, seed + 2)
    Bm = synth.normal_f16((N, r), 0.01, seed + 3)
    dY = synth.normal_f16((M, N), 1.0, seed + 4)
    return X, W, A, Bm, dY


@pytest.mark.parametrize("n,k,dist", [(1, 128, "normal"), (3, 256, "special"), (300, 128, "special"),
                                      (257, 11008, "outlier"), (1000, 4096, "normal"), (64, 1024, "tiny")])
def test_quantize_bitexact(n, k, dist):
    B = _dev()
    _say("f16 quantize", n, k, dist)
    w = _weight(n, k, dist, n * 13 + k)
    q = B.qlora_quantize(_t(w), B.device_codebook())
    assert q.dtype == torch.float16
    torch.cuda.synchronize()
    c, qs, st, wd = _oracle(w)
    cs, qss = onf4.to_storage(c, qs, n, k)
    assert np.array_equal(q.codes.cpu().numpy(), cs)
    assert np.array_equal(q.qscale.cpu().numpy(), qss)
    assert np.array_equal(q.step.cpu().numpy().view(np.uint32), st.view(np.uint32))
    d = B.qlora_dequantize(q, B.device_codebook())
    torch.cuda.synchronize()
    assert d.dtype == torch.float16
    _same(_bits(d), wd, ("dequant", n, k, dist))
    if dist == "tiny":
        sub = (wd & 0x7C00) == 0
        assert np.count_nonzero(sub & ((wd & 0x3FF) != 0)) > 1000   # subnormal outputs exercised


@pytest.mark.parametrize("path", ["gemm", "gemv"])
@pytest.mark.parametrize("dist", ["special", "tiny"])
def test_fused_identity_fwd(path, dist):
    B = _dev()
    n, k = 200, 512
    w = _weight(n, k, dist, 97)
    q = B.qlora_quantize(_t(w), B.device_codebook())
    wd = onf4.f16_to_f32(_oracle(w)[3])
    for r0 in (range(0, k, 32) if path == "gemv" else [0]):
        m = 32 if path == "gemv" else k
        eye = np.zeros((m, k), dtype=np.float32)
        eye[np.arange(m), r0 + np.arange(m)] = 1.0
        X = torch.from_numpy(eye).to(torch.float16).cuda()
        Y, _ = B.qlora_linear_fwd(q, B.device_codebook(), X, path=path)
        torch.cuda.synchronize()
        _same(Y.cpu().numpy(), wd[:, r0:r0 + m].T, (path, dist, r0))


@pytest.mark.parametrize("n,k", [(300, 384), (200, 640)])
def test_fused_identity_dx(n, k):
    B = _dev()
    w = _weight(n, k, "outlier", 98 + n)
    q = B.qlora_quantize(_t(w), B.device_codebook())
    wd = onf4.f16_to_f32(_oracle(w)[3])
    dY = torch.eye(n, dtype=torch.float16).cuda()
    dX, _, _ = B.qlora_linear_bwd(q, B.device_codebook(), None, dY)
    torch.cuda.synchronize()
    _same(dX.cpu().numpy(), wd, (n, k))


CASES = [(1, 4096, 4096, 8, "gemv"), (16, 4096, 4096, 8, "gemv"), (17, 257, 320, 16, "gemv"),
         (16, 4096, 4096, 8, "gemm"), (130, 300, 512, 16, "gemm"), (257, 513, 640, 64, "gemm"),
         (512, 1024, 1024, 8, "auto"), (1024, 512, 2048, 64, "auto"), (2048, 4096, 4096, 8, "auto")]


@pytest.mark.parametrize("M,N,K,r,path", CASES)
def test_linear_parity(M, N, K, r, path):
    """Forward (Y, T) and backward (dX, dA, dB) in fp32 against the oracle;
    the small-M cases run the split-K and split-dX reductions, the r = 64
    cases the split rank projections and the two-tile adapter gradients."""
    B = _dev()
    _say("f16 linear", M, N, K, r, path)
    s = 2.0
    cb = B.device_codebook()
    X, W, A, Bm, dY = _inputs(M, N, K, r, seed=M + 5 * N + K + r)
    q = B.qlora_quantize(_t(W), cb)
    Xd, Ad, Bd, dYd = _t(X), _t(A), _t(Bm), _t(dY)
    Y, T = B.qlora_linear_fwd(q, cb, Xd, Ad, Bd, s, path=path)
    dX, dA, dB = B.qlora_linear_bwd(q, cb, Xd, dYd, Ad, Bd, s, T=T)
    torch.cuda.synchronize()
    Wd = _oracle(W)[3]
    ms = np.arange(M) if M <= 512 else np.sort(synth.rng(6).choice(M, 48, replace=False))
    Yo, To = olin.forward(Wd, X[ms], A, Bm, s, dtype=F16)
    assert _rel(Y.cpu().numpy()[ms], Yo) <= REL_TOL
    assert _rel(T.cpu().numpy()[ms], To) <= REL_TOL
    dXo = olin.backward(Wd, X[ms], dY[ms], A, Bm, s, dtype=F16)[0]
    assert _rel(dX.cpu().numpy()[ms], dXo) <= REL_TOL
    if M <= 1024:
        _, dAo, dBo = olin.backward(Wd, X, dY, A, Bm, s, dtype=F16)
        assert _rel(dA.cpu().numpy(), dAo) <= REL_TOL
        assert _rel(dB.cpu().numpy(), dBo) <= REL_TOL


@pytest.mark.parametrize("M,N,K,r", [(16, 4096, 4096, 8), (5, 1024, 8192, 24), (32, 2048, 4096, 64)])
def test_small_m_recomputed_t_bit_identical(M, N, K, r):
    """fp16 operands on the small-m streaming path (path AUTO), where T and U
    are formed inside the split reduces.  A backward given no T forms T again,
    one row per workgroup in the same summation order, so its dX, dA and dB
    equal, byte for byte, those of the backward given the saved T; both
    against the oracle in fp32."""
    B = _dev()
    _say("f16 recomputed T", M, N, K, r)
    s = 2.0
    cb = B.device_codebook()
    X, W, A, Bm, dY = _inputs(M, N, K, r, seed=7 * M + N + K + r)
    q = B.qlora_quantize(_t(W), cb)
    Xd, Ad, Bd, dYd = _t(X), _t(A), _t(Bm), _t(dY)
    Y, T = B.qlora_linear_fwd(q, cb, Xd, Ad, Bd, s)
    dX, dA, dB = B.qlora_linear_bwd(q, cb, Xd, dYd, Ad, Bd, s, T=T)
    dXr, dAr, dBr = B.qlora_linear_bwd(q, cb, Xd, dYd, Ad, Bd, s)
    torch.cuda.synchronize()
    assert torch.equal(dX, dXr) and torch.equal(dA, dAr) and torch.equal(dB, dBr)
    Wd = _oracle(W)[3]
    Yo, To = olin.forward(Wd, X, A, Bm, s, dtype=F16)
    dXo, dAo, dBo = olin.backward(Wd, X, dY, A, Bm, s, dtype=F16)
    for got, ref in [(Y, Yo), (T, To), (dX, dXo), (dA, dAo), (dB, dBo)]:
        assert _rel(got.cpu().numpy(), ref) <= REL_TOL


@pytest.mark.parametrize("M,path", [(16, "gemv"), (200, "gemm")])
def test_lora_only(M, path):
    """W = 0 isolates the adapter terms of Y and dX."""
    B = _dev()
    N, K, r, s = 384, 512, 16, 2.0
    X, _, A, Bm, dY = _inputs(M, N, K, r, seed=5)
    W = np.zeros((N, K), dtype=np.uint16)
    cb = B.device_codebook()
    q = B.qlora_quantize(_t(W), cb)
    Y, T = B.qlora_linear_fwd(q, cb, _t(X), _t(A), _t(Bm), s, path=path)
    dX, _, _ = B.qlora_linear_bwd(q, cb, _t(X), _t(dY), _t(A), _t(Bm), s, T=T)
    torch.cuda.synchronize()
    Wd = _oracle(W)[3]
    assert _rel(Y.cpu().numpy(), olin.forward(Wd, X, A, Bm, s, dtype=F16)[0]) <= REL_TOL
    assert _rel(dX.cpu().numpy(), olin.backward(Wd, X, dY, A, Bm, s, dtype=F16)[0]) <= REL_TOL


def test_f16_outputs_within_one_ulp():
    """fp16 outputs are the fp32 results rounded once: within one fp16 ulp of
    themselves plus the fp32 accumulation bound of the exact value."""
    B = _dev()
    M, N, K, r, s = 32, 512, 1024, 8, 2.0
    X, W, A, Bm, dY = _inputs(M, N, K, r, seed=9)
    cb = B.device_codebook()
    q = B.qlora_quantize(_t(W), cb)
    Wd = _oracle(W)[3]
    Yo, To = olin.forward(Wd, X, A, Bm, s, dtype=F16)
    f = lambda b: np.abs(onf4.f16_to_f32(b).astype(np.float64))
    gamma = (K + r) * 2.0 ** -24 * (f(X) @ f(Wd).T + s * np.abs(To) @ f(Bm).T)
    for path in ("gemv", "gemm"):
        Y, _ = B.qlora_linear_fwd(q, cb, _t(X), _t(A), _t(Bm), s, y_dtype=torch.float16, path=path)
        torch.cuda.synchronize()
        y = Y.float().cpu().numpy().astype(np.float64)
        ulp = np.spacing(np.abs(y).astype(np.float16)).astype(np.float64)
        assert np.all(np.abs(y - Yo) <= ulp + gamma), path
    dX, _, _ = B.qlora_linear_bwd(q, cb, _t(X), _t(dY), _t(A), _t(Bm), s, dx_dtype=torch.float16)
    torch.cuda.synchronize()
    dXo = olin.backward(Wd, X, dY, A, Bm, s, dtype=F16)[0]
    U = f(dY) @ f(Bm)
    gdx = (N + r) * 2.0 ** -24 * (f(dY) @ f(Wd) + s * U @ f(A))
    x = dX.float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(x - dXo) <= np.spacing(np.abs(x).astype(np.float16)).astype(np.float64) + gdx)


@pytest.mark.parametrize("M", [1, 16])
def test_grouped_forward(M):
    B = _dev()
    cb = B.device_codebook()
    jobs, ref = [], []
    for i, (N, K, r) in enumerate([(4096, 4096, 8), (300, 384, 0), (257, 11008, 8), (64, 128, 0)]):
        X, W, A, Bm, _ = _inputs(M, N, K, r, seed=700 + M + 13 * i)
        q = B.qlora_quantize(_t(W), cb)
        j = dict(w=q, X=_t(X), Y=torch.full((M, N), float("nan"), device="cuda"))
        if r:
            j.update(A=_t(A), B=_t(Bm), scaling=2.0, T=torch.full((M, r), float("nan"), device="cuda"))
        jobs.append(j)
        ref.append((W, X, A if r else None, Bm if r else None))
    g = B.qlora_group_init(jobs, M, y_dtype=torch.float32)
    B.qlora_linear_fwd_grouped(g, cb)
    torch.cuda.synchronize()
    for j, (W, X, A, Bm) in zip(jobs, ref):
        Yo, _ = olin.forward(_oracle(W)[3], X, A, Bm, 2.0, dtype=F16)
        assert _rel(j["Y"].cpu().numpy(), Yo) <= REL_TOL


@pytest.mark.parametrize("N,K,r", [(300, 512, 8), (1024, 2048, 64)])
def test_merge_and_requantize(N, K, r):
    """Merged fp16 weight bit-exact against the merge oracle; requantized
    arrays bit-exact against the fp16 quantizer of the merged weight."""
    B = _dev()
    s = 2.0
    W = synth.normal_f16((N, K), 0.02, N + K + r)
    A = synth.normal_f16((r, K), 0.01, N + K + r + 1)
    Bm = synth.normal_f16((N, r), 0.01, N + K + r + 2)
    cb = B.device_codebook()
    q = B.qlora_quantize(_t(W), cb)
    out = B.NF4Weight.empty(N, K, "cuda", dtype=torch.float16)
    M, out = B.qlora_merge(q, cb, _t(A), _t(Bm), s, out=out)
    torch.cuda.synchronize()
    Mo = omerge.merged_weight(_oracle(W)[3], A, Bm, s, dtype=F16)
    _same(_bits(M).astype(np.int64), Mo.astype(np.int64), ("merged", N, K, r))
    c, qs, st = onf4.quantize(Mo, MID, dtype=F16)
    cs, qss = onf4.to_storage(c, qs, N, K)
    assert np.array_equal(out.codes.cpu().numpy(), cs)
    assert np.array_equal(out.qscale.cpu().numpy(), qss)
    assert np.array_equal(out.step.cpu().numpy().view(np.uint32), st.view(np.uint32))


def test_same_bytes_as_bf16_on_common_values():
    """A weight exact in both types packs to the same bytes from either."""
    B = _dev()
    n, k = 256, 1024
    ints = synth.rng(11).integers(-255, 256, size=(n, k)).astype(np.float32) * np.float32(2.0 ** -12)
    b16 = torch.from_numpy(ints).to(torch.bfloat16).cuda()
    h16 = torch.from_numpy(ints).to(torch.float16).cuda()
    cb = B.device_codebook()
    qb, qh = B.qlora_quantize(b16, cb), B.qlora_quantize(h16, cb)
    torch.cuda.synchronize()
    assert torch.equal(qb.codes, qh.codes) and torch.equal(qb.qscale, qh.qscale)
    assert torch.equal(qb.step.view(torch.int32), qh.step.view(torch.int32))


def test_quantize_quotients_near_decision_midpoints():
    """fp16 blocks whose elements sit a few fp16 ulps around absmax * midpoint
    for every midpoint, over absmax values across the fp16 exponent range
    (subnormal elements included): the kernel's quotient (reciprocal and one
    fma correction, argued exact for 11-bit significands) must round exactly as
    binary32 division does, so the codes match the oracle bit for bit."""
    B = _dev()
    g = np.random.default_rng(2025)
    nblk = 32768
    exps = g.integers(1, 31, nblk)                  # every normal fp16 binade
    mants = g.integers(0, 1024, nblk)
    a_bits = ((exps << 10) | mants).astype(np.uint16)
    a = onf4.f16_to_f32(a_bits).astype(np.float64)
    blocks = np.empty((nblk, 64), dtype=np.uint16)
    blocks[:, 0] = a_bits
    for j in range(1, 64):
        k = (j - 1) % 15
        off = (j - 1) // 15 - 2                      # -2 .. 2 fp16 ulps around the target
        tgt = onf4.f32_to_f16_rne((a * MID.astype(np.float64)[k]).astype(np.float32))
        sgn = tgt & 0x8000
        mag = np.clip((tgt & 0x7FFF).astype(np.int32) + off, 0, 0x7BFF)
        blocks[:, j] = (sgn | mag).astype(np.uint16)
    xf = np.abs(onf4.f16_to_f32(blocks).astype(np.float64))
    over = xf > a[:, None]
    blocks[over] = (blocks[over] & 0x8000) | np.repeat(a_bits[:, None], 64, axis=1)[over]
    w = blocks.reshape(2048, 1024)
    q = B.qlora_quantize(_t(w), B.device_codebook())
    torch.cuda.synchronize()
    c, qs, st, _ = _oracle(w)
    cs, qss = onf4.to_storage(c, qs, 2048, 1024)
    assert np.array_equal(q.codes.cpu().numpy(), cs)
    assert np.array_equal(q.qscale.cpu().numpy(), qss)
