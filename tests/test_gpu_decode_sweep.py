"""GPU parity of the decode sweep at its full size, in the launch configuration
the decode workload times: 32 layers x the seven 7B-style projections (q, k,
v, o 4096 x 4096; gate, up 11008 x 4096; down 4096 x 11008), 6.48e9 NF4 +
double-quantized weights (3.34 GB packed) resident at once, LoRA r = 8, s = 2
on q, k, v, o, covered by ONE grouped forward launch per sweep at m = 1, 4
and 16 (kwkr.cn/news/627310 §1.2: a generated token reads every weight
once).

The oracle checks sampled projections (first, middle and last layers, each
shape, with and without LoRA) in full: packed codes and scales bit-exact, Y and T by relative
Frobenius error <= 2e-3 in fp32.  Every other projection of the sweep is
checked against the single-projection streaming call on the same inputs
(same kernel family, so a grouped-launch job-mapping mistake -- a workgroup
reading another job's weight, activations or outputs -- shows there).
"""
import sys

import numpy as np
import pytest
import torch

import synth
from oracle import linear as olin
from oracle import nf4 as onf4

pytestmark = pytest.mark.gpu

REL_TOL = 2e-3
LAYERS = 32
# (name, out_features n, in_features k, LoRA rank)
PROJ = [("q", 4096, 4096, 8), ("k", 4096, 4096, 8), ("v", 4096, 4096, 8), ("o", 4096, 4096, 8),
        ("gate", 11008, 4096, 0), ("up", 11008, 4096, 0), ("down", 4096, 11008, 0)]
SCALING = 2.0
# (layer, projection index) pairs checked against the oracle
SAMPLED = [(0, 0), (15, 4), (16, 3), (31, 6)]


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _rel(a, ref):
    ref = np.asarray(ref, dtype=np.float64)
    num = np.linalg.norm(np.asarray(a, dtype=np.float64) - ref)
    den = np.linalg.norm(ref)
    return num / den if den > 0 else num


@pytest.fixture(scope="module")
def sweep():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from qlora_fine_tuning_nf4_amd import binding as B
    B.lib()
    cb = B.device_codebook()
    weights, kept = [], {}
    for layer in range(LAYERS):
        for i, (name, n, k, r) in enumerate(PROJ):
            W = synth.device_normal_bf16((n, k), 0.02, synth.tensor_seed(3, 100 * layer + 10 * i))
            q = B.qlora_quantize(W, cb)
            if (layer, i) in SAMPLED:
                kept[(layer, i)] = _bits(W)
            weights.append((layer, i, q, n, k, r))
            del W
    torch.cuda.synchronize()
    _say("decode sweep: quantized", len(weights), "projections,",
         sum(q.nbytes() for _, _, q, *_ in weights), "packed bytes")
    # the oracle's quantization of each sampled projection, and its dequantized
    # bf16 weight, computed once
    lv, mid = onf4.codebook()
    oracle = {}
    for key, w_bits in kept.items():
        c, qs, st = onf4.quantize(w_bits, mid)
        oracle[key] = (c, qs, st, onf4.dequantize(c, qs, st, lv).reshape(w_bits.shape))
    del kept
    yield B, cb, weights, oracle


def test_sweep_quantized_bitexact_on_sampled(sweep):
    B, cb, weights, oracle = sweep
    for layer, i, q, n, k, r in weights:
        if (layer, i) not in oracle:
            continue
        c, qs, st, _ = oracle[(layer, i)]
        cst, qst = onf4.to_storage(c, qs, n, k)
        assert np.array_equal(q.codes.cpu().numpy(), cst), (layer, i)
        assert np.array_equal(q.qscale.cpu().numpy(), qst), (layer, i)
        assert np.array_equal(q.step.cpu().numpy().view(np.uint32), st.view(np.uint32)), (layer, i)


@pytest.mark.parametrize("M", [1, 4, 16])
def test_sweep_one_grouped_launch(sweep, M):
    B, cb, weights, oracle = sweep
    _say("decode sweep, one grouped launch, m =", M)
    jobs, inputs = [], []
    for idx, (layer, i, q, n, k, r) in enumerate(weights):
        X = synth.device_normal_bf16((M, k), 1.0, synth.tensor_seed(3, 20000 + idx))
        j = dict(w=q, X=X, Y=torch.full((M, n), float("nan"), device="cuda"))
        if r:
            j.update(A=synth.device_normal_bf16((r, k), 0.01, synth.tensor_seed(3, 40000 + idx)),
                     B=synth.device_normal_bf16((n, r), 0.01, synth.tensor_seed(3, 60000 + idx)),
                     scaling=SCALING, T=torch.full((M, r), float("nan"), device="cuda"))
        jobs.append(j)
        inputs.append((layer, i, n, k, r))
    g = B.qlora_group_init(jobs, M, y_dtype=torch.float32)
    B.qlora_linear_fwd_grouped(g, cb)
    torch.cuda.synchronize()

    worst = 0.0
    for j, (layer, i, n, k, r) in zip(jobs, inputs):
        Y = j["Y"]
        assert not torch.isnan(Y).any(), (layer, i)
        # the same projection through the single-projection streaming call
        Ys, Ts = B.qlora_linear_fwd(j["w"], cb, j["X"], j.get("A"), j.get("B"), SCALING if r else 0.0,
                                    path="gemv")
        d = _rel(Y.cpu().numpy(), Ys.cpu().numpy())
        worst = max(worst, d)
        assert d <= 1e-5, (layer, i, d)
        if r:
            assert _rel(j["T"].cpu().numpy(), Ts.cpu().numpy()) <= 1e-5, (layer, i)
        if (layer, i) in oracle:
            Wd = oracle[(layer, i)][3]
            A = _bits(j["A"]) if r else None
            Bm = _bits(j["B"]) if r else None
            Yo, To = olin.forward(Wd, _bits(j["X"]), A, Bm, SCALING)
            err = _rel(Y.cpu().numpy(), Yo)
            _say(f"  layer {layer} {PROJ[i][0]} ({n} x {k}) rel_fro(Y) = {err:.3e}")
            assert err <= REL_TOL, (layer, i, err)
            if r:
                assert _rel(j["T"].cpu().numpy(), To) <= REL_TOL
    _say(f"  grouped vs single calls, worst relative difference {worst:.2e}")
    del g, jobs
