"""GPU check of the adapter-gradient reduction folded into the input-gradient
GEMM (the split partials of dA = s U^T X and dB = s dY^T T added up by the GEMM's
producer waves instead of a reduction launch of their own).

Both routes add the same partials in the same split order, so dA and dB from
a backward that computes dX on the tiled GEMM path (folded) equal those of
the same backward without dX (own reduction launch) bit for bit.  Shapes:
ragged m and n, r = 12 (not a multiple of 8: U through a transposed copy),
r = 64 (one 64-rank tile) and r = 128 (two), a grid with fewer producer threads than outputs
(the fold loops), fp16 compute, 7B projections at m = 2048 and 4096, and B
not 16-byte aligned (U through a transposed copy).  Agreement with the
oracle is covered by the backward parity tests, which run the folded route
at these sizes.
"""
import sys

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from qlora_fine_tuning_nf4_amd import binding
    binding.lib()
    return binding


def _t(bits, f16=False):
    dt = torch.float16 if f16 else torch.bfloat16
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(dt).cuda()


# (m, n, k, r, fp16, B offset in elements): n < 128 or enough tiles keep the
# GEMM at one split
CASES = [(600, 100, 384, 16, False, 0), (600, 120, 320, 24, False, 0), (600, 100, 384, 12, False, 0), (600, 100, 384, 64, False, 0),
         (600, 100, 384, 16, True, 0), (1500, 4096, 4096, 8, False, 0), (2048, 11008, 4096, 64, False, 0),
         (2048, 4096, 4096, 8, False, 0), (2048, 4096, 4096, 8, False, 1), (4096, 4096, 4096, 8, False, 0),
         (600, 100, 384, 128, False, 0), (2048, 4096, 4096, 128, False, 0)]


@pytest.mark.parametrize("m,n,k,r,f16,boff", CASES)
def test_folded_wgrad_reduction_matches_own_launch(m, n, k, r, f16, boff):
    B = _dev()
    print("wgrad fold", m, n, k, r, f16, boff, file=sys.stderr, flush=True)
    seed = m + 3 * n + 7 * k + r
    gen = synth.normal_f16 if f16 else synth.normal_bf16
    X = _t(gen((m, k), 1.0, seed), f16)
    W = _t(gen((n, k), 0.02, seed + 1), f16)
    A = _t(gen((r, k), 0.01, seed + 2), f16)
    Bm = _t(gen((n, r), 0.01, seed + 3), f16)
    if boff:   # the same values at an address 2 bytes past a 16-byte boundary
        buf = torch.empty(n * r + boff, dtype=Bm.dtype, device=Bm.device)
        buf[boff:] = Bm.reshape(-1)
        Bm = buf[boff:].view(n, r)
        assert Bm.data_ptr() % 16 != 0
    dY = _t(gen((m, n), 1.0, seed + 4), f16)
    cb = B.device_codebook()
    q = B.qlora_quantize(W, cb)
    dX, dA, dB = B.qlora_linear_bwd(q, cb, X, dY, A, Bm, 2.0, path="gemm")
    _, dA0, dB0 = B.qlora_linear_bwd(q, cb, X, dY, A, Bm, 2.0, need_dX=False, path="gemm")
    torch.cuda.synchronize()
    assert torch.isfinite(dX).all()
    assert torch.equal(dA, dA0), (dA - dA0).abs().max().item()
    assert torch.equal(dB, dB0), (dB - dB0).abs().max().item()
    assert dA.abs().sum().item() > 0 and dB.abs().sum().item() > 0
