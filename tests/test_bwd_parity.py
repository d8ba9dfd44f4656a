"""GPU parity of the backward kernels (fa_bwd) against the fp64 oracle, through the C ABI.

The GPU backward takes O and LSE from the GPU forward (its real inputs); the oracle
computes the exact gradients of the forward's definition from Q, K, V and dO alone.
Tolerance (tests.parity.check_grad): per element 1e-2 plus half a bf16 spacing at the exact
value plus k 2^-8 times the element's sensitivity to the k bf16 roundings of one factor of
every product term (and of O inside D = dO . O); per tensor, rel-L2 4e-3 plus twice the
expected RMS of those roundings. The full-size workloads are checked element by element in
test_full_parity.py.
"""
import math

import numpy as np
import pytest
import torch

from oracle.attention import attention_bwd_ref, widen_bf16
from synth import make_grad_out, make_qkv
from tests.parity import check_grad, down, up

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import io_aware_exact_21_amd as fa
    return fa


def _gpu_bwd(fa, q, k, v, do, causal, scale):
    tq, tk, tv, tdo = up(q), up(k), up(v), up(do)
    o, lse = fa.fwd(tq, tk, tv, causal=causal, scale=scale)
    dq, dk, dv = fa.bwd(tq, tk, tv, o, lse, tdo, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return dq, dk, dv


def _check(dq, dk, dv, ref):
    gq, gk, gv, aq, ak, av, rq, rk, rv = ref
    info = (check_grad(down(dq), gq, aq, rq, "dQ"), check_grad(down(dk), gk, ak, rk, "dK"),
            check_grad(down(dv), gv, av, rv, "dV"))
    print("  dQ/dK/dV:", [{k: round(v, 5) for k, v in i.items()} for i in info], flush=True)
    return info


SMALL = [
    # B, Hq, Hkv, Sq, Skv, d
    (1, 1, 1, 1, 1, 64), (1, 2, 2, 7, 7, 128), (1, 2, 2, 200, 200, 128), (2, 4, 2, 130, 257, 64),
    (1, 4, 1, 96, 64, 128), (1, 2, 2, 64, 300, 128), (1, 8, 2, 257, 257, 128), (2, 2, 1, 300, 129, 64),
    (1, 3, 3, 129, 129, 64), (1, 2, 1, 5, 70, 128),
    # d = 128 dQ workgroups of 2, 6 and 8 key tiles (ring depth 4, the last tiles without barriers)
    (1, 2, 2, 100, 100, 128), (1, 2, 1, 383, 383, 128), (1, 2, 2, 190, 450, 128),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SMALL, ids=[str(s) for s in SMALL])
def test_small_shapes(fa, shape, causal):
    B, Hq, Hkv, Sq, Skv, d = shape
    seed = 500 + Sq + 7 * Skv + d
    print(f"case {shape} causal={causal}", flush=True)
    q, k, v = make_qkv(B, Hq, Hkv, Sq, Skv, d, seed=seed)
    do = make_grad_out(B, Sq, Hq, d, seed)
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv = _gpu_bwd(fa, q, k, v, do, causal, scale)
    ref = attention_bwd_ref(widen_bf16(q), widen_bf16(k), widen_bf16(v), widen_bf16(do), causal=causal,
                            scale=scale, abs_terms=True)
    _check(dq, dk, dv, ref)


@pytest.mark.parametrize("scale", [-0.3, 0.0, 0.25])
def test_scale_sign_and_zero(fa, scale):
    B, Hq, Hkv, Sq, Skv, d = 1, 4, 2, 150, 150, 128
    q, k, v = make_qkv(B, Hq, Hkv, Sq, Skv, d, seed=77)
    do = make_grad_out(B, Sq, Hq, d, 77)
    dq, dk, dv = _gpu_bwd(fa, q, k, v, do, True, scale)
    ref = attention_bwd_ref(widen_bf16(q), widen_bf16(k), widen_bf16(v), widen_bf16(do), causal=True,
                            scale=scale, abs_terms=True)
    _check(dq, dk, dv, ref)
    if scale == 0.0:
        assert torch.count_nonzero(dq) == 0 and torch.count_nonzero(dk) == 0


def test_deterministic(fa):
    q, k, v = make_qkv(1, 4, 2, 333, 333, 128, seed=78)
    do = make_grad_out(1, 333, 4, 128, 78)
    a = _gpu_bwd(fa, q, k, v, do, True, 128 ** -0.5)
    b = _gpu_bwd(fa, q, k, v, do, True, 128 ** -0.5)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
