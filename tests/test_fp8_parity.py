"""GPU parity of the fp8 (e4m3) forward (fa_fwd_fp8) against the fp64 oracle, through the C ABI.

The oracle is exact attention on the dequantised inputs (attention_fp8_ref). The kernel
rounds P to e4m3 before the P.V product (its normaliser sums the unrounded p), so the
tolerance is derived from that rounding rather than taken from the bf16 bar:
  * a normal e4m3 value is within 2^-4 of p (relative); below 2^-6 the error is
    absolute, at most 2^-10 in units where the row's largest p is >= 1;
  * so per element |O - O_ref| <= 1e-2 + half a bf16 spacing + 2^-4 A + Bs with
    A = sum_j P_ij |V_j| and Bs = sum_j min(P_ij, 2^-10 Pmax_i) |V_j|;
  * per tensor, twice the expected RMS of those roundings (uniform errors, RMS 1/sqrt 3 of
    their bound): ||err|| <= 4e-3 ||O|| + (2 / sqrt 3) (2^-4 ||R|| + ||Rs||) with
    R = (sum_j P_ij^2 V_j^2)^(1/2) and Rs = (sum_j min(P_ij, 2^-10 Pmax_i)^2 V_j^2)^(1/2);
  * LSE (unrounded normaliser): max-abs 1e-2 and rel-L2 4e-3 as for bf16.
The sensitivities A, Bs, R, Rs are computed here from the dequantised inputs.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle.attention import attention_fp8_ref, e4m3_value, kv_head_of
from synth import WORKLOADS
from synth.fp8 import make_fp8_qkv, quantize_heads, v_transposed
from oracle import fullcheck as fc
from tests.parity import check_lse

pytestmark = pytest.mark.gpu
U8 = fc.FP8_P_ROUNDING


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import io_aware_exact_21_amd as fa
    return fa


def _dequant(q8, k8, vt8, qs, ks, vs, Skv):
    Q = e4m3_value(q8) * qs.astype(np.float64)[:, None, :, None]
    K = e4m3_value(k8) * ks.astype(np.float64)[:, None, :, None]
    V = e4m3_value(vt8[..., :Skv]).transpose(0, 3, 1, 2) * vs.astype(np.float64)[:, None, :, None]
    return Q, K, V


def _sensitivities(q_rows, K, V, rows, Sq, causal, scale):
    """A, Bs, R, Rs [n, d] for query rows ``rows`` of one head (see module docstring)."""
    return fc.fp8_sensitivities(q_rows, K, V, rows, Sq, causal, scale)


def _check(o, O, A, Bs, R, Rs, what="O(fp8)"):
    err = np.abs(o - O)
    bound = fc.fp8_bound(O, A, Bs)
    worst = np.unravel_index(np.argmax(err / bound), err.shape)
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    assert (err <= bound).all(), (f"{what}: |err| {err[worst]:.4e} > bound {bound[worst]:.4e} at {worst} "
                                  f"(gpu {o[worst]}, ref {O[worst]})")
    nO = np.linalg.norm(O)
    rel = np.linalg.norm(o - O) / nO
    rel_bound = 4e-3 + 2.0 / math.sqrt(3.0) * (U8 * np.linalg.norm(R) + np.linalg.norm(Rs)) / nO
    assert rel <= rel_bound, f"{what}: rel-L2 {rel:.3e} > {rel_bound:.3e}"
    return {"max_abs": float(err.max()), "max_err_over_bound": float((err / bound).max()), "rel_l2": float(rel),
            "rel_l2_bound": float(rel_bound)}


def _gpu(fa, q8, k8, vt8, qs, ks, vs, causal, scale):
    dev = "cuda"
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    o, lse = fa.fwd_fp8(to(q8), to(k8), to(vt8), to(qs), to(ks), to(vs), causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


SMALL = [
    # B, Hq, Hkv, Sq, Skv, d
    (1, 1, 1, 1, 1, 64), (1, 2, 2, 7, 7, 128), (1, 2, 1, 200, 200, 128), (2, 4, 2, 130, 257, 64),
    (1, 4, 1, 300, 100, 128), (1, 2, 2, 64, 333, 128), (1, 8, 2, 257, 257, 128), (2, 2, 1, 100, 190, 64),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SMALL, ids=[str(s) for s in SMALL])
def test_small_shapes(fa, shape, causal):
    B, Hq, Hkv, Sq, Skv, d = shape
    print(f"case {shape} causal={causal}", flush=True)
    q8, k8, vt8, qs, ks, vs, ldv = make_fp8_qkv(B, Hq, Hkv, Sq, Skv, d, seed=700 + Sq + 3 * Skv + d,
                                                k_stress_frac=0.02)
    scale = 1.0 / math.sqrt(d)
    o, lse = _gpu(fa, q8, k8, vt8, qs, ks, vs, causal, scale)
    O, L = attention_fp8_ref(q8, k8, vt8, qs, ks, vs, causal=causal, scale=scale)
    Q, K, V = _dequant(q8, k8, vt8, qs, ks, vs, Skv)
    sens = [np.zeros((B, Sq, Hq, d)) for _ in range(4)]
    for b in range(B):
        for h in range(Hq):
            hk = kv_head_of(h, Hq, Hkv)
            for x, y in zip(sens, _sensitivities(Q[b, :, h], K[b, :, hk], V[b, :, hk], np.arange(Sq), Sq, causal,
                                                 scale)):
                x[b, :, h] = y
    info = _check(o, O, *sens)
    check_lse(lse, L)
    print("  ", info, flush=True)


@pytest.mark.parametrize("causal", [False, True])
def test_late_max_jumps(fa, causal):
    """Row maxima that jump far above the running max inside the unmasked tiles, where the
    kernel first tries the max-free step; the lane sums exceed its bound there and the full
    step reruns on the same scores. Head 0 jumps at keys 700 and 960, head 1 at key 896."""
    rng = np.random.default_rng(74)
    B, S, H, d = 1, 1024, 2, 128
    q = 1.0 + 0.3 * rng.standard_normal((B, S, H, d))       # every row points the same way
    k = 0.3 * rng.standard_normal((B, S, H, d))
    v = rng.standard_normal((B, S, H, d))
    k[0, 700, 0, :] = 3.0                                     # about 49 powers of two up
    k[0, 960, 0, :] = 6.0                                     # another 49
    k[0, 896, 1, :] = 6.0
    q8, qs = quantize_heads(q)
    k8, ks = quantize_heads(k)
    v8, vs = quantize_heads(v)
    vt8, _ = v_transposed(v8)
    scale = 1.0 / math.sqrt(d)
    o, lse = _gpu(fa, q8, k8, vt8, qs, ks, vs, causal, scale)
    O, L = attention_fp8_ref(q8, k8, vt8, qs, ks, vs, causal=causal, scale=scale)
    Q, K, V = _dequant(q8, k8, vt8, qs, ks, vs, S)
    sens = [np.zeros((B, S, H, d)) for _ in range(4)]
    for h in range(H):
        for x, y in zip(sens, _sensitivities(Q[0, :, h], K[0, :, h], V[0, :, h], np.arange(S), S, causal, scale)):
            x[0, :, h] = y
    _check(o, O, *sens)
    check_lse(lse, L)


@pytest.mark.parametrize("scale", [-0.2, 0.0])
def test_scale_sign_and_zero(fa, scale):
    q8, k8, vt8, qs, ks, vs, ldv = make_fp8_qkv(1, 4, 2, 150, 150, 128, seed=71)
    o, lse = _gpu(fa, q8, k8, vt8, qs, ks, vs, True, scale)
    O, L = attention_fp8_ref(q8, k8, vt8, qs, ks, vs, causal=True, scale=scale)
    Q, K, V = _dequant(q8, k8, vt8, qs, ks, vs, 150)
    sens = [np.zeros((1, 150, 4, 128)) for _ in range(4)]
    for h in range(4):
        for x, y in zip(sens, _sensitivities(Q[0, :, h], K[0, :, h // 2], V[0, :, h // 2], np.arange(150), 150,
                                             True, scale)):
            x[0, :, h] = y
    _check(o, O, *sens)
    check_lse(lse, L)


def test_deterministic(fa):
    q8, k8, vt8, qs, ks, vs, ldv = make_fp8_qkv(1, 4, 2, 333, 333, 128, seed=72)
    a = _gpu(fa, q8, k8, vt8, qs, ks, vs, True, 128 ** -0.5)
    b = _gpu(fa, q8, k8, vt8, qs, ks, vs, True, 128 ** -0.5)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_full_size_long_prefill_every_element(fa):
    """fp8 version of the MHA long prefill (B2 H32 S8192 d128 causal, K x4 on 1% of
    positions) in the launch configuration the benchmark times: every element of O and
    LSE against the oracle on the dequantised inputs (oracle.fullcheck.check_fp8)."""
    w = WORKLOADS["mha8k"]
    q8, k8, vt8, qs, ks, vs, ldv = make_fp8_qkv(w.B, w.Hq, w.Hkv, w.Sq, w.Skv, w.d, w.seed, w.k_stress_frac)
    print(f"full-size fp8 {w.name}", flush=True)
    o, lse = _gpu(fa, q8, k8, vt8, qs, ks, vs, True, w.scale)
    res = fc.check_fp8(q8, k8, vt8, qs, ks, vs, o, lse, causal=True, scale=w.scale,
                       progress=lambda m: print("  ", m, flush=True))
    print("  ", res, flush=True)
    path = os.environ.get("FA_PARITY_REPORT")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"workload": "e4m3 " + w.name, "label": "pass" if fc.fp8_ok(res) else "fail",
                                "fp8": res}) + "\n")
    assert fc.fp8_ok(res), res
