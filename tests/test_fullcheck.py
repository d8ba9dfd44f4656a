"""The whole-tensor stated check (oracle/fullcheck.py) on the CPU: its statistics, its
pass / floor-limited / fail labels, and its process-pool drivers on small cases with
outputs derived from the oracle itself (the correctly rounded answer must pass; a
planted error must fail)."""
import numpy as np
import pytest

from oracle import fullcheck as fc
from oracle.attention import attention_ref, decode_ref, widen_bf16
from synth import bf16_rne_bits, make_qkv


def test_bf16_rounding_matches_the_input_recipe():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(20000) * np.exp2(rng.integers(-20, 20, 20000))
    np.testing.assert_array_equal(fc.bf16_rne(x), widen_bf16(bf16_rne_bits(x)))
    assert fc.bf16_ulp(np.array([1.0, 1.5, 4.0, 5.9, -0.3]))[2] == 2.0 ** -5
    assert fc.bf16_ulp(np.array([1.0]))[0] == 2.0 ** -7


def _summ(o, ref, lse=None, lref=None):
    return fc.summarise(fc.o_stats(o, ref), None if lse is None else fc.lse_stats(lse, lref))


def test_labels():
    ref = np.array([[5.3, 0.1, -0.7], [0.2, 0.3, 0.4]])
    L = np.array([1.0, -np.inf])
    good = _summ(ref + 1e-3, ref, L, L)
    assert fc.label(good, None) == "pass"
    rounded = _summ(fc.bf16_rne(ref), ref, L, L)       # 5.3 -> 5.3125: 0.0125 > 1e-2, within one ulp
    assert rounded["O_max_abs"] > 1e-2 and rounded["O_over_1e-2_beyond_1ulp"] == 0
    assert rounded["O_ref_at_worst"] == 5.3 and rounded["O_worst_error_bf16_ulps"] == pytest.approx(0.4)
    assert rounded["O_widened_bound_misses"] == 0
    assert fc.label(rounded, good) == "floor-limited"
    assert fc.label(rounded, None) == "fail"           # no fp32 run: not labelled floor-limited
    bad_f32 = _summ(ref + 2e-2, ref, L, L)
    assert fc.label(rounded, bad_f32) == "fail"
    two_ulps = ref.copy(); two_ulps[0, 0] += 2 * 2.0 ** -5
    assert fc.label(_summ(two_ulps, ref, L, L), good) == "fail"
    lse_bad = _summ(ref, ref, L + np.array([0.02, 0.0]), L)
    assert fc.label(lse_bad, good) == "fail"
    ninf_bad = _summ(ref, ref, np.array([1.0, 3.0]), L)
    assert ninf_bad["LSE_ninf_mismatch"] == 1 and fc.label(ninf_bad, good) == "fail"
    nan_o = ref.copy(); nan_o[1, 1] = np.nan
    assert fc.label(_summ(nan_o, ref, L, L), good) == "fail"


def test_merge_equals_whole():
    rng = np.random.default_rng(2)
    ref = rng.standard_normal((40, 8)); o = ref + rng.standard_normal((40, 8)) * 1e-3
    whole = fc.summarise(fc.o_stats(o, ref), None)
    parts = fc.summarise(fc.merge_stats([fc.o_stats(o[:13], ref[:13]), fc.o_stats(o[13:], ref[13:])]), None)
    for k in whole:
        assert whole[k] == pytest.approx(parts[k], rel=1e-12), k


@pytest.fixture(scope="module")
def pool():
    return fc.start_pool(2 if fc._pool is None else None)


def test_check_prefill_pool(pool):
    """Pool driver on a causal GQA case: the oracle's own answer rounded to bf16 passes,
    the same with one element moved by 0.05 fails."""
    B, Hq, Hkv, S, d = 2, 4, 2, 70, 64
    q, k, v = make_qkv(B, Hq, Hkv, S, S, d, seed=41)
    O, L = attention_ref(widen_bf16(q), widen_bf16(k), widen_bf16(v), causal=True, scale=0.125)
    o_bf = fc.bf16_rne(O).astype(np.float32)
    res = fc.check_prefill(q, k, v, {"bf16": (o_bf, L.astype(np.float32)), "f32": (O.astype(np.float32), L)},
                           causal=True, scale=0.125)
    assert fc.label(res["bf16"], res["f32"]) == "pass"
    assert res["bf16"]["O_elements"] == O.size and res["bf16"]["LSE_finite_entries"] == L.size
    assert res["_oracle"]["shares"] == B * Hq
    o_bad = o_bf.copy(); o_bad[1, 33, 3, 7] += 0.05
    res = fc.check_prefill(q, k, v, {"bf16": (o_bad, L)}, causal=True, scale=0.125, heads=[(1, 3), (0, 0)])
    assert res["bf16"]["O_max_abs"] > 0.04 and fc.label(res["bf16"], None) == "fail"


def test_check_decode_pool(pool):
    B, Hq, Hkv, Skv, d = 3, 8, 2, 300, 128
    q, k, v = make_qkv(B, Hq, Hkv, 1, Skv, d, seed=42)
    q = q.reshape(B, Hq, d)
    O, L = decode_ref(widen_bf16(q), widen_bf16(k), widen_bf16(v), scale=d ** -0.5)
    res = fc.check_decode(q, k, v, {"bf16": (fc.bf16_rne(O), L)}, scale=d ** -0.5)
    assert fc.label(res["bf16"], None) == "pass" and res["bf16"]["O_elements"] == O.size
    o_bad = fc.bf16_rne(O); o_bad[2, 5, 100] -= 0.03
    res = fc.check_decode(q, k, v, {"bf16": (o_bad, L)}, scale=d ** -0.5)
    assert fc.label(res["bf16"], None) == "fail"


def test_grad_bound_and_merge():
    """The gradient bound: 1e-2 + half a bf16 spacing + k 2^-8 times the worst-case
    sensitivity; statistics merged over shares equal those of the whole tensor."""
    ref = np.array([1.0, -3.0, 0.02])
    a = np.array([0.0, 100.0, 2.0])
    np.testing.assert_allclose(fc.grad_bound(ref, a, 2), [1e-2 + 2.0 ** -8, 1e-2 + 2.0 ** -7 + 200 * 2.0 ** -8,
                                                          1e-2 + 2.0 ** -14 + 4 * 2.0 ** -8])
    assert fc.grad_rel_bound(2.0, 0.0, 1) == fc.REL_L2
    assert fc.grad_rel_bound(2.0, 4.0, 1) == pytest.approx(fc.REL_L2 + 2 * 2.0 ** -8 / np.sqrt(3) * 2)
    rng = np.random.default_rng(5)
    g_ref = rng.standard_normal(50); a_r = np.abs(rng.standard_normal(50)); r_r = a_r / 3
    g = g_ref + rng.standard_normal(50) * 1e-3
    whole = fc.grad_summary([fc.grad_stats(g, g_ref, a_r, r_r, 2)], 2)
    parts = fc.grad_summary([fc.grad_stats(g[:17], g_ref[:17], a_r[:17], r_r[:17], 2),
                             fc.grad_stats(g[17:], g_ref[17:], a_r[17:], r_r[17:], 2)], 2)
    for key in whole:
        assert whole[key] == pytest.approx(parts[key], rel=1e-12), key
    assert fc.grad_ok(whole)
    g2 = g.copy(); g2[3] = np.nan
    assert not fc.grad_ok(fc.grad_summary([fc.grad_stats(g2, g_ref, a_r, r_r, 2)], 2))


def test_check_backward_pool(pool):
    """Pool driver of the gradient check on a causal GQA case: the oracle's own gradients
    rounded to bf16 pass; dK with one element moved by 0.05 fails, and only dK."""
    from oracle.attention import attention_bwd_ref
    from synth import make_grad_out
    B, Hq, Hkv, S, d = 2, 4, 2, 70, 64
    q, k, v = make_qkv(B, Hq, Hkv, S, S, d, seed=43)
    do = make_grad_out(B, S, Hq, d, 43)
    g = attention_bwd_ref(widen_bf16(q), widen_bf16(k), widen_bf16(v), widen_bf16(do), causal=True, scale=0.125)
    grads = tuple(fc.bf16_rne(x).astype(np.float32) for x in g)
    res = fc.check_backward(q, k, v, do, grads, causal=True, scale=0.125)
    assert all(fc.grad_ok(res[n]) for n in ("dQ", "dK", "dV"))
    assert res["dQ"]["elements"] == q.size and res["dK"]["elements"] == k.size and res["_oracle"]["shares"] == B * Hkv
    bad = grads[1].copy(); bad[1, 20, 1, 5] += 0.05
    res = fc.check_backward(q, k, v, do, (grads[0], bad, grads[2]), causal=True, scale=0.125)
    assert fc.grad_ok(res["dQ"]) and fc.grad_ok(res["dV"]) and not fc.grad_ok(res["dK"])
    assert res["dK"]["over_bound"] == 1


def test_attention_outputs_and_ffn_check(pool):
    """attention_outputs equals attention_ref; check_ffn passes the oracle's own layer
    output rounded to bf16 (in several row blocks) and fails one element moved by 0.1."""
    from oracle.attention import ffn_ref
    from synth import make_ffn_weights
    B, Hq, Hkv, S, d = 2, 2, 1, 50, 64
    q, k, v = make_qkv(B, Hq, Hkv, S, S, d, seed=44)
    O = fc.attention_outputs(q, k, v, causal=True, scale=0.125)
    np.testing.assert_array_equal(O, attention_ref(widen_bf16(q), widen_bf16(k), widen_bf16(v), causal=True,
                                                   scale=0.125)[0])
    dm = Hq * d
    w = make_ffn_weights(dm, 4 * dm, seed=45)
    h = O.reshape(B * S, dm)
    y = ffn_ref(h, *[widen_bf16(x) for x in w])
    res = fc.check_ffn(h, w, fc.bf16_rne(y), row_block=32)
    assert fc.ffn_ok(res) and res["elements"] == y.size and res["max_abs"] > 0
    bad = fc.bf16_rne(y); bad[77, 3] += 0.1
    res = fc.check_ffn(h, w, bad, row_block=32)
    assert not fc.ffn_ok(res) and res["over_bound"] == 1


def test_check_fp8_pool(pool):
    """The fp8 whole-tensor check: the oracle's own O rounded to bf16 with its LSE passes;
    one O element moved by 0.2 (far beyond the e4m3 rounding bound) fails."""
    from oracle.attention import attention_fp8_ref
    from synth.fp8 import make_fp8_qkv
    q8, k8, vt8, qs, ks, vs, ldv = make_fp8_qkv(1, 4, 2, 90, 90, 64, seed=46, k_stress_frac=0.05)
    O, L = attention_fp8_ref(q8, k8, vt8, qs, ks, vs, causal=True, scale=0.125)
    res = fc.check_fp8(q8, k8, vt8, qs, ks, vs, fc.bf16_rne(O), L, causal=True, scale=0.125)
    assert fc.fp8_ok(res) and res["O"]["elements"] == O.size and res["_oracle"]["shares"] == 4
    bad = fc.bf16_rne(O); bad[0, 50, 3, 9] += 0.2
    res = fc.check_fp8(q8, k8, vt8, qs, ks, vs, bad, L, causal=True, scale=0.125)
    assert not fc.fp8_ok(res) and res["O"]["over_bound"] == 1
    lbad = L.copy(); lbad[0, 1, 7] += 0.05
    assert not fc.fp8_ok(fc.check_fp8(q8, k8, vt8, qs, ks, vs, fc.bf16_rne(O), lbad, causal=True, scale=0.125))
