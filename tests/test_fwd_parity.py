"""GPU parity of the fused forward kernel against the fp64 oracle (through the C ABI)."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle.attention import attention_ref, widen_bf16
from synth import WORKLOADS, make_qkv, make_workload
from tests.parity import check_lse, check_o, down, up

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import io_aware_exact_21_amd as fa
    return fa


def _run_full(fa, q, k, v, causal, scale=None, d=None, out_f32=False):
    d = q.shape[-1]
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    o, lse = fa.fwd(up(q), up(k), up(v), causal=causal, scale=sc, out_f32=out_f32)
    torch.cuda.synchronize()
    O, L = attention_ref(widen_bf16(q), widen_bf16(k), widen_bf16(v), causal=causal, scale=sc)
    return down(o), down(lse), O, L


SMALL = [
    # B, Hq, Hkv, Sq, Skv, d
    (1, 1, 1, 1, 1, 64), (2, 2, 2, 7, 7, 64), (1, 4, 1, 33, 33, 128), (2, 4, 2, 130, 130, 64),
    (1, 2, 1, 257, 257, 128), (1, 8, 8, 64, 64, 128), (2, 8, 2, 200, 200, 128), (1, 2, 2, 5, 70, 64),
    (1, 2, 1, 70, 5, 128), (1, 16, 2, 129, 300, 128), (1, 1, 1, 300, 129, 64), (3, 3, 1, 97, 97, 64),
    # d = 128 workgroups of 2, 6 and 8 key tiles: the copy distance and the barrier-free last
    # tiles at and just past the ring depth
    (1, 4, 2, 100, 100, 128), (1, 2, 2, 383, 383, 128), (1, 2, 1, 190, 450, 128),
    # four query heads per KV head at d = 128: one workgroup per KV group and 64-row Q tile
    (1, 8, 2, 130, 250, 128), (2, 4, 1, 300, 300, 128), (1, 8, 2, 250, 130, 128),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SMALL, ids=[str(s) for s in SMALL])
def test_small_shapes(fa, shape, causal):
    B, Hq, Hkv, Sq, Skv, d = shape
    q, k, v = make_qkv(B, Hq, Hkv, Sq, Skv, d, seed=100 + Sq + 7 * Skv + d)
    print(f"case {shape} causal={causal}", flush=True)
    o, l, O, L = _run_full(fa, q, k, v, causal)
    check_o(o, O, bf16=True)
    check_lse(l, L)


# More query tiles than the chip has CUs: many workgroups per CU and per XCD, so these cover
# the work order across heads and tiles (ragged tiles, GQA, Sq != Skv).
MANY_UNITS = [
    # B, Hq, Hkv, Sq, Skv, d
    (3, 40, 8, 700, 700, 128), (2, 48, 16, 600, 900, 128), (3, 40, 8, 700, 700, 64), (1, 96, 96, 333, 333, 64),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", MANY_UNITS, ids=[str(s) for s in MANY_UNITS])
def test_many_work_units(fa, shape, causal):
    B, Hq, Hkv, Sq, Skv, d = shape
    q, k, v = make_qkv(B, Hq, Hkv, Sq, Skv, d, seed=300 + Sq + Skv + d)
    print(f"case {shape} causal={causal}", flush=True)
    o, l, O, L = _run_full(fa, q, k, v, causal)
    check_o(o, O, bf16=True)
    check_lse(l, L)


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("causal", [False, True])
def test_fp32_output_arithmetic(fa, causal, d):
    """fp32-output instantiation: the kernel arithmetic meets 1e-2 / 4e-3 with no output rounding."""
    q, k, v = make_qkv(2, 8, 2, 300, 300, d, seed=31)
    o, l, O, L = _run_full(fa, q, k, v, causal, out_f32=True)
    info = check_o(o, O, bf16=False)
    assert info["max_abs"] < 5e-3
    check_lse(l, L)


def test_tiny_workload(fa):
    w = WORKLOADS["tiny"]
    q, k, v = make_workload(w)
    o, l, O, L = _run_full(fa, q, k, v, w.causal, scale=w.scale)
    check_o(o, O, bf16=True)
    check_lse(l, L)


@pytest.mark.parametrize("name", ["small_causal_gqa_d64", "small_noncausal_d128"])
def test_golden(fa, name):
    with open(os.path.join(GOLDEN, name + ".json")) as f:
        g = json.load(f)
    q, k, v = make_qkv(g["B"], g["Hq"], g["Hkv"], g["Sq"], g["Skv"], g["d"], g["seed"])
    o, lse = fa.fwd(up(q), up(k), up(v), causal=g["causal"], scale=g["scale"])
    torch.cuda.synchronize()
    O = np.array([float.fromhex(x) for x in g["O"]]).reshape(g["B"], g["Sq"], g["Hq"], g["d"])
    L = np.array([float.fromhex(x) for x in g["LSE"]]).reshape(g["B"], g["Hq"], g["Sq"])
    check_o(down(o), O, bf16=True)
    check_lse(down(lse), L)


def _bits(x):
    from synth import bf16_rne_bits
    return bf16_rne_bits(x)


def test_identical_keys(fa):
    """All keys equal -> O is the mean of the visible V rows (closed form)."""
    rng = np.random.default_rng(3)
    B, S, H, d = 1, 150, 2, 128
    q = _bits(rng.standard_normal((B, S, H, d)))
    k = np.broadcast_to(_bits(rng.standard_normal((1, 1, H, d))), (B, S, H, d)).copy()
    v = _bits(rng.standard_normal((B, S, H, d)))
    o, l, O, L = _run_full(fa, q, k, v, True)
    vv = widen_bf16(v)
    mean = np.cumsum(vv, axis=1) / np.arange(1, S + 1)[None, :, None, None]
    np.testing.assert_allclose(O, mean, rtol=1e-12, atol=1e-12)
    check_o(o, O, bf16=True)
    check_lse(l, L)


def test_dominant_key(fa):
    """One key scores far above the rest of every row -> O equals that key's V row."""
    rng = np.random.default_rng(4)
    B, S, H, d = 1, 96, 1, 64
    q = np.zeros((B, S, H, d)); q[..., 0] = 1.0
    k = rng.standard_normal((B, S, H, d)) * 0.05; k[..., 0] = 0.0; k[0, 40, 0, 0] = 64.0
    v = rng.standard_normal((B, S, H, d))
    q, k, v = _bits(q), _bits(k), _bits(v)
    o, l, O, L = _run_full(fa, q, k, v, False, scale=1.0)
    assert np.abs(o - widen_bf16(v)[0, 40, 0][None, None, None, :]).max() == 0.0
    check_lse(l, L)


def test_huge_scores_no_overflow(fa):
    """Scores around 1e4 stay finite and match the oracle (running max keeps exp finite)."""
    rng = np.random.default_rng(5)
    B, S, H, d = 1, 200, 2, 64
    q = rng.standard_normal((B, S, H, d)); k = rng.standard_normal((B, S, H, d))
    v = rng.standard_normal((B, S, H, d))
    q[..., 0] = 640.0; k[..., 0] = 128.0           # every score gains 0.125 * 640 * 128 = 10240
    q, k, v = _bits(q), _bits(k), _bits(v)
    o, l, O, L = _run_full(fa, q, k, v, True, scale=0.125)
    assert np.isfinite(o).all() and np.isfinite(l).all()
    check_o(o, O, bf16=True)
    check_lse(l, L)
    assert abs(float(np.median(l - L))) < 1e-2 and l.min() > 10000


@pytest.mark.parametrize("causal", [False, True])
def test_late_max_jumps(fa, causal):
    """Row maxima that jump far above the running max deep inside the unmasked tiles, where
    the kernel forms probabilities without a max reduction and must redo the unit with the
    full step. Head 0 jumps at key 700 (an odd 32-key unit) and again at key 960 (even
    unit), head 1 at key 896 (even unit); each jump is over 100 powers of two."""
    rng = np.random.default_rng(11)
    B, S, H, d = 1, 1024, 2, 128
    q = rng.standard_normal((B, S, H, d))
    k = rng.standard_normal((B, S, H, d))
    v = rng.standard_normal((B, S, H, d))
    q[..., 0] = 1.0
    k[0, 700, 0, 0] = 1024.0          # score about 1024 / sqrt(128): 130 powers of two up
    k[0, 960, 0, 0] = 3072.0          # a second jump in the same rows
    k[0, 896, 1, 0] = 2048.0
    o, l, O, L = _run_full(fa, _bits(q), _bits(k), _bits(v), causal)
    check_o(o, O, bf16=True)
    check_lse(l, L)
    seen = np.arange(S) >= (960 if causal else 0)
    ref = widen_bf16(_bits(v))[0, 960, 0]
    assert np.abs(o[0, seen, 0] - ref[None, :]).max() < 1e-2   # the dominant key's V row


@pytest.mark.parametrize("jump", [400.0, 1024.0])
def test_large_values_with_late_jumps(fa, jump):
    """V scaled by 2^40 (exact in bf16) with a row max that jumps late: about 51 powers of two
    (inside the max-free step's 2^64 bound on the normaliser, so probabilities up to about
    2^51 multiply values up to 2^42) or about 130 (the unit is redone with the full step).
    Every product and sum in the kernel then scales by exactly 2^40, so O must be exactly
    2^40 times the unscaled result and the LSE identical; both also match the oracle."""
    rng = np.random.default_rng(12)
    B, S, H, d = 1, 1024, 2, 128
    q = rng.standard_normal((B, S, H, d))
    k = rng.standard_normal((B, S, H, d))
    v = rng.standard_normal((B, S, H, d))
    q[..., 0] = 1.0
    k[0, 700, 0, 0] = jump
    k[0, 900, 1, 0] = jump
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    vb40 = _bits(widen_bf16(vb) * 2.0 ** 40)
    assert np.array_equal(widen_bf16(vb40), widen_bf16(vb) * 2.0 ** 40)
    tq, tk = up(qb), up(kb)
    o1, l1 = fa.fwd(tq, tk, up(vb), causal=False)
    o2, l2 = fa.fwd(tq, tk, up(vb40), causal=False)
    torch.cuda.synchronize()
    assert torch.isfinite(o2.float()).all()
    assert torch.equal(o2.float(), o1.float() * 2.0 ** 40)
    assert torch.equal(l1, l2)
    o, l, O, L = _run_full(fa, qb, kb, vb40, False)
    check_o(o / 2.0 ** 40, O / 2.0 ** 40, bf16=True)
    check_lse(l, L)


@pytest.mark.parametrize("scale", [-0.09, 0.0, 0.5])
def test_other_scales(fa, scale):
    q, k, v = make_qkv(1, 4, 2, 100, 100, 128, seed=9)
    o, l, O, L = _run_full(fa, q, k, v, True, scale=scale)
    check_o(o, O, bf16=True)
    check_lse(l, L)


def test_deterministic(fa):
    q, k, v = make_qkv(1, 8, 2, 513, 513, 128, seed=10)
    tq, tk, tv = up(q), up(k), up(v)
    o1, l1 = fa.fwd(tq, tk, tv, causal=True)
    o2, l2 = fa.fwd(tq, tk, tv, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
