"""Seeded input generators: bf16 rounding, reproducibility and workload structure."""
import json
import os

import numpy as np

from oracle.attention import attention_ref, widen_bf16
from synth import WORKLOADS, bf16_rne_bits, make_qkv, stress_positions
from synth.inputs import bf16_bits_to_f32, normal_bf16, times4_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_rne_hand_patterns():
    # value -> expected bf16 bits, worked out by hand from the bfloat16 format
    cases = [
        (1.0, 0x3F80), (-3.0, 0xC040), (0.0, 0x0000),
        (1.0 + 2.0 ** -8, 0x3F80),            # tie between 1 and 1+2^-7 -> even (1)
        (1.0 + 3 * 2.0 ** -8, 0x3F82),        # tie between 1+2^-7 and 1+2^-6 -> even (1+2^-6)
        (1.0 + 2.0 ** -8 + 2.0 ** -30, 0x3F81),  # just above the tie -> up
        (3.140625, 0x4049), (2.0 ** -133, 0x0001), (2.0 ** -126, 0x0080),
        (-(2.0 ** 127) * (2 - 2.0 ** -7), 0xFF7F),
    ]
    for x, bits in cases:
        assert int(bf16_rne_bits(np.array([x]))[0]) == bits, (x, hex(bits))


def test_bf16_rne_is_nearest():
    x = np.random.default_rng(3).standard_normal(200000) * 7
    b = bf16_rne_bits(x)
    r = bf16_bits_to_f32(b).astype(np.float64)
    up = bf16_bits_to_f32(b + 1).astype(np.float64)          # neighbours in the bf16 grid
    dn = bf16_bits_to_f32(b - 1).astype(np.float64)
    err = np.abs(x - r)
    assert (err <= np.abs(x - up)).all() and (err <= np.abs(x - dn)).all()


def test_seeded_and_blocked():
    a = normal_bf16((2, 3000, 2, 8), 5, 1)
    b = normal_bf16((2, 3000, 2, 8), 5, 1)
    assert np.array_equal(a, b)
    c = normal_bf16((2, 3000, 2, 8), 6, 1)
    assert not np.array_equal(a, c)
    v = bf16_bits_to_f32(a)
    assert abs(float(v.mean())) < 0.02 and abs(float(v.std()) - 1.0) < 0.02


def test_stress_positions_and_times4():
    w = WORKLOADS["mha8k"]
    for b in range(w.B):
        p = stress_positions(w.seed, b, w.Skv, w.k_stress_frac)
        assert len(p) == 82 and len(np.unique(p)) == 82 and p.max() < w.Skv
    bits = bf16_rne_bits(np.array([1.5, -0.3, 2.0 ** -100]))
    assert np.array_equal(bf16_bits_to_f32(times4_bf16(bits)), bf16_bits_to_f32(bits) * 4)
    q, k, v = make_qkv(1, 1, 2, 4, 1000, 8, 9, k_stress_frac=0.01)
    q2, k2, v2 = make_qkv(1, 1, 2, 4, 1000, 8, 9)
    p = stress_positions(9, 0, 1000, 0.01)
    assert np.array_equal(bf16_bits_to_f32(k[0, p]), 4 * bf16_bits_to_f32(k2[0, p]))
    rest = np.setdiff1d(np.arange(1000), p)
    assert np.array_equal(k[0, rest], k2[0, rest]) and np.array_equal(v, v2)


def test_workload_shapes():
    w = WORKLOADS
    assert (w["tiny"].B, w["tiny"].Sq, w["tiny"].d, w["tiny"].causal) == (1, 256, 64, False)
    assert (w["mha8k"].Hq, w["mha8k"].Skv, w["mha8k"].d) == (32, 8192, 128)
    assert (w["gqa32k"].Hq, w["gqa32k"].Hkv, w["gqa32k"].Sq) == (32, 8, 32768)
    assert w["decode"].decode and w["decode"].Sq == 1 and w["decode"].B == 64
    assert w["mha8k"].scale == float(np.float32(1 / np.sqrt(128)))


def test_golden_fixtures_reproduce():
    """The stored oracle outputs are reproduced exactly from the seeded inputs."""
    for name in ("small_causal_gqa_d64", "small_noncausal_d128"):
        with open(os.path.join(GOLDEN, name + ".json")) as f:
            g = json.load(f)
        q, k, v = make_qkv(g["B"], g["Hq"], g["Hkv"], g["Sq"], g["Skv"], g["d"], g["seed"])
        O, L = attention_ref(widen_bf16(q), widen_bf16(k), widen_bf16(v), causal=g["causal"], scale=g["scale"])
        assert np.array_equal(O.ravel(), np.array([float.fromhex(x) for x in g["O"]]))
        assert np.array_equal(L.ravel(), np.array([float.fromhex(x) for x in g["LSE"]]))
