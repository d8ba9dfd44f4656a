"""Pins for the fp8 oracle pieces: the e4m3 decoder against values the OCP format fixes,
the input quantiser (round-to-nearest-even, per-head scale), and the fp8 reference
against the pinned attention oracle on the dequantised inputs."""
import numpy as np
import pytest

from oracle.attention import attention_fp8_ref, attention_ref, e4m3_value
from synth.fp8 import e4m3_rne_codes, make_fp8_qkv, quantize_heads, v_transposed


def test_e4m3_known_values():
    # smallest subnormal, largest subnormal, smallest normal, one, largest finite, negatives
    codes = np.array([0x00, 0x01, 0x07, 0x08, 0x30, 0x38, 0x39, 0x40, 0x77, 0x7E, 0x80, 0x81, 0xB8, 0xFE],
                     dtype=np.uint8)
    want = [0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 0.5, 1.0, 1.125, 2.0, 240.0, 448.0, -0.0, -(2.0 ** -9),
            -1.0, -448.0]
    np.testing.assert_array_equal(e4m3_value(codes), want)
    assert np.isnan(e4m3_value(np.array([0x7F, 0xFF], np.uint8))).all()


def test_e4m3_every_code_is_monotone_and_spaced():
    v = e4m3_value(np.arange(0x7F, dtype=np.uint8))
    d = np.diff(v)
    assert np.all(d > 0)
    # three mantissa bits: 8 equal steps per binade, subnormal steps equal the first normal step
    for e in range(1, 15):
        seg = v[8 * e:8 * e + 8]
        assert np.allclose(np.diff(seg), seg[1] - seg[0])
    assert v[8] - v[7] == v[1] - v[0] == 2.0 ** -9


def test_quantiser_rounds_to_nearest_even():
    vals = e4m3_value(np.arange(0x7F, dtype=np.uint8))
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.uniform(-448, 448, 20000), rng.standard_normal(5000) * 2 ** -7,
                        (vals[1:] + vals[:-1]) / 2, -(vals[1:] + vals[:-1]) / 2])
    c = e4m3_rne_codes(x)
    got = e4m3_value(c)
    err = np.abs(got - x)
    # nearest: no representable value is closer
    best = np.min(np.abs(vals[None, :] - np.abs(x)[:, None]), axis=1)
    assert np.all(err <= best + 0.0)
    ties = np.isclose(np.abs(x)[:, None], (vals[1:] + vals[:-1])[None, :] / 2, rtol=0, atol=0).any(axis=1)
    assert np.all((c[ties] & 1) == 0)


def test_quantiser_scale_maps_amax_to_448():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((2, 50, 3, 16))
    c, s = quantize_heads(x)
    assert s.dtype == np.float32 and s.shape == (2, 3)
    deq = e4m3_value(c) * s.astype(np.float64)[:, None, :, None]
    # relative rounding of a normal e4m3 value is at most 2^-4; tiny values are absolute
    amax = np.abs(x).max(axis=(1, 3))[:, None, :, None]
    assert np.all(np.abs(deq - x) <= np.maximum(2.0 ** -4 * np.abs(x), amax / 448 * 2.0 ** -9) * 1.0001)
    assert np.abs(e4m3_value(c)).max() == 448.0


def test_v_transposed_layout():
    rng = np.random.default_rng(5)
    v = rng.integers(0, 0x7E, size=(2, 37, 3, 8), dtype=np.uint8)
    vt, ldv = v_transposed(v)
    assert ldv == 48 and vt.shape == (2, 3, 8, 48)
    assert np.array_equal(vt[..., :37], v.transpose(0, 2, 3, 1)) and not vt[..., 37:].any()


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_reference_is_attention_of_dequantised_inputs(causal):
    q8, k8, vt8, qs, ks, vs, ldv = make_fp8_qkv(2, 4, 2, 40, 53, 16, seed=9, k_stress_frac=0.05)
    O, L = attention_fp8_ref(q8, k8, vt8, qs, ks, vs, causal=causal, scale=0.25)
    # independent dequantisation path: per-element float math on the transposed-back V codes
    Q = np.vectorize(lambda c: float(e4m3_value(np.array([c], np.uint8))[0]))(q8) * qs[:, None, :, None]
    K = e4m3_value(k8) * ks[:, None, :, None].astype(np.float64)
    V = e4m3_value(np.ascontiguousarray(vt8[..., :53].transpose(0, 3, 1, 2))) * vs[:, None, :, None].astype(np.float64)
    O2, L2 = attention_ref(Q, K, V, causal=causal, scale=0.25)
    np.testing.assert_allclose(O, O2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(L, L2, rtol=0, atol=1e-13)
    # the quantised inputs stay close to the unquantised draws' attention (sanity, loose)
    assert np.isfinite(O).all()
