"""Pins of the paged-cache decode oracle against the contiguous decode oracle.

The paged oracle gathers sequence b's token t from page block_table[b, t // page_size],
slot t % page_size. These tests build a paged pool from a known contiguous cache (pages
shuffled, spare pages filled with values that would dominate any score) and require the
plain decode of the contiguous cache: a wrong page, slot, order or length changes the
result.
"""
import numpy as np
import pytest

from oracle.attention import decode_ref, paged_decode_ref, widen_bf16
from synth import make_qkv, paged_layout


def _to_pages(kc, vc, table, P, page_size, fill=0.0):
    """Scatter contiguous caches [B, Smax, Hkv, d] into a pool of P pages per the table."""
    B, Smax, Hkv, d = kc.shape
    kp = np.full((P, page_size, Hkv, d), fill)
    vp = np.full((P, page_size, Hkv, d), fill)
    for b in range(B):
        for n in range((Smax + page_size - 1) // page_size):
            lo, hi = n * page_size, min(Smax, (n + 1) * page_size)
            kp[table[b, n], :hi - lo] = kc[b, lo:hi]
            vp[table[b, n], :hi - lo] = vc[b, lo:hi]
    return kp, vp


@pytest.mark.parametrize("page_size", [16, 32, 64])
def test_paged_equals_contiguous_full_lengths(page_size):
    B, Hq, Hkv, S, d = 3, 8, 2, 200, 64
    q, k, v = make_qkv(B, Hq, Hkv, 1, S, d, seed=71)
    q, k, v = widen_bf16(q).reshape(B, Hq, d), widen_bf16(k), widen_bf16(v)
    lens = np.full(B, S, dtype=np.int32)
    mb = (S + page_size - 1) // page_size
    table, P = paged_layout(B, page_size, lens, mb, seed=5, spare_pages=7)
    assert sorted(table.ravel().tolist()) == sorted(set(table.ravel().tolist()))   # pages distinct
    kp, vp = _to_pages(k, v, table, P, page_size, fill=1e4)   # spare pages would dominate if read
    O, L = paged_decode_ref(q, kp, vp, table, lens, scale=d ** -0.5)
    O2, L2 = decode_ref(q, k, v, scale=d ** -0.5)
    np.testing.assert_allclose(O, O2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, L2, rtol=0, atol=1e-12)


def test_paged_truncated_and_empty_sequences():
    B, Hq, Hkv, S, d, ps = 4, 4, 4, 130, 64, 16
    q, k, v = make_qkv(B, Hq, Hkv, 1, S, d, seed=72)
    q, k, v = widen_bf16(q).reshape(B, Hq, d), widen_bf16(k), widen_bf16(v)
    lens = np.array([130, 1, 0, 47], dtype=np.int32)
    mb = (S + ps - 1) // ps
    table, P = paged_layout(B, ps, np.full(B, S), mb, seed=6)
    kp, vp = _to_pages(k, v, table, P, ps)
    O, L = paged_decode_ref(q, kp, vp, table, lens, scale=0.125)
    for b in range(B):
        n = int(lens[b])
        if n == 0:
            assert np.all(O[b] == 0.0) and np.all(np.isneginf(L[b]))
            continue
        o, l = decode_ref(q[b:b + 1], k[b:b + 1, :n], v[b:b + 1, :n], scale=0.125)
        np.testing.assert_allclose(O[b], o[0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(L[b], l[0], rtol=0, atol=1e-12)
    # one token: the output is that token's value row
    hk = np.arange(Hq) * Hkv // Hq
    np.testing.assert_allclose(O[1], v[1, 0, hk], rtol=0, atol=1e-12)


def test_page_permutation_does_not_change_result():
    B, Hq, Hkv, S, d, ps = 2, 4, 2, 96, 64, 32
    q, k, v = make_qkv(B, Hq, Hkv, 1, S, d, seed=73)
    q, k, v = widen_bf16(q).reshape(B, Hq, d), widen_bf16(k), widen_bf16(v)
    lens = np.array([96, 70], dtype=np.int32)
    t1, P1 = paged_layout(B, ps, lens, 3, seed=1, spare_pages=3)
    t2, P2 = paged_layout(B, ps, lens, 3, seed=2, spare_pages=3)
    assert not np.array_equal(t1, t2)
    a = paged_decode_ref(q, *_to_pages(k, v, t1, P1, ps, fill=-7.0), t1, lens, scale=0.2)
    c = paged_decode_ref(q, *_to_pages(k, v, t2, P2, ps, fill=3.0), t2, lens, scale=0.2)
    np.testing.assert_array_equal(a[0], c[0])
    np.testing.assert_array_equal(a[1], c[1])


def test_paged_layout_is_seeded_and_covers_lengths():
    lens = np.array([0, 1, 16, 17, 100], dtype=np.int32)
    t, P = paged_layout(5, 16, lens, 7, seed=9, spare_pages=2)
    t2, P2 = paged_layout(5, 16, lens, 7, seed=9, spare_pages=2)
    assert np.array_equal(t, t2) and P == P2
    need = [0, 1, 1, 2, 7]
    assert P == sum(need) + 2
    used = np.concatenate([t[b, :need[b]] for b in range(5)])
    assert len(set(used.tolist())) == len(used)
    assert used.min() >= 0 and used.max() < P
