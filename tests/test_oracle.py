"""Pins for the fp64 oracle: closed forms, invariants, brute force and library routines.

Each pin is a function of the oracle module so that the planted-mistake test at
the bottom can run every pin against deliberately broken copies of the oracle
and check that at least one pin notices.
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp, softmax

import oracle.attention as oa

RNG = np.random.default_rng


def _bf16ish(rng, shape, scale=1.0):
    """Random values that are exact in bf16 (8 significant bits), as float64."""
    x = rng.standard_normal(shape) * scale
    e = np.floor(np.log2(np.abs(x) + 1e-300))
    q = 2.0 ** (e - 7)
    return np.round(x / q) * q


# ---------------------------------------------------------------- pins
def pin_online_equals_oneshot(m):
    """P-1. [ILP, Code / Deep dive]: the streamed softmax equals the one-shot one to
    machine precision, for any block size (block 1: an update after every key)."""
    rng = RNG(11)
    for d in (4, 8, 64):
        for S in (1, 5, 17, 64):
            q = _bf16ish(rng, (1, S, 1, d)); k = _bf16ish(rng, (1, S, 1, d)); v = _bf16ish(rng, (1, S, 1, d))
            sc = 1.0 / math.sqrt(d)
            O, L = m.attention_ref(q, k, v, causal=False, scale=sc)
            for i in (0, S - 1):
                for block in (1, 2, 3, 7, S):
                    o, l = m.online_ref(q[0, i, 0], k[0, :, 0], v[0, :, 0], scale=sc, block=block)
                    np.testing.assert_allclose(o, O[0, i, 0], rtol=1e-12, atol=1e-13)
                    assert abs(l - L[0, 0, i]) <= 1e-12 * max(1.0, abs(l))


def pin_weights_are_softmax(m):
    """P-2. With V = I the output rows are the softmax weights themselves: they match
    scipy's softmax of the scaled scores, sum to 1 ([GRASP, section 2]) and, when
    causal, vanish above the diagonal."""
    rng = RNG(12)
    S, d = 9, 16
    q = _bf16ish(rng, (S, d)); k = _bf16ish(rng, (S, d))
    sc = 0.25
    s = sc * (q @ k.T)
    W, L = m.attention_rows(q, k, np.eye(S), np.arange(S), S, False, sc)
    np.testing.assert_allclose(W, softmax(s, axis=1), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(W.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    np.testing.assert_allclose(L, logsumexp(s, axis=1), rtol=1e-13)
    Wc, _ = m.attention_rows(q, k, np.eye(S), np.arange(S), S, True, sc)
    assert (np.triu(Wc, 1) == 0).all()
    np.testing.assert_allclose(Wc.sum(axis=1), 1.0, rtol=0, atol=1e-14)


def pin_identical_keys(m):
    """P-3. All keys equal: every visible key gets the same weight, so O is the mean
    of the visible V rows and LSE = s + ln |A(i)| (closed form)."""
    rng = RNG(13)
    S, d = 12, 8
    q = _bf16ish(rng, (1, S, 1, d)); kk = _bf16ish(rng, (d,)); v = _bf16ish(rng, (1, S, 1, d))
    k = np.broadcast_to(kk, (1, S, 1, d)).copy()
    sc = 0.5
    for causal in (False, True):
        O, L = m.attention_ref(q, k, v, causal=causal, scale=sc)
        for i in range(S):
            n = i + 1 if causal else S
            np.testing.assert_allclose(O[0, i, 0], v[0, :n, 0].mean(axis=0), rtol=1e-13, atol=1e-14)
            assert abs(L[0, 0, i] - (sc * float(q[0, i, 0] @ kk) + math.log(n))) < 1e-12


def pin_dominant_score(m):
    """P-4. One score 60 above all others: O is that key's V row, LSE its score."""
    rng = RNG(14)
    S, d = 10, 8
    q = np.zeros((1, 1, 1, d)); q[..., 0] = 1.0
    k = _bf16ish(rng, (1, S, 1, d)) * 0.1; k[..., 0] = 0.0
    k[0, 6, 0, 0] = 60.0
    v = _bf16ish(rng, (1, S, 1, d))
    O, L = m.attention_ref(q, k, v, causal=False, scale=1.0)
    np.testing.assert_allclose(O[0, 0, 0], v[0, 6, 0], rtol=1e-20, atol=1e-24)
    assert abs(L[0, 0, 0] - 60.0) < 1e-20 + 1e-24 + S * math.exp(-59)


def pin_huge_scores(m):
    """P-5. Scores near 1e4 stay finite (the running max, [ILP, Interviewer follow-ups]);
    a component shared by every score of a row shifts LSE by it and leaves O alone."""
    rng = RNG(15)
    B, S, H, d = 1, 16, 2, 64
    q = _bf16ish(rng, (B, S, H, d)); k = _bf16ish(rng, (B, S, H, d)); v = _bf16ish(rng, (B, S, H, d))
    q[..., 0] = 0.0; k[..., 0] = 0.0
    O0, L0 = m.attention_ref(q, k, v, causal=True, scale=0.125)
    q[..., 0] = 640.0; k[..., 0] = 128.0                       # adds 0.125*640*128 = 10240
    O1, L1 = m.attention_ref(q, k, v, causal=True, scale=0.125)
    assert np.isfinite(O1).all() and np.isfinite(L1).all()
    np.testing.assert_allclose(O1, O0, rtol=1e-9, atol=1e-9)
    np.testing.assert_allclose(L1 - 10240.0, L0, rtol=0, atol=1e-9)


def pin_causal_bruteforce(m):
    """P-6. Causal masking brute-forced at S <= 8: explicit -inf mask + scipy softmax,
    bottom-right aligned when Sq != Skv; rows with no visible key give O = 0, LSE = -inf."""
    rng = RNG(16)
    d = 4
    for Sq, Skv in ((1, 1), (5, 5), (8, 8), (3, 8), (1, 8), (8, 3)):
        q = _bf16ish(rng, (1, Sq, 1, d)); k = _bf16ish(rng, (1, Skv, 1, d)); v = _bf16ish(rng, (1, Skv, 1, d))
        O, L = m.attention_ref(q, k, v, causal=True, scale=0.5)
        for i in range(Sq):
            mask = np.array([0.0 if j <= i + Skv - Sq else -np.inf for j in range(Skv)])
            s = 0.5 * (q[0, i, 0] @ k[0, :, 0].T) + mask
            if np.isinf(s).all():
                assert (O[0, i, 0] == 0).all() and L[0, 0, i] == -np.inf
                continue
            w = softmax(s)
            np.testing.assert_allclose(O[0, i, 0], w @ v[0, :, 0], rtol=1e-13, atol=1e-14)
            assert abs(L[0, 0, i] - logsumexp(s)) < 1e-13


def pin_gqa_is_repeated_mha(m):
    """P-7. Grouped-query attention equals MHA with each KV head repeated for its
    group of consecutive query heads ([IOP, FlashAttention] names GQA)."""
    rng = RNG(17)
    B, S, Hq, Hkv, d = 2, 6, 8, 2, 8
    q = _bf16ish(rng, (B, S, Hq, d)); k = _bf16ish(rng, (B, S, Hkv, d)); v = _bf16ish(rng, (B, S, Hkv, d))
    O, L = m.attention_ref(q, k, v, causal=True, scale=0.3)
    kr = np.repeat(k, Hq // Hkv, axis=2); vr = np.repeat(v, Hq // Hkv, axis=2)
    O2, L2 = m.attention_ref(q, kr, vr, causal=True, scale=0.3)
    assert np.array_equal(O, O2) and np.array_equal(L, L2)
    # and heads really do differ: swapping KV heads must change the result
    O3, _ = m.attention_ref(q, k[:, :, ::-1], v[:, :, ::-1], causal=True, scale=0.3)
    assert not np.allclose(O, O3)


def pin_decode_is_prefill_row(m):
    """P-8. A decode step equals a one-row non-causal prefill and equals the last row
    of a causal prefill over the same keys ([ILP, Direct answer])."""
    rng = RNG(18)
    B, Skv, Hq, Hkv, d = 2, 11, 4, 2, 8
    k = _bf16ish(rng, (B, Skv, Hkv, d)); v = _bf16ish(rng, (B, Skv, Hkv, d))
    qs = _bf16ish(rng, (B, Skv, Hq, d))
    Od, Ld = m.decode_ref(qs[:, -1], k, v, scale=0.35)
    Op, Lp = m.attention_ref(qs[:, -1:], k, v, causal=False, scale=0.35)
    Oc, Lc = m.attention_ref(qs, k, v, causal=True, scale=0.35)
    np.testing.assert_array_equal(Od, Op[:, 0]); np.testing.assert_array_equal(Ld, Lp[:, :, 0])
    np.testing.assert_allclose(Od, Oc[:, -1], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(Ld, Lc[:, :, -1], rtol=1e-13)


def pin_split_combine(m):
    """P-9. Split-KV partials merged by log-sum-exp equal the unsplit decode, for even,
    uneven and empty chunks ([ILP, Deep dive]: FlashDecoding splits the KV length)."""
    rng = RNG(19)
    B, Skv, Hq, Hkv, d = 2, 37, 4, 2, 8
    q = _bf16ish(rng, (B, Hq, d)); k = _bf16ish(rng, (B, Skv, Hkv, d)); v = _bf16ish(rng, (B, Skv, Hkv, d))
    O, L = m.decode_ref(q, k, v, scale=0.4)
    for bounds in ([0, 37], [0, 18, 37], [0, 13, 26, 37], list(range(0, 37, 3)) + [37],
                   [0, 5, 5, 30, 37], [0, 0, 37, 37]):
        po, pl = m.split_partials_ref(q, k, v, scale=0.4, bounds=bounds)
        Oc, Lc = m.combine_ref(po, pl)
        np.testing.assert_allclose(Oc, O, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(Lc, L, rtol=1e-12)
    po = np.zeros((1, 1, 3, d)); pl = np.full((1, 1, 3), -np.inf)
    Oc, Lc = m.combine_ref(po, pl)
    assert (Oc == 0).all() and Lc[0, 0] == -np.inf


def pin_single_key(m):
    """P-10. One key: its weight is 1, so O = V_0 and LSE = s_00."""
    rng = RNG(20)
    q = _bf16ish(rng, (1, 1, 1, 16)); k = _bf16ish(rng, (1, 1, 1, 16)); v = _bf16ish(rng, (1, 1, 1, 16))
    O, L = m.attention_ref(q, k, v, causal=True, scale=0.25)
    np.testing.assert_array_equal(O[0, 0, 0], v[0, 0, 0])
    assert L[0, 0, 0] == 0.25 * float(q[0, 0, 0] @ k[0, 0, 0])


def pin_permutation(m):
    """P-11. Without a mask, permuting the (key, value) pairs changes nothing."""
    rng = RNG(21)
    B, S, H, d = 1, 20, 2, 8
    q = _bf16ish(rng, (B, S, H, d)); k = _bf16ish(rng, (B, S, H, d)); v = _bf16ish(rng, (B, S, H, d))
    O, L = m.attention_ref(q, k, v, causal=False, scale=0.3)
    p = rng.permutation(S)
    O2, L2 = m.attention_ref(q, k[:, p], v[:, p], causal=False, scale=0.3)
    np.testing.assert_allclose(O2, O, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(L2, L, rtol=1e-12)


def pin_convexity(m):
    """P-12. Each output is a convex combination of the visible V rows."""
    rng = RNG(22)
    B, S, H, d = 1, 24, 2, 8
    q = _bf16ish(rng, (B, S, H, d), 3.0); k = _bf16ish(rng, (B, S, H, d)); v = _bf16ish(rng, (B, S, H, d))
    O, _ = m.attention_ref(q, k, v, causal=True, scale=0.3)
    for i in range(S):
        lo = v[0, :i + 1].min(axis=0); hi = v[0, :i + 1].max(axis=0)
        assert (O[0, i] >= lo - 1e-12).all() and (O[0, i] <= hi + 1e-12).all()


def pin_closed_form_two_keys(m):
    """Hand-worked case: scores 0 and 1 give weights 1/(1+e), e/(1+e);
    V = I then makes O exactly those weights and LSE = ln(1+e)."""
    q = np.zeros((1, 1, 1, 2)); q[0, 0, 0] = [1.0, 0.0]
    k = np.zeros((1, 2, 1, 2)); k[0, 1, 0] = [1.0, 0.0]
    v = np.zeros((1, 2, 1, 2)); v[0, 0, 0] = [1.0, 0.0]; v[0, 1, 0] = [0.0, 1.0]
    O, L = m.attention_ref(q, k, v, causal=False, scale=1.0)
    e = math.e
    np.testing.assert_allclose(O[0, 0, 0], [1 / (1 + e), e / (1 + e)], rtol=1e-15)
    assert abs(L[0, 0, 0] - math.log1p(e)) < 1e-15


def pin_matches_torch_sdpa_fp64(m):
    """Cross-check with torch's scaled_dot_product_attention in float64 on the CPU
    (an independent library implementation of the same definition), including GQA,
    causal masks with Sq < Skv (explicit bottom-right mask) and the LSE."""
    rng = RNG(23)
    for (B, Sq, Skv, Hq, Hkv, d, causal) in ((2, 33, 33, 4, 4, 16, True), (1, 7, 40, 8, 2, 32, True),
                                             (2, 19, 50, 6, 3, 8, False)):
        q = _bf16ish(rng, (B, Sq, Hq, d)); k = _bf16ish(rng, (B, Skv, Hkv, d)); v = _bf16ish(rng, (B, Skv, Hkv, d))
        sc = 1.0 / math.sqrt(d)
        O, L = m.attention_ref(q, k, v, causal=causal, scale=sc)
        tq = torch.from_numpy(q).permute(0, 2, 1, 3)
        tk = torch.from_numpy(np.repeat(k, Hq // Hkv, axis=2)).permute(0, 2, 1, 3)
        tv = torch.from_numpy(np.repeat(v, Hq // Hkv, axis=2)).permute(0, 2, 1, 3)
        mask = None
        if causal:
            mask = torch.from_numpy(np.arange(Skv)[None, :] <= np.arange(Sq)[:, None] + Skv - Sq)
        sig = float(np.float32(sc))
        to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=sig)
        np.testing.assert_allclose(O, to.permute(0, 2, 1, 3).numpy(), rtol=1e-12, atol=1e-13)
        s = sig * (tq @ tk.transpose(-1, -2))
        if mask is not None:
            s = s.masked_fill(~mask, -math.inf)
        np.testing.assert_allclose(L, torch.logsumexp(s, dim=-1).numpy(), rtol=1e-12)


def pin_widen_bf16(m):
    """bf16 bits widen exactly: 0x3F80 = 1, 0xC040 = -3, 0x0001 = 2^-133, 0x7F80 = inf."""
    bits = np.array([0x3F80, 0xC040, 0x0001, 0x7F80, 0x4049], dtype=np.uint16)
    w = m.widen_bf16(bits)
    assert w[0] == 1.0 and w[1] == -3.0 and w[2] == 2.0 ** -133 and w[3] == np.inf
    assert w[4] == 3.140625


PINS = [pin_online_equals_oneshot, pin_weights_are_softmax, pin_identical_keys, pin_dominant_score,
        pin_huge_scores, pin_causal_bruteforce, pin_gqa_is_repeated_mha, pin_decode_is_prefill_row,
        pin_split_combine, pin_single_key, pin_permutation, pin_convexity, pin_closed_form_two_keys,
        pin_matches_torch_sdpa_fp64, pin_widen_bf16]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(oa)


# ---------------------------------------------------------------- planted mistakes
def _mutant_causal_off_by_one(mp):
    mp.setattr(oa, "visible_keys", lambda i, Sq, Skv, causal: Skv if not causal else max(0, min(Skv, i + Skv - Sq)))


def _mutant_causal_top_left(mp):
    mp.setattr(oa, "visible_keys", lambda i, Sq, Skv, causal: Skv if not causal else max(0, min(Skv, i + 1)))


def _mutant_scale_dropped(mp):
    mp.setattr(oa, "_sigma", lambda s: 1.0)


def _mutant_scale_sign(mp):
    mp.setattr(oa, "_sigma", lambda s: -float(np.float32(s)))


def _mutant_scale_sqrt(mp):
    mp.setattr(oa, "_sigma", lambda s: math.sqrt(float(np.float32(s))))


def _mutant_gqa_modulo(mp):
    mp.setattr(oa, "kv_head_of", lambda h, Hq, Hkv: h % Hkv)


def _wrap_rows(mp, post):
    orig = oa.attention_rows

    def rows(q_rows, K, V, rows, Sq, causal, scale):
        return post(*orig(q_rows, K, V, rows, Sq, causal, scale), q_rows=q_rows, K=K, V=V)
    mp.setattr(oa, "attention_rows", rows)


def _mutant_lse_log2(mp):
    _wrap_rows(mp, lambda O, L, **kw: (O, L / math.log(2)))


def _mutant_lse_missing_max(mp):
    orig = oa.attention_rows

    def rows(q_rows, K, V, rows, Sq, causal, scale):
        O, L = orig(q_rows, K, V, rows, Sq, causal, scale)
        s = float(np.float32(scale)) * (q_rows @ K.T)
        return O, L - s.max(axis=1)
    mp.setattr(oa, "attention_rows", rows)


def _mutant_value_reversed(mp):
    orig = oa.attention_rows
    mp.setattr(oa, "attention_rows", lambda q_rows, K, V, rows, Sq, causal, scale:
               orig(q_rows, K, V[::-1], rows, Sq, causal, scale))


def _mutant_no_normalise(mp):
    def rows(q_rows, K, V, rows, Sq, causal, scale):
        sigma, Skv = float(np.float32(scale)), K.shape[0]
        s = sigma * (q_rows @ K.T)
        nvis = np.array([oa.visible_keys(int(i), Sq, Skv, causal) for i in rows])
        s = np.where(np.arange(Skv)[None, :] < nvis[:, None], s, -np.inf)
        M = s.max(axis=1)
        w = np.exp(s - M[:, None])
        return w @ V, M + np.log(w.sum(axis=1))          # forgot to divide by the sum
    mp.setattr(oa, "attention_rows", rows)


def _mutant_combine_linear(mp):
    def combine(part_o, part_lse):
        mx = part_lse.max(axis=-1)
        fin = np.isfinite(mx)
        w = np.where(np.isfinite(part_lse), 1.0, 0.0)
        W = np.maximum(w.sum(axis=-1), 1)
        O = np.where(fin[..., None], (w[..., None] * part_o).sum(axis=-2) / W[..., None], 0.0)
        return O, np.where(fin, mx, -np.inf)
    mp.setattr(oa, "combine_ref", combine)


def _mutant_online_no_rescale(mp):
    real_merge = oa._merge_running

    def merge(a, b):                                         # forgot to rescale the running acc
        m, l, acc = real_merge(a, b)
        wb = math.exp(b[0] - m) if b[0] != -math.inf else 0.0
        return m, l, a[2] + wb * b[2]
    mp.setattr(oa, "_merge_running", merge)


MUTANTS = [_mutant_causal_off_by_one, _mutant_causal_top_left, _mutant_scale_dropped, _mutant_scale_sign,
           _mutant_scale_sqrt, _mutant_gqa_modulo, _mutant_lse_log2, _mutant_lse_missing_max,
           _mutant_value_reversed, _mutant_no_normalise, _mutant_combine_linear, _mutant_online_no_rescale]


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m.__name__ for m in MUTANTS])
def test_planted_mistake_is_caught(mutant, monkeypatch):
    """A plausible mistake planted in the oracle (on the CPU) makes some pin fail."""
    mutant(monkeypatch)
    failed = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(oa)
        except (AssertionError, FloatingPointError, ValueError, ZeroDivisionError):
            failed.append(pin.__name__)
    assert failed, f"{mutant.__name__} passed every pin"
