"""Pins for the backward oracle (attention_bwd_ref) against facts it does not share code with.

The oracle writes the chain rule out by hand. These tests hold it to:
  * central finite differences of the forward oracle (itself pinned in test_oracle.py),
    element by element on tiny shapes and along random directions on larger ones;
  * reverse-mode autodiff (torch, float64, CPU) of a plain masked-softmax formula;
  * exact identities of the gradient: sum_j dK_j = 0, sum_j dV_j = sum of dO over rows
    that see a key, dQ = 0 for a row with one key or with none, zero scale;
  * the grouped-query reduction: a KV head's gradient is the sum over its query heads.
"""
import numpy as np
import pytest
import torch

from oracle.attention import attention_bwd_ref, attention_ref, visible_keys

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _inputs(B, Sq, Skv, Hq, Hkv, d, seed, spread=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Sq, Hq, d)) * spread
    k = rng.standard_normal((B, Skv, Hkv, d)) * spread
    v = rng.standard_normal((B, Skv, Hkv, d))
    do = rng.standard_normal((B, Sq, Hq, d))
    return q, k, v, do


def _loss(q, k, v, do, causal, scale):
    return float((attention_ref(q, k, v, causal=causal, scale=scale)[0] * do).sum())


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 5, 7, 2, 1, 4), (2, 6, 4, 2, 2, 3), (1, 4, 4, 3, 1, 2)])
def test_elementwise_finite_differences(causal, shape):
    # (1,6,4,...) with causal has rows that see no key (Sq > Skv, bottom-right alignment)
    q, k, v, do = _inputs(*shape, seed=11)
    scale = 0.7
    dq, dk, dv = attention_bwd_ref(q, k, v, do, causal=causal, scale=scale)
    h = 1e-5
    args = {"q": q, "k": k, "v": v}
    for name, g in (("q", dq), ("k", dk), ("v", dv)):
        x = args[name]
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            fd = (_loss(**{**args, name: xp}, do=do, causal=causal, scale=scale)
                  - _loss(**{**args, name: xm}, do=do, causal=causal, scale=scale)) / (2 * h)
            assert abs(fd - g[idx]) < 1e-8 * max(1.0, abs(fd)), (name, idx, fd, g[idx])


@pytest.mark.parametrize("causal", [False, True])
def test_directional_derivative(causal):
    # larger shape, grouped heads, several row blocks of the oracle
    q, k, v, do = _inputs(2, 40, 56, 4, 2, 16, seed=12, spread=1.5)
    scale = 16 ** -0.5
    dq, dk, dv = attention_bwd_ref(q, k, v, do, causal=causal, scale=scale, row_block=16)
    rng = np.random.default_rng(13)
    for name in ("q", "k", "v"):
        args = {"q": q, "k": k, "v": v}
        dirn = rng.standard_normal(args[name].shape)
        g = {"q": dq, "k": dk, "v": dv}[name]
        h = 1e-5
        lp = _loss(**{**args, name: args[name] + h * dirn}, do=do, causal=causal, scale=scale)
        lm = _loss(**{**args, name: args[name] - h * dirn}, do=do, causal=causal, scale=scale)
        fd = (lp - lm) / (2 * h)
        an = float((g * dirn).sum())
        assert abs(fd - an) < 1e-7 * max(1.0, abs(fd)), (name, fd, an)


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_autograd(causal):
    B, Sq, Skv, Hq, Hkv, d = 1, 33, 47, 4, 2, 8
    q, k, v, do = _inputs(B, Sq, Skv, Hq, Hkv, d, seed=14, spread=2.0)
    scale = float(np.float32(0.35))
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    g = Hq // Hkv
    ke = tk.repeat_interleave(g, dim=2)                        # [B,Skv,Hq,d]
    ve = tv.repeat_interleave(g, dim=2)
    s = torch.einsum("bihc,bjhc->bhij", tq, ke) * scale
    if causal:
        i = torch.arange(Sq)[:, None]
        j = torch.arange(Skv)[None, :]
        s = s.masked_fill(j > i + Skv - Sq, float("-inf"))
    p = torch.softmax(s, dim=-1)
    o = torch.einsum("bhij,bjhc->bihc", p, ve)
    (o * torch.tensor(do)).sum().backward()
    dq, dk, dv = attention_bwd_ref(q, k, v, do, causal=causal, scale=scale, row_block=8)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_identities(causal):
    B, Sq, Skv, Hq, Hkv, d = 2, 24, 20, 4, 2, 8
    q, k, v, do = _inputs(B, Sq, Skv, Hq, Hkv, d, seed=15)
    dq, dk, dv = attention_bwd_ref(q, k, v, do, causal=causal, scale=0.4, row_block=7)
    # softmax rows sum to one: the score gradient of a row sums to zero, so sum_j dK_j = 0
    np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-12)
    # and sum_j dV_j = sum of dO over the rows (of every query head of the group) that see a key
    seen = np.array([visible_keys(i, Sq, Skv, causal) > 0 for i in range(Sq)])
    g = Hq // Hkv
    want = (do * seen[None, :, None, None]).sum(axis=1).reshape(B, Hkv, g, d).sum(axis=2)
    np.testing.assert_allclose(dv.sum(axis=1), want, atol=1e-12)
    # a row that sees exactly one key has P = 1 and dS = 0; a row that sees none has no gradient
    for i in range(Sq):
        if visible_keys(i, Sq, Skv, causal) <= 1:
            assert np.all(dq[:, i] == 0.0)


def test_single_key_and_zero_scale():
    q, k, v, do = _inputs(1, 6, 1, 2, 1, 4, seed=16)
    dq, dk, dv = attention_bwd_ref(q, k, v, do, causal=False, scale=0.9)
    assert np.all(dq == 0) and np.all(dk == 0)
    np.testing.assert_allclose(dv[0, 0, 0], do[0].sum(axis=(0, 1)), atol=1e-14)
    # zero scale: uniform weights, dQ = dK = 0, dV_j = sum_i dO_i / n
    q, k, v, do = _inputs(1, 5, 9, 1, 1, 4, seed=17)
    dq, dk, dv = attention_bwd_ref(q, k, v, do, causal=False, scale=0.0)
    assert np.all(dq == 0) and np.all(dk == 0)
    np.testing.assert_allclose(dv[0, :, 0], np.broadcast_to(do[0, :, 0].sum(axis=0) / 9, (9, 4)), atol=1e-14)


def test_grouped_heads_sum_over_group():
    B, Sq, Skv, Hq, Hkv, d = 1, 12, 16, 6, 2, 4
    q, k, v, do = _inputs(B, Sq, Skv, Hq, Hkv, d, seed=18)
    dq, dk, dv = attention_bwd_ref(q, k, v, do, causal=True, scale=0.5)
    g = Hq // Hkv
    ke, ve = np.repeat(k, g, axis=2), np.repeat(v, g, axis=2)   # one KV head per query head
    dq1, dk1, dv1 = attention_bwd_ref(q, ke, ve, do, causal=True, scale=0.5)
    np.testing.assert_allclose(dq, dq1, atol=1e-13)
    np.testing.assert_allclose(dk, dk1.reshape(B, Skv, Hkv, g, d).sum(axis=3), atol=1e-13)
    np.testing.assert_allclose(dv, dv1.reshape(B, Skv, Hkv, g, d).sum(axis=3), atol=1e-13)


def test_sensitivity_sums():
    # the sensitivity sums bound the gradients (triangle inequality), equal dV when every
    # term has one sign (dO >= 0; dV does not depend on D), and do not change the gradients
    q, k, v, do = _inputs(1, 30, 40, 4, 2, 8, seed=19)
    for causal in (False, True):
        g = attention_bwd_ref(q, k, v, do, causal=causal, scale=-0.45, row_block=11)
        ga = attention_bwd_ref(q, k, v, do, causal=causal, scale=-0.45, row_block=11, abs_terms=True)
        assert len(g) == 3 and len(ga) == 9
        for x, y, a, r in zip(g, ga[:3], ga[3:6], ga[6:]):
            np.testing.assert_array_equal(x, y)
            assert np.all(np.abs(x) <= a + 1e-12)
            assert np.all(r <= a + 1e-12)                      # root-sum-square <= sum of magnitudes
        pos = np.abs(do)
        dv, adv = attention_bwd_ref(q, k, v, pos, causal=causal, scale=0.3, abs_terms=True)[2:6:3]
        np.testing.assert_allclose(dv, adv, rtol=1e-13, atol=1e-15)


def test_sensitivity_bounds_rounding_of_o_in_d():
    # Rounding O to bf16 inside D = dO . O moves dQ and dK by at most u * (sensitivity):
    # recompute the gradients with D from a bf16-rounded O and compare.
    from oracle.attention import visible_keys as vk
    from synth import bf16_rne_bits
    q, k, v, do = _inputs(1, 24, 24, 2, 1, 16, seed=20, spread=2.5)
    scale = -0.6                                               # peaked rows: dS = P (dP - D) cancels
    dq, dk, dv, aq, ak, av = attention_bwd_ref(q, k, v, do, causal=True, scale=scale, abs_terms=True)[:6]
    O = attention_ref(q, k, v, causal=True, scale=scale)[0]
    Ob = (bf16_rne_bits(O).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    sig = float(np.float32(scale))
    gq = np.zeros_like(dq)
    gk = np.zeros_like(dk)
    for h in range(2):
        for i in range(24):
            n = vk(i, 24, 24, True)
            s = sig * (k[0, :n, 0] @ q[0, i, h])
            P = np.exp(s - s.max())
            P /= P.sum()
            dS = P * (v[0, :n, 0] @ do[0, i, h] - (do[0, i, h] * Ob[0, i, h]).sum())
            gq[0, i, h] = sig * (dS @ k[0, :n, 0])
            gk[0, :n, 0] += sig * np.outer(dS, q[0, i, h])
    u = 2.0 ** -8
    assert np.all(np.abs(gq - dq) <= u * aq + 1e-12)
    assert np.all(np.abs(gk - dk) <= u * ak + 1e-12)
    assert np.abs(gq - dq).max() > 1e-3                       # the effect is real, not negligible


def test_rss_sensitivity_matches_simulated_rounding():
    # Perturb every rounded factor by an independent relative error uniform in [-u, u]
    # (dS, P, and each O element inside D) and compare the RMS change of the gradients
    # with (u / sqrt(3)) times the oracle's root-sum-square sensitivity.
    from oracle.attention import visible_keys as vk
    B, Sq, Skv, Hq, Hkv, d = 1, 20, 20, 2, 1, 8
    q, k, v, do = _inputs(B, Sq, Skv, Hq, Hkv, d, seed=21, spread=2.0)
    scale, u, T = 0.55, 2.0 ** -8, 300
    res = attention_bwd_ref(q, k, v, do, causal=True, scale=scale, abs_terms=True)
    g, r = res[:3], res[6:]
    rng = np.random.default_rng(22)
    sq = [np.zeros_like(x) for x in g]
    sig = float(np.float32(scale))
    for _ in range(T):
        gq, gk, gv = np.zeros_like(g[0]), np.zeros_like(g[1]), np.zeros_like(g[2])
        for h in range(Hq):
            for i in range(Sq):
                n = vk(i, Sq, Skv, True)
                s = sig * (k[0, :n, 0] @ q[0, i, h])
                P = np.exp(s - s.max())
                P /= P.sum()
                O = P @ v[0, :n, 0]
                Dp = (do[0, i, h] * O * (1 + u * rng.uniform(-1, 1, d))).sum()
                dS = P * (v[0, :n, 0] @ do[0, i, h] - Dp) * (1 + u * rng.uniform(-1, 1, n))
                Pp = P * (1 + u * rng.uniform(-1, 1, n))
                gq[0, i, h] = sig * (dS @ k[0, :n, 0])
                gk[0, :n, 0] += sig * np.outer(dS, q[0, i, h])
                gv[0, :n, 0] += np.outer(Pp, do[0, i, h])
        for acc, x, y in zip(sq, (gq, gk, gv), g):
            acc += (x - y) ** 2
    for acc, rr in zip(sq, r):
        ratio = np.linalg.norm(np.sqrt(acc / T)) / np.linalg.norm(u / np.sqrt(3.0) * rr)
        assert 0.9 < ratio < 1.1, ratio
