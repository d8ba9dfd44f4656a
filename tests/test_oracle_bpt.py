"""Pins for the feed-forward oracle (ffn_ref) and the attention + FFN layer (bpt_layer_ref)."""
import itertools

import numpy as np

from oracle.attention import attention_ref, bpt_layer_ref, ffn_ref, widen_bf16
from synth import make_ffn_weights


def test_ffn_closed_form_identity():
    # W1 = [I; -I] (out = 2d rows), W2 = [I, -I], no bias: relu(h) - relu(-h) = h
    d = 6
    rng = np.random.default_rng(1)
    h = rng.standard_normal((5, d))
    w1 = np.concatenate([np.eye(d), -np.eye(d)], axis=0)
    w2 = np.concatenate([np.eye(d), -np.eye(d)], axis=1)
    np.testing.assert_allclose(ffn_ref(h, w1, np.zeros(2 * d), w2, np.zeros(d)), h, atol=1e-15)


def test_ffn_brute_force_loops():
    rng = np.random.default_rng(2)
    dm, dff = 3, 5
    # weights stored as linear layers: w1[j, k] maps input k to hidden unit j, w2[n, j]
    # maps hidden unit j to output n
    h, w1, b1 = rng.standard_normal((4, dm)), rng.standard_normal((dff, dm)), rng.standard_normal(dff)
    w2, b2 = rng.standard_normal((dm, dff)), rng.standard_normal(dm)
    y = ffn_ref(h, w1, b1, w2, b2)
    for t, n in itertools.product(range(4), range(dm)):
        acc = b2[n]
        for j in range(dff):
            z = b1[j] + sum(h[t, kk] * w1[j, kk] for kk in range(dm))
            acc += max(z, 0.0) * w2[n, j]
        assert abs(acc - y[t, n]) < 1e-12


def test_ffn_acts_per_token():
    # each output row depends only on its own input row: permuting tokens permutes outputs
    rng = np.random.default_rng(3)
    h = rng.standard_normal((9, 4))
    w1, b1, w2, b2 = rng.standard_normal((8, 4)), rng.standard_normal(8), rng.standard_normal((4, 8)), rng.standard_normal(4)
    perm = rng.permutation(9)
    np.testing.assert_allclose(ffn_ref(h[perm], w1, b1, w2, b2), ffn_ref(h, w1, b1, w2, b2)[perm], atol=1e-14)


def test_layer_is_ffn_of_attention_and_blockwise_equal():
    rng = np.random.default_rng(4)
    B, S, H, d = 2, 20, 2, 4
    q, k, v = (rng.standard_normal((B, S, H, d)) for _ in range(3))
    w1, b1, w2, b2 = rng.standard_normal((32, H * d)), rng.standard_normal(32), rng.standard_normal((H * d, 32)), rng.standard_normal(H * d)
    y = bpt_layer_ref(q, k, v, w1, b1, w2, b2, causal=True, scale=0.5)
    O = attention_ref(q, k, v, causal=True, scale=0.5)[0].reshape(B, S, H * d)
    np.testing.assert_allclose(y, ffn_ref(O, w1, b1, w2, b2), atol=1e-13)
    # the blockwise schedule: FFN of each query block's attention output, blocks of 7 rows
    blocks = [ffn_ref(O[:, r0:r0 + 7], w1, b1, w2, b2) for r0 in range(0, S, 7)]
    np.testing.assert_allclose(np.concatenate(blocks, axis=1), y, atol=1e-13)


def test_ffn_weights_recipe():
    w1, b1, w2, b2 = make_ffn_weights(64, 256, seed=5)
    assert w1.shape == (256, 64) and b1.shape == (256,) and w2.shape == (64, 256) and b2.shape == (64,)
    assert abs(widen_bf16(w1).std() * 8 - 1) < 0.05 and abs(widen_bf16(w2).std() * 16 - 1) < 0.05
    assert abs(widen_bf16(b1).std() * 10 - 1) < 0.2
    w1b = make_ffn_weights(64, 256, seed=5)[0]
    assert np.array_equal(w1, w1b)
