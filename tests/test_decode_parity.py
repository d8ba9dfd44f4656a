"""GPU parity of the split-KV decode kernels (partials + log-sum-exp merge) against the oracle."""
import math

import numpy as np
import pytest
import torch

from oracle.attention import combine_ref, decode_ref, split_partials_ref, widen_bf16
from synth import make_qkv
from tests.parity import check_lse, check_o, down, up

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import io_aware_exact_21_amd as fa
    return fa


def _inputs(B, Hq, Hkv, Skv, d, seed):
    q, k, v = make_qkv(B, Hq, Hkv, 1, Skv, d, seed)
    return q.reshape(B, Hq, d), k, v


CASES = [
    # B, Hq, Hkv, Skv, d, num_splits
    (1, 1, 1, 1, 64, 1), (2, 4, 1, 37, 128, 1), (2, 8, 2, 64, 128, 2), (2, 8, 2, 65, 128, 3),
    (3, 4, 4, 300, 64, 2), (2, 32, 8, 1000, 128, 8), (1, 8, 1, 1000, 128, 32), (2, 16, 4, 777, 64, 5),
    (1, 32, 1, 513, 128, 4), (2, 2, 2, 130, 128, 7),
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_decode_small(fa, case):
    B, Hq, Hkv, Skv, d, ns = case
    print(f"decode case {case}", flush=True)
    q, k, v = _inputs(B, Hq, Hkv, Skv, d, seed=200 + Skv + ns)
    sc = 1.0 / math.sqrt(d)
    o, lse = fa.decode(up(q), up(k), up(v), num_splits=ns)
    torch.cuda.synchronize()
    O, L = decode_ref(widen_bf16(q), widen_bf16(k), widen_bf16(v), scale=sc)
    check_o(down(o), O, bf16=True)
    check_lse(down(lse), L)


@pytest.mark.parametrize("case", CASES[1:7], ids=[str(c) for c in CASES[1:7]])
def test_partials_match_chunk_oracle(fa, case):
    """Each chunk's normalised output and LSE match the oracle over the same key range
    (empty chunks give 0 and -inf)."""
    B, Hq, Hkv, Skv, d, ns = case
    q, k, v = _inputs(B, Hq, Hkv, Skv, d, seed=300 + Skv)
    sc = 1.0 / math.sqrt(d)
    po, pl = fa.decode_partials(up(q), up(k), up(v), ns)
    torch.cuda.synchronize()
    bounds = fa.decode_chunk_bounds(Skv, ns)
    PO, PL = split_partials_ref(widen_bf16(q), widen_bf16(k), widen_bf16(v), scale=sc, bounds=bounds)
    check_o(down(po), PO, bf16=False, what="part_o")
    check_lse(down(pl), PL, what="part_lse")


def test_combine_alone(fa):
    """The merge kernel on synthetic partials, including chunks and whole rows with lambda = -inf."""
    rng = np.random.default_rng(7)
    B, Hq, n, d = 3, 5, 6, 128
    po = rng.standard_normal((B, Hq, n, d)).astype(np.float32)
    pl = (rng.standard_normal((B, Hq, n)) * 3 + 5).astype(np.float32)
    pl[0, 1, 2] = -np.inf
    pl[1, 2, :] = -np.inf
    po[1, 2, :] = 0.0
    o, lse = fa.decode_combine(torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda())
    torch.cuda.synchronize()
    O, L = combine_ref(po.astype(np.float64), pl.astype(np.float64))
    check_o(down(o), O, bf16=True)
    check_lse(down(lse), L)
    assert (down(o)[1, 2] == 0).all() and np.isneginf(down(lse)[1, 2])


def test_split_count_invariance(fa):
    q, k, v = _inputs(2, 8, 2, 2000, 128, seed=11)
    tq, tk, tv = up(q), up(k), up(v)
    ref = None
    for ns in (1, 2, 3, 8, 32, 64):
        o, lse = fa.decode(tq, tk, tv, num_splits=ns)
        torch.cuda.synchronize()
        if ref is None:
            ref = (down(o), down(lse))
        else:
            assert np.abs(down(o) - ref[0]).max() <= 2 * 2.0 ** -8 * max(1.0, np.abs(ref[0]).max())
            assert np.abs(down(lse) - ref[1]).max() < 1e-4


def test_decode_deterministic(fa):
    q, k, v = _inputs(4, 8, 2, 4000, 128, seed=12)
    tq, tk, tv = up(q), up(k), up(v)
    o1, l1 = fa.decode(tq, tk, tv)
    o2, l2 = fa.decode(tq, tk, tv)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
