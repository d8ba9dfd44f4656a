"""fa_decode_noalloc (partials in the library's per-GPU scratch) against fa_decode (caller's
workspace), through the C ABI: the same kernels on the same inputs, so the outputs must be
bitwise equal. Two calls in a row, the second smaller, so the second reads scratch that the
first left behind."""
import numpy as np
import pytest
import torch

from oracle.attention import decode_ref, widen_bf16
from synth import make_qkv
from tests.parity import check_lse, check_o, down, up

pytestmark = pytest.mark.gpu

CASES = [
    # B, Hq, Hkv, Skv, d, num_splits
    (16, 32, 8, 4100, 128, 3),
    (3, 8, 2, 700, 64, 2),
]


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import io_aware_exact_21_amd as fa
    return fa


def _inputs(B, Hq, Hkv, Skv, d, seed):
    q, k, v = make_qkv(B, Hq, Hkv, 1, Skv, d, seed=seed)
    return q.reshape(B, Hq, d), k, v


def test_noalloc_matches_decode_twice(fa):
    prev = None
    for i, (B, Hq, Hkv, Skv, d, ns) in enumerate(CASES):
        print(f"noalloc case {i}: B{B} Hq{Hq} Hkv{Hkv} Skv{Skv} d{d} splits {ns}", flush=True)
        q, k, v = _inputs(B, Hq, Hkv, Skv, d, seed=60 + i)
        tq, tk, tv = up(q), up(k), up(v)
        o_ref, l_ref = fa.decode(tq, tk, tv, num_splits=ns)
        o_na, l_na = fa.decode_noalloc(tq, tk, tv, num_splits=ns)
        torch.cuda.synchronize()
        assert torch.equal(o_na, o_ref) and torch.equal(l_na, l_ref)
        O, L = decode_ref(widen_bf16(q), widen_bf16(k), widen_bf16(v), scale=d ** -0.5)
        check_o(down(o_na), O, bf16=True)
        check_lse(down(l_na), L)
        if prev is not None:
            assert prev[0].shape != o_na.shape          # the second call is the smaller one
        prev = (o_na, l_na)


def test_noalloc_default_splits_and_limit(fa):
    from io_aware_exact_21_amd._lib import FA_ERR_WORKSPACE, FaError
    q, k, v = _inputs(4, 8, 2, 1000, 128, seed=70)
    tq, tk, tv = up(q), up(k), up(v)
    o_ref, l_ref = fa.decode(tq, tk, tv)
    o_na, l_na = fa.decode_noalloc(tq, tk, tv)
    torch.cuda.synchronize()
    assert torch.equal(o_na, o_ref) and torch.equal(l_na, l_ref)
    # 4 * 8 * 64 splits * 128 * 4 B = 1 MiB fits; a split count past the scratch size is refused
    big_q = torch.zeros((64, 32, 128), dtype=torch.bfloat16, device="cuda")
    big_kv = torch.zeros((64, 64 * 40, 8, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(FaError) as e:
        fa.decode_noalloc(big_q, big_kv, big_kv, num_splits=40)
    assert e.value.status == FA_ERR_WORKSPACE
