"""GPU parity of the paged-cache split-KV decode against the paged oracle."""
import numpy as np
import pytest
import torch

from oracle.attention import paged_decode_ref, widen_bf16
from synth import PAGED_WORKLOADS, make_paged_decode, make_paged_workload
from tests.parity import check_lse, check_o, down, up

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import io_aware_exact_21_amd as fa
    return fa


def _run(fa, q, kp, vp, table, lens, ns, scale):
    dev = torch.device("cuda:0")
    o, lse = fa.decode_paged(up(q), up(kp), up(vp), torch.from_numpy(table).to(dev),
                             torch.from_numpy(np.asarray(lens, dtype=np.int32)).to(dev), scale=scale, num_splits=ns)
    torch.cuda.synchronize()
    return down(o), down(lse)


CASES = [
    # B, Hq, Hkv, d, page_size, lengths, num_splits
    (3, 8, 2, 128, 16, [200, 1, 17], 1),
    (3, 8, 2, 128, 16, [200, 1, 17], 3),
    (4, 4, 4, 64, 32, [0, 63, 64, 65], 2),
    (2, 32, 8, 128, 64, [1000, 333], 4),
    (2, 16, 1, 128, 128, [129, 1024], 8),
    (5, 8, 8, 64, 16, [15, 16, 31, 600, 2], 5),
    (1, 32, 1, 128, 256, [700], 2),
    (2, 8, 2, 128, 16, [40, 7], 16),       # more splits than 64-key tiles: leading chunks empty
    (2, 8, 2, 128, 32, [0, 0], 2),
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_paged_small(fa, case):
    B, Hq, Hkv, d, ps, lens, ns = case
    print(f"paged case {case}", flush=True)
    q, kp, vp, table, sl = make_paged_decode(B, Hq, Hkv, d, ps, lens, seed=400 + ps + ns, spare_pages=5)
    sc = float(np.float32(d ** -0.5))
    o, lse = _run(fa, q, kp, vp, table, sl, ns, sc)
    O, L = paged_decode_ref(widen_bf16(q), widen_bf16(kp), widen_bf16(vp), table, sl, scale=sc)
    check_o(o, O, bf16=True)
    check_lse(lse, L)


def test_paged_split_counts_agree(fa):
    """Every split count gives the oracle's answer (within tolerance)."""
    q, kp, vp, table, sl = make_paged_decode(2, 8, 2, 128, 16, [999, 512], seed=77, spare_pages=3)
    sc = float(np.float32(128 ** -0.5))
    O, L = paged_decode_ref(widen_bf16(q), widen_bf16(kp), widen_bf16(vp), table, sl, scale=sc)
    for ns in (1, 2, 3, 8, 16):
        o, lse = _run(fa, q, kp, vp, table, sl, ns, sc)
        check_o(o, O, bf16=True)
        check_lse(lse, L)


def test_paged_workload_full(fa):
    """The benchmark's paged workload at full size, every sequence and head."""
    w = PAGED_WORKLOADS["paged"]
    q, kp, vp, table, sl = make_paged_workload(w)
    o, lse = _run(fa, q, kp, vp, table, sl, 0, w.scale)
    O, L = paged_decode_ref(widen_bf16(q), widen_bf16(kp), widen_bf16(vp), table, sl, scale=w.scale)
    check_o(o, O, bf16=True)
    check_lse(lse, L)


def test_paged_deterministic(fa):
    q, kp, vp, table, sl = make_paged_decode(2, 16, 4, 128, 32, [800, 77], seed=78)
    a = _run(fa, q, kp, vp, table, sl, 4, 0.1)
    b = _run(fa, q, kp, vp, table, sl, 4, 0.1)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
