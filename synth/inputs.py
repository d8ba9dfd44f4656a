"""Seeded synthetic inputs for the attention workloads.

This module holds no attention arithmetic. It draws standard-normal samples,
rounds them to bfloat16 storage (raw uint16 bit patterns) and lays them out in
the [B, S, H, d] shapes of the five workloads. The oracle tests, the GPU parity
tests and the benchmark all take their inputs from here, so both sides of every
comparison see the same bits.

Recipe (the pages state only "i.i.d. N(0,1) from seed"; this is the reading):

* Every tensor is split into blocks of ``ROWS_PER_BLOCK`` token rows per batch
  element. Block (tensor t, batch b, block n) draws float64 standard normals
  from ``default_rng(SeedSequence(seed, spawn_key=(t, b, n)))`` (PCG64). The
  tensor ids are Q=0, K=1, V=2. Blocks are independent, so generation runs in
  parallel threads and the seed -> tensor map is fixed.
* Each float64 sample is rounded straight to bfloat16, round-to-nearest-even.
* The long-prefill workload then multiplies K by 4 at round(0.01 * Skv)
  distinct token positions per batch element (all KV heads). The positions come
  from ``default_rng(SeedSequence(seed, spawn_key=(3, b))).choice(Skv, n,
  replace=False)``. Multiplying by 4 only adds 2 to the exponent, so it is exact.
* The loss gradient dO of a backward step is drawn like Q (same shape, same
  recipe) with tensor id 5.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

ROWS_PER_BLOCK = 1024
TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_STRESS, TENSOR_PAGES, TENSOR_DO = 0, 1, 2, 3, 4, 5


@dataclass(frozen=True)
class Workload:
    """One attention workload: shapes, mask, seed and input structure."""
    name: str
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Skv: int
    d: int
    causal: bool
    seed: int
    decode: bool = False          # q_len = 1 against a KV cache, split-KV path
    k_stress_frac: float = 0.0    # fraction of K token positions multiplied by 4

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(d), as the fp32 value the library receives."""
        return float(np.float32(1.0 / np.sqrt(self.d)))

    def describe(self) -> dict:
        return {"workload": self.name, "B": self.B, "Hq": self.Hq, "Hkv": self.Hkv,
                "Sq": self.Sq, "Skv": self.Skv, "d": self.d, "causal": self.causal,
                "dtype_io": "bf16", "layout": "[B,S,H,d]"}


WORKLOADS = {
    "tiny": Workload("tiny exact-check B1 H1 S256 d64 non-causal",
                     1, 1, 1, 256, 256, 64, False, 1001),
    "mha2k": Workload("MHA prefill B4 H16 S2048 d64 causal",
                      4, 16, 16, 2048, 2048, 64, True, 1002),
    "mha8k": Workload("MHA long prefill B2 H32 S8192 d128 causal, K x4 on 1% of positions",
                      2, 32, 32, 8192, 8192, 128, True, 1003, k_stress_frac=0.01),
    "gqa32k": Workload("GQA prefill B1 Hq32 Hkv8 S32768 d128 causal",
                       1, 32, 8, 32768, 32768, 128, True, 1004),
    "decode": Workload("split-KV decode B64 Hq32 Hkv8 Skv16384 d128",
                       64, 32, 8, 1, 16384, 128, False, 1005, decode=True),
}


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def bf16_rne_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16 (round-to-nearest-even); return uint16 bits.

    bfloat16 keeps 8 significant bits. For a value with binary exponent e
    (x = f * 2**e, 0.5 <= |f| < 1) the representable spacing is 2**(e-8), and
    never finer than the subnormal spacing 2**-133. ``np.rint`` rounds half to
    even, so rint(x / spacing) * spacing is the RNE result, exact in float64.
    The rounded value fits float32 exactly, whose upper 16 bits are the bf16
    pattern. Values beyond the bf16 range become +-inf; NaN stays NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    spacing = np.ldexp(1.0, np.maximum(e, -125) - 8)
    r = np.rint(x / spacing) * spacing
    with np.errstate(over="ignore"):
        r32 = r.astype(np.float32)
    big = np.abs(r) >= 2.0 ** 128
    if big.any():
        r32 = np.where(big, np.copysign(np.float32(np.inf), r32), r32)
    return (r32.view(np.uint32) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _fill_block(out: np.ndarray, seed: int, key: tuple) -> None:
    rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=key))
    out[...] = bf16_rne_bits(rng.standard_normal(out.shape))


def normal_bf16(shape: tuple, seed: int, tensor_id: int, pool=None) -> np.ndarray:
    """i.i.d. N(0,1) rounded to bf16, shape [B, S, H, d], as uint16 bits."""
    B, S = shape[0], shape[1]
    out = np.empty(shape, dtype=np.uint16)
    jobs = []
    for b in range(B):
        for n, s0 in enumerate(range(0, S, ROWS_PER_BLOCK)):
            jobs.append((out[b, s0:s0 + ROWS_PER_BLOCK], (tensor_id, b, n)))
    if pool is None or len(jobs) == 1:
        for view, key in jobs:
            _fill_block(view, seed, key)
    else:
        list(pool.map(lambda j: _fill_block(j[0], seed, j[1]), jobs))
    return out


def stress_positions(seed: int, b: int, Skv: int, frac: float) -> np.ndarray:
    """Token positions of batch element b whose K rows are multiplied by 4."""
    n = int(round(frac * Skv))
    rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(TENSOR_STRESS, b)))
    return np.sort(rng.choice(Skv, size=n, replace=False))


def times4_bf16(bits: np.ndarray) -> np.ndarray:
    """Multiply bf16 values by 4 (exact: exponent + 2), returning bits."""
    f = bf16_bits_to_f32(bits) * np.float32(4.0)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def make_qkv(B: int, Hq: int, Hkv: int, Sq: int, Skv: int, d: int, seed: int,
             k_stress_frac: float = 0.0):
    """Q [B,Sq,Hq,d], K and V [B,Skv,Hkv,d] as bf16 bit arrays (uint16)."""
    with ThreadPoolExecutor(_threads()) as pool:
        q = normal_bf16((B, Sq, Hq, d), seed, TENSOR_Q, pool)
        k = normal_bf16((B, Skv, Hkv, d), seed, TENSOR_K, pool)
        v = normal_bf16((B, Skv, Hkv, d), seed, TENSOR_V, pool)
    if k_stress_frac > 0.0:
        for b in range(B):
            pos = stress_positions(seed, b, Skv, k_stress_frac)
            k[b, pos] = times4_bf16(k[b, pos])
    return q, k, v


def make_grad_out(B: int, Sq: int, Hq: int, d: int, seed: int) -> np.ndarray:
    """Loss gradient dO [B,Sq,Hq,d] for a backward step, bf16 bits (tensor id 5)."""
    with ThreadPoolExecutor(_threads()) as pool:
        return normal_bf16((B, Sq, Hq, d), seed, TENSOR_DO, pool)


def make_workload(w: Workload):
    """Inputs of a named workload. Decode q is [B,Hq,d] (= [B,1,Hq,d])."""
    q, k, v = make_qkv(w.B, w.Hq, w.Hkv, w.Sq, w.Skv, w.d, w.seed, w.k_stress_frac)
    if w.decode:
        q = q.reshape(w.B, w.Hq, w.d)
    return q, k, v


@dataclass(frozen=True)
class PagedWorkload:
    """A decode step over a paged KV cache: variable lengths, shuffled pages."""
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    page_size: int
    max_len: int          # longest sequence (max_blocks = max_len / page_size)
    min_len: int          # shortest sequence
    seed: int
    spare_pages: int = 64  # pages that belong to no sequence (filled with data too)

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / np.sqrt(self.d)))

    def describe(self) -> dict:
        return {"workload": self.name, "B": self.B, "Hq": self.Hq, "Hkv": self.Hkv, "d": self.d,
                "page_size": self.page_size, "seq_len_range": [self.min_len, self.max_len],
                "dtype_io": "bf16", "layout": "pages [P, page, Hkv, d], block table [B, max_blocks]"}


PAGED_WORKLOADS = {
    "paged": PagedWorkload("paged split-KV decode B64 Hq32 Hkv8 d128 page16, lengths 4096..16384",
                           64, 32, 8, 128, 16, 16384, 4096, 1006),
}


def paged_layout(B: int, page_size: int, seq_lens: np.ndarray, max_blocks: int, seed: int,
                 spare_pages: int = 0):
    """Block table [B, max_blocks] int32 and the page count for the given lengths.

    Sequence b uses ceil(seq_lens[b] / page_size) pages. All used pages plus
    ``spare_pages`` unused ones are numbered, shuffled with
    ``default_rng(SeedSequence(seed, spawn_key=(4,)))`` and dealt out in sequence
    order; unused table slots point at page 0.
    """
    need = [(int(n) + page_size - 1) // page_size for n in seq_lens]
    total = sum(need) + spare_pages
    rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(TENSOR_PAGES,)))
    perm = rng.permutation(total).astype(np.int32)
    table = np.zeros((B, max_blocks), dtype=np.int32)
    pos = 0
    for b in range(B):
        table[b, :need[b]] = perm[pos:pos + need[b]]
        pos += need[b]
    return table, total


def make_paged_decode(B: int, Hq: int, Hkv: int, d: int, page_size: int, seq_lens, seed: int,
                      spare_pages: int = 0, max_blocks: int | None = None):
    """q [B,Hq,d], k_pages/v_pages [P,page,Hkv,d] (bf16 bits), block table, seq_lens.

    The page pools are i.i.d. N(0,1) rounded to bf16 (pages drawn like token rows
    of a [1, P*page, Hkv, d] tensor); q likewise.
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    mb = max_blocks if max_blocks is not None else max(1, int(max((int(n) + page_size - 1) // page_size
                                                                for n in seq_lens)))
    table, P = paged_layout(B, page_size, seq_lens, mb, seed, spare_pages)
    with ThreadPoolExecutor(_threads()) as pool:
        q = normal_bf16((B, 1, Hq, d), seed, TENSOR_Q, pool).reshape(B, Hq, d)
        k = normal_bf16((1, P * page_size, Hkv, d), seed, TENSOR_K, pool).reshape(P, page_size, Hkv, d)
        v = normal_bf16((1, P * page_size, Hkv, d), seed, TENSOR_V, pool).reshape(P, page_size, Hkv, d)
    return q, k, v, table, seq_lens


def paged_seq_lens(w: PagedWorkload) -> np.ndarray:
    """Lengths of a paged workload: uniform integers in [min_len, max_len]."""
    rng = np.random.default_rng(np.random.SeedSequence(w.seed, spawn_key=(TENSOR_PAGES, 1)))
    return rng.integers(w.min_len, w.max_len + 1, size=w.B).astype(np.int32)


def make_paged_workload(w: PagedWorkload):
    lens = paged_seq_lens(w)
    return make_paged_decode(w.B, w.Hq, w.Hkv, w.d, w.page_size, lens, w.seed, w.spare_pages,
                             max_blocks=w.max_len // w.page_size)


TENSOR_W1, TENSOR_B1, TENSOR_W2, TENSOR_B2 = 6, 7, 8, 9


def _normal_2d(rows: int, cols: int, seed: int, tensor_id: int) -> np.ndarray:
    out = np.empty((rows, cols), dtype=np.float64)
    for n, r0 in enumerate(range(0, rows, ROWS_PER_BLOCK)):
        rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(tensor_id, 0, n)))
        out[r0:r0 + ROWS_PER_BLOCK] = rng.standard_normal(out[r0:r0 + ROWS_PER_BLOCK].shape)
    return out


def make_ffn_weights(d_model: int, d_ff: int, seed: int):
    """Feed-forward weights as bf16 bits, each layer as a linear layer's [out, in] weight:
    W1 [d_ff, d_model], b1 [d_ff], W2 [d_model, d_ff], b2 [d_model]. W1 and W2 are
    N(0,1) / sqrt(fan-in) (so activations stay of order one), the biases N(0,1) / 10;
    blocks of 1024 rows seeded SeedSequence(seed, (id, 0, n)) with ids 6, 7, 8, 9;
    rounded to bf16 (RNE)."""
    w1 = bf16_rne_bits(_normal_2d(d_ff, d_model, seed, TENSOR_W1) / np.sqrt(d_model))
    b1 = bf16_rne_bits(_normal_2d(1, d_ff, seed, TENSOR_B1)[0] / 10.0)
    w2 = bf16_rne_bits(_normal_2d(d_model, d_ff, seed, TENSOR_W2) / np.sqrt(d_ff))
    b2 = bf16_rne_bits(_normal_2d(1, d_model, seed, TENSOR_B2)[0] / 10.0)
    return w1, b1, w2, b2
