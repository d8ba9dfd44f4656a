"""Seeded fp8 (OCP e4m3) inputs for the fp8 attention variant.

Input preparation only: no attention arithmetic. The same float64 standard-normal
draws as the bf16 workloads (``synth.inputs`` recipe, tensor ids Q=0, K=1, V=2, the
same K x4 stress positions) are quantised per (batch, head) to OCP e4m3 codes:

* scale = float32(amax / 448), amax = the largest |x| of that (batch, head) slice,
  so the largest value maps onto the largest finite code (448);
* code = round-to-nearest-even of x / scale to e4m3 (sign, 4 exponent bits with
  bias 7, 3 mantissa bits; subnormals below 2^-6; no infinities; 0x7F and 0xFF are
  NaN and never produced here);
* the dequantised value is decode(code) * scale.

Layouts: q [B, Sq, Hq, d] and k [B, Skv, Hkv, d] as uint8 codes; v is stored
transposed, [B, Hkv, d, ldv] with ldv = Skv rounded up to 16 and zero padding;
descales q_scale [B, Hq], k_scale and v_scale [B, Hkv] float32.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .inputs import (ROWS_PER_BLOCK, TENSOR_K, TENSOR_Q, TENSOR_V, _threads, stress_positions)

E4M3_MAX = 448.0


def _e4m3_table() -> tuple:
    codes = np.arange(128, dtype=np.uint8)
    e = (codes >> 3).astype(np.int64)
    m = (codes & 7).astype(np.float64)
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    return codes[:127], val[:127]          # 0x7F is NaN


_CODES, _VALS = _e4m3_table()


def e4m3_rne_codes(x: np.ndarray) -> np.ndarray:
    """float64 -> e4m3 codes, round to nearest, ties to the even code. |x| must be <= 448."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(~np.isfinite(x)) or np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("values outside the finite e4m3 range")
    a = np.abs(x)
    hi = np.searchsorted(_VALS, a, side="left")               # first value >= a
    hi = np.minimum(hi, len(_VALS) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = a - _VALS[lo], _VALS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (_CODES[hi] % 2 == 0))
    idx = np.where(a <= _VALS[0], 0, np.where(pick_hi, hi, lo))
    mag = _CODES[idx]
    return np.where(np.signbit(x) & (mag != 0), mag | 0x80, mag).astype(np.uint8)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """e4m3 codes -> float64 (for input preparation and checks in this module)."""
    c = np.asarray(codes, dtype=np.uint8)
    v = _VALS[np.minimum(c & 0x7F, 126)]
    v = np.where((c & 0x7F) == 0x7F, np.nan, v)
    return np.where(c & 0x80, -v, v)


def _fill_f64(out: np.ndarray, seed: int, key: tuple) -> None:
    rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=key))
    out[...] = rng.standard_normal(out.shape)


def normal_f64(shape: tuple, seed: int, tensor_id: int, pool=None) -> np.ndarray:
    """The float64 draws behind ``normal_bf16`` (same blocks and seeds), unrounded."""
    B, S = shape[0], shape[1]
    out = np.empty(shape, dtype=np.float64)
    jobs = [(out[b, s0:s0 + ROWS_PER_BLOCK], (tensor_id, b, n))
            for b in range(B) for n, s0 in enumerate(range(0, S, ROWS_PER_BLOCK))]
    if pool is None or len(jobs) == 1:
        for view, key in jobs:
            _fill_f64(view, seed, key)
    else:
        list(pool.map(lambda j: _fill_f64(j[0], seed, j[1]), jobs))
    return out


def quantize_heads(x: np.ndarray) -> tuple:
    """x [B, S, H, d] float64 -> (codes uint8 [B, S, H, d], scale float32 [B, H])."""
    amax = np.abs(x).max(axis=(1, 3))                          # [B, H]
    scale = (amax / E4M3_MAX).astype(np.float32)
    scale = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    y = x / scale.astype(np.float64)[:, None, :, None]
    y = np.clip(y, -E4M3_MAX, E4M3_MAX)                        # float32 scale may round amax/scale above 448
    return e4m3_rne_codes(y), scale


def v_transposed(v_codes: np.ndarray) -> tuple:
    """v codes [B, Skv, Hkv, d] -> ([B, Hkv, d, ldv] with ldv = Skv rounded up to 16, zero padded, ldv)."""
    B, Skv, Hkv, d = v_codes.shape
    ldv = (Skv + 15) // 16 * 16
    vt = np.zeros((B, Hkv, d, ldv), dtype=np.uint8)
    vt[..., :Skv] = v_codes.transpose(0, 2, 3, 1)
    return vt, ldv


def make_fp8_qkv(B: int, Hq: int, Hkv: int, Sq: int, Skv: int, d: int, seed: int, k_stress_frac: float = 0.0):
    """(q8, k8, vt8, q_scale, k_scale, v_scale, ldv) for the fp8 variant, from the bf16 recipe's draws."""
    with ThreadPoolExecutor(_threads()) as pool:
        q = normal_f64((B, Sq, Hq, d), seed, TENSOR_Q, pool)
        k = normal_f64((B, Skv, Hkv, d), seed, TENSOR_K, pool)
        v = normal_f64((B, Skv, Hkv, d), seed, TENSOR_V, pool)
    if k_stress_frac > 0.0:
        for b in range(B):
            k[b, stress_positions(seed, b, Skv, k_stress_frac)] *= 4.0
    q8, qs = quantize_heads(q)
    del q
    k8, ks = quantize_heads(k)
    del k
    v8, vs = quantize_heads(v)
    del v
    vt8, ldv = v_transposed(v8)
    return q8, k8, vt8, qs, ks, vs, ldv
