"""Whole-tensor comparison of device results with the fp64 oracle, over a process pool.

TEST INFRASTRUCTURE ONLY, like the rest of this package: the tests and the benchmark's
oracle leg use it; the library never does.

The stated check for bf16 I/O with fp32 accumulation is max-abs <= 1e-2 and relative
L2 <= 4e-3 for O and for the finite LSE entries, over the whole tensor, with -inf LSE
entries matching exactly. A bf16 output cannot come closer to the exact value than
half a bf16 spacing, which exceeds 1e-2 once |O| >= 4, so next to the stated check
this module reports:
  * the floor: max |RNE_bf16(O_ref) - O_ref|, what a correctly rounded O would miss by;
  * the worst element's error in bf16 ulps (spacings at its exact value);
  * the same check on an fp32 output of the same kernel (no output rounding).
A config gets the label "pass" when the stated check holds as written. A miss of the
O max-abs is labelled "floor-limited" only when every element beyond 1e-2 lies within
one bf16 ulp of O_ref, the rel-L2 and LSE checks hold, and the fp32-output run passes
the stated check as written; anything else is "fail".

Work is split by (batch, query head) -- or, for decode, by batch element -- and each
worker runs the oracle on its share and returns only error statistics, which add up
over shares. Workers are separate spawned interpreters with one BLAS thread each; start
the pool before the calling process initialises a GPU.
"""
from __future__ import annotations

import math
import multiprocessing as mp
import os
import time

import numpy as np

from .attention import (attention_bwd_ref, attention_rows, e4m3_value, ffn_ref, kv_head_of, visible_keys,
                        widen_bf16)

MAX_ABS = 1e-2
REL_L2 = 4e-3
ROW_BLOCK = 512
# Gradients: unit roundoff of bf16 (8 significant bits), and how many bf16 roundings of
# one factor of every product term each gradient's arithmetic contains. dQ: dS rounded
# for its product. dV: P rounded for its product. dK: dS rounded for its product, and at
# d = 128 formed from the P already rounded for the dV product (a second rounding of
# the same factor; at d = 64 the bound is one rounding looser than needed).
GRAD_TERM = 2.0 ** -8
GRAD_ROUNDINGS = {"dQ": 1, "dK": 2, "dV": 1}

_pool = None
_pool_size = 0


# ---------------------------------------------------------------- pool
def _init_worker() -> None:
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except Exception:
        pass


def pool_workers() -> int:
    """Workers for this host: its CPU affinity, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def start_pool(n: int | None = None):
    """Start (once) the spawned worker pool and return it."""
    global _pool, _pool_size
    if _pool is None:
        _pool_size = n or pool_workers()
        _pool = mp.get_context("spawn").Pool(_pool_size, initializer=_init_worker)
    return _pool


def pool_size() -> int:
    return _pool_size


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ---------------------------------------------------------------- statistics
def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values (8 significant bits) at |x|; normal range assumed below 2^-126."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return np.ldexp(1.0, (e - 7).astype(np.int64))


def bf16_rne(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest bf16 value (ties to even), as float64."""
    sp = bf16_ulp(x)
    return np.rint(x / sp) * sp


def o_stats(o: np.ndarray, ref: np.ndarray) -> dict:
    """Mergeable error statistics of one output share against the oracle."""
    o = np.asarray(o, dtype=np.float64)
    err = np.abs(o - ref)
    fin = np.isfinite(o)
    ulp = bf16_ulp(ref)
    over = err > MAX_ABS
    err_f = np.where(fin, err, np.inf)                       # a non-finite output counts as infinitely wrong
    worst = int(np.argmax(err_f)) if err.size else 0
    return {"n": int(err.size), "nonfinite": int((~fin).sum()),
            "sse": float(np.square(np.where(fin, o - ref, 0.0)).sum()), "ssr": float(np.square(ref).sum()),
            "max_abs": float(err_f.flat[worst]) if err.size else 0.0,
            "ulps_at_max": float(err_f.flat[worst] / ulp.flat[worst]) if err.size else 0.0,
            "ref_at_max": float(ref.flat[worst]) if err.size else 0.0,
            "floor": float(np.abs(bf16_rne(ref) - ref).max()) if err.size else 0.0,
            "over": int(over.sum()), "over_beyond_ulp": int((over & (err > ulp)).sum()),
            "widened_bad": int((err > MAX_ABS + 0.5 * ulp).sum())}


def lse_stats(lse: np.ndarray, ref: np.ndarray) -> dict:
    lse = np.asarray(lse, dtype=np.float64)
    ninf = np.isneginf(ref)
    g, r = lse[~ninf], ref[~ninf]
    err = np.abs(g - r)
    return {"n": int(g.size), "ninf_mismatch": int((np.isneginf(lse) != ninf).sum()),
            "nonfinite": int((~np.isfinite(g)).sum()),
            "sse": float(np.square(np.where(np.isfinite(g), g - r, 0.0)).sum()), "ssr": float(np.square(r).sum()),
            "max_abs": float(np.where(np.isfinite(err), err, np.inf).max()) if g.size else 0.0}


def merge_stats(parts: list) -> dict:
    if not parts:
        return {}
    out = {}
    top = max(parts, key=lambda p: p["max_abs"])           # the share holding the worst element
    for k in parts[0]:
        if k in ("max_abs", "ulps_at_max", "ref_at_max"):
            out[k] = top[k]
        elif k == "floor":
            out[k] = max(p[k] for p in parts)
        else:
            out[k] = sum(p[k] for p in parts)
    return out


def summarise(o: dict, lse: dict | None) -> dict:
    """Stated-check numbers of merged statistics."""
    rel_o = math.sqrt(o["sse"] / o["ssr"]) if o["ssr"] > 0 else math.sqrt(o["sse"])
    res = {"O_max_abs": o["max_abs"], "O_rel_l2": rel_o, "O_floor": o["floor"],
           "O_worst_error_bf16_ulps": o["ulps_at_max"], "O_ref_at_worst": o["ref_at_max"],
           "O_over_1e-2": o["over"], "O_over_1e-2_beyond_1ulp": o["over_beyond_ulp"],
           "O_widened_bound_misses": o["widened_bad"], "O_nonfinite": o["nonfinite"], "O_elements": o["n"]}
    if lse is not None:
        rel_l = math.sqrt(lse["sse"] / lse["ssr"]) if lse["ssr"] > 0 else math.sqrt(lse["sse"])
        res.update({"LSE_max_abs": lse["max_abs"], "LSE_rel_l2": rel_l, "LSE_ninf_mismatch": lse["ninf_mismatch"],
                    "LSE_nonfinite": lse["nonfinite"], "LSE_finite_entries": lse["n"]})
    return res


def grad_bound(ref: np.ndarray, a_ref: np.ndarray, roundings: int) -> np.ndarray:
    """Per-element gradient bound: 1e-2, plus half a bf16 spacing at the exact value (the
    output rounding), plus the worst case of ``roundings`` relative roundings of size at
    most 2^-8 of one factor of every product term (a_ref: the oracle's worst-case
    sensitivity to relative changes of that factor and of O inside D_i = dO_i . O_i)."""
    return MAX_ABS + 0.5 * bf16_ulp(ref) + roundings * GRAD_TERM * a_ref


def grad_rel_bound(nref: float, nr: float, roundings: int) -> float:
    """Per-tensor rel-L2 bound: the stated 4e-3 plus twice the expected RMS of the
    roundings (each independent, uniform in [-u, u], RMS u / sqrt(3); nr: the norm of the
    oracle's root-sum-square sensitivity)."""
    return REL_L2 + 2.0 * math.sqrt(roundings) * (GRAD_TERM / math.sqrt(3.0)) * (nr / nref if nref > 0 else 0.0)


def grad_stats(g: np.ndarray, ref: np.ndarray, a_ref: np.ndarray, r_ref: np.ndarray, roundings: int) -> dict:
    """Mergeable statistics of one gradient share against the oracle."""
    g = np.asarray(g, dtype=np.float64)
    fin = np.isfinite(g)
    err = np.where(fin, np.abs(g - ref), np.inf)
    bound = grad_bound(ref, a_ref, roundings)
    return {"n": int(err.size), "nonfinite": int((~fin).sum()),
            "sse": float(np.square(np.where(fin, g - ref, 0.0)).sum()), "ssr": float(np.square(ref).sum()),
            "ssq_sens": float(np.square(r_ref).sum()),
            "max_abs": float(err.max()) if err.size else 0.0,
            "max_err_over_bound": float((err / bound).max()) if err.size else 0.0,
            "over_bound": int((err > bound).sum()),
            "over_1e-2": int((err > MAX_ABS).sum())}


def grad_summary(parts: list, roundings: int) -> dict:
    t = {k: sum(p[k] for p in parts) for k in ("n", "nonfinite", "sse", "ssr", "ssq_sens", "over_bound", "over_1e-2")}
    nref = math.sqrt(t["ssr"])
    rel = math.sqrt(t["sse"]) / nref if nref > 0 else math.sqrt(t["sse"])
    return {"elements": t["n"], "nonfinite": t["nonfinite"], "max_abs": max(p["max_abs"] for p in parts),
            "rel_l2": rel, "rel_l2_bound": grad_rel_bound(nref, math.sqrt(t["ssq_sens"]), roundings),
            "max_err_over_bound": max(p["max_err_over_bound"] for p in parts),
            "over_bound": t["over_bound"], "over_1e-2": t["over_1e-2"], "roundings": roundings}


def grad_ok(s: dict) -> bool:
    return s["nonfinite"] == 0 and s["over_bound"] == 0 and s["rel_l2"] <= s["rel_l2_bound"]


def stated_ok(s: dict) -> bool:
    ok = s["O_nonfinite"] == 0 and s["O_max_abs"] <= MAX_ABS and s["O_rel_l2"] <= REL_L2
    if "LSE_max_abs" in s:
        ok = ok and s["LSE_ninf_mismatch"] == 0 and s["LSE_nonfinite"] == 0 and s["LSE_max_abs"] <= MAX_ABS \
            and s["LSE_rel_l2"] <= REL_L2
    return ok


def label(bf16: dict, f32: dict | None) -> str:
    """'pass', 'floor-limited' or 'fail' for a bf16-output summary (see the module docstring)."""
    if stated_ok(bf16):
        return "pass"
    rest = dict(bf16, O_max_abs=0.0)                 # everything but the O max-abs
    if stated_ok(rest) and bf16["O_over_1e-2_beyond_1ulp"] == 0 and f32 is not None and stated_ok(f32):
        return "floor-limited"
    return "fail"


# ---------------------------------------------------------------- worker
def _oracle_rows(q_bits, k_bits, v_bits, rows, Sq, causal, scale):
    Q, K, V = widen_bf16(q_bits), widen_bf16(k_bits), widen_bf16(v_bits)
    O = np.zeros((len(rows), Q.shape[1]))
    L = np.full(len(rows), -np.inf)
    for r0 in range(0, len(rows), ROW_BLOCK):
        sl = slice(r0, r0 + ROW_BLOCK)
        O[sl], L[sl] = attention_rows(Q[sl], K, V, rows[sl], Sq, causal, scale)
    return O, L


def _share_task(args):
    """One share: oracle O, LSE for its query rows, then error statistics of each device output."""
    key, q_bits, k_bits, v_bits, rows, Sq, causal, scale, outputs = args
    t0 = time.perf_counter()
    O, L = _oracle_rows(q_bits, k_bits, v_bits, rows, Sq, causal, scale)
    dt = time.perf_counter() - t0
    stats = {}
    for name, o, lse in outputs:
        stats[name] = (o_stats(o, O), lse_stats(lse, L) if lse is not None else None)
    return key, stats, dt


def _decode_task(args):
    """One batch element of a decode step: every query head against its KV head."""
    key, q_bits, k_bits, v_bits, Hkv, scale, outputs = args
    Hq = q_bits.shape[0]
    t0 = time.perf_counter()
    O = np.zeros((Hq, q_bits.shape[1]))
    L = np.full(Hq, -np.inf)
    for h in range(Hq):
        hk = kv_head_of(h, Hq, Hkv)
        o, l = attention_rows(widen_bf16(q_bits[h:h + 1]), widen_bf16(k_bits[:, hk]), widen_bf16(v_bits[:, hk]),
                              np.zeros(1, dtype=np.int64), 1, False, scale)
        O[h], L[h] = o[0], l[0]
    dt = time.perf_counter() - t0
    stats = {name: (o_stats(o, O), lse_stats(lse, L)) for name, o, lse in outputs}
    return key, stats, dt


def _bwd_task(args):
    """One KV head of one batch element with every query head of its group: the oracle's
    gradients and sensitivities, then statistics of each device gradient."""
    key, q_bits, k_bits, v_bits, do_bits, causal, scale, dev = args
    t0 = time.perf_counter()
    ref = attention_bwd_ref(widen_bf16(q_bits), widen_bf16(k_bits), widen_bf16(v_bits), widen_bf16(do_bits),
                            causal=causal, scale=scale, abs_terms=True)
    dt = time.perf_counter() - t0
    stats = {}
    for i, name in enumerate(("dQ", "dK", "dV")):
        stats[name] = grad_stats(dev[i], ref[i], ref[3 + i], ref[6 + i], GRAD_ROUNDINGS[name])
    return key, stats, dt


# ---------------------------------------------------------------- drivers
def prefill_flops(Sq: int, Skv: int, d: int, causal: bool) -> float:
    """Counted FLOPs of one (batch, head) under the 4 d per visible (query, key) rule."""
    if causal:
        nvis = sum(visible_keys(i, Sq, Skv, True) for i in range(Sq))
    else:
        nvis = Sq * Skv
    return 4.0 * d * nvis


def check_prefill(q, k, v, outputs: dict, *, causal: bool, scale: float, heads=None, progress=None) -> dict:
    """Compare device outputs of a prefill with the oracle over every (batch, head) (or ``heads``).

    q [B,Sq,Hq,d], k and v [B,Skv,Hkv,d] are bf16 bit arrays (uint16); ``outputs`` maps a
    name to (O [B,Sq,Hq,d] float32 or float64, LSE [B,Hq,Sq] or None). Returns, per
    output name, the merged statistics summary, plus timing of the oracle itself.
    """
    B, Sq, Hq, d = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    heads = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else list(heads)
    rows = np.arange(Sq)

    def tasks():
        for b, h in heads:
            hk = kv_head_of(h, Hq, Hkv)
            outs = [(name, np.ascontiguousarray(o[b, :, h, :]),
                     None if lse is None else np.ascontiguousarray(lse[b, h, :])) for name, (o, lse) in outputs.items()]
            yield ((b, h), np.ascontiguousarray(q[b, :, h, :]), np.ascontiguousarray(k[b, :, hk, :]),
                   np.ascontiguousarray(v[b, :, hk, :]), rows, Sq, causal, scale, outs)

    return _run(_share_task, tasks(), len(heads), list(outputs), prefill_flops(Sq, Skv, d, causal), progress)


def check_decode(q, k, v, outputs: dict, *, scale: float, batches=None, progress=None) -> dict:
    """Decode: q [B,Hq,d], caches [B,Skv,Hkv,d] (bf16 bits); outputs name -> (O [B,Hq,d], LSE [B,Hq])."""
    B, Hq, d = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    batches = range(B) if batches is None else list(batches)

    def tasks():
        for b in batches:
            outs = [(name, np.ascontiguousarray(o[b]), np.ascontiguousarray(lse[b])) for name, (o, lse) in outputs.items()]
            yield (b, np.ascontiguousarray(q[b]), np.ascontiguousarray(k[b]), np.ascontiguousarray(v[b]), Hkv, scale, outs)

    return _run(_decode_task, tasks(), len(batches), list(outputs), 4.0 * d * Skv * Hq, progress)


def _rows_task(args):
    """One (batch, query head): the oracle's O for every row (returned whole)."""
    key, q_bits, k_bits, v_bits, rows, Sq, causal, scale = args
    t0 = time.perf_counter()
    O, _ = _oracle_rows(q_bits, k_bits, v_bits, rows, Sq, causal, scale)
    return key, O, time.perf_counter() - t0


def attention_outputs(q, k, v, *, causal: bool, scale: float, progress=None) -> np.ndarray:
    """The oracle's attention output O [B,Sq,Hq,d] (float64) of bf16 bit arrays q, k, v,
    computed over the pool, one share per (batch, query head)."""
    B, Sq, Hq, d = q.shape
    Hkv = k.shape[2]
    rows = np.arange(Sq)
    out = np.zeros((B, Sq, Hq, d))

    def tasks():
        for b in range(B):
            for h in range(Hq):
                hk = kv_head_of(h, Hq, Hkv)
                yield ((b, h), np.ascontiguousarray(q[b, :, h, :]), np.ascontiguousarray(k[b, :, hk, :]),
                       np.ascontiguousarray(v[b, :, hk, :]), rows, Sq, causal, scale)

    t0, done, n = time.perf_counter(), 0, B * Hq
    for (b, h), O, _ in start_pool().imap_unordered(_rows_task, tasks(), chunksize=1):
        out[b, :, h, :] = O
        done += 1
        if progress is not None and (done == n or done % max(1, n // 8) == 0):
            progress(f"oracle attention: {done}/{n} heads, {time.perf_counter() - t0:.1f} s")
    return out


FFN_SIGMAS = 6.0


def ffn_sigma(h: np.ndarray, w1: np.ndarray, b1: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """Standard deviation of the rounding error of the feed-forward output y, given the
    fp64 input rows h [n, d_model] and weights (W1 [d_ff, d_model], W2 [d_model, d_ff]).
    h reaches the first product rounded to bf16 (relative 2^-8), the hidden activations
    m = relu(h W1^T + b1) are rounded to bf16 after the ReLU (1-Lipschitz), and y once
    more at the output (half a spacing, bounded separately). Each element of y sums
    thousands of independently rounded terms, so its error is close to normal with
    standard deviation (2^-8 / sqrt 3) r, r_n^2 = sum_j (sum_k h_k^2 W1_jk^2 + m_j^2) W2_nj^2."""
    m = np.maximum(h @ w1.T + b1, 0.0)
    r2 = ((h ** 2) @ (w1 ** 2).T + m ** 2) @ (w2 ** 2).T
    return GRAD_TERM / math.sqrt(3.0) * np.sqrt(r2)


def ffn_bound(y: np.ndarray, sigma: np.ndarray) -> np.ndarray:
    """Per-element bound of the blockwise layer's output: 1e-2 + half a bf16 spacing of y
    + 6 sigma (the worst case, sums of absolute values, would not catch an error in a
    single element at d_model 4096)."""
    return MAX_ABS + 0.5 * bf16_ulp(y) + FFN_SIGMAS * sigma


def check_ffn(h: np.ndarray, w_bits, y_dev: np.ndarray, *, row_block: int = 2048, progress=None) -> dict:
    """Every element of a device feed-forward output y_dev [n, d_model] against
    ffn_ref(h) of the oracle's rows h [n, d_model] (float64) and the bf16 weight bits
    (W1, b1, W2, b2), in blocks of rows (multithreaded BLAS in this process). Returns
    max-abs, rel-L2 and its bound (4e-3 + 2 ||sigma|| / ||y||), the worst error over the
    per-element bound and the count of elements beyond it."""
    W = [widen_bf16(x) for x in w_bits]
    sse = ssr = ssig = 0.0
    max_abs = worst = 0.0
    over = nonfinite = 0
    t0 = time.perf_counter()
    for r0 in range(0, h.shape[0], row_block):
        hb = h[r0:r0 + row_block]
        y = ffn_ref(hb, *W)
        sig = ffn_sigma(hb, W[0], W[1], W[2])
        g = np.asarray(y_dev[r0:r0 + row_block], dtype=np.float64)
        fin = np.isfinite(g)
        err = np.where(fin, np.abs(g - y), np.inf)
        bound = ffn_bound(y, sig)
        nonfinite += int((~fin).sum())
        sse += float(np.square(np.where(fin, g - y, 0.0)).sum())
        ssr += float(np.square(y).sum())
        ssig += float(np.square(sig).sum())
        max_abs = max(max_abs, float(err.max()))
        worst = max(worst, float((err / bound).max()))
        over += int((err > bound).sum())
        if progress is not None:
            progress(f"oracle feed-forward: rows {r0 + len(hb)}/{h.shape[0]}, {time.perf_counter() - t0:.1f} s")
    ny = math.sqrt(ssr)
    return {"elements": int(y_dev.size), "nonfinite": nonfinite, "max_abs": max_abs,
            "rel_l2": math.sqrt(sse) / ny if ny > 0 else math.sqrt(sse),
            "rel_l2_bound": REL_L2 + 2.0 * math.sqrt(ssig) / ny if ny > 0 else REL_L2,
            "max_err_over_bound": worst, "over_bound": over, "wall_s": time.perf_counter() - t0}


def ffn_ok(s: dict) -> bool:
    return s["nonfinite"] == 0 and s["over_bound"] == 0 and s["rel_l2"] <= s["rel_l2_bound"]


FP8_P_ROUNDING = 2.0 ** -4        # relative rounding of a normal e4m3 value
FP8_P_SUB = 2.0 ** -10            # absolute rounding below e4m3's normal range, in units of the row max


def fp8_sensitivities(Q, K, V, rows, Sq: int, causal: bool, scale: float):
    """Sensitivities of O to the e4m3 rounding of P for query rows ``rows`` of one head
    (dequantised float64 Q [n, d], K, V [Skv, d]): A = sum_j P_ij |V_j|,
    Bs = sum_j min(P_ij, 2^-10 Pmax_i) |V_j| and their root-sum-square forms R, Rs.
    A normal e4m3 value is within 2^-4 of p (relative); below 2^-6 the error is absolute,
    at most 2^-10 in units where the row's largest p is >= 1."""
    sigma = float(np.float32(scale))
    Skv = K.shape[0]
    s = sigma * (Q @ K.T)
    nvis = np.array([visible_keys(int(i), Sq, Skv, causal) for i in rows])
    keep = np.arange(Skv)[None, :] < nvis[:, None]
    s = np.where(keep, s, -np.inf)
    P = np.zeros_like(s)
    live = nvis > 0
    if live.any():
        w = np.exp(s[live] - s[live].max(axis=1, keepdims=True))
        P[live] = w / w.sum(axis=1, keepdims=True)
    aV = np.abs(V)
    small = np.minimum(P, FP8_P_SUB * P.max(axis=1, keepdims=True))
    return P @ aV, small @ aV, np.sqrt((P ** 2) @ (V ** 2)), np.sqrt((small ** 2) @ (V ** 2))


def fp8_bound(O_ref, A, Bs):
    """Per-element bound of the fp8 forward's O: 1e-2 + half a bf16 spacing + 2^-4 A + Bs."""
    return MAX_ABS + 0.5 * bf16_ulp(O_ref) + FP8_P_ROUNDING * A + Bs


def _fp8_task(args):
    """One (batch, query head) of the fp8 forward: the oracle on the dequantised inputs,
    the rounding sensitivities, then statistics of the device O and LSE."""
    key, q8, k8, vt8, qsc, ksc, vsc, Sq, causal, scale, o_dev, lse_dev = args
    t0 = time.perf_counter()
    Skv = k8.shape[0]
    Q = e4m3_value(q8) * float(qsc)
    K = e4m3_value(k8) * float(ksc)
    V = e4m3_value(vt8[:, :Skv]).T * float(vsc)
    st = {"n": 0, "nonfinite": 0, "sse": 0.0, "ssr": 0.0, "ssR": 0.0, "ssRs": 0.0, "max_abs": 0.0,
          "max_err_over_bound": 0.0, "over_bound": 0, "over_1e-2": 0}
    L = np.full(Sq, -np.inf)
    for r0 in range(0, Sq, ROW_BLOCK):
        rows = np.arange(r0, min(Sq, r0 + ROW_BLOCK))
        O, L[rows] = attention_rows(Q[rows], K, V, rows, Sq, causal, scale)
        A, Bs, R, Rs = fp8_sensitivities(Q[rows], K, V, rows, Sq, causal, scale)
        g = np.asarray(o_dev[rows], dtype=np.float64)
        fin = np.isfinite(g)
        err = np.where(fin, np.abs(g - O), np.inf)
        bound = fp8_bound(O, A, Bs)
        st["n"] += int(err.size)
        st["nonfinite"] += int((~fin).sum())
        st["sse"] += float(np.square(np.where(fin, g - O, 0.0)).sum())
        st["ssr"] += float(np.square(O).sum())
        st["ssR"] += float(np.square(R).sum())
        st["ssRs"] += float(np.square(Rs).sum())
        st["max_abs"] = max(st["max_abs"], float(err.max()))
        st["max_err_over_bound"] = max(st["max_err_over_bound"], float((err / bound).max()))
        st["over_bound"] += int((err > bound).sum())
        st["over_1e-2"] += int((err > MAX_ABS).sum())
    return key, (st, lse_stats(lse_dev, L)), time.perf_counter() - t0


def check_fp8(q8, k8, vt8, q_scale, k_scale, v_scale, o, lse, *, causal: bool, scale: float, progress=None) -> dict:
    """Every element of the fp8 forward's O (bound ``fp8_bound``; per tensor rel-L2 <=
    4e-3 + (2 / sqrt 3)(2^-4 ||R|| + ||Rs||) / ||O||) and LSE (the stated bf16 bar: its
    normaliser sums unrounded p) against the oracle on the dequantised inputs, over the
    pool, one share per (batch, query head). q8 [B,Sq,Hq,d], k8 [B,Skv,Hkv,d], vt8
    [B,Hkv,d,ldv] e4m3 codes; scales [B,H]; o [B,Sq,Hq,d], lse [B,Hq,Sq] device results."""
    B, Sq, Hq, d = q8.shape
    Hkv = k8.shape[2]

    def tasks():
        for b in range(B):
            for h in range(Hq):
                hk = kv_head_of(h, Hq, Hkv)
                yield ((b, h), np.ascontiguousarray(q8[b, :, h]), np.ascontiguousarray(k8[b, :, hk]),
                       np.ascontiguousarray(vt8[b, hk]), q_scale[b, h], k_scale[b, hk], v_scale[b, hk], Sq, causal,
                       scale, np.ascontiguousarray(o[b, :, h]), np.ascontiguousarray(lse[b, h]))

    parts, lparts = [], []
    t0, done, n = time.perf_counter(), 0, B * Hq
    for _, (st, sl), _ in start_pool().imap_unordered(_fp8_task, tasks(), chunksize=1):
        parts.append(st)
        lparts.append(sl)
        done += 1
        if progress is not None and (done == n or done % max(1, n // 8) == 0):
            progress(f"oracle fp8: {done}/{n} heads, {time.perf_counter() - t0:.1f} s")
    t = {k: sum(p[k] for p in parts) for k in ("n", "nonfinite", "sse", "ssr", "ssR", "ssRs", "over_bound", "over_1e-2")}
    nO = math.sqrt(t["ssr"])
    res = {"O": {"elements": t["n"], "nonfinite": t["nonfinite"], "max_abs": max(p["max_abs"] for p in parts),
                 "rel_l2": math.sqrt(t["sse"]) / nO if nO > 0 else math.sqrt(t["sse"]),
                 "rel_l2_bound": REL_L2 + 2.0 / math.sqrt(3.0) * (FP8_P_ROUNDING * math.sqrt(t["ssR"])
                                                                  + math.sqrt(t["ssRs"])) / nO if nO > 0 else REL_L2,
                 "max_err_over_bound": max(p["max_err_over_bound"] for p in parts), "over_bound": t["over_bound"],
                 "over_1e-2": t["over_1e-2"]}}
    lm = merge_stats(lparts)
    res["LSE"] = {"max_abs": lm["max_abs"], "rel_l2": math.sqrt(lm["sse"] / lm["ssr"]) if lm["ssr"] > 0 else 0.0,
                  "ninf_mismatch": lm["ninf_mismatch"], "nonfinite": lm["nonfinite"], "finite_entries": lm["n"]}
    res["_oracle"] = {"shares": n, "wall_s": time.perf_counter() - t0, "workers": pool_size(), "cpu_model": cpu_model()}
    return res


def fp8_ok(res: dict) -> bool:
    o, lse = res["O"], res["LSE"]
    return (o["nonfinite"] == 0 and o["over_bound"] == 0 and o["rel_l2"] <= o["rel_l2_bound"]
            and lse["ninf_mismatch"] == 0 and lse["nonfinite"] == 0 and lse["max_abs"] <= MAX_ABS
            and lse["rel_l2"] <= REL_L2)


def check_backward(q, k, v, do, grads, *, causal: bool, scale: float, progress=None) -> dict:
    """Compare device gradients (dQ, dK, dV as float arrays in the layouts of q and k) with
    the oracle over every (batch, KV head) group. q, do [B,Sq,Hq,d] and k, v [B,Skv,Hkv,d]
    are bf16 bit arrays. Returns per gradient the merged summary (``grad_summary``) and
    the oracle's timing."""
    B, Sq, Hq, d = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    grp = Hq // Hkv
    dq, dk, dv = grads

    def tasks():
        for b in range(B):
            for hk in range(Hkv):
                hs = slice(hk * grp, (hk + 1) * grp)
                qs, ks = (slice(b, b + 1), slice(None), hs), (slice(b, b + 1), slice(None), slice(hk, hk + 1))
                yield ((b, hk), np.ascontiguousarray(q[qs]), np.ascontiguousarray(k[ks]), np.ascontiguousarray(v[ks]),
                       np.ascontiguousarray(do[qs]), causal, scale,
                       (np.ascontiguousarray(dq[qs]), np.ascontiguousarray(dk[ks]), np.ascontiguousarray(dv[ks])))

    pool = start_pool()
    parts = {n: [] for n in GRAD_ROUNDINGS}
    busy, done, n = 0.0, 0, B * Hkv
    t0 = time.perf_counter()
    for _, stats, dt in pool.imap_unordered(_bwd_task, tasks(), chunksize=1):
        busy += dt
        for name, st in stats.items():
            parts[name].append(st)
        done += 1
        if progress is not None and (done == n or done % max(1, n // 8) == 0):
            progress(f"oracle: {done}/{n} KV heads, {time.perf_counter() - t0:.1f} s")
    res = {name: grad_summary(p, GRAD_ROUNDINGS[name]) for name, p in parts.items()}
    res["_oracle"] = {"shares": n, "wall_s": time.perf_counter() - t0, "worker_busy_s": busy, "workers": pool_size(),
                      "cpu_model": cpu_model()}
    return res


def _run(fn, tasks, ntasks: int, names: list, flops_per_task: float, progress) -> dict:
    pool = start_pool()
    parts = {n: ([], []) for n in names}
    busy = 0.0
    t0 = time.perf_counter()
    done = 0
    for _, stats, dt in pool.imap_unordered(fn, tasks, chunksize=1):
        busy += dt
        for n, (so, sl) in stats.items():
            parts[n][0].append(so)
            if sl is not None:
                parts[n][1].append(sl)
        done += 1
        if progress is not None and (done == ntasks or done % max(1, ntasks // 8) == 0):
            progress(f"oracle: {done}/{ntasks} shares, {time.perf_counter() - t0:.1f} s")
    wall = time.perf_counter() - t0
    res = {n: summarise(merge_stats(po), merge_stats(pl) if pl else None) for n, (po, pl) in parts.items()}
    res["_oracle"] = {"shares": ntasks, "wall_s": wall, "worker_busy_s": busy, "workers": pool_size(),
                      "flops": flops_per_task * ntasks, "gflops_per_s": flops_per_task * ntasks / wall / 1e9,
                      "cpu_model": cpu_model()}
    return res
