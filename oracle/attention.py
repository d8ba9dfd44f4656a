"""Plain fp64 CPU oracle for exact attention, its gradients, its streamed form and the split-KV merge.

TEST INFRASTRUCTURE ONLY. This module is the yardstick the GPU library is
checked against. Only the tests, the smoke check and the benchmark's CPU
baseline may import it; the library itself never calls it and has no CPU
fallback.

Sources (three web pages on IO-aware attention):
  [IOP]   "I/O-Aware Kernels", IOP Systems blog, sections "The Memory Bottleneck"
          and "FlashAttention".
  [GRASP] "Tracing Tiled QKV Data Movement in FlashAttention's Memory
          Hierarchy", grasp.study lesson, sections 2 and 3.
  [ILP]   "FlashAttention & IO-aware attention", inference-learning-path
          interview page, sections "Direct answer", "Deep dive", "Code",
          "Interviewer follow-ups".

What is computed. [IOP, The Memory Bottleneck] and [ILP, Direct answer] define
attention as scores Q K^T, a row softmax, and a product with V; [ILP, Direct
answer] states that the streamed (online-softmax) form yields exactly that
function. So the oracle is the definition itself, evaluated in float64 on the
bf16 input values widened exactly:

    s_ij   = scale * sum_c Q[i,c] K[j,c]          for j in A(i)
    M_i    = max_{j in A(i)} s_ij
    w_ij   = exp(s_ij - M_i),  L_i = sum_j w_ij
    O[i,:] = sum_j w_ij V[j,:] / L_i
    LSE_i  = M_i + ln L_i                          (natural log)

Readings where the pages are silent (each one is listed in the design notes):
  * A(i) is every key when not causal; when causal it is {j : j <= i + Skv - Sq}
    (bottom-right alignment, equal to j <= i when Sq == Skv).
  * A row with no visible key has O = 0 and LSE = -inf.
  * Grouped-query heads: query head h reads KV head floor(h * Hkv / Hq).
  * ``scale`` is used as the float32 value the library receives, widened.
  * Subtracting M_i leaves the result unchanged mathematically; it keeps
    exp() finite ([ILP, Interviewer follow-ups] on why the running max exists).

Score rows are formed one block of query rows at a time; nothing else is
blocked, fused or reordered.
"""
from __future__ import annotations

import math

import numpy as np


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly (bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def _sigma(scale: float) -> float:
    return float(np.float32(scale))


def kv_head_of(h: int, Hq: int, Hkv: int) -> int:
    """KV head read by query head h: contiguous groups of Hq / Hkv query heads."""
    return (h * Hkv) // Hq


def visible_keys(i: int, Sq: int, Skv: int, causal: bool) -> int:
    """Number of keys query row i may attend to; keys are 0 .. n-1."""
    if not causal:
        return Skv
    return max(0, min(Skv, i + Skv - Sq + 1))


def attention_rows(q_rows: np.ndarray, K: np.ndarray, V: np.ndarray, rows: np.ndarray,
                   Sq: int, causal: bool, scale: float):
    """Exact attention for selected query rows of one (batch, head).

    q_rows [n, d] f64 are the query vectors of rows ``rows`` (indices into the
    Sq query positions); K, V [Skv, d] f64 are that head's keys and values.
    Returns O [n, d] and LSE [n] in float64.
    """
    rows = np.asarray(rows)
    Skv = K.shape[0]
    sigma = _sigma(scale)
    nvis = np.array([visible_keys(int(i), Sq, Skv, causal) for i in rows], dtype=np.int64)
    # keys past the largest visible count are masked for every row of the block (weight
    # exactly 0), so only the first nk keys enter the products
    nk = int(nvis.max()) if len(rows) else 0
    s = sigma * (q_rows @ K[:nk].T)                              # [n, nk]
    keep = np.arange(nk)[None, :] < nvis[:, None]
    s = np.where(keep, s, -np.inf)
    O = np.zeros((len(rows), V.shape[1]))
    LSE = np.full(len(rows), -np.inf)
    live = nvis > 0
    if live.any():
        sl = s[live]
        M = sl.max(axis=1)
        w = np.exp(sl - M[:, None])                              # masked -> exp(-inf) = 0
        L = w.sum(axis=1)
        O[live] = (w @ V[:nk]) / L[:, None]
        LSE[live] = M + np.log(L)
    return O, LSE


def attention_ref(q: np.ndarray, k: np.ndarray, v: np.ndarray, *, causal: bool,
                  scale: float, row_block: int = 512):
    """Exact attention over whole tensors.

    q [B,Sq,Hq,d], k and v [B,Skv,Hkv,d], all float64.
    Returns O [B,Sq,Hq,d] and LSE [B,Hq,Sq], float64.
    """
    B, Sq, Hq, d = q.shape
    Bk, Skv, Hkv, dk = k.shape
    if Bk != B or dk != d or v.shape != k.shape or Hq % Hkv != 0:
        raise ValueError("inconsistent shapes")
    O = np.zeros((B, Sq, Hq, d))
    LSE = np.full((B, Hq, Sq), -np.inf)
    for b in range(B):
        for h in range(Hq):
            hk = kv_head_of(h, Hq, Hkv)
            K, V = k[b, :, hk, :], v[b, :, hk, :]
            for r0 in range(0, Sq, row_block):
                rows = np.arange(r0, min(Sq, r0 + row_block))
                o, l = attention_rows(q[b, rows, h, :], K, V, rows, Sq, causal, scale)
                O[b, rows, h, :] = o
                LSE[b, h, rows] = l
    return O, LSE


def decode_ref(q: np.ndarray, kc: np.ndarray, vc: np.ndarray, *, scale: float):
    """Single-query decode: q [B,Hq,d], caches [B,Skv,Hkv,d] -> O [B,Hq,d], LSE [B,Hq].

    [ILP, Direct answer]: a decode step has one query, so its scores are a
    1 x Skv vector over every cached key (no mask).
    """
    O, LSE = attention_ref(q[:, None], kc, vc, causal=False, scale=scale)
    return O[:, 0], LSE[:, :, 0]


def online_ref(q: np.ndarray, K: np.ndarray, V: np.ndarray, *, scale: float, block: int = 2):
    """Streamed softmax for one query row: the running-statistics form.

    [ILP, Direct answer] and [IOP, FlashAttention]: the keys are visited left to right
    in blocks, and only three running quantities survive between blocks: the largest
    scaled score m seen so far, the normaliser l = sum exp(s_j - m) and the accumulator
    acc = sum exp(s_j - m) v_j over the keys seen. A block is first summarised by the
    same three quantities over its own keys; the running state and the block summary
    are then brought to their common maximum, each scaled by exp(its m - common m),
    and added. The output is acc / l and the log-sum-exp m + ln l. ``block = 1``
    updates the statistics after every key.
    Returns (o [d], lse) in float64.
    """
    sigma = _sigma(scale)
    state = (-math.inf, 0.0, np.zeros(V.shape[1]))          # (m, l, acc) over no keys
    for j0 in range(0, K.shape[0], block):
        scores = sigma * (K[j0:j0 + block] @ q)
        m_blk = float(scores.max())
        e_blk = np.exp(scores - m_blk)
        summary = (m_blk, float(e_blk.sum()), e_blk @ V[j0:j0 + block])
        state = _merge_running(state, summary)
    m, l, acc = state
    if l == 0.0:
        return np.zeros(V.shape[1]), -math.inf
    return acc / l, m + math.log(l)


def _merge_running(a, b):
    """Two (m, l, acc) summaries of disjoint key sets -> the summary of their union.
    A summary of no keys has m = -inf and weight 0 (never exponentiated)."""
    m = max(a[0], b[0])
    wa = math.exp(a[0] - m) if a[0] != -math.inf else 0.0
    wb = math.exp(b[0] - m) if b[0] != -math.inf else 0.0
    return m, wa * a[1] + wb * b[1], wa * a[2] + wb * b[2]


def split_partials_ref(q: np.ndarray, kc: np.ndarray, vc: np.ndarray, *, scale: float,
                       bounds: list):
    """Per-chunk decode partials, each chunk normalised on its own.

    [ILP, Deep dive] names splitting the KV length across compute units for
    decode. Chunk c covers keys bounds[c] .. bounds[c+1]-1 and yields the
    attention of the query over those keys alone: O_c and lambda_c (its LSE).
    An empty chunk gives O_c = 0 and lambda_c = -inf.
    Returns part_o [B,Hq,n,d] and part_lse [B,Hq,n].
    """
    B, Hq, d = q.shape
    n = len(bounds) - 1
    part_o = np.zeros((B, Hq, n, d))
    part_lse = np.full((B, Hq, n), -np.inf)
    for c in range(n):
        lo, hi = bounds[c], bounds[c + 1]
        if hi > lo:
            o, l = decode_ref(q, kc[:, lo:hi], vc[:, lo:hi], scale=scale)
            part_o[:, :, c] = o
            part_lse[:, :, c] = l
    return part_o, part_lse


def combine_ref(part_o: np.ndarray, part_lse: np.ndarray):
    """Merge chunk partials by log-sum-exp.

    The chunk-level form of the running-max rescale ([ILP, Direct answer]):
    chunk c stands for exp(lambda_c) total weight with normalised output O_c, so
        Lambda = ln sum_c exp(lambda_c),   O = sum_c exp(lambda_c - Lambda) O_c.
    The largest lambda is subtracted first to keep exp() finite. Chunks with
    lambda = -inf carry no weight; if every chunk is empty, O = 0, LSE = -inf.
    part_o [..., n, d], part_lse [..., n] -> O [..., d], LSE [...].
    """
    mx = part_lse.max(axis=-1)
    finite = np.isfinite(mx)
    safe = np.where(finite, mx, 0.0)
    w = np.exp(part_lse - safe[..., None])                       # -inf chunks -> 0
    W = w.sum(axis=-1)
    with np.errstate(invalid="ignore", divide="ignore"):
        O = np.where(finite[..., None], (w[..., None] * part_o).sum(axis=-2) / W[..., None], 0.0)
        LSE = np.where(finite, safe + np.log(W), -np.inf)
    return O, LSE


def paged_decode_ref(q: np.ndarray, k_pages: np.ndarray, v_pages: np.ndarray, block_table: np.ndarray,
                     seq_lens: np.ndarray, *, scale: float):
    """Single-query decode over a paged KV cache.

    [IOP, FlashAttention] mentions paged KV caches; the layout is this library's
    reading: pools k_pages, v_pages [num_pages, page_size, Hkv, d], and sequence b's
    token t lives in page block_table[b, t // page_size] at slot t % page_size; the
    sequence holds seq_lens[b] tokens, all visible to its query. The result is the
    plain decode over the tokens gathered in order. A sequence with no token gets
    O = 0 and LSE = -inf.
    q [B,Hq,d] -> O [B,Hq,d], LSE [B,Hq] (float64).
    """
    B, Hq, d = q.shape
    page_size = k_pages.shape[1]
    O = np.zeros((B, Hq, d))
    LSE = np.full((B, Hq), -np.inf)
    for b in range(B):
        n = int(seq_lens[b])
        if n <= 0:
            continue
        t = np.arange(n)
        pages = np.asarray(block_table[b])[t // page_size]
        kc = k_pages[pages, t % page_size]                      # [n, Hkv, d]
        vc = v_pages[pages, t % page_size]
        o, l = decode_ref(q[b:b + 1], kc[None], vc[None], scale=scale)
        O[b], LSE[b] = o[0], l[0]
    return O, LSE


def attention_bwd_rows(q_rows: np.ndarray, do_rows: np.ndarray, K: np.ndarray, V: np.ndarray,
                       rows: np.ndarray, Sq: int, causal: bool, scale: float, abs_terms: bool = False):
    """Gradients from selected query rows of one (batch, query head).

    [GRASP, Conclusion] says the backward pass recomputes the attention matrix
    instead of storing it. The pages give no formulas, so this is the derivative of
    the forward definition above by the chain rule, with the probabilities rebuilt
    from Q and K (nothing from the forward is reused). For loss gradient dO:

        P_ij   = softmax_j(s_ij) over j in A(i),  s_ij = scale * Q_i . K_j
        dV_j  += sum_i P_ij dO_i
        dP_ij  = dO_i . V_j
        dS_ij  = P_ij (dP_ij - sum_k P_ik dP_ik)     (gradient of the scaled score)
        dQ_i   = scale * sum_j dS_ij K_j
        dK_j  += scale * sum_i dS_ij Q_i

    q_rows, do_rows [n, d] are rows ``rows`` of that head; K, V [Skv, d] its KV head.
    Returns dQ [n, d] and this block's contributions dK, dV [Skv, d] (float64). A row
    with no visible key contributes nothing and gets dQ = 0.

    With ``abs_terms`` it also returns two sensitivity measures per output element, for
    relative perturbations of the factor dS (dQ, dK) or P (dV) of every product term
    and of every element of the output O entering D_i = dO_i . O_i (a backward pass
    receives O rounded to the output format). With E_i = sum_c |dO_ic| |O_ic| and
    F_i = (sum_c dO_ic^2 O_ic^2)^(1/2):
      * worst case (all perturbations of size 1, signs adversarial):
          dQ: |scale| (sum_j |dS_ij| |K_j| + E_i sum_j P_ij |K_j|)
          dK: |scale| (sum_i |dS_ij| |Q_i| + sum_i P_ij E_i |Q_i|)
          dV: sum_i P_ij |dO_i|
      * root-sum-square (independent perturbations of unit variance):
          dQ: |scale| (sum_j dS_ij^2 K_j^2 + F_i^2 (sum_j P_ij K_j)^2)^(1/2)
          dK: |scale| (sum_i dS_ij^2 Q_i^2 + sum_i P_ij^2 F_i^2 Q_i^2)^(1/2)
          dV: (sum_i P_ij^2 dO_i^2)^(1/2)
    (elementwise over the head dimension). In ``attention_bwd_ref`` the squared
    root-sum-square terms add over row blocks, so this function returns them squared.
    """
    rows = np.asarray(rows)
    Skv = K.shape[0]
    sigma = _sigma(scale)
    s = sigma * (q_rows @ K.T)                                   # [n, Skv]
    nvis = np.array([visible_keys(int(i), Sq, Skv, causal) for i in rows])
    keep = np.arange(Skv)[None, :] < nvis[:, None]
    P = np.zeros_like(s)
    live = nvis > 0
    if live.any():
        sl = np.where(keep[live], s[live], -np.inf)
        w = np.exp(sl - sl.max(axis=1, keepdims=True))
        P[live] = w / w.sum(axis=1, keepdims=True)
    dP = do_rows @ V.T                                           # [n, Skv]
    dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
    grads = (sigma * (dS @ K), sigma * (dS.T @ q_rows), P.T @ do_rows)
    if not abs_terms:
        return grads
    aS = abs(sigma) * np.abs(dS)
    O = P @ V
    E = (np.abs(do_rows) * np.abs(O)).sum(axis=1)                 # sum_c |dO_ic| |O_ic|
    F2 = (do_rows ** 2 * O ** 2).sum(axis=1)                      # sum_c dO_ic^2 O_ic^2
    aK, aQ = np.abs(K), np.abs(q_rows)
    s2 = sigma * sigma
    worst = (aS @ aK + abs(sigma) * E[:, None] * (P @ aK),
             aS.T @ aQ + abs(sigma) * (P.T @ (E[:, None] * aQ)),
             P.T @ np.abs(do_rows))
    rss2 = (s2 * ((dS ** 2) @ (K ** 2) + F2[:, None] * (P @ K) ** 2),
            s2 * ((dS ** 2).T @ (q_rows ** 2) + (P ** 2).T @ (F2[:, None] * q_rows ** 2)),
            (P ** 2).T @ (do_rows ** 2))
    return grads + worst + rss2


def attention_bwd_ref(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray, *, causal: bool,
                      scale: float, row_block: int = 512, abs_terms: bool = False):
    """Gradients of exact attention with respect to Q, K and V.

    q, do [B,Sq,Hq,d]; k, v [B,Skv,Hkv,d]; all float64. The loss gradient dO is the
    gradient with respect to the output O of ``attention_ref``. A KV head's gradients
    sum the contributions of every query head that reads it.
    Returns dQ [B,Sq,Hq,d], dK and dV [B,Skv,Hkv,d] (float64); with ``abs_terms`` also
    the worst-case and the root-sum-square sensitivities of ``attention_bwd_rows`` for
    dQ, dK, dV, in the same shapes (nine arrays in all).
    """
    B, Sq, Hq, d = q.shape
    Bk, Skv, Hkv, dk = k.shape
    if Bk != B or dk != d or v.shape != k.shape or do.shape != q.shape or Hq % Hkv != 0:
        raise ValueError("inconsistent shapes")
    out = [np.zeros((B, Sq, Hq, d)), np.zeros((B, Skv, Hkv, d)), np.zeros((B, Skv, Hkv, d))]
    if abs_terms:
        for _ in range(2):
            out += [np.zeros((B, Sq, Hq, d)), np.zeros((B, Skv, Hkv, d)), np.zeros((B, Skv, Hkv, d))]
    for b in range(B):
        for h in range(Hq):
            hk = kv_head_of(h, Hq, Hkv)
            K, V = k[b, :, hk, :], v[b, :, hk, :]
            for r0 in range(0, Sq, row_block):
                rows = np.arange(r0, min(Sq, r0 + row_block))
                res = attention_bwd_rows(q[b, rows, h, :], do[b, rows, h, :], K, V, rows, Sq, causal, scale,
                                         abs_terms)
                for n in range(0, len(res), 3):
                    out[n][b, rows, h, :] = res[n]
                    out[n + 1][b, :, hk, :] += res[n + 1]
                    out[n + 2][b, :, hk, :] += res[n + 2]
    if abs_terms:
        for n in (6, 7, 8):
            out[n] = np.sqrt(out[n])
    return tuple(out)


def e4m3_value(codes: np.ndarray) -> np.ndarray:
    """OCP fp8 e4m3 codes (uint8) -> float64, exactly.

    Bit layout s eeee mmm, exponent bias 7: e = 0 gives the subnormals m * 2^-9,
    otherwise (8 + m) * 2^(e - 10); 0x7F and 0xFF are NaN; there is no infinity.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.ldexp(1.0, e - 10))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return np.where(c >= 128, -mag, mag)


def attention_fp8_ref(q8: np.ndarray, k8: np.ndarray, vt8: np.ndarray, q_scale: np.ndarray,
                      k_scale: np.ndarray, v_scale: np.ndarray, *, causal: bool, scale: float):
    """Exact attention of fp8-quantised inputs (the fp8 variant FlashAttention-3 adds).

    [ILP, Deep dive] names an FP8 variant and nothing more; the reading is attention
    on the dequantised tensors: Q = e4m3(q8) * q_scale[b, h], K likewise, and V from
    the transposed codes vt8 [B, Hkv, d, ldv] (columns past Skv ignored). The result
    is ``attention_ref`` on those float64 values.
    q8 [B,Sq,Hq,d], k8 [B,Skv,Hkv,d] uint8; scales [B,H] -> O [B,Sq,Hq,d], LSE [B,Hq,Sq].
    """
    Skv = k8.shape[1]
    Q = e4m3_value(q8) * np.asarray(q_scale, np.float64)[:, None, :, None]
    K = e4m3_value(k8) * np.asarray(k_scale, np.float64)[:, None, :, None]
    V = e4m3_value(vt8[..., :Skv]).transpose(0, 3, 1, 2) * np.asarray(v_scale, np.float64)[:, None, :, None]
    return attention_ref(Q, K, V, causal=causal, scale=scale)


def ffn_ref(h: np.ndarray, w1: np.ndarray, b1: np.ndarray, w2: np.ndarray, b2: np.ndarray) -> np.ndarray:
    """Position-wise feed-forward network on rows h [..., d_model] (float64).

    [IOP, Blockwise Parallel Transformers] applies the transformer's feed-forward
    network to the attention output and notes that it acts on every token on its own.
    The pages do not write the network out; the reading is the classic two-layer form
    with a ReLU, each layer stored as a linear layer's [out, in] weight:
    relu(h W1^T + b1) W2^T + b2, W1 [d_ff, d_model], W2 [d_model, d_ff].
    """
    return np.maximum(h @ w1.T + b1, 0.0) @ w2.T + b2


def bpt_layer_ref(q: np.ndarray, k: np.ndarray, v: np.ndarray, w1: np.ndarray, b1: np.ndarray, w2: np.ndarray,
                  b2: np.ndarray, *, causal: bool, scale: float) -> np.ndarray:
    """Attention followed by the feed-forward network, over the whole sequence.

    [IOP, Blockwise Parallel Transformers]: the attention output of every query row,
    heads concatenated (d_model = Hq * d), goes through ``ffn_ref``. The blockwise
    schedule the pages describe computes this same function one query block at a time.
    q [B,S,Hq,d], k, v [B,S,Hkv,d] -> y [B,S,Hq*d] (float64).
    """
    O, _ = attention_ref(q, k, v, causal=causal, scale=scale)
    B, S, Hq, d = O.shape
    return ffn_ref(O.reshape(B, S, Hq * d), w1, b1, w2, b2)
