/*
 * fa.h - exact attention (FlashAttention forward) and split-KV decode for AMD
 * Instinct MI355X (gfx950). C ABI: plain pointers and sizes only.
 *
 * What is computed. For every batch b, query head h and query row i
 *
 *     O[b,i,h,:] = sum_{j in A(i)} softmax_j(scale * q_i . k_j) * v_j
 *     LSE[b,h,i] = ln sum_{j in A(i)} exp(scale * q_i . k_j)
 *
 * i.e. softmax(scale * Q K^T) V, evaluated as one fused pass that keeps tiles of
 * Q on chip, streams K/V tiles through on-chip memory and never writes the
 * score matrix to device memory ("I/O-Aware Kernels", section FlashAttention;
 * "FlashAttention & IO-aware attention", Direct answer). The streamed result is
 * the exact function, up to floating-point rounding order.
 *
 * Conventions shared by every entry point
 *  - Device pointers. Every tensor pointer is a device (HBM) pointer allocated
 *    by the caller; the library allocates nothing and keeps no per-call state.
 *  - bf16 tensors are raw 16-bit bfloat16 storage; all tensors are dense and
 *    contiguous in the stated layout; every pointer must be 16-byte aligned.
 *  - Head mapping (grouped-query attention): query head h reads KV head
 *    floor(h * Hkv / Hq); Hq must be a multiple of Hkv.
 *  - Causal mask (when requested) is aligned bottom-right: row i sees keys
 *    j <= i + Skv - Sq. A row that sees no key gets O = 0 and LSE = -inf.
 *  - Arithmetic: bf16 inputs, fp32 scores/softmax/accumulation; O is rounded
 *    once to bf16 (round-to-nearest-even) at the end. LSE is natural-log fp32.
 *  - `stream` is a hipStream_t (NULL = the default stream). Every call is
 *    asynchronous on that stream and never synchronises.
 *  - Errors: arguments are validated before anything is launched; on a
 *    validation error nothing runs and a FA_ERR_* code is returned. A failed
 *    launch returns FA_ERR_HIP. Faults inside a kernel surface at the caller's
 *    next synchronisation of `stream`. Unsupported head sizes return
 *    FA_ERR_UNSUPPORTED; there is no fallback path ("FlashAttention &
 *    IO-aware attention", Interviewer follow-ups: a silent fall-back to a
 *    materialising path defeats the method).
 *  - Thread safety: all entry points are reentrant.
 *  - Results are deterministic run to run (no atomics, fixed split counts).
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = 1,        /* a required pointer is NULL                          */
  FA_ERR_SHAPE = 2,       /* a size is < 1, Hq % Hkv != 0, or sizes overflow      */
  FA_ERR_UNSUPPORTED = 3, /* head size not in {64, 128}, or GQA group too large   */
  FA_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned                     */
  FA_ERR_WORKSPACE = 5,   /* decode workspace missing or too small                */
  FA_ERR_HIP = 6          /* the HIP runtime reported an error at launch          */
} fa_status;

/* Human-readable name of a status code (static string, never NULL). */
const char* fa_status_string(int status);

/*
 * fa_fwd - fused exact attention forward ("I/O-Aware Kernels", section
 * FlashAttention: Q blocks resident, K/V streamed blockwise, online softmax).
 *
 *   q   : bf16 [B, Sq,  Hq,  d]     k, v : bf16 [B, Skv, Hkv, d]
 *   o   : bf16 [B, Sq,  Hq,  d]     (written)
 *   lse : fp32 [B, Hq, Sq]          (written; may be NULL to skip)
 *   d in {64, 128}; B, Hq, Hkv, Sq, Skv >= 1; causal is 0 or 1;
 *   scale multiplies Q K^T before the softmax (1/sqrt(d) in the usual case).
 * Returns FA_OK or a fa_status error code.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int Hq, int Hkv, int Sq, int Skv, int d,
           int causal, float scale, void* stream);

/*
 * fa_fwd_f32out - the same computation as fa_fwd with O written as fp32
 * [B, Sq, Hq, d] instead of bf16 (no final output rounding). Used to check the
 * kernel's arithmetic apart from output quantisation; same errors as fa_fwd.
 */
int fa_fwd_f32out(const void* q, const void* k, const void* v, float* o, float* lse,
                  int B, int Hq, int Hkv, int Sq, int Skv, int d,
                  int causal, float scale, void* stream);

/*
 * Split-KV decode ("FlashAttention & IO-aware attention", Deep dive and
 * Interviewer follow-ups: for one query per sequence, split the KV length
 * across compute units, then merge).
 *
 * The Skv keys are cut into num_splits chunks of L = 64 * ceil(ceil(Skv/64) /
 * num_splits) keys: chunk c covers keys [c*L, min(Skv, (c+1)*L)); trailing
 * chunks may be empty. Each chunk yields its own normalised output O_c and
 * log-sum-exp lambda_c; the merge is
 *     LSE = ln sum_c exp(lambda_c),   O = sum_c exp(lambda_c - LSE) * O_c
 * (an empty chunk has lambda_c = -inf and weight 0).
 */

/* Heuristic split count used when num_splits <= 0 (always >= 1): about two
 * workgroups (one per (sequence, KV head, chunk)) per compute unit, chunks of at
 * least 512 keys, at most 64 chunks. */
int fa_decode_default_splits(int B, int Hkv, int Skv, int d);

/* Bytes of workspace fa_decode needs for this shape and split count
 * (num_splits >= 1; pass fa_decode_default_splits(...) for the heuristic's
 * count). Returns 0 on invalid sizes. */
size_t fa_decode_workspace_bytes(int B, int Hq, int d, int num_splits);

/*
 * fa_decode - one decode step: chunk partials, then the merge, both launched on
 * `stream` (no host synchronisation between them). num_splits <= 0 selects
 * fa_decode_default_splits(B, Hkv, Skv, d).
 *   q        : bf16 [B, Hq, d]   (a single query row per sequence and head)
 *   k_cache, v_cache : bf16 [B, Skv, Hkv, d]  (no mask: every key is visible)
 *   o        : bf16 [B, Hq, d]   (written)
 *   lse      : fp32 [B, Hq]      (written; may be NULL)
 *   workspace: device buffer of at least fa_decode_workspace_bytes(B, Hq, d,
 *              num_splits) bytes, owned by the caller, 256-byte aligned. It holds
 *              the fp32 partials [B, Hq, num_splits, d] followed (at the next
 *              256-byte boundary) by the fp32 chunk LSEs [B, Hq, num_splits].
 *   Hq / Hkv must be <= 32 (the query heads of one KV head share one tile).
 */
int fa_decode(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
              int B, int Hq, int Hkv, int Skv, int d, float scale,
              int num_splits, void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_decode_partials - the first half of fa_decode alone: writes the per-chunk
 * normalised outputs part_o fp32 [B, Hq, num_splits, d] and chunk LSEs
 * part_lse fp32 [B, Hq, num_splits]. num_splits must be >= 1.
 */
int fa_decode_partials(const void* q, const void* k_cache, const void* v_cache,
                       float* part_o, float* part_lse,
                       int B, int Hq, int Hkv, int Skv, int d, float scale,
                       int num_splits, void* stream);

/*
 * fa_decode_combine - the merge alone: part_o fp32 [B, Hq, num_splits, d],
 * part_lse fp32 [B, Hq, num_splits] -> o bf16 [B, Hq, d], lse fp32 [B, Hq]
 * (lse may be NULL). If every chunk of a row is empty, O = 0 and LSE = -inf.
 */
int fa_decode_combine(const float* part_o, const float* part_lse, void* o, float* lse,
                      int B, int Hq, int d, int num_splits, void* stream);

/* Bytes of device scratch behind fa_decode_noalloc (16 MiB per GPU). */
#define FA_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * fa_decode_noalloc - fa_decode for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). Same arguments, results and errors as fa_decode without the
 * workspace: the chunk partials go to a scratch array inside the library, one
 * copy per GPU, FA_NOALLOC_SCRATCH_BYTES long, held until the process ends. Its
 * address is looked up once per device on the first call made with that device
 * current; later calls allocate nothing and call no allocating routine.
 *  - The current device must be the device of `stream` and of every pointer.
 *  - Calls whose fa_decode_workspace_bytes(B, Hq, d, num_splits) exceeds
 *    FA_NOALLOC_SCRATCH_BYTES return FA_ERR_WORKSPACE and launch nothing.
 *  - Every call on one GPU shares that GPU's scratch: calls that overlap on one
 *    GPU (different streams, or threads without ordering) race and give
 *    undefined results. Calls ordered on one stream are safe; each call writes
 *    every partial it reads, so nothing needs clearing between calls.
 * Returns FA_OK or a fa_status error code (FA_ERR_HIP if the scratch address
 * cannot be obtained).
 */
int fa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                      int B, int Hq, int Hkv, int Skv, int d, float scale, int num_splits, void* stream);

/*
 * fa_decode_paged - one decode step over a paged KV cache (the paged KV layout
 * that "I/O-Aware Kernels", section FlashAttention, mentions for FlashInfer's
 * kernels; the layout below is this library's own).
 *
 *   q           : bf16 [B, Hq, d]
 *   k_pages, v_pages : bf16 [num_pages, page_size, Hkv, d]  (page pools)
 *   block_table : int32 [B, max_blocks_per_seq]; sequence b's token t lives in
 *                 page block_table[b, t / page_size], slot t % page_size
 *   seq_lens    : int32 [B]; sequence b holds seq_lens[b] tokens, all visible
 *   o, lse      : bf16 [B, Hq, d] and fp32 [B, Hq] (lse may be NULL)
 *   page_size is a power of two in [16, 2^20]; Hq / Hkv <= 32.
 * Chunks are cut from the T = ceil(max_blocks_per_seq * page_size / 64) tiles of
 * 64 keys of the longest possible sequence, the same boundaries for every
 * sequence: chunk c (0 <= c < n = num_splits) covers tiles
 * [floor(T c (2n - c) / n^2), floor(T (c + 1) (2n - c - 1) / n^2)), so chunk
 * sizes fall linearly from about 2 T/n to T/n^2 and the grid, which issues every
 * sequence's first chunk before any second one, runs the largest pieces first.
 * A sequence's chunks past its own length are empty. The merge is fa_decode's. num_splits <= 0 selects the larger
 * of fa_decode_default_splits(B, Hkv, max_blocks_per_seq * page_size, d) and
 * ceil(max_blocks_per_seq * page_size / 2048) (at most 64). The workspace is
 * fa_decode's: fa_decode_workspace_bytes(B, Hq, d, num_splits) bytes, 256-byte
 * aligned; to size it for the default count, pass the count computed above.
 * block_table and seq_lens are device memory and are not read by the host:
 * lengths are clamped to [0, max_blocks_per_seq * page_size] and page ids to
 * [0, num_pages - 1], so bad entries give unspecified results for that
 * sequence but never an out-of-bounds access. A sequence of length 0 gets
 * O = 0 and LSE = -inf. block_table and seq_lens must be 4-byte aligned.
 */
int fa_decode_paged(const void* q, const void* k_pages, const void* v_pages, const int* block_table,
                    const int* seq_lens, void* o, float* lse, int B, int Hq, int Hkv, int d, int page_size,
                    int max_blocks_per_seq, int num_pages, float scale, int num_splits, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * fa_bwd_workspace_bytes - bytes of device workspace fa_bwd needs: one fp32 per
 * query row and head (D_i = dO_i . O_i), rounded up to 256. 0 for bad sizes.
 */
size_t fa_bwd_workspace_bytes(int B, int Hq, int Sq);

/*
 * fa_bwd - backward pass of exact attention: dQ, dK, dV for the forward of fa_fwd
 * with the same q, k, v, causal flag and scale. The backward recomputes the
 * attention probabilities instead of storing them ("Tracing Tiled QKV Data Movement
 * in FlashAttention's Memory Hierarchy", Conclusion); the gradients are those of the
 * forward's definition (chain rule through the row softmax):
 *   P_ij = exp(scale * q_i.k_j - LSE_i) for visible j, D_i = dO_i . O_i,
 *   dS_ij = P_ij (dO_i . v_j - D_i),
 *   dV_j = sum_i P_ij dO_i, dK_j = scale sum_i dS_ij q_i, dQ_i = scale sum_j dS_ij k_j,
 * where a KV head sums over every query head of its group (GQA). Arithmetic: bf16
 * matrix-core products with fp32 accumulation; each product's bf16 factor (P for dV, dS
 * for dQ and dK) is rounded to nearest even, D uses the bf16 O, and at d = 128 the dS of
 * dK is formed from P as rounded for the dV product. Results are deterministic.
 *
 *   q, o, dout, dq : bf16 [B, Sq, Hq, d]   (o and lse: outputs of fa_fwd)
 *   k, v, dk, dv   : bf16 [B, Skv, Hkv, d]
 *   lse            : fp32 [B, Hq, Sq], natural log (-inf for rows with no visible key)
 *   workspace      : device memory of at least fa_bwd_workspace_bytes(B, Hq, Sq)
 *                    bytes (overwritten; no state is kept between calls)
 * All pointers are device memory, 16-byte aligned, caller-owned; outputs are fully
 * overwritten (no accumulation into dq, dk, dv). Same shape and head-size rules as
 * fa_fwd (d = 64 or 128, Hq % Hkv == 0); scale must be finite (any sign). Causal
 * masking is aligned bottom-right as in fa_fwd. Rows with no visible key get dQ = 0.
 * Two kernels run on `stream` in order (dQ and D, then dK and dV); nothing is
 * allocated or synchronised. Returns FA_OK or an FA_ERR_* code before launching.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
           void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq, int Skv, int d, int causal, float scale,
           void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_fwd_fp8 - exact attention forward on fp8 inputs (the FP8 variant that
 * FlashAttention-3 adds: "FlashAttention & IO-aware attention", Deep dive). The
 * result approximates softmax(scale * Q K^T) V of the dequantised tensors
 *   Q = e4m3(q8) * q_scale[b, h],  K = e4m3(k8) * k_scale[b, hk],
 *   V[b, j, hk, :] = e4m3(vt8[b, hk, :, j]) * v_scale[b, hk],
 * with both products on the fp8 matrix cores (P rounded to e4m3 before the P.V
 * product; the normaliser sums the unrounded probabilities).
 *
 *   q8   : e4m3 codes (OCP: sign, 4 exponent bits with bias 7, 3 mantissa bits; 0x7F
 *          and 0xFF are NaN) [B, Sq, Hq, d]
 *   k8   : e4m3 codes [B, Skv, Hkv, d]
 *   vt8  : e4m3 codes of V transposed, [B, Hkv, d, ldv]; columns j < Skv are keys,
 *          columns Skv .. ldv-1 are padding that must hold finite codes (zeros, say)
 *   q_scale [B, Hq], k_scale [B, Hkv], v_scale [B, Hkv]: fp32 dequantisation scales
 *   o    : bf16 [B, Sq, Hq, d];  lse: fp32 [B, Hq, Sq] natural log, or NULL
 *   ldv  : multiple of 16, >= Skv rounded up to 16, with d * ldv <= 2e9
 * d = 64 or 128, Hq % Hkv == 0, causal aligned bottom-right as in fa_fwd, scale finite.
 * Device pointers: q8, k8, vt8, o, lse 16-byte aligned; the scales 4-byte aligned.
 * Inputs must be finite. One launch on `stream`; nothing is allocated. Returns FA_OK or
 * an FA_ERR_* code before launching.
 */
int fa_fwd_fp8(const void* q8, const void* k8, const void* vt8, const float* q_scale, const float* k_scale,
               const float* v_scale, void* o, float* lse, int B, int Hq, int Hkv, int Sq, int Skv, int ldv, int d,
               int causal, float scale, void* stream);

/*
 * fa_bpt_workspace_bytes - device workspace fa_bpt_layer needs: for one block of
 * R = min(block_rows, S) query rows of every batch element, the block's attention output
 * (bf16, B*R x Hq*d) and its hidden activations (bf16, B*R x d_ff), each rounded up to
 * 256 bytes. 0 for bad sizes.
 */
size_t fa_bpt_workspace_bytes(int B, int S, int block_rows, int Hq, int d, int d_ff);

/*
 * fa_bpt_layer - attention followed by the position-wise feed-forward network, run
 * blockwise ("I/O-Aware Kernels", section Blockwise Parallel Transformers): for each
 * block of `block_rows` query rows (taken from every batch element at once), the
 * attention output of the block (fa_fwd's kernel, causal positions taken from the whole
 * sequence) goes straight through
 *     y = relu(h W1^T + b1) W2^T + b2,   h = the block's attention output, heads concatenated,
 * so only one block's activations ever exist (the workspace), not the sequence's. Both
 * products run on this library's bf16 matrix-core GEMM kernel (fp32 accumulation, the
 * bias and ReLU applied to the fp32 sums, one bf16 rounding at the store).
 *
 *   q : bf16 [B, S, Hq, d];  k, v : bf16 [B, S, Hkv, d]  (self-attention, Sq = Skv = S)
 *   w1: bf16 [d_ff, Hq*d] (a linear layer's [out, in] weight);  b1: bf16 [d_ff]
 *   w2: bf16 [Hq*d, d_ff];  b2: bf16 [Hq*d]
 *   y : bf16 [B, S, Hq*d]
 *   workspace: at least fa_bpt_workspace_bytes(B, S, block_rows, Hq, d, d_ff) bytes,
 *              256-byte aligned, caller-owned, overwritten.
 * The block's attention output and the hidden activations are rounded to bf16. Same
 * shape rules as fa_fwd; d_ff a positive multiple of 64; block_rows >= 1 (values >= S
 * give the whole-sequence schedule). All tensors are device memory, 16-byte aligned.
 * Per block, three kernels run on `stream` in order; nothing is allocated or
 * synchronised. Returns FA_OK or an FA_ERR_* code (FA_ERR_HIP for a failed launch, after
 * earlier blocks may have run).
 */
int fa_bpt_layer(const void* q, const void* k, const void* v, const void* w1, const void* b1, const void* w2,
                 const void* b2, void* y, int B, int Hq, int Hkv, int S, int d, int d_ff, int causal, float scale,
                 int block_rows, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
