// Internal launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Waves per prefill workgroup (32 query rows each, two waves per SIMD) and per
// decode-split workgroup (each wave takes 32 keys of every KV tile).
constexpr int kFwdWaves = 8;
// At d = 64 a prefill workgroup has four waves (128 query rows) and three workgroups
// share a CU (168 registers): the finer grain shortens the causal tail of the small-head
// shapes.
constexpr int fwd_waves(int d) { return d == 64 ? 4 : kFwdWaves; }
constexpr int kDecWaves = 2;
constexpr int kDecTile = 32 * kDecWaves;   // keys per decode KV tile
constexpr int kSplitAlign = 64;            // decode chunk lengths are multiples of this

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  void* o;
  float* lse;
  int B, Hq, Hkv, Sq, Skv, d;
  // elements between batch elements of q, of k and v, and of o (Sq*Hq*d, Skv*Hkv*d and
  // Sq*Hq*d for contiguous tensors; the blockwise layer runs one row block of every
  // batch element at once); lse is always contiguous [B, Hq, Sq]
  int64_t q_bstride, kv_bstride, o_bstride;
  float c;          // |scale| * log2(e), or 1 when scale == 0 (then Q is zeroed)
  unsigned qsign;   // 0x80008000 when scale < 0 (negates Q exactly), else 0
  unsigned qmask;   // 0 when scale == 0 (every score is exactly 0), else all ones
};

struct DecParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  float* part_o;    // [B, Hq, nsplit, d]
  float* part_lse;  // [B, Hq, nsplit]
  int B, Hq, Hkv, Skv, d;
  int nsplit, chunk;  // chunk = keys per split (multiple of kSplitAlign); contiguous caches only
  float c;
  unsigned qsign;
  unsigned qmask;
  // Paged caches only: k and v are page pools [num_pages, page_size, Hkv, d];
  // sequence b's token t lives in page block_table[b * max_blocks + t / page_size]
  // at slot t % page_size, and the sequence holds seq_lens[b] tokens.
  const int* block_table;   // [B, max_blocks]
  const int* seq_lens;      // [B]
  int page_log2, max_blocks, num_pages;
};

struct CombineParams {
  const float* part_o;
  const float* part_lse;
  uint16_t* o;
  float* lse;
  int rows;         // B * Hq
  int d, nsplit;
};

long long fwd_grid_size(int B, int Hq, int Sq, int d);
hipError_t launch_fwd(const FwdParams& p, bool causal, bool out_f32, hipStream_t stream);
hipError_t launch_decode_partials(const DecParams& p, hipStream_t stream);
hipError_t launch_decode_paged_partials(const DecParams& p, hipStream_t stream);
hipError_t launch_decode_combine(const CombineParams& p, hipStream_t stream);

}  // namespace fa
