// C ABI of the attention library: argument validation, then one launch per step on the
// caller's stream. Nothing here allocates memory or synchronises.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "fa.h"
#include "fa_bpt.hpp"
#include "fa_bwd.hpp"
#include "fa_fp8.hpp"
#include "fa_launch.hpp"

// Device memory the allocation-free decode (fa_decode_noalloc) uses for its chunk
// partials. Each GPU the library runs on holds one copy until the process ends. In host
// code the array's name is only a stand-in: its device address is obtained once per
// device with hipGetSymbolAddress (with that device current) and kept in scratch_addr.
static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr unsigned kQsignMask = 0x80008000u;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_common(int B, int Hq, int Hkv, int Sq, int Skv, int d) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Skv < 1) return FA_ERR_SHAPE;
  if (Hq % Hkv != 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  // element counts must stay well inside int64 and row indices inside int32
  const double q_elems = (double)B * Sq * Hq * d;
  const double kv_elems = (double)B * Skv * Hkv * d;
  if (q_elems > 4.0e18 || kv_elems > 4.0e18) return FA_ERR_SHAPE;
  if ((double)B * Sq > 2.0e9 || (double)B * Skv * Hkv > 2.0e9 || (double)B * Hq > 2.0e9) return FA_ERR_SHAPE;
  return FA_OK;
}

// The streaming kernels address the rows of one tile with 32-bit per-lane byte offsets
// from the tile's first row: `rows` rows of `row_bytes` each must span less than 2^32 bytes.
bool tile_offsets_fit(int rows, double row_bytes) { return (double)rows * row_bytes <= 4294967296.0; }

// The kernels need a positive exponent factor c = |scale| * log2(e). A negative scale
// is folded into Q by flipping its sign bits (exact in bf16). With scale == 0 every
// score is exactly 0, which is what a zeroed Q gives for any c, so Q is masked to 0.
int scale_terms(float scale, float* c, unsigned* qsign, unsigned* qmask) {
  if (!isfinite(scale)) return FA_ERR_SHAPE;
  *c = scale == 0.f ? 1.f : fabsf(scale) * 1.4426950408889634f;
  *qsign = scale < 0.f ? kQsignMask : 0u;
  *qmask = scale == 0.f ? 0u : 0xFFFFFFFFu;
  return FA_OK;
}

int fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
             int Sq, int Skv, int d, int causal, float scale, void* stream, bool out_f32) {
  if (!q || !k || !v || !o) return FA_ERR_NULL;
  int st = check_common(B, Hq, Hkv, Sq, Skv, d);
  if (st != FA_OK) return st;
  if (causal != 0 && causal != 1) return FA_ERR_SHAPE;
  if (!tile_offsets_fit(64, (double)Hkv * d * 2)) return FA_ERR_SHAPE;   // 64-key K/V tiles
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (lse && !aligned16(lse)))
    return FA_ERR_ALIGN;
  fa::FwdParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = o;
  p.lse = lse;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Sq = Sq; p.Skv = Skv; p.d = d;
  p.q_bstride = p.o_bstride = (int64_t)Sq * Hq * d;
  p.kv_bstride = (int64_t)Skv * Hkv * d;
  st = scale_terms(scale, &p.c, &p.qsign, &p.qmask);
  if (st != FA_OK) return st;
  if (fa::fwd_grid_size(B, Hq, Sq, d) > 0x7fffffffLL) return FA_ERR_SHAPE;
  (void)hipGetLastError();
  if (fa::launch_fwd(p, causal != 0, out_f32, static_cast<hipStream_t>(stream)) != hipSuccess) return FA_ERR_HIP;
  return FA_OK;
}

int split_chunk(int Skv, int nsplit) {
  const int tiles = (Skv + fa::kSplitAlign - 1) / fa::kSplitAlign;
  return fa::kSplitAlign * ((tiles + nsplit - 1) / nsplit);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int decode_args(const void* q, const void* k, const void* v, int B, int Hq, int Hkv, int Skv, int d,
                int nsplit) {
  if (!q || !k || !v) return FA_ERR_NULL;
  int st = check_common(B, Hq, Hkv, 1, Skv, d);
  if (st != FA_OK) return st;
  if (Hq / Hkv > 32) return FA_ERR_UNSUPPORTED;
  if (nsplit < 1 || (double)B * Hkv * nsplit > 2.0e9) return FA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return FA_ERR_ALIGN;
  return FA_OK;
}

int combine_impl(const float* part_o, const float* part_lse, void* o, float* lse, int B, int Hq, int d,
                 int nsplit, hipStream_t stream) {
  fa::CombineParams c;
  c.part_o = part_o;
  c.part_lse = part_lse;
  c.o = static_cast<uint16_t*>(o);
  c.lse = lse;
  c.rows = B * Hq;
  c.d = d;
  c.nsplit = nsplit;
  (void)hipGetLastError();
  if (fa::launch_decode_combine(c, stream) != hipSuccess) return FA_ERR_HIP;
  return FA_OK;
}

int partials_impl(const void* q, const void* k, const void* v, float* part_o, float* part_lse, int B, int Hq,
                  int Hkv, int Skv, int d, float scale, int nsplit, hipStream_t stream) {
  fa::DecParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.part_o = part_o;
  p.part_lse = part_lse;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Skv = Skv; p.d = d;
  p.nsplit = nsplit;
  p.chunk = split_chunk(Skv, nsplit);
  int st = scale_terms(scale, &p.c, &p.qsign, &p.qmask);
  if (st != FA_OK) return st;
  (void)hipGetLastError();
  if (fa::launch_decode_partials(p, stream) != hipSuccess) return FA_ERR_HIP;
  return FA_OK;
}

int paged_partials_impl(const void* q, const void* k_pages, const void* v_pages, const int* block_table,
                        const int* seq_lens, float* part_o, float* part_lse, int B, int Hq, int Hkv, int d,
                        int page_log2, int max_blocks, int num_pages, float scale, int nsplit, hipStream_t stream) {
  fa::DecParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k_pages);
  p.v = static_cast<const uint16_t*>(v_pages);
  p.part_o = part_o;
  p.part_lse = part_lse;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.d = d;
  p.Skv = max_blocks << page_log2;
  p.nsplit = nsplit;
  p.chunk = split_chunk(p.Skv, nsplit);
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.page_log2 = page_log2;
  p.max_blocks = max_blocks;
  p.num_pages = num_pages;
  int st = scale_terms(scale, &p.c, &p.qsign, &p.qmask);
  if (st != FA_OK) return st;
  (void)hipGetLastError();
  if (fa::launch_decode_paged_partials(p, stream) != hipSuccess) return FA_ERR_HIP;
  return FA_OK;
}

// Argument checks of one decode step (everything but the workspace).
int decode_checks(const void* q, const void* k, const void* v, const void* o, const float* lse, int B, int Hq,
                  int Hkv, int Skv, int d, int nsplit) {
  int st = decode_args(q, k, v, B, Hq, Hkv, Skv, d, nsplit);
  if (st != FA_OK) return st;
  if (!o) return FA_ERR_NULL;
  if (!aligned16(o) || (lse && !aligned16(lse))) return FA_ERR_ALIGN;
  return FA_OK;
}

// Chunk partials into `workspace` (laid out as fa_decode_workspace_bytes describes), then the merge.
int decode_launch(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int Skv,
                  int d, float scale, int nsplit, void* workspace, hipStream_t s) {
  float* part_o = static_cast<float*>(workspace);
  float* part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                             align256((size_t)B * Hq * nsplit * d * sizeof(float)));
  int st = partials_impl(q, k, v, part_o, part_lse, B, Hq, Hkv, Skv, d, scale, nsplit, s);
  if (st != FA_OK) return st;
  return combine_impl(part_o, part_lse, o, lse, B, Hq, d, nsplit, s);
}

// ---- scratch of the allocation-free decode ------------------------------------------
constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_addr[kMaxDevices];
std::mutex scratch_mu;

// Device address of the current device's scratch array (looked up on the first call per device).
int scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_HIP;
  void* ptr = scratch_addr[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    std::lock_guard<std::mutex> lock(scratch_mu);
    ptr = scratch_addr[dev].load(std::memory_order_relaxed);
    if (ptr == nullptr) {
      if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return FA_ERR_HIP;
      scratch_addr[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return FA_OK;
}

int log2_exact(int x) {
  int l = 0;
  while ((1 << l) < x && l < 30) ++l;
  return (1 << l) == x ? l : -1;
}

}  // namespace

extern "C" {

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: invalid sizes, head counts or scale";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: head size must be 64 or 128 (decode: Hq/Hkv <= 32)";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: every pointer must be 16-byte aligned";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: decode workspace missing, misaligned or too small";
    case FA_ERR_HIP: return "FA_ERR_HIP: the HIP runtime rejected the launch";
    default: return "unknown fa_status";
  }
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int Sq,
           int Skv, int d, int causal, float scale, void* stream) {
  return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, d, causal, scale, stream, false);
}

int fa_fwd_f32out(const void* q, const void* k, const void* v, float* o, float* lse, int B, int Hq, int Hkv,
                  int Sq, int Skv, int d, int causal, float scale, void* stream) {
  return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, d, causal, scale, stream, true);
}

int fa_decode_default_splits(int B, int Hkv, int Skv, int d) {
  (void)d;
  if (B < 1 || Hkv < 1 || Skv < 1) return 1;
  // Aim for about two workgroups per compute unit (256 CUs) while keeping every chunk
  // at least 512 keys long: with non-temporal cache loads, 512 workgroups of long chunks
  // stream HBM faster than more, shorter ones (B 4..64, Hkv 8, Skv 4096..16384, d 128).
  const long long units = (long long)B * Hkv;
  long long want = (2LL * 256 + units - 1) / units;
  long long most = (Skv + 511) / 512;
  if (want > most) want = most;
  if (want > 64) want = 64;
  if (want < 1) want = 1;
  return (int)want;
}

size_t fa_decode_workspace_bytes(int B, int Hq, int d, int num_splits) {
  if (B < 1 || Hq < 1 || d < 1) return 0;
  if (num_splits <= 0) return 0;
  const size_t rows = (size_t)B * Hq * num_splits;
  return align256(rows * d * sizeof(float)) + align256(rows * sizeof(float));
}

int fa_decode_partials(const void* q, const void* k_cache, const void* v_cache, float* part_o, float* part_lse,
                       int B, int Hq, int Hkv, int Skv, int d, float scale, int num_splits, void* stream) {
  int st = decode_args(q, k_cache, v_cache, B, Hq, Hkv, Skv, d, num_splits);
  if (st != FA_OK) return st;
  if (!part_o || !part_lse) return FA_ERR_NULL;
  if (!aligned16(part_o) || !aligned16(part_lse)) return FA_ERR_ALIGN;
  return partials_impl(q, k_cache, v_cache, part_o, part_lse, B, Hq, Hkv, Skv, d, scale, num_splits,
                       static_cast<hipStream_t>(stream));
}

int fa_decode_combine(const float* part_o, const float* part_lse, void* o, float* lse, int B, int Hq, int d,
                      int num_splits, void* stream) {
  if (!part_o || !part_lse || !o) return FA_ERR_NULL;
  if (B < 1 || Hq < 1 || num_splits < 1 || (double)B * Hq > 2.0e9) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (!aligned16(part_o) || !aligned16(part_lse) || !aligned16(o) || (lse && !aligned16(lse)))
    return FA_ERR_ALIGN;
  return combine_impl(part_o, part_lse, o, lse, B, Hq, d, num_splits, static_cast<hipStream_t>(stream));
}

int fa_decode(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse, int B, int Hq,
              int Hkv, int Skv, int d, float scale, int num_splits, void* workspace, size_t workspace_bytes,
              void* stream) {
  if (num_splits <= 0) num_splits = fa_decode_default_splits(B, Hkv, Skv, d);
  int st = decode_checks(q, k_cache, v_cache, o, lse, B, Hq, Hkv, Skv, d, num_splits);
  if (st != FA_OK) return st;
  const size_t need = fa_decode_workspace_bytes(B, Hq, d, num_splits);
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 || workspace_bytes < need)
    return FA_ERR_WORKSPACE;
  return decode_launch(q, k_cache, v_cache, o, lse, B, Hq, Hkv, Skv, d, scale, num_splits, workspace,
                       static_cast<hipStream_t>(stream));
}

int fa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse, int B, int Hq,
                      int Hkv, int Skv, int d, float scale, int num_splits, void* stream) {
  if (num_splits <= 0) num_splits = fa_decode_default_splits(B, Hkv, Skv, d);
  int st = decode_checks(q, k_cache, v_cache, o, lse, B, Hq, Hkv, Skv, d, num_splits);
  if (st != FA_OK) return st;
  // the limit is checked before the device is touched, so an oversized call launches nothing
  if (fa_decode_workspace_bytes(B, Hq, d, num_splits) > (size_t)FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_WORKSPACE;
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != FA_OK) return st;
  return decode_launch(q, k_cache, v_cache, o, lse, B, Hq, Hkv, Skv, d, scale, num_splits, ws,
                       static_cast<hipStream_t>(stream));
}

int fa_decode_paged(const void* q, const void* k_pages, const void* v_pages, const int* block_table,
                    const int* seq_lens, void* o, float* lse, int B, int Hq, int Hkv, int d, int page_size,
                    int max_blocks_per_seq, int num_pages, float scale, int num_splits, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (!q || !k_pages || !v_pages || !block_table || !seq_lens || !o) return FA_ERR_NULL;
  if (B < 1 || Hq < 1 || Hkv < 1 || max_blocks_per_seq < 1 || num_pages < 1) return FA_ERR_SHAPE;
  if (Hq % Hkv != 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (Hq / Hkv > 32) return FA_ERR_UNSUPPORTED;
  const int page_log2 = log2_exact(page_size);
  if (page_log2 < 4 || page_log2 > 20) return FA_ERR_SHAPE;     // power of two, 16 .. 2^20 tokens
  const double max_len = (double)max_blocks_per_seq * page_size;
  if (max_len > 2.0e9 || (double)num_pages * page_size * Hkv * d > 4.0e18 || (double)B * max_blocks_per_seq > 2.0e9 ||
      (double)B * Hq > 2.0e9)
    return FA_ERR_SHAPE;
  if (num_splits <= 0) {
    // lengths vary per sequence: besides filling the CUs, keep chunks near 2048 keys so
    // that long and short sequences spread over many equal workgroups
    num_splits = fa_decode_default_splits(B, Hkv, (int)max_len, d);
    const long long by_len = ((long long)max_len + 2047) / 2048;
    if (by_len > num_splits) num_splits = (int)(by_len < 64 ? by_len : 64);
  }
  if (num_splits < 1 || (double)B * Hkv * num_splits > 2.0e9) return FA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages) || !aligned16(o) || (lse && !aligned16(lse)) ||
      (reinterpret_cast<uintptr_t>(block_table) & 3u) || (reinterpret_cast<uintptr_t>(seq_lens) & 3u))
    return FA_ERR_ALIGN;
  const size_t need = fa_decode_workspace_bytes(B, Hq, d, num_splits);
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 || workspace_bytes < need)
    return FA_ERR_WORKSPACE;
  float* part_o = static_cast<float*>(workspace);
  float* part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                             align256((size_t)B * Hq * num_splits * d * sizeof(float)));
  hipStream_t s = static_cast<hipStream_t>(stream);
  int st = paged_partials_impl(q, k_pages, v_pages, block_table, seq_lens, part_o, part_lse, B, Hq, Hkv, d,
                               page_log2, max_blocks_per_seq, num_pages, scale, num_splits, s);
  if (st != FA_OK) return st;
  return combine_impl(part_o, part_lse, o, lse, B, Hq, d, num_splits, s);
}

size_t fa_bwd_workspace_bytes(int B, int Hq, int Sq) {
  if (B < 1 || Hq < 1 || Sq < 1) return 0;
  return align256((size_t)B * Hq * Sq * sizeof(float));
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout, void* dq,
           void* dk, void* dv, int B, int Hq, int Hkv, int Sq, int Skv, int d, int causal, float scale,
           void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return FA_ERR_NULL;
  int st = check_common(B, Hq, Hkv, Sq, Skv, d);
  if (st != FA_OK) return st;
  if (causal != 0 && causal != 1) return FA_ERR_SHAPE;
  if (!isfinite(scale)) return FA_ERR_SHAPE;
  // 64-row K/V tiles (dQ kernel) and 128-row Q/dO tiles (dK/dV kernel)
  if (!tile_offsets_fit(64, (double)Hkv * d * 2) || !tile_offsets_fit(128, (double)Hq * d * 2)) return FA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv) || !aligned16(lse))
    return FA_ERR_ALIGN;
  if (!workspace || workspace_bytes < fa_bwd_workspace_bytes(B, Hq, Sq)) return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_ALIGN;
  if (fa::bwd_dq_grid(B, Hq, Sq, d) > 0x7fffffffLL || fa::bwd_dkdv_grid(B, Hkv, Skv) > 0x7fffffffLL) return FA_ERR_SHAPE;
  fa::BwdParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<const uint16_t*>(o);
  p.dout = static_cast<const uint16_t*>(dout);
  p.lse = lse;
  p.dq = static_cast<uint16_t*>(dq);
  p.dk = static_cast<uint16_t*>(dk);
  p.dv = static_cast<uint16_t*>(dv);
  p.dsum = static_cast<float*>(workspace);
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Sq = Sq; p.Skv = Skv; p.d = d;
  p.scale = scale;
  p.c = scale * 1.4426950408889634f;
  (void)hipGetLastError();
  if (fa::launch_bwd(p, causal != 0, static_cast<hipStream_t>(stream)) != hipSuccess) return FA_ERR_HIP;
  return FA_OK;
}

int fa_fwd_fp8(const void* q8, const void* k8, const void* vt8, const float* q_scale, const float* k_scale,
               const float* v_scale, void* o, float* lse, int B, int Hq, int Hkv, int Sq, int Skv, int ldv, int d,
               int causal, float scale, void* stream) {
  if (!q8 || !k8 || !vt8 || !q_scale || !k_scale || !v_scale || !o) return FA_ERR_NULL;
  int st = check_common(B, Hq, Hkv, Sq, Skv, d);
  if (st != FA_OK) return st;
  if (causal != 0 && causal != 1) return FA_ERR_SHAPE;
  if (!isfinite(scale)) return FA_ERR_SHAPE;
  // V^T rows: at least Skv rounded up to 16 bytes, a multiple of 16, and small enough
  // that d rows of one head stay within 32-bit byte offsets
  if (ldv % 16 != 0 || ldv < (Skv + 15) / 16 * 16 || (double)ldv * d > 2.0e9) return FA_ERR_SHAPE;
  if ((double)B * Hkv * d * ldv > 4.0e18) return FA_ERR_SHAPE;
  if (!tile_offsets_fit(64, (double)Hkv * d)) return FA_ERR_SHAPE;        // 64-key e4m3 K tiles
  if (!aligned16(q8) || !aligned16(k8) || !aligned16(vt8) || !aligned16(o) || (lse && !aligned16(lse)))
    return FA_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(q_scale) | reinterpret_cast<uintptr_t>(k_scale) |
       reinterpret_cast<uintptr_t>(v_scale)) & 3u)
    return FA_ERR_ALIGN;
  if (fa::fp8_grid_size(B, Hq, Sq, d) > 0x7fffffffLL) return FA_ERR_SHAPE;
  fa::Fp8Params p;
  p.q = static_cast<const uint8_t*>(q8);
  p.k = static_cast<const uint8_t*>(k8);
  p.vt = static_cast<const uint8_t*>(vt8);
  p.q_scale = q_scale;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Sq = Sq; p.Skv = Skv; p.d = d; p.ldv = ldv;
  p.c = scale * 1.4426950408889634f;
  (void)hipGetLastError();
  if (fa::launch_fwd_fp8(p, causal != 0, static_cast<hipStream_t>(stream)) != hipSuccess) return FA_ERR_HIP;
  return FA_OK;
}

size_t fa_bpt_workspace_bytes(int B, int S, int block_rows, int Hq, int d, int d_ff) {
  if (B < 1 || S < 1 || block_rows < 1 || Hq < 1 || d < 1 || d_ff < 1) return 0;
  const size_t rows = (size_t)B * (block_rows < S ? block_rows : S);
  return align256(rows * Hq * d * 2) + align256(rows * d_ff * 2);
}

int fa_bpt_layer(const void* q, const void* k, const void* v, const void* w1, const void* b1, const void* w2,
                 const void* b2, void* y, int B, int Hq, int Hkv, int S, int d, int d_ff, int causal, float scale,
                 int block_rows, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !w1 || !b1 || !w2 || !b2 || !y) return FA_ERR_NULL;
  int st = check_common(B, Hq, Hkv, S, S, d);
  if (st != FA_OK) return st;
  if (causal != 0 && causal != 1) return FA_ERR_SHAPE;
  if (!tile_offsets_fit(64, (double)Hkv * d * 2)) return FA_ERR_SHAPE;
  // the GEMMs take K in steps of 64 and N in blocks of 32, and address a 256-row tile with
  // 32-bit offsets (d_model = Hq * d is a multiple of 64 already)
  if (d_ff < 64 || d_ff % 64 != 0 || block_rows < 1 || (double)Hq * d * d_ff > 2.0e9 ||
      (double)B * S * Hq * d > 4.0e18 || !tile_offsets_fit(256, (double)d_ff * 2) ||
      !tile_offsets_fit(256, (double)Hq * d * 2))
    return FA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(w1) || !aligned16(b1) || !aligned16(w2) ||
      !aligned16(b2) || !aligned16(y))
    return FA_ERR_ALIGN;
  const int rows_max = block_rows < S ? block_rows : S;
  // one block of rows of every batch element runs at once
  if ((double)B * rows_max > 2.0e9 || fa::fwd_grid_size(B, Hq, rows_max, d) > 0x7fffffffLL ||
      fa::ffn_gemm_grid(B * rows_max, d_ff) > 0x7fffffffLL)
    return FA_ERR_SHAPE;
  if (!workspace || workspace_bytes < fa_bpt_workspace_bytes(B, S, block_rows, Hq, d, d_ff)) return FA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return FA_ERR_ALIGN;
  fa::FwdParams p;
  st = scale_terms(scale, &p.c, &p.qsign, &p.qmask);
  if (st != FA_OK) return st;
  // workspace: the attention output of one row block of every batch element
  // [B * rows, Hq * d], then its hidden activations [B * rows, d_ff]
  const int dm = Hq * d;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  uint16_t* attn = reinterpret_cast<uint16_t*>(ws);
  uint16_t* mid = reinterpret_cast<uint16_t*>(ws + align256((size_t)B * rows_max * dm * 2));
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  for (int r0 = 0; r0 < S; r0 += rows_max) {
    const int rows = S - r0 < rows_max ? S - r0 : rows_max;
    // attention of query rows r0 .. r0 + rows - 1 of every batch element: causal rows see
    // keys up to their own position, which the bottom-right alignment gives with
    // Skv = r0 + rows; q and k/v keep the whole sequence's batch strides
    p.q = static_cast<const uint16_t*>(q) + (int64_t)r0 * dm;
    p.k = static_cast<const uint16_t*>(k);
    p.v = static_cast<const uint16_t*>(v);
    p.o = attn;
    p.lse = nullptr;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Sq = rows; p.Skv = causal ? r0 + rows : S; p.d = d;
    p.q_bstride = (int64_t)S * dm;
    p.kv_bstride = (int64_t)S * Hkv * d;
    p.o_bstride = (int64_t)rows * dm;
    if (fa::launch_fwd(p, causal != 0, false, hs) != hipSuccess) return FA_ERR_HIP;
    // feed-forward network of the block: mid = relu(attn W1^T + b1), y = mid W2^T + b2
    fa::FfnGemmParams g1;
    g1.x = attn; g1.w = static_cast<const uint16_t*>(w1); g1.bias = static_cast<const uint16_t*>(b1); g1.c = mid;
    g1.M = B * rows; g1.N = d_ff; g1.K = dm; g1.ldc = d_ff; g1.group_rows = g1.M; g1.group_stride = g1.M;
    if (fa::launch_ffn_gemm(g1, true, hs) != hipSuccess) return FA_ERR_HIP;
    fa::FfnGemmParams g2;
    g2.x = mid; g2.w = static_cast<const uint16_t*>(w2); g2.bias = static_cast<const uint16_t*>(b2);
    g2.c = static_cast<uint16_t*>(y) + (int64_t)r0 * dm;          // row b * rows + i -> y[b, r0 + i]
    g2.M = B * rows; g2.N = dm; g2.K = d_ff; g2.ldc = dm; g2.group_rows = rows; g2.group_stride = S;
    if (fa::launch_ffn_gemm(g2, false, hs) != hipSuccess) return FA_ERR_HIP;
  }
  return FA_OK;
}

}  // extern "C"
