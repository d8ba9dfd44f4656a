// Split-KV decode for gfx950: one query row per (sequence, query head).
//
// A decode step has a single query, so its scores are a 1 x Skv vector and the step
// is bound by reading the KV cache ("FlashAttention & IO-aware attention", Direct
// answer and Interviewer follow-ups). To occupy every compute unit the KV length is
// cut into chunks that run in separate workgroups (Deep dive: FlashDecoding splits
// the KV length across SMs), each producing a chunk-normalised output and its
// log-sum-exp; a second kernel merges the chunks by log-sum-exp.
//
// The query heads that share one KV head (grouped-query attention, "I/O-Aware
// Kernels", section FlashAttention) are the columns of one MFMA tile, so every K/V
// byte is read once for the whole group. Inside a workgroup each wave takes its own
// 32 keys of every tile; the waves' partial statistics are merged through LDS.
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

// Copy of one K tile and one V tile of a paged cache (global -> registers -> LDS).
// Thread t copies 16-byte column t % CPR of PER_T consecutive keys, starting at key
// (t / CPR) * PER_T of the tile. Those keys share one page (pages hold at least 16
// tokens and PER_T <= 8 divides 16), so a thread needs a single page-table entry per
// tile, looked up one tile ahead by fetch_page.
template <int D, int BCT, int NT>
struct PagedTileCopy : TileCopy<D, BCT, NT> {
  using Base = TileCopy<D, BCT, NT>;
  using Base::CPR;
  using Base::PER_T;
  static_assert(Base::CHUNKS == PER_T * NT && NT % CPR == 0, "every thread copies PER_T whole chunks");
  static_assert(PER_T <= 16 && 16 % PER_T == 0, "a thread's keys must stay inside one 16-token page");

  __device__ __forceinline__ static int first_key(int tid) { return (tid / CPR) * PER_T; }

  // Page id of this thread's keys in the tile starting at key k0 (0 when they are all
  // at or past kmax). Ids outside [0, num_pages) are clamped, so a bad table entry
  // cannot read outside the page pool.
  __device__ __forceinline__ static int fetch_page(const int* __restrict__ bt_row, int k0, int kmax,
                                                   int page_log2, int num_pages, int tid) {
    const int key = k0 + first_key(tid);
    return key < kmax ? min(max(bt_row[key >> page_log2], 0), num_pages - 1) : 0;
  }

  // kp / vp: page pool base + this head's offset; row_stride = Hkv * D elements.
  __device__ __forceinline__ void load_paged(const uint16_t* __restrict__ kp, const uint16_t* __restrict__ vp,
                                             int64_t row_stride, int page_log2, int k0, int kmax, int pid,
                                             int tid) {
    const int pmask = (1 << page_log2) - 1;
    const int key0 = k0 + first_key(tid), c = tid % CPR;
    const int64_t base = (((int64_t)pid << page_log2) + (key0 & pmask)) * row_stride + c * 8;
#pragma unroll
    for (int p = 0; p < PER_T; ++p) {
      u32x4 zk = {0u, 0u, 0u, 0u}, zv = {0u, 0u, 0u, 0u};
      if (key0 + p < kmax) {
        zk = stream_load16(kp + base + p * row_stride);
        zv = stream_load16(vp + base + p * row_stride);
      }
      this->kr[p] = zk;
      this->vr[p] = zv;
    }
  }

  __device__ __forceinline__ void store_paged(uint16_t* ks, uint16_t* vs, int tid) const {
    const int key0 = first_key(tid), c = tid % CPR;
#pragma unroll
    for (int p = 0; p < PER_T; ++p) {
      const int key = key0 + p;
      *reinterpret_cast<u32x4*>(ks + key * D + ((c ^ k_swz<D>(key)) << 3)) = this->kr[p];
      *reinterpret_cast<u32x4*>(vs + key * D + ((c ^ v_swz<D>(key)) << 3)) = this->vr[p];
    }
  }
};

// Register budget: two waves per SIMD (<= 256 VGPRs), so four workgroups share a CU
// and each keeps its next tile in flight in registers while the current one sits in
// its single LDS buffer: twice the bytes in flight per CU of one wave per SIMD.
template <int D, int NW, bool PAGED>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void fa_decode_split_kernel(DecParams p) {
  constexpr int BCT = 32 * NW;
  constexpr int NT = NW * 64;
  using Copy = PagedTileCopy<D, BCT, NT>;
  // One LDS buffer for the current K and V tiles, reused for the final merge of the
  // waves' partial results.
  constexpr int KV_BYTES = 2 * BCT * D * 2;
  constexpr int MERGE_BYTES = NW * 32 * (D + 2) * 4;
  __shared__ __attribute__((aligned(16))) uint16_t smem_raw[(KV_BYTES > MERGE_BYTES ? KV_BYTES : MERGE_BYTES) / 2];
  uint16_t* const ksm = smem_raw;
  uint16_t* const vsm = smem_raw + BCT * D;

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  // Chunk-major order: every (sequence, head) takes its first chunk before any takes
  // its second. Workgroups are dealt round-robin to the XCDs, so this hands each XCD the
  // same mix of chunk indices; with variable lengths the empty chunks (high indices of
  // short sequences) come last instead of all landing on the XCDs of those indices.
  const int units = p.B * p.Hkv;
  const int cidx = blockIdx.x / units;
  const int bh = blockIdx.x - cidx * units;
  const int b = bh / p.Hkv, hk = bh - b * p.Hkv;
  const int grp = p.Hq / p.Hkv;                       // query heads per KV head (<= 32)
  // Keys of this sequence and this chunk. Chunks have one length for every sequence
  // (cut from the longest possible one), so workgroups carry equal work whatever the
  // mix of lengths; a paged sequence holds seq_lens[b] tokens (clamped to its table)
  // and its chunks past that length are empty.
  int skv = p.Skv;
  if (PAGED) skv = min(max(p.seq_lens[b], 0), p.max_blocks << p.page_log2);
  int c0, c1;
  if (PAGED) {
    // paged: chunk c covers tiles [T c (2n - c) / n^2, ...) of the T tiles of the longest
    // possible sequence (n = nsplit): sizes fall linearly from about 2 T/n to T/n^2, so the
    // chunk-major grid issues the largest pieces first and ends on small ones
    const long long T = (p.Skv + kSplitAlign - 1) / kSplitAlign, n = p.nsplit, cc = cidx;
    const long long d2 = n * n;
    c0 = kSplitAlign * (int)(T * cc * (2 * n - cc) / d2);
    c1 = min(skv, kSplitAlign * (int)(T * (cc + 1) * (2 * n - cc - 1) / d2));
  } else {
    c0 = cidx * p.chunk;
    c1 = min(skv, c0 + p.chunk);
  }
  const int nk = c1 > c0 ? c1 - c0 : 0;
  const int ntiles = (nk + BCT - 1) / BCT;

  const LaneGeom g = make_geom<D>(lane);
  const bool real = g.lr < grp;
  const int h = hk * grp + g.lr;

  u32x4 qop[D / 16];
  {
    const uint16_t* qp = p.q + ((int64_t)b * p.Hq + h) * D + 8 * g.hh;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      u32x4 z = {0u, 0u, 0u, 0u};
      if (real) z = *reinterpret_cast<const u32x4*>(qp + 16 * s);
      qop[s] = (z ^ p.qsign) & p.qmask;
    }
  }

  const int64_t kv_stride = (int64_t)p.Hkv * D;
  // contiguous: this sequence's rows; paged: the page pool, offset to this KV head
  const uint16_t* kb = PAGED ? p.k + (int64_t)hk * D : p.k + ((int64_t)b * p.Skv * p.Hkv + hk) * D;
  const uint16_t* vb = PAGED ? p.v + (int64_t)hk * D : p.v + ((int64_t)b * p.Skv * p.Hkv + hk) * D;
  const int* bt_row = PAGED ? p.block_table + (int64_t)b * p.max_blocks : nullptr;

  f32x16 O[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) O[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float c = p.c;

  Copy cp;
  int pid = 0;               // paged: page of this thread's keys in the next tile to copy
  if (ntiles > 0) {
    if (PAGED) {
      pid = Copy::fetch_page(bt_row, c0, c1, p.page_log2, p.num_pages, tid);
      cp.load_paged(kb, vb, kv_stride, p.page_log2, c0, c1, pid, tid);
      pid = Copy::fetch_page(bt_row, c0 + BCT, c1, p.page_log2, p.num_pages, tid);
      cp.store_paged(ksm, vsm, tid);
    } else {
      cp.load(kb, vb, kv_stride, c0, c1, tid);
      cp.store(ksm, vsm, tid);
    }
  }
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int k0 = c0 + j * BCT;
    const bool more = j + 1 < ntiles;
    if (more) {
      if (PAGED) {
        cp.load_paged(kb, vb, kv_stride, p.page_log2, k0 + BCT, c1, pid, tid);
        // page of the tile after next, one tile ahead of its use
        pid = Copy::fetch_page(bt_row, k0 + 2 * BCT, c1, p.page_log2, p.num_pages, tid);
      } else {
        cp.load(kb, vb, kv_stride, k0 + BCT, c1, tid);
      }
    }
    const uint16_t* ks = ksm;
    const uint16_t* vs = vsm;

    const int kw = k0 + 32 * w;
    if (kw < c1) {
      f32x16 S = scores_block<D>(ks, g, 32 * w, qop);
      if (kw + 32 > c1) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kw + 8 * (e >> 2) + 4 * g.hh + (e & 3);
          if (key >= c1) S[e] = -INFINITY;
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, S[e]);
      mx = pair_max(mx);
      const float m_new = fmaxf(m_run, mx * c);
      const bool need = m_new > m_run + kRescaleGap;
      if (__ballot(need)) {
        const float alpha = need ? fast_exp2(m_run - m_new) : 1.f;
        if (need) m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < D / 32; ++i) O[i] *= alpha;
      }
      const float nm = m_run == -INFINITY ? 0.f : -m_run;
      float ls = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float pe = fast_exp2(fmaf(S[e], c, nm));
        S[e] = pe;
        ls += pe;
      }
      l_run += ls;
      pv_step<D>(vs, g, 2 * w, p_operand(S, 0), O);
      pv_step<D>(vs, g, 2 * w + 1, p_operand(S, 1), O);
    }

    __syncthreads();    // every wave is done with tile j in LDS
    if (more) {
      if (PAGED) cp.store_paged(ksm, vsm, tid);
      else cp.store(ksm, vsm, tid);
    }
    __syncthreads();
  }

  // ---- merge the NW waves' partial results through LDS ------------------------------
  float* mrow = reinterpret_cast<float*>(smem_raw);         // [NW][32]
  float* lrow = mrow + NW * 32;                              // [NW][32]
  float* obuf = lrow + NW * 32;                              // [NW][32][D]
  const float l_tot = pair_sum(l_run);
  if (g.hh == 0) {
    mrow[w * 32 + g.lr] = m_run;
    lrow[w * 32 + g.lr] = l_tot;
  }
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e)
      obuf[(w * 32 + g.lr) * D + 32 * db + 8 * (e >> 2) + 4 * g.hh + (e & 3)] = O[db][e];
  __syncthreads();

  for (int idx = tid; idx < grp * D; idx += NT) {
    const int r = idx / D, dim = idx - r * D;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, mrow[ww * 32 + r]);
    float lt = 0.f, o = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        const float sc = fast_exp2(mrow[ww * 32 + r] - M);
        lt += lrow[ww * 32 + r] * sc;
        o += obuf[(ww * 32 + r) * D + dim] * sc;
      }
    }
    const int hq = hk * grp + r;
    const int64_t prow = ((int64_t)b * p.Hq + hq) * p.nsplit + cidx;
    p.part_o[prow * D + dim] = lt > 0.f ? o / lt : 0.f;
    if (dim == 0) p.part_lse[prow] = lt > 0.f ? (M + fast_log2(lt)) * kLn2 : -INFINITY;
  }
}

// Log-sum-exp merge of the chunk partials; one wave per (sequence, query head).
template <int D>
__global__ __launch_bounds__(256) void fa_decode_combine_kernel(CombineParams p) {
  constexpr int PER = D / 64;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + w;
  if (row >= p.rows) return;
  const float* pl = p.part_lse + (int64_t)row * p.nsplit;
  float M = -INFINITY;
  for (int c = 0; c < p.nsplit; ++c) M = fmaxf(M, pl[c]);
  float acc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] = 0.f;
  float W = 0.f;
  if (M != -INFINITY) {
    for (int c = 0; c < p.nsplit; ++c) {
      const float wc = fast_exp2((pl[c] - M) * kLog2e);
      W += wc;
      const float* po = p.part_o + ((int64_t)row * p.nsplit + c) * D + lane * PER;
#pragma unroll
      for (int k = 0; k < PER; ++k) acc[k] += wc * po[k];
    }
  }
  const float inv = W > 0.f ? 1.f / W : 0.f;
  uint16_t* op = p.o + (int64_t)row * D + lane * PER;
  if (PER == 2) {
    *reinterpret_cast<unsigned*>(op) = pack_bf16x2(acc[0] * inv, acc[PER - 1] * inv);
  } else {
    op[0] = (uint16_t)(pack_bf16x2(acc[0] * inv, 0.f) & 0xFFFFu);
  }
  if (p.lse != nullptr && lane == 0) p.lse[row] = W > 0.f ? M + fast_log2(W) * kLn2 : -INFINITY;
}

template <bool PAGED>
static hipError_t launch_split(const DecParams& p, hipStream_t stream) {
  const long long grid = (long long)p.B * p.Hkv * p.nsplit;
  if (p.d == 128)
    hipLaunchKernelGGL((fa_decode_split_kernel<128, kDecWaves, PAGED>), dim3((unsigned)grid), dim3(kDecWaves * 64),
                       0, stream, p);
  else
    hipLaunchKernelGGL((fa_decode_split_kernel<64, kDecWaves, PAGED>), dim3((unsigned)grid), dim3(kDecWaves * 64),
                       0, stream, p);
  return hipGetLastError();
}

hipError_t launch_decode_partials(const DecParams& p, hipStream_t stream) { return launch_split<false>(p, stream); }
hipError_t launch_decode_paged_partials(const DecParams& p, hipStream_t stream) { return launch_split<true>(p, stream); }

hipError_t launch_decode_combine(const CombineParams& p, hipStream_t stream) {
  const unsigned grid = (unsigned)((p.rows + 3) / 4);
  if (p.d == 128)
    hipLaunchKernelGGL((fa_decode_combine_kernel<128>), dim3(grid), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((fa_decode_combine_kernel<64>), dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace fa
