// Exact attention forward on fp8 (OCP e4m3) inputs for gfx950 (CDNA4).
//
// The fp8 variant of FlashAttention that FlashAttention-3 adds ("FlashAttention &
// IO-aware attention", Deep dive) with the same blockwise online softmax as the bf16
// kernel ("I/O-Aware Kernels", section FlashAttention): Q tiles stay resident, K and V
// tiles stream through LDS, and a running max m and normaliser l rescale the output
// accumulator. Both products run on v_mfma_f32_32x32x64_f8f6f4 (64 fp8 values of k per
// lane row, twice the bf16 rate): S^T = K Q^T over the head dimension, and O^T = V^T P^T
// over 64 keys with P rounded to e4m3. V arrives transposed ([d][keys]) so that each
// lane's 32 keys of V^T are one contiguous 32-byte read.
//
// Inputs are e4m3 codes with one float32 dequantisation scale per (batch, head); the
// Q and K scales fold into the exponent factor and the V scale into the epilogue.
//
// Score rows are permuted within each 64-key tile: S^T tile t (t = 0, 1) puts the key
// 32 h + 16 t + e into element e of the lanes of half h (h = lane / 32), so the 32
// score registers of a lane are exactly the 32 consecutive keys its B operand of the
// P.V product must hold, in order. The row max and sum stay lane-local except for one
// exchange between lanes l and l ^ 32.
//
// Overflow: e4m3 has no infinity and converts values above 448 to NaN. The running max
// moves whenever a row's scores exceed it by more than 2^8, so every p <= 256.
//
// The normaliser sums the unrounded fp32 p. (Summing the e4m3 P instead, on the matrix
// cores against an all-ones operand, leaves the vector ALUs free of those additions but
// moves the LSE by up to the e4m3 rounding of the few largest p: several hundredths.)
#include "fa_device.hpp"
#include "fa_dma.hpp"
#include "fa_fp8.hpp"
#include "fa_walk.hpp"

#include <type_traits>

namespace fa {

namespace {

constexpr int kTile = 64;      // keys per LDS tile
constexpr int kStages = 3;     // LDS ring depth
constexpr float kGap = 8.0f;   // log2 units; keeps p <= 2^8 (e4m3 max is 448)
// Bound of the max-free step: a lane's sum of its p bounds each of them, so a sum at or
// below 2^8 keeps every p inside e4m3's finite range as the full step does.
constexpr float kPBound = 256.0f;

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  // format codes 0 / 0: both operands e4m3; block scales 127 = 2^0
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ i32x8 join(u32x4 lo, u32x4 hi) {
  i32x8 r = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  return r;
}

// Key (tile row) that output row m of S^T tile t is formed from.
__device__ __forceinline__ int key_of_row(int t, int m) {
  return 16 * t + 32 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3);
}

// 16-byte chunk c of a K tile row r (d bytes) is stored at c ^ kswz(r); chunk c of a
// V^T tile row (64 bytes) at c ^ vswz(r). Sixteen lanes reading one chunk of the rows
// key_of_row(t, 0..15) (K) or of 16 consecutive rows (V^T) hit distinct banks.
template <int D>
__device__ __forceinline__ int kswz(int r) {
  return D == 128 ? (((r >> 1) & 1) | (((r >> 2) & 1) << 1) | (((r >> 5) & 1) << 2))
                  : (((r >> 2) & 1) | (((r >> 5) & 1) << 1));
}
__device__ __forceinline__ int vswz(int r) { return (r >> 2) & 3; }

template <int D>
struct Ring {
  static constexpr unsigned kTileBytes = kTile * D;      // one K tile or one V^T tile
  static constexpr unsigned kVBase = kStages * kTileBytes;
  static constexpr unsigned kBytes = 2 * kStages * kTileBytes;
};

// Direct copies of one K tile (64 rows x D bytes) and one V^T tile (D rows x 64 bytes)
// into a ring stage: D/8 wave-level copies of 64 x 16 bytes, dealt to the waves.
template <int D, int NW>
struct Fp8Dma {
  static constexpr int KCPR = D / 16;             // chunks per K row
  static constexpr int NK = kTile * KCPR / 64;    // K copies per tile
  static constexpr int NI = 2 * NK;               // K + V^T copies per tile
  static constexpr int NPW = NI / NW;             // copies per wave and tile
  static_assert(NI % NW == 0, "copies must split evenly over the waves");
  unsigned off[NPW];                              // per-lane byte offsets (full tiles)

  __device__ __forceinline__ void init(int kstride, int ldv, int w, int lane) {
#pragma unroll
    for (int n = 0; n < NPW; ++n) {
      const int j = w + NW * n;
      if (j < NK) {
        const int L = j * 64 + lane, r = L / KCPR, cl = L % KCPR;
        off[n] = (unsigned)(r * kstride) + (unsigned)((cl ^ kswz<D>(r)) << 4);
      } else {
        const int L = (j - NK) * 64 + lane, r = L / 4, cl = L % 4;
        off[n] = (unsigned)(r * ldv) + (unsigned)((cl ^ vswz(r)) << 4);
      }
    }
  }

  // Tile t into stage t % kStages. Keys at or past Skv re-read key Skv - 1 (K) or the
  // last 16-key chunk of the V^T rows (their weights are masked to 0).
  __device__ __forceinline__ void issue(const uint8_t* kb, const uint8_t* vb, int kstride, int ldv, int Skv, int t,
                                        unsigned ring, int w, int lane) const {
    using R = Ring<D>;
    const int k0 = t * kTile;
    const unsigned kst = ring + (unsigned)(t % kStages) * R::kTileBytes;
    const unsigned vst = kst + R::kVBase;
    const uint8_t* kt = kb + (int64_t)k0 * kstride;
    const uint8_t* vt = vb + k0;
    const bool full = k0 + kTile <= Skv;
#pragma unroll
    for (int n = 0; n < NPW; ++n) {
      const int j = w + NW * n;
      if (j < NK) {
        unsigned o = off[n];
        if (!full) {
          const int L = j * 64 + lane, r = L / KCPR, cl = L % KCPR;
          o = (unsigned)(min(r, Skv - 1 - k0) * kstride) + (unsigned)((cl ^ kswz<D>(r)) << 4);
        }
        dma::copy16(kt, o, kst + j * 1024);
      } else {
        unsigned o = off[n];
        if (!full) {
          const int L = (j - NK) * 64 + lane, r = L / 4, cl = L % 4;
          const int c = cl ^ vswz(r);
          const int last = (ldv - k0) / 16 - 1;   // last chunk inside the row
          o = (unsigned)(r * ldv) + (unsigned)(min(c, last) << 4);
        }
        dma::copy16(vt, o, vst + (j - NK) * 1024);
      }
    }
  }
};

__device__ __forceinline__ unsigned pack_fp8x4(float a, float b, float c, float d) {
  unsigned w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0u, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

}  // namespace

template <int D, bool CAUSAL>
__global__ __launch_bounds__(fp8_waves(D) * 64, kFp8WavesPerSimd) void fa_fwd_fp8_kernel(Fp8Params p) {
  constexpr int NW = fp8_waves(D), BR = fp8_rows(D);
  using R = Ring<D>;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[R::kBytes];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, hh = lane >> 5;

  // work unit: heaviest causal query tiles first, whole heads per XCD
  const int n_qt = (p.Sq + BR - 1) / BR;
  int hl, rr;
  prefill_work_unit(blockIdx.x, p.B * p.Hq, n_qt, hl, rr);
  const int qt = CAUSAL ? n_qt - 1 - rr : rr;
  const int b = hl / p.Hq, h = hl - b * p.Hq;
  const int hk = (h * p.Hkv) / p.Hq;
  const int q0 = qt * BR;
  const int diag = p.Skv - p.Sq;                         // row i sees keys j <= i + diag

  int kend = p.Skv;
  if (CAUSAL) kend = max(0, min(p.Skv, min(p.Sq, q0 + BR) + diag));
  const int ntiles = (kend + kTile - 1) / kTile;

  const int row = q0 + 32 * w + lr;
  const bool valid = row < p.Sq;
  const int row_lo = q0 + 32 * w;
  const int row_hi = min(row_lo + 31, p.Sq - 1);
  int kw = row_lo < p.Sq ? p.Skv : 0;                    // keys this wave needs
  if (CAUSAL && row_lo < p.Sq) kw = max(0, min(p.Skv, row_hi + diag + 1));
  const int nt_w = (kw + kTile - 1) / kTile;
  int tmask = p.Skv / kTile;                             // tiles below need no mask
  if (CAUSAL) tmask = min(tmask, max(0, row_lo + diag + 1) / kTile);
  const int lim = valid ? (CAUSAL ? min(p.Skv - 1, row + diag) : p.Skv - 1) : -1;

  // exponent factor: |softmax scale| * log2(e) * the Q and K dequantisation scales (the
  // sign of the scale is folded into Q's sign bits, so the row max can be taken on the
  // raw products); a zero scale zeroes Q, which makes every score exactly 0
  const float qks = p.q_scale[b * p.Hq + h] * p.k_scale[b * p.Hkv + hk];
  const float c = p.c == 0.f ? 1.f : fabsf(p.c) * qks;
  const unsigned qsign = p.c < 0.f ? 0x80808080u : 0u;
  const unsigned qmask = p.c == 0.f ? 0u : 0xFFFFFFFFu;
  const float vsc = p.v_scale[b * p.Hkv + hk];

  // ---- resident Q operand: row `row`, bytes 64 ks + 32 hh .. + 31 -------------------
  // Rows past the end of the sequence load row Sq - 1 (finite scores, output not stored),
  // so the loads need no per-row branch and go out together. They are waited for with the
  // copies of the first two tiles, below.
  u32x4 qraw[D / 32];
  i32x8 qop[D / 64];
  {
    const uint8_t* qp = p.q + ((int64_t)(b * p.Sq + min(row, p.Sq - 1)) * p.Hq + h) * D + 32 * hh;
#pragma unroll
    for (int ks = 0; ks < D / 64; ++ks) {
      qraw[2 * ks] = *reinterpret_cast<const u32x4*>(qp + 64 * ks);
      qraw[2 * ks + 1] = *reinterpret_cast<const u32x4*>(qp + 64 * ks + 16);
    }
  }

  // ---- per-lane LDS offsets: K rows of S^T tile 0 (tile 1 is 16 rows on, an immediate),
  // V^T rows 32 db + lr (db steps are immediates)
  unsigned kofs[D / 64][2];
  {
    const int r = key_of_row(0, lr);
#pragma unroll
    for (int ks = 0; ks < D / 64; ++ks)
#pragma unroll
      for (int x = 0; x < 2; ++x) kofs[ks][x] = (unsigned)(r * D + (((4 * ks + 2 * hh + x) ^ kswz<D>(r)) << 4));
  }
  unsigned vofs[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) vofs[x] = (unsigned)(lr * 64 + (((2 * hh + x) ^ vswz(lr)) << 4));

  const unsigned ring = dma::lds_addr(smem);
  const int kstride = p.Hkv * D;
  const uint8_t* kb = p.k + ((int64_t)b * p.Skv * p.Hkv + hk) * D;
  const uint8_t* vb = p.vt + ((int64_t)b * p.Hkv + hk) * D * (int64_t)p.ldv;
  Fp8Dma<D, NW> cp;
  cp.init(kstride, p.ldv, w, lane);

  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // one 64-key tile; MASK (a compile-time tag) applies the causal / key-count limit per
  // element
  auto tile = [&](unsigned kst, unsigned vst, int j, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    unsigned ka[D / 64][2];
#pragma unroll
    for (int ks = 0; ks < D / 64; ++ks)
#pragma unroll
      for (int x = 0; x < 2; ++x) ka[ks][x] = kst + kofs[ks][x];
    f32x16 s0 = {}, s1 = {};
#pragma unroll
    for (int ks = 0; ks < D / 64; ++ks) {
      const i32x8 a0 = join(*reinterpret_cast<const lds_u32x4*>(dma::lds_ptr(ka[ks][0])),
                            *reinterpret_cast<const lds_u32x4*>(dma::lds_ptr(ka[ks][1])));
      const i32x8 a1 = join(*reinterpret_cast<const lds_u32x4*>(dma::lds_ptr(ka[ks][0]) + 16 * D),
                            *reinterpret_cast<const lds_u32x4*>(dma::lds_ptr(ka[ks][1]) + 16 * D));
      s0 = mfma_fp8(a0, qop[ks], s0);
      s1 = mfma_fp8(a1, qop[ks], s1);
    }
    // this lane's 32 keys: 64 j + 32 hh + e (s0, e < 16) and + 16 + e (s1)
    if (MASK) {
      const int kl = 64 * j + 32 * hh;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        if (kl + e > lim) s0[e] = -INFINITY;
        if (kl + 16 + e > lim) s1[e] = -INFINITY;
      }
    }
    float pv[32];
    bool done = false;
    if (!MASK) {
      // max-free step on unmasked tiles once every row has a finite running max: p against
      // the current max; when some lane's sum exceeds kPBound the full step below redoes
      // the tile's softmax from the same scores
      if (!__ballot(m_run == -INFINITY)) {
        const float nm = -m_run;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          pv[e] = fast_exp2(fmaf(s0[e], c, nm));
          pv[16 + e] = fast_exp2(fmaf(s1[e], c, nm));
        }
        float ls = 0.f;
#pragma unroll
        for (int e = 0; e < 32; ++e) ls += pv[e];
        if (!__ballot(!(ls <= kPBound))) {
          l_run += ls;
          done = true;
        }
      }
    }
    if (!done) {
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, fmaxf(s0[e], s1[e]));
      mx = pair_max(mx) * c;
      const bool need = mx > m_run + kGap;
      if (__ballot(need)) {
        const float alpha = need ? fast_exp2(m_run - mx) : 1.f;   // m_run = -inf gives 0
        if (need) m_run = mx;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < D / 32; ++i)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[i][e] *= alpha;
      }
      const float nm = m_run == -INFINITY ? 0.f : -m_run;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        pv[e] = fast_exp2(fmaf(s0[e], c, nm));
        pv[16 + e] = fast_exp2(fmaf(s1[e], c, nm));
      }
      float ls = 0.f;
#pragma unroll
      for (int e = 0; e < 32; ++e) ls += pv[e];
      l_run += ls;
    }
    i32x8 pb;
#pragma unroll
    for (int i = 0; i < 8; ++i) pb[i] = (int)pack_fp8x4(pv[4 * i], pv[4 * i + 1], pv[4 * i + 2], pv[4 * i + 3]);
    const unsigned va0 = vst + vofs[0], va1 = vst + vofs[1];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const i32x8 a = join(*reinterpret_cast<const lds_u32x4*>(dma::lds_ptr(va0) + db * 2048),
                           *reinterpret_cast<const lds_u32x4*>(dma::lds_ptr(va1) + db * 2048));
      o[db] = mfma_fp8(a, pb, o[db]);
    }
  };

  // The Q loads and the copies of tiles 0 and 1 complete together; after this wait only
  // tile copies are in flight, which the per-tile waits below count. (The wait the
  // compiler places before the first use of the Q registers does not see the copies and
  // waits for every outstanding load: it is kept after this one.)
  if (ntiles > 0) cp.issue(kb, vb, kstride, p.ldv, p.Skv, 0, ring, w, lane);
  if (ntiles > 1) cp.issue(kb, vb, kstride, p.ldv, p.Skv, 1, ring, w, lane);
  dma::wait_vmcnt<0>();
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    asm volatile("" : "+v"(qraw[i]));
    qraw[i] = (qraw[i] ^ qsign) & qmask;
  }
#pragma unroll
  for (int ks = 0; ks < D / 64; ++ks) qop[ks] = join(qraw[2 * ks], qraw[2 * ks + 1]);
  // Iteration j waits for its tile and issues tile j + 2 into the stage of tile j - 1 after
  // the barrier. Once no copies are left to issue, one full wait and barrier (at iteration
  // max(0, ntiles - 2)) makes the last tiles resident everywhere, and the last iteration
  // runs without either.
  auto sync = [&](int j) {
    if (j + 2 < ntiles) {
      dma::wait_vmcnt<Fp8Dma<D, NW>::NPW>();
      __syncthreads();                                   // tile j landed everywhere; tile j - 1 is free
      cp.issue(kb, vb, kstride, p.ldv, p.Skv, j + 2, ring, w, lane);
    } else if (j == max(0, ntiles - 2)) {
      dma::wait_vmcnt<0>();
      __syncthreads();
    }
  };
  // Tiles below tmask need no mask: one loop with the mask-free body, then the rest.
  // Every wave calls sync for every tile in either loop, and whether it waits and passes a
  // barrier depends only on j, so the barriers still match.
  int j = 0;
  const int split = min(tmask, min(nt_w, ntiles));
  for (; j < split; ++j) {
    sync(j);
    const unsigned kst = ring + (unsigned)(j % kStages) * R::kTileBytes;
    tile(kst, kst + R::kVBase, j, std::false_type{});
  }
  for (; j < ntiles; ++j) {
    sync(j);
    if (j >= nt_w) continue;
    const unsigned kst = ring + (unsigned)(j % kStages) * R::kTileBytes;
    tile(kst, kst + R::kVBase, j, std::true_type{});
  }

  // ---- epilogue: O = v_scale * acc / l, LSE = ln2 * (m + log2 l) -------------------------
  const float lt = pair_sum(l_run);
  const float inv = lt > 0.f ? vsc / lt : 0.f;
  if (valid) {
    uint16_t* dst = p.o + ((int64_t)(b * p.Sq + row) * p.Hq + h) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x2 v2 = {pack_bf16x2(o[db][4 * i] * inv, o[db][4 * i + 1] * inv),
                    pack_bf16x2(o[db][4 * i + 2] * inv, o[db][4 * i + 3] * inv)};
        *reinterpret_cast<u32x2*>(dst + 32 * db + 8 * i + 4 * hh) = v2;
      }
    if (p.lse && hh == 0)
      p.lse[((int64_t)b * p.Hq + h) * p.Sq + row] = lt > 0.f ? (m_run + fast_log2(lt)) * kLn2 : -INFINITY;
  }
}

long long fp8_grid_size(int B, int Hq, int Sq, int d) {
  return (long long)B * Hq * ((Sq + fp8_rows(d) - 1) / fp8_rows(d));
}

hipError_t launch_fwd_fp8(const Fp8Params& p, bool causal, hipStream_t stream) {
  const dim3 grid((unsigned)fp8_grid_size(p.B, p.Hq, p.Sq, p.d)), block(fp8_waves(p.d) * 64);
  if (p.d == 128) {
    if (causal) hipLaunchKernelGGL((fa_fwd_fp8_kernel<128, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((fa_fwd_fp8_kernel<128, false>), grid, block, 0, stream, p);
  } else {
    if (causal) hipLaunchKernelGGL((fa_fwd_fp8_kernel<64, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((fa_fwd_fp8_kernel<64, false>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace fa
