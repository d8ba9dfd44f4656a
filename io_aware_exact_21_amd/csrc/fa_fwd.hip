// Fused exact attention forward for gfx950.
//
// One workgroup of eight waves (two per SIMD) owns BR = 256 query rows of one
// (batch, query head); each wave owns 32 of them, the 32 columns of its MFMA tiles.
// The Q rows stay in registers for the whole kernel while K/V tiles of 64 keys
// stream through a three-stage LDS ring filled by direct global->LDS loads
// ("I/O-Aware Kernels", section FlashAttention: Q blocks resident, K and V streamed
// blockwise). Scores never leave registers; an online softmax keeps the running max
// m, the normaliser l and the output accumulator of every row and rescales them by
// 2^(m_old - m_new) when the max grows ("FlashAttention & IO-aware attention",
// Direct answer). Division by l happens once, in the epilogue.
//
// Work is software-pipelined in units of 32 keys. While the matrix cores run the
// P.V product of unit u and the Q.K^T product of unit u + 2, the vector ALUs run the
// softmax of unit u + 1, so MFMA and VALU work of one wave overlap; the second wave
// on each SIMD fills the remaining gaps.
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

namespace {

constexpr int kFwdTile = 64;      // keys per LDS tile
constexpr int kFwdStages = 3;     // LDS ring depth (tiles)

// One wave-level direct global -> LDS copy: every lane fetches 16 bytes from its own
// global address and the wave writes them to 64 consecutive 16-byte LDS chunks
// starting at byte address `lds` (wave-uniform, passed in m0). Issued as inline
// assembly so that the compiler does not serialise later LDS reads of other ring
// stages behind it; completion is tracked explicitly with wait_vmcnt + a barrier.
__device__ __forceinline__ void lds_dma16(const void* gptr, unsigned lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "s"(lds)
               : "memory", "m0");
}

__device__ __forceinline__ unsigned lds_addr(const uint16_t* p) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) uint16_t*)p;
}

// Direct global -> LDS copy of one K tile and one V tile (bf16, BCT keys x D) into
// one ring stage. The lane that fills LDS chunk (key, c) fetches global chunk
// c ^ swz(key), which stores the tile row-major with the XOR swizzle the operand
// reads expect. Keys at or past `kmax` re-read key kmax - 1 (finite data that the
// softmax masks to weight 0).
template <int D, int BCT, int NW>
__device__ __forceinline__ void dma_tile(const uint16_t* __restrict__ kb, const uint16_t* __restrict__ vb,
                                         int64_t row_stride, int k0, int kmax, const uint16_t* ks,
                                         const uint16_t* vs, int w, int lane) {
  constexpr int CPR = D / 8;              // 16-byte chunks per key row
  constexpr int KPI = 64 / CPR;           // keys per wave-level copy
  constexpr int NI = BCT / KPI;           // copies per tensor and tile
  static_assert(NI % NW == 0, "copies must split evenly over the waves");
  const int kl = lane / CPR, cl = lane % CPR;
  const unsigned ka = lds_addr(ks), va = lds_addr(vs);
#pragma unroll
  for (int n = 0; n < NI / NW; ++n) {
    const int i = w + NW * n;
    const int key = KPI * i + kl;
    const int kg = min(k0 + key, kmax - 1);
    const int64_t roff = (int64_t)kg * row_stride;
    lds_dma16(kb + roff + ((cl ^ k_swz<D>(key)) << 3), ka + i * 1024);
    lds_dma16(vb + roff + ((cl ^ v_swz<D>(key)) << 3), va + i * 1024);
  }
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// S^T = K Q^T for one 32-key unit (kr0 = first key row of the unit in the tile).
template <int D>
__device__ __forceinline__ f32x16 qk_unit(const uint16_t* ks, const LaneGeom& g, int kr0,
                                          const u32x4 (&q)[D / 16]) {
  f32x16 s = {};
#pragma unroll
  for (int st = 0; st < D / 16; ++st) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(ks + kr0 * D + g.kbase[st]);
    s = mfma_32x32x16(a, q[st], s);
  }
  return s;
}

// O^T += V^T P^T for one 32-key unit (two 16-key steps starting at step t0 of the tile).
template <int D>
__device__ __forceinline__ void pv_unit(const uint16_t* vs, const LaneGeom& g, int t0, const u32x4 (&pp)[2],
                                        f32x16 (&o)[D / 32]) {
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const uint16_t* a0p = vs + (16 * (t0 + tt)) * D + g.vbase[db];
      const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a0p));
      const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a0p + 8 * D));
      const u32x2 x0 = __builtin_bit_cast(u32x2, r0), x1 = __builtin_bit_cast(u32x2, r1);
      const u32x4 a = {x0[0], x0[1], x1[0], x1[1]};
      o[db] = mfma_32x32x16(a, pp[tt], o[db]);
    }
  }
}

__device__ __forceinline__ unsigned bf16_pair_sum_weights() { return 0x3F803F80u; }   // (1.0, 1.0)

// Online-softmax step of one 32-row group over one 32-key unit. `s` holds this lane's
// 16 raw scores of query row (lane % 32); they become probabilities 2^(s*c - m) packed
// to bf16 as the two P operands of the unit. With MASK, element e (key offset
// 8*(e/4) + e%4 past this lane's first key) gets weight 0 when the offset exceeds `t`.
// The running max only moves when the unit's max exceeds it by more than kRescaleGap;
// the accumulator factor is left in `alpha` for the caller to apply.
template <bool MASK>
__device__ __forceinline__ void softmax_unit(f32x16 s, float& m, float& l, float& alpha, u32x4 (&pout)[2],
                                             float c, int t) {
  if (MASK) {
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (8 * (e >> 2) + (e & 3) > t) s[e] = -INFINITY;
  }
  float mx = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
  for (int e = 3; e < 15; e += 2) mx = fmaxf(fmaxf(mx, s[e]), s[e + 1]);
  mx = fmaxf(mx, s[15]);
  mx = pair_max(mx);
  const float m_new = fmaxf(m, mx * c);
  const bool need = m_new > m + kRescaleGap;
  alpha = need ? fast_exp2(m - m_new) : 1.f;
  m = need ? m_new : m;
  const float nm = m == -INFINITY ? 0.f : -m;
  float ls = 0.f;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    unsigned pk[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = fast_exp2(fmaf(s[8 * h + 2 * i], c, nm));
      const float b = fast_exp2(fmaf(s[8 * h + 2 * i + 1], c, nm));
      pk[i] = pack_bf16x2(a, b);
      ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[i]),
                                           __builtin_bit_cast(bf16x2, bf16_pair_sum_weights()), ls, false);
    }
    pout[h] = u32x4{pk[0], pk[1], pk[2], pk[3]};
  }
  l = fmaf(l, alpha, ls);
}

}  // namespace

template <int D, bool CAUSAL, bool OUT_F32>
__global__ __launch_bounds__(kFwdWaves * 64) void fa_fwd_kernel(FwdParams p) {
  constexpr int NW = kFwdWaves;
  constexpr int BCT = kFwdTile;
  constexpr int NS = kFwdStages;
  constexpr int BR = 32 * NW;
  constexpr int TE = BCT * D;                           // bf16 per K (or V) tile
  __shared__ __attribute__((aligned(1024))) uint16_t smem[NS][2][TE];   // [stage][K|V]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: per-wave branches stay scalar

  // ---- work unit: heaviest causal tiles first; whole heads kept on one XCD ----------
  const int n_qt = (p.Sq + BR - 1) / BR;
  const int total = p.B * p.Hq * n_qt;
  int L = blockIdx.x;
  if ((total & 7) == 0) L = (L & 7) * (total >> 3) + (L >> 3);
  const int hl = L / n_qt, rr = L - hl * n_qt;
  const int qt = CAUSAL ? (n_qt - 1 - rr) : rr;
  const int b = hl / p.Hq, h = hl - b * p.Hq;
  const int hk = (h * p.Hkv) / p.Hq;
  const int q0 = qt * BR;
  const int diag = p.Skv - p.Sq;                       // row i sees keys j <= i + diag

  int kend = p.Skv;                                    // keys any row of the workgroup sees
  if (CAUSAL) kend = min(p.Skv, min(p.Sq, q0 + BR) + diag);
  const int ntiles = kend > 0 ? (kend + BCT - 1) / BCT : 0;

  const LaneGeom g = make_geom<D>(lane);
  const int row_lo = q0 + 32 * w;                      // first query row of this wave
  const int row_hi = min(row_lo + 31, p.Sq - 1);       // last real row of this wave
  // keys this wave needs, in 32-key units
  int kw = row_lo < p.Sq ? p.Skv : 0;
  if (CAUSAL && row_lo < p.Sq) kw = max(0, min(p.Skv, row_hi + diag + 1));
  const int nu = (kw + 31) / 32;
  // units [0, umask) need no per-element mask (neither the causal diagonal nor the tail)
  int umask = p.Skv / 32;
  if (CAUSAL) umask = min(umask, row_lo + diag + 1 > 0 ? (row_lo + diag + 1) / 32 : 0);

  // ---- Q^T operand, resident in registers --------------------------------------------
  const int qrow = row_lo + g.lr;
  u32x4 q[D / 16];
  {
    const uint16_t* qp = p.q + ((int64_t)(b * p.Sq + qrow) * p.Hq + h) * D + 8 * g.hh;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      u32x4 z = {0u, 0u, 0u, 0u};
      if (qrow < p.Sq) z = *reinterpret_cast<const u32x4*>(qp + 16 * s);
      q[s] = (z ^ p.qsign) & p.qmask;                  // the sign of the scale is folded into Q
    }
  }
  // unit u masks this lane's key offsets above t - 32u
  const int lim = CAUSAL ? min(p.Skv - 1, qrow + diag) : p.Skv - 1;
  const int tmask = lim - 4 * g.hh;

  const int64_t kv_stride = (int64_t)p.Hkv * D;
  const uint16_t* kb = p.k + ((int64_t)b * p.Skv * p.Hkv + hk) * D;
  const uint16_t* vb = p.v + ((int64_t)b * p.Skv * p.Hkv + hk) * D;

  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = f32x16{};
  float m = -INFINITY, l = 0.f, alpha = 1.f;
  const float c = p.c;

  f32x16 s0, s1;               // scores of the even / odd unit in flight
  u32x4 p0[2], p1[2];          // bf16 probabilities of the even / odd unit

  // ---- prologue: tiles 0 and 1 resident, then Q.K^T of units 0, 1 and softmax of 0 --
  if (ntiles > 0) dma_tile<D, BCT, NW>(kb, vb, kv_stride, 0, p.Skv, smem[0][0], smem[0][1], w, lane);
  if (ntiles > 1) dma_tile<D, BCT, NW>(kb, vb, kv_stride, BCT, p.Skv, smem[1][0], smem[1][1], w, lane);
  wait_vmcnt<0>();     // iteration 0 reads K of tile 1 already
  __syncthreads();

  auto softmax_any = [&](const f32x16& sc, u32x4 (&pp)[2], int u) {
    if (u >= umask) softmax_unit<true>(sc, m, l, alpha, pp, c, tmask - 32 * u);
    else softmax_unit<false>(sc, m, l, alpha, pp, c, 0);
  };
  // Apply the factor of the unit just softmaxed to the accumulator: after the P.V
  // product of the previous unit, before the next one. Rare: the max moves lazily.
  auto rescale = [&]() {
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int i = 0; i < D / 32; ++i) o[i] *= alpha;
    }
  };

  if (nu > 0) {
    s0 = qk_unit<D>(smem[0][0], g, 0, q);
    if (nu > 1) s1 = qk_unit<D>(smem[0][0], g, 32, q);
    softmax_any(s0, p0, 0);    // o is zero here, so unit 0's factor needs no application
  }

  // ---- main loop: one tile (two units) per iteration ------------------------------
  // Tiles [0, jf) have all four pipeline units live and unmasked for this wave and run
  // without guards; the rest (causal diagonal, ragged tail, finished waves) run guarded.
  // Every wave passes the same number of barriers.
  int jf = min(nu - 3, umask - 2);
  jf = jf > 0 ? min((jf + 1) / 2, ntiles) : 0;
  int j = 0;
  for (; j < jf; ++j) {
    if (j + 2 < ntiles) {
      const int st2 = (j + 2) % NS;
      dma_tile<D, BCT, NW>(kb, vb, kv_stride, (j + 2) * BCT, p.Skv, smem[st2][0], smem[st2][1], w, lane);
    }
    const uint16_t* vs = smem[j % NS][1];
    const uint16_t* ks1 = smem[(j + 1) % NS][0];
    pv_unit<D>(vs, g, 0, p0, o);                  // PV(2j)
    s0 = qk_unit<D>(ks1, g, 0, q);                // QK(2j + 2)
    softmax_unit<false>(s1, m, l, alpha, p1, c, 0);   // softmax(2j + 1)
    rescale();
    pv_unit<D>(vs, g, 2, p1, o);                  // PV(2j + 1)
    s1 = qk_unit<D>(ks1, g, 32, q);               // QK(2j + 3)
    softmax_unit<false>(s0, m, l, alpha, p0, c, 0);   // softmax(2j + 2)
    rescale();
    if (j + 2 < ntiles) wait_vmcnt<0>();
    __syncthreads();
  }
  for (; j < ntiles; ++j) {
    if (j + 2 < ntiles) {
      const int st2 = (j + 2) % NS;
      dma_tile<D, BCT, NW>(kb, vb, kv_stride, (j + 2) * BCT, p.Skv, smem[st2][0], smem[st2][1], w, lane);
    }
    const uint16_t* vs = smem[j % NS][1];
    const uint16_t* ks1 = smem[(j + 1) % NS][0];
    const int u0 = 2 * j;
    if (u0 < nu) {
      pv_unit<D>(vs, g, 0, p0, o);
      if (u0 + 2 < nu) s0 = qk_unit<D>(ks1, g, 0, q);
      if (u0 + 1 < nu) {
        softmax_any(s1, p1, u0 + 1);
        rescale();
      }
    }
    if (u0 + 1 < nu) {
      pv_unit<D>(vs, g, 2, p1, o);
      if (u0 + 3 < nu) s1 = qk_unit<D>(ks1, g, 32, q);
      if (u0 + 2 < nu) {
        softmax_any(s0, p0, u0 + 2);
        rescale();
      }
    }
    if (j + 2 < ntiles) wait_vmcnt<0>();
    __syncthreads();
  }

  // ---- epilogue: O = acc / l, LSE = ln2 * (m + log2 l) -------------------------------
  const float lt = pair_sum(l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (qrow < p.Sq) {
    const int64_t obase = ((int64_t)(b * p.Sq + qrow) * p.Hq + h) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int dim = 32 * db + 8 * i + 4 * g.hh;
        const float o0 = o[db][4 * i + 0] * inv, o1 = o[db][4 * i + 1] * inv;
        const float o2 = o[db][4 * i + 2] * inv, o3 = o[db][4 * i + 3] * inv;
        if (OUT_F32) {
          float4 v4 = make_float4(o0, o1, o2, o3);
          *reinterpret_cast<float4*>(static_cast<float*>(p.o) + obase + dim) = v4;
        } else {
          u32x2 v2 = {pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.o) + obase + dim) = v2;
        }
      }
    if (p.lse != nullptr && g.hh == 0)
      p.lse[(int64_t)(b * p.Hq + h) * p.Sq + qrow] = lt > 0.f ? (m + fast_log2(lt)) * kLn2 : -INFINITY;
  }
}

template <int D, bool CAUSAL, bool OUT_F32>
static hipError_t launch_fwd_t(const FwdParams& p, hipStream_t stream) {
  const long long total = fwd_grid_size(p.B, p.Hq, p.Sq);
  hipLaunchKernelGGL((fa_fwd_kernel<D, CAUSAL, OUT_F32>), dim3((unsigned)total), dim3(kFwdWaves * 64), 0,
                     stream, p);
  return hipGetLastError();
}

long long fwd_grid_size(int B, int Hq, int Sq) {
  constexpr int BR = 32 * kFwdWaves;
  return (long long)B * Hq * ((Sq + BR - 1) / BR);
}

hipError_t launch_fwd(const FwdParams& p, bool causal, bool out_f32, hipStream_t stream) {
  if (p.d == 128) {
    if (causal) return out_f32 ? launch_fwd_t<128, true, true>(p, stream) : launch_fwd_t<128, true, false>(p, stream);
    return out_f32 ? launch_fwd_t<128, false, true>(p, stream) : launch_fwd_t<128, false, false>(p, stream);
  }
  if (causal) return out_f32 ? launch_fwd_t<64, true, true>(p, stream) : launch_fwd_t<64, true, false>(p, stream);
  return out_f32 ? launch_fwd_t<64, false, true>(p, stream) : launch_fwd_t<64, false, false>(p, stream);
}

}  // namespace fa
