// Fused exact attention forward for gfx950.
//
// One workgroup owns BR = 32 * NW query rows of one (batch, query head); each of its
// NW waves owns 32 of those rows. The Q rows stay in registers for the whole kernel
// while the K/V tiles of BCT = 64 keys stream through a two-stage LDS buffer
// ("I/O-Aware Kernels", section FlashAttention: Q blocks resident, K and V
// streamed blockwise). For each tile a wave forms its 32 x 64 score block on MFMA,
// updates the running max m and normaliser l of every row, rescales its output
// accumulator by 2^(m_old - m_new) when the max has grown, and adds P V on MFMA
// ("FlashAttention & IO-aware attention", Direct answer: online softmax with running
// max, normaliser and accumulator). Division by l happens once, in the epilogue.
// Scores never leave registers.
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

template <int D, int NW, bool CAUSAL, bool OUT_F32>
__global__ __launch_bounds__(NW * 64) void fa_fwd_kernel(FwdParams p) {
  constexpr int BCT = 64;
  constexpr int NT = NW * 64;
  constexpr int BR = 32 * NW;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2][2][BCT * D];   // [stage][K|V]

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;

  // ---- work unit: heaviest causal tiles first; whole heads kept on one XCD ----------
  const int n_qt = (p.Sq + BR - 1) / BR;
  const int total = p.B * p.Hq * n_qt;
  int L = blockIdx.x;
  if ((total & 7) == 0) L = (L & 7) * (total >> 3) + (L >> 3);
  const int hl = L / n_qt, r = L - hl * n_qt;
  const int qt = CAUSAL ? (n_qt - 1 - r) : r;
  const int b = hl / p.Hq, h = hl - b * p.Hq;
  const int hk = (h * p.Hkv) / p.Hq;
  const int q0 = qt * BR;
  const int diag = p.Skv - p.Sq;                     // row i sees keys j <= i + diag

  int kend = p.Skv;
  if (CAUSAL) kend = min(p.Skv, min(p.Sq, q0 + BR) + diag);
  const int ntiles = kend > 0 ? (kend + BCT - 1) / BCT : 0;

  const LaneGeom g = make_geom<D>(lane);
  const int row_lo = q0 + 32 * w;                    // first query row of this wave
  const int qrow = row_lo + g.lr;

  // ---- Q^T operand, resident in registers ------------------------------------------
  u32x4 qop[D / 16];
  {
    const uint16_t* qp = p.q + ((int64_t)(b * p.Sq + qrow) * p.Hq + h) * D + 8 * g.hh;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      u32x4 z = {0u, 0u, 0u, 0u};
      if (qrow < p.Sq) z = *reinterpret_cast<const u32x4*>(qp + 16 * s);
      qop[s] = (z ^ p.qsign) & p.qmask;              // the sign of the scale is folded into Q
    }
  }

  const int64_t kv_stride = (int64_t)p.Hkv * D;
  const uint16_t* kb = p.k + ((int64_t)b * p.Skv * p.Hkv + hk) * D;
  const uint16_t* vb = p.v + ((int64_t)b * p.Skv * p.Hkv + hk) * D;

  f32x16 O[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) O[i] = f32x16{};
  float m_run = -INFINITY;   // running max of t = s * c (log2 units), lazily updated
  float l_run = 0.f;         // this lane's half of the row normaliser, relative to m_run
  const float c = p.c;       // |scale| * log2(e)

  TileCopy<D, BCT, NT> cp;
  if (ntiles > 0) {
    cp.load(kb, vb, kv_stride, 0, p.Skv, tid);
    cp.store(smem[0][0], smem[0][1], tid);
  }
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int k0 = j * BCT;
    const bool more = j + 1 < ntiles;
    if (more) cp.load(kb, vb, kv_stride, k0 + BCT, p.Skv, tid);
    const uint16_t* ks = smem[j & 1][0];
    const uint16_t* vs = smem[j & 1][1];

    const bool wave_live = row_lo < p.Sq && (!CAUSAL || k0 <= row_lo + 31 + diag);
    if (wave_live) {
      f32x16 S[BCT / 32];
#pragma unroll
      for (int kb2 = 0; kb2 < BCT / 32; ++kb2) S[kb2] = scores_block<D>(ks, g, 32 * kb2, qop);

      const bool need_mask = (k0 + BCT > p.Skv) || (CAUSAL && k0 + BCT - 1 > row_lo + diag);
      if (need_mask) {
        const int lim = CAUSAL ? min(p.Skv - 1, qrow + diag) : p.Skv - 1;
#pragma unroll
        for (int kb2 = 0; kb2 < BCT / 32; ++kb2)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = k0 + 32 * kb2 + 8 * (e >> 2) + 4 * g.hh + (e & 3);
            if (key > lim) S[kb2][e] = -INFINITY;
          }
      }

      float mx = -INFINITY;
#pragma unroll
      for (int kb2 = 0; kb2 < BCT / 32; ++kb2)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, S[kb2][e]);
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
      for (int kb2 = 0; kb2 < BCT / 32; ++kb2)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float pe = fast_exp2(fmaf(S[kb2][e], c, nm));
          S[kb2][e] = pe;
          ls += pe;
        }
      l_run += ls;

#pragma unroll
      for (int t = 0; t < BCT / 16; ++t) pv_step<D>(vs, g, t, p_operand(S[t >> 1], t & 1), O);
    }

    if (more) cp.store(smem[(j + 1) & 1][0], smem[(j + 1) & 1][1], tid);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l, LSE = ln2 * (m + log2 l) -------------------------------
  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qrow < p.Sq) {
    const int64_t obase = ((int64_t)(b * p.Sq + qrow) * p.Hq + h) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int dim = 32 * db + 8 * i + 4 * g.hh;
        const float o0 = O[db][4 * i + 0] * inv, o1 = O[db][4 * i + 1] * inv;
        const float o2 = O[db][4 * i + 2] * inv, o3 = O[db][4 * i + 3] * inv;
        if (OUT_F32) {
          float4 v4 = make_float4(o0, o1, o2, o3);
          *reinterpret_cast<float4*>(static_cast<float*>(p.o) + obase + dim) = v4;
        } else {
          u32x2 v2 = {pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.o) + obase + dim) = v2;
        }
      }
    if (p.lse != nullptr && g.hh == 0)
      p.lse[(int64_t)(b * p.Hq + h) * p.Sq + qrow] =
          l_tot > 0.f ? (m_run + fast_log2(l_tot)) * kLn2 : -INFINITY;
  }
}

template <int D, int NW, bool CAUSAL, bool OUT_F32>
static hipError_t launch_fwd_t(const FwdParams& p, hipStream_t stream) {
  constexpr int BR = 32 * NW;
  const int n_qt = (p.Sq + BR - 1) / BR;
  const long long total = (long long)p.B * p.Hq * n_qt;
  hipLaunchKernelGGL((fa_fwd_kernel<D, NW, CAUSAL, OUT_F32>), dim3((unsigned)total), dim3(NW * 64), 0,
                     stream, p);
  return hipGetLastError();
}

long long fwd_grid_size(int B, int Hq, int Sq) {
  constexpr int BR = 32 * kFwdWaves;
  return (long long)B * Hq * ((Sq + BR - 1) / BR);
}

hipError_t launch_fwd(const FwdParams& p, bool causal, bool out_f32, hipStream_t stream) {
  constexpr int NW = kFwdWaves;
  if (p.d == 128) {
    if (causal) return out_f32 ? launch_fwd_t<128, NW, true, true>(p, stream) : launch_fwd_t<128, NW, true, false>(p, stream);
    return out_f32 ? launch_fwd_t<128, NW, false, true>(p, stream) : launch_fwd_t<128, NW, false, false>(p, stream);
  }
  if (causal) return out_f32 ? launch_fwd_t<64, NW, true, true>(p, stream) : launch_fwd_t<64, NW, true, false>(p, stream);
  return out_f32 ? launch_fwd_t<64, NW, false, true>(p, stream) : launch_fwd_t<64, NW, false, false>(p, stream);
}

}  // namespace fa
