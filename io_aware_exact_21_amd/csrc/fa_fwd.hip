// Fused exact attention forward for gfx950.
//
// One workgroup of eight waves (two per SIMD; at d = 64 four waves, three workgroups per
// CU) owns BR = 256 (128) query rows of one (batch, query head); each wave owns 32 of
// them, the 32 columns of its MFMA tiles.
// The Q rows stay in registers for the whole kernel while K/V tiles of 64 keys
// stream through an LDS ring (five tiles at d = 128, three at d = 64) filled by direct global->LDS loads
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
#include "fa_dma.hpp"
#include "fa_launch.hpp"
#include "fa_walk.hpp"

namespace fa {

namespace {

constexpr int kFwdTile = 64;      // keys per LDS tile
// LDS ring depth in tiles; copies run NS - 1 tiles ahead of the tile in use. At d = 128
// (one workgroup per CU) the ring holds five tiles, the whole 160 KB of LDS, so that the
// last four tiles of a workgroup are resident together and its waves finish them without
// barriers; at d = 64 three workgroups share a CU and the ring holds three tiles.
constexpr int fwd_stages(int d) { return d == 128 ? 5 : 3; }
// Query heads packed per workgroup: at d = 128 with four query heads per KV head. Bitwise
// the same output as one head per workgroup; +1% on B4 Hq32 Hkv8 S4096 causal (the finer
// 64-row grain of the causal diagonal), unchanged on the 32k GQA prefill.
__host__ __device__ constexpr bool fwd_packs_gqa(int d, int Hq, int Hkv) {
  return d == 128 && fwd_waves(d) == 8 && Hq == 4 * Hkv;
}
// Bound on the probabilities of the max-free softmax step. A row's running normaliser
// (the sum of its probabilities against the current reference m) bounds each of them;
// while it stays at or below 2^64, every p is at most 2^64 and every fp32 sum of p * v
// stays finite for |v| < 2^63, so the running max only has to move when a row's scores
// jump by more than about 64 (log2 units) above it.
constexpr float kRescaleBound = 18446744073709551616.0f;   // 2^64

typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
using dma::lds_addr;
using dma::lds_ptr;
using dma::lds_u8;
using dma::wait_vmcnt;

// LDS ring: the NS K tiles first, then the NS V tiles (BCT keys x D bf16 each, row-major,
// 16-byte chunks XOR-swizzled by key). Keeping K and V apart keeps every operand read
// within a 16-bit immediate of one per-lane base address.
template <int D, int BCT, int NS>
struct Ring {
  static constexpr unsigned kTileBytes = BCT * D * 2;
  static constexpr unsigned kVBase = NS * kTileBytes;
  static constexpr unsigned kBytes = 2 * NS * kTileBytes;
};

// Direct global -> LDS copies of one K tile and one V tile into one ring stage. The
// lane that fills LDS chunk (key, c) fetches global chunk c ^ swz(key). The tile
// base is wave-uniform (SGPRs); per-lane byte offsets within a tile are fixed. Keys
// at or past `kmax` (only in the last tile) re-read key kmax - 1: finite data that the
// softmax gives weight 0.
template <int D, int BCT, int NW, int NS>
struct KvDma {
  static constexpr int CPR = D / 8;              // 16-byte chunks per key row
  static constexpr int KPI = 64 / CPR;           // keys per wave-level copy
  static constexpr int NI = BCT / KPI;           // copies per tensor and tile
  static constexpr int NPW = NI / NW;            // copies per wave, tensor and tile
  static_assert(NI % NW == 0, "copies must split evenly over the waves");
  unsigned koff[NPW], voff[NPW];                 // byte offsets within a tile

  __device__ __forceinline__ static int key_of(int n, int w, int lane) { return KPI * (w + NW * n) + lane / CPR; }

  __device__ __forceinline__ void init(int64_t row_stride, int w, int lane) {
    const int cl = lane % CPR;
#pragma unroll
    for (int n = 0; n < NPW; ++n) {
      const int key = key_of(n, w, lane);
      koff[n] = (unsigned)(key * row_stride * 2) + ((cl ^ k_swz<D>(key)) << 4);
      voff[n] = (unsigned)(key * row_stride * 2) + ((cl ^ v_swz<D>(key)) << 4);
    }
  }

  // Copy tile t (keys t*BCT ...) into ring stage t % NS.
  __device__ __forceinline__ void issue(const uint16_t* kb, const uint16_t* vb, int64_t row_stride, int t,
                                        int kmax, unsigned ring, int w, int lane) const {
    using R = Ring<D, BCT, NS>;
    const int k0 = t * BCT;
    const unsigned kst = ring + (unsigned)(t % NS) * R::kTileBytes;
    const unsigned vst = kst + R::kVBase;
    const uint16_t* kt = kb + (int64_t)k0 * row_stride;
    const uint16_t* vt = vb + (int64_t)k0 * row_stride;
    if (k0 + BCT <= kmax) {
#pragma unroll
      for (int n = 0; n < NPW; ++n) {
        dma::copy16(kt, koff[n], kst + (w + NW * n) * 1024);
        dma::copy16(vt, voff[n], vst + (w + NW * n) * 1024);
      }
    } else {
      const int cl = lane % CPR;
#pragma unroll
      for (int n = 0; n < NPW; ++n) {
        const int key = key_of(n, w, lane);
        const unsigned roff = (unsigned)((int64_t)min(key, kmax - 1 - k0) * row_stride * 2);
        dma::copy16(kt, roff + ((cl ^ k_swz<D>(key)) << 4), kst + (w + NW * n) * 1024);
        dma::copy16(vt, roff + ((cl ^ v_swz<D>(key)) << 4), vst + (w + NW * n) * 1024);
      }
    }
  }
};

// S^T = K Q^T for one 32-key unit. `ka[st]` + `imm` = LDS byte address of this lane's K
// operand chunk for 16-dim step st; `imm` selects the ring stage and the unit's rows.
template <int D>
__device__ __forceinline__ f32x16 qk_unit(const unsigned (&ka)[D / 16], unsigned imm, const u32x4 (&q)[D / 16]) {
  f32x16 s = {};
#pragma unroll
  for (int st = 0; st < D / 16; ++st) {
    const u32x4 a = *reinterpret_cast<const lds_u32x4*>(lds_ptr(ka[st]) + imm);
    s = mfma_32x32x16(a, q[st], s);
  }
  return s;
}

// O^T += V^T P^T for one 32-key unit: two 16-key steps, D/32 dim blocks. `va[db]` +
// `imm` = LDS byte address of this lane's transposing-read origin for dim block db at
// the unit's first 16-key step.
template <int D>
__device__ __forceinline__ void pv_unit(const unsigned (&va)[D / 32], unsigned imm, const u32x4 (&pp)[2],
                                        f32x16 (&o)[D / 32]) {
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const lds_u8* a0p = lds_ptr(va[db]) + imm + tt * 16 * D * 2;
      const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a0p));
      const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a0p + 8 * D * 2));
      const u32x2 x0 = __builtin_bit_cast(u32x2, r0), x1 = __builtin_bit_cast(u32x2, r1);
      const u32x4 a = {x0[0], x0[1], x1[0], x1[1]};
      o[db] = mfma_32x32x16(a, pp[tt], o[db]);
    }
  }
}

// Order of the steps of a hot-loop slot: position p runs step at[p] (steps below NQK are
// Q.K^T, the rest P.V). Two Q.K^T steps open the slot, then P.V and Q.K^T alternate until
// the Q.K^T steps run out, so the K and V operand reads spread evenly over the slot and
// the scores' dependent chain still ends a few steps before the slot does.
template <int NQK, int NPV>
struct SlotOrder {
  int at[NQK + NPV];
  constexpr SlotOrder() : at() {
    int q = 0, v = 0, p = 0;
    at[p++] = q++;
    at[p++] = q++;
    while (q < NQK) {
      at[p++] = NQK + v++;
      at[p++] = q++;
    }
    while (v < NPV) at[p++] = NQK + v++;
  }
};

__device__ __forceinline__ unsigned bf16_pair_sum_weights() { return 0x3F803F80u; }   // (1.0, 1.0)

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Row sums of the probabilities on the matrix cores. A P operand of the P.V product
// (32x32x16 B layout: lane l holds query l % 32 and 8 of the 16 keys of a step, the other
// 8 in lane l ^ 32), read as the B operand of v_mfma_f32_16x16x32_bf16, places query c's
// 16 values at k-slots 0-7 and 16-23 and query 16 + c's at 8-15 and 24-31 of column c
// (c = l % 16). With A row 0 = ones on k-slots 0-7 and 16-23, A row 4 = ones on 8-15 and
// 24-31 and every other row zero, D[0][c] is query c's sum and D[4][c] query 16 + c's;
// in the D layout (lane l: column l % 16, rows 4 (l / 16) + 0..3) element 0 of lane
// l < 32 is then the sum of query l, and element 0 of lanes 32-63 stays unchanged. The
// sums are exact fp32 sums of the bf16 probabilities, as the packed pair sums were.
__device__ __forceinline__ u32x4 rowsum_ones(int lane) {
  const bool on = ((lane & 15) == 0 && ((lane >> 4) & 1) == 0) || ((lane & 15) == 4 && ((lane >> 4) & 1) == 1);
  const unsigned w = on ? bf16_pair_sum_weights() : 0u;
  return u32x4{w, w, w, w};
}
__device__ __forceinline__ f32x4 rowsum_mfma(const u32x4& ones, const u32x4& p, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ones), __builtin_bit_cast(bf16x8, p),
                                                  acc, 0, 0, 0);
}

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

// Per-wave state of the forward pass and its per-tile steps.
template <int D, bool CAUSAL>
struct FwdWave {
  static constexpr int BCT = kFwdTile;
  static constexpr int NS = fwd_stages(D);
  using R = Ring<D, BCT, NS>;

  u32x4 q[D / 16];            // Q^T operand (this wave's 32 rows)
  f32x16 o[D / 32];           // O^T accumulator
  f32x16 s0, s1;              // scores of the even / odd unit in flight
  u32x4 p0[2], p1[2];         // bf16 probabilities of the even / odd unit
  float m, alpha, c;          // running max (log2 units), pending factor, |scale|*log2 e
  // running normaliser in element 0 (a lane's share of its row's sum: lanes l and l ^ 32
  // together hold it); the matrix-core row sums accumulate here, elements 1-3 stay 0
  f32x4 lacc;
  u32x4 ones;                 // A operand of the row-sum product (rowsum_ones)
  unsigned kb_[D / 16];       // K operand read bases (ring stage 0)
  unsigned vb_[D / 32];       // V^T operand read bases (ring stage 0)
  int nu, umask, tmask;       // live units, first masked unit, mask threshold

  __device__ __forceinline__ void softmax_any(const f32x16& sc, u32x4 (&pp)[2], int u) {
    float l = lacc[0];
    if (u >= umask) softmax_unit<true>(sc, m, l, alpha, pp, c, tmask - 32 * u);
    else softmax_unit<false>(sc, m, l, alpha, pp, c, 0);
    lacc[0] = l;
  }
  // Apply the factor of the unit just softmaxed to the accumulator: after the P.V
  // product of the previous unit, before the next one. Rare: the max moves lazily.
  __device__ __forceinline__ void rescale() {
    if (__ballot(alpha != 1.f)) {
      // element by element: a vector-times-scalar product would splat alpha into a
      // 16-register vector first
#pragma unroll
      for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[i][e] *= alpha;
    }
  }

  // One hot-loop slot: Q.K^T of the unit two ahead into `sout`, then P.V of the unit in
  // `pin`, with the softmax of the unit in between (`sin` -> `pout`) spread over them.
  // One MFMA per step: a step first reads the operand of the MFMA two steps ahead, then
  // issues its MFMA and a share of the softmax; a scheduling fence after every step keeps
  // that order (the compiler's own schedule left most LDS reads exposed). Q.K^T goes first
  // so that its dependent MFMA chain has finished long before the next slot's softmax
  // reads the scores.
  // The softmax step skips the max reduction: p = 2^(s*c - m) against the current running
  // max, packed to bf16. The rounded p are summed into the running normaliser on the
  // matrix cores (two 16x16x32 products with the rowsum_ones operand per unit, the first
  // issued as soon as the unit's first 16 keys are packed). Every p is <= kRescaleBound
  // whenever the normaliser is, so when some row's normaliser exceeds that bound the slot
  // restores the normaliser, returns false, and the caller redoes the unit with the full
  // step (which may move m) before its P.V product; the result is then the same as taking
  // the full step directly.
  __device__ __forceinline__ bool fast_slot(const unsigned (&ka)[D / 16], const unsigned (&va)[D / 32],
                                            unsigned imm, const u32x4 (&pin)[2], f32x16& sout,
                                            const f32x16& sin, u32x4 (&pout)[2]) {
    constexpr int NDB = D / 32;
    constexpr int NPV = 2 * NDB;          // P.V MFMAs (16-key step tt, dim block db)
    constexpr int NQK = D / 16;           // Q.K^T MFMAs
    constexpr int N = NPV + NQK;
    constexpr int E = 16 / N;             // softmax elements per step
    constexpr int I1 = 8 / E;             // step at which the unit's first 8 elements are packed
    const float nm = -m;
    const float lprev = lacc[0];
    u32x4 op[N];
    float pe[16];
    unsigned pk[8];
    // steps [0, NQK): Q.K^T; steps [NQK, N): P.V; position i runs step ord.at[i]
    constexpr SlotOrder<NQK, NPV> ord;
    auto load = [&](int pos) {
      const int i = ord.at[pos];
      if (i >= NQK) {
        const int tt = (i - NQK) / NDB, db = (i - NQK) % NDB;
        const lds_u8* a0p = lds_ptr(va[db]) + imm + tt * 16 * D * 2;
        const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a0p));
        const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a0p + 8 * D * 2));
        const u32x2 x0 = __builtin_bit_cast(u32x2, r0), x1 = __builtin_bit_cast(u32x2, r1);
        op[pos] = u32x4{x0[0], x0[1], x1[0], x1[1]};
      } else {
        op[pos] = *reinterpret_cast<const lds_u32x4*>(lds_ptr(ka[i]) + imm);
      }
    };
    // At d = 128 (one softmax element per step) the element's three dependent operations are
    // spread over consecutive steps: a step takes the exponential of its element, whose
    // exponent the step before formed, forms the next element's exponent and packs the pair
    // finished by the step before, so no operation waits on one issued just ahead of it
    // (+1% on the d = 128 prefills; at d = 64, two elements per step, it was 2% slower).
    constexpr bool LAG = D == 128;
    float tx[16];
    load(0);
    load(1);
    if constexpr (LAG) {
#pragma unroll
      for (int e = 0; e < E; ++e) tx[e] = fmaf(sin[e], c, nm);
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x16 s = {};
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if (i + 2 < N) load(i + 2);
      const int st = ord.at[i];
      if (st >= NQK) {
        const int tt = (st - NQK) / NDB, db = (st - NQK) % NDB;
        o[db] = mfma_32x32x16(op[i], pin[tt], o[db]);
      } else {
        s = mfma_32x32x16(op[i], q[st], s);
      }
      if constexpr (LAG) {
#pragma unroll
        for (int e = E * i; e < E * i + E; ++e) pe[e] = fast_exp2(tx[e]);
        if (i + 1 < N) {
#pragma unroll
          for (int e = E * (i + 1); e < E * (i + 1) + E; ++e) tx[e] = fmaf(sin[e], c, nm);
        }
        if (i >= 1) {
#pragma unroll
          for (int e = E * (i - 1); e < E * i; ++e)
            if (e & 1) pk[e >> 1] = pack_bf16x2(pe[e - 1], pe[e]);
        }
        if (i == I1) {                    // elements 0-7 were packed by this step
          pout[0] = u32x4{pk[0], pk[1], pk[2], pk[3]};
          lacc = rowsum_mfma(ones, pout[0], lacc);
        }
      } else {
        if (i == I1) {
          pout[0] = u32x4{pk[0], pk[1], pk[2], pk[3]};
          lacc = rowsum_mfma(ones, pout[0], lacc);
        }
#pragma unroll
        for (int e = E * i; e < E * i + E; ++e) {
          pe[e] = fast_exp2(fmaf(sin[e], c, nm));
          if (e & 1) pk[e >> 1] = pack_bf16x2(pe[e - 1], pe[e]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (LAG) {
#pragma unroll
      for (int e = E * (N - 1); e < E * N; ++e)
        if (e & 1) pk[e >> 1] = pack_bf16x2(pe[e - 1], pe[e]);
    }
    pout[1] = u32x4{pk[4], pk[5], pk[6], pk[7]};
    lacc = rowsum_mfma(ones, pout[1], lacc);
    sout = s;
    // An overflowing p (+inf) reaches other rows' sums as 0 * inf = NaN, and this file is
    // compiled without NaN semantics, so the bound is tested on the magnitude bits, where
    // inf and NaN compare above every finite value.
    if (__ballot((__float_as_uint(lacc[0]) & 0x7fffffffu) > __float_as_uint(kRescaleBound))) {
      lacc[0] = lprev;
      return false;
    }
    return true;
  }
  // Slot A of tile j (units 2j .. 2j + 3 live, unmasked, finite running max): PV(2j),
  // QK(2j + 2) and the max-free softmax of unit 2j + 1. Returns false when some row's
  // probabilities exceed the bound (its max jumped); unit 2j + 1 must then be redone with
  // redo_a before slot B.
  __device__ __forceinline__ bool fast_slot_a(const unsigned (&ka)[D / 16], const unsigned (&va)[D / 32]) {
    return fast_slot(ka, va, 0, p0, s0, s1, p1);
  }
  // Slot B of tile j: PV(2j + 1), QK(2j + 3) and the max-free softmax of unit 2j + 2.
  __device__ __forceinline__ bool fast_slot_b(const unsigned (&ka)[D / 16], const unsigned (&va)[D / 32]) {
    return fast_slot(ka, va, 32 * D * 2, p1, s1, s0, p0);
  }
  // Redo the softmax of a unit with the full step (which moves the running max) and
  // rescale the accumulator. The unit's scores are formed again from its K tile, still
  // resident in LDS: the same MFMAs in the same order give bitwise the same scores.
  __device__ __forceinline__ void redo_unit(const unsigned (&ka)[D / 16], unsigned imm, u32x4 (&pp)[2]) {
    float l = lacc[0];
    softmax_unit<false>(qk_unit<D>(ka, imm, q), m, l, alpha, pp, c, 0);
    lacc[0] = l;
    rescale();
  }
  __device__ __forceinline__ void tile_addrs(int j, unsigned (&ka)[D / 16], unsigned (&va)[D / 32],
                                             unsigned (&kj)[D / 16]) const {
    const unsigned kv = (unsigned)(j % NS) * R::kTileBytes;
    const unsigned kk = (unsigned)((j + 1) % NS) * R::kTileBytes;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
      ka[i] = kb_[i] + kk;
      kj[i] = kb_[i] + kv;
    }
#pragma unroll
    for (int i = 0; i < D / 32; ++i) va[i] = vb_[i] + kv;
  }

  // Tile j with per-unit guards (causal diagonal, ragged tail, finished waves).
  __device__ __forceinline__ void guarded_tile(int j) {
    const unsigned kv = (unsigned)(j % NS) * R::kTileBytes;
    const unsigned kk = (unsigned)((j + 1) % NS) * R::kTileBytes;
    unsigned ka[D / 16], va[D / 32];
#pragma unroll
    for (int i = 0; i < D / 16; ++i) ka[i] = kb_[i] + kk;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) va[i] = vb_[i] + kv;
    const int u0 = 2 * j;
    if (u0 < nu) {
      pv_unit<D>(va, 0, p0, o);
      if (u0 + 2 < nu) s0 = qk_unit<D>(ka, 0, q);
      if (u0 + 1 < nu) {
        softmax_any(s1, p1, u0 + 1);
        rescale();
      }
    }
    if (u0 + 1 < nu) {
      pv_unit<D>(va, 32 * D * 2, p1, o);
      if (u0 + 3 < nu) s1 = qk_unit<D>(ka, 32 * D * 2, q);
      if (u0 + 2 < nu) {
        softmax_any(s0, p0, u0 + 2);
        rescale();
      }
    }
  }
};

}  // namespace

// The lane index (0..63) as a fresh value the compiler cannot reuse from earlier code:
// recomputing lane-dependent values from it late keeps them out of the registers of the
// tile loop.
__device__ __forceinline__ unsigned opaque_lane() {
  unsigned ln;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
  return ln;
}

template <int D, bool CAUSAL, bool OUT_F32>
__global__ __launch_bounds__(fwd_waves(D) * 64, 2) void fa_fwd_kernel(FwdParams p) {
  constexpr int NW = fwd_waves(D);
  constexpr int BCT = kFwdTile;
  constexpr int NS = fwd_stages(D);
  constexpr int DIST = NS - 1;        // copies run DIST tiles ahead
  constexpr int BR = 32 * NW;
  using R = Ring<D, BCT, NS>;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[R::kBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: per-wave branches stay scalar

  // ---- work unit (heaviest causal query tiles first, whole heads per XCD) -------------
  // With four query heads per KV head (d = 128) a workgroup takes one 64-row Q tile of all
  // four heads of a KV group ("I/O-Aware Kernels", FlashAttention: query heads of a group
  // share their K/V): wave w works on query head 4 hk + (w & 3), rows 32 (w >> 2) of the
  // tile, so waves w and w + 4 on one SIMD hold the two row blocks of one head.
  const bool pack = fwd_packs_gqa(D, p.Hq, p.Hkv);
  const int RT = pack ? BR / 4 : BR;                   // query rows of one head per workgroup
  const int n_qt = (p.Sq + RT - 1) / RT;
  int hl, rr;
  prefill_work_unit(blockIdx.x, p.B * (pack ? p.Hkv : p.Hq), n_qt, hl, rr);
  const int qt = CAUSAL ? (n_qt - 1 - rr) : rr;
  int b, h, hk;
  if (pack) {
    b = hl / p.Hkv;
    hk = hl - b * p.Hkv;
    h = 4 * hk + (w & 3);
  } else {
    b = hl / p.Hq;
    h = hl - b * p.Hq;
    hk = (h * p.Hkv) / p.Hq;
  }
  const int q0 = qt * RT;
  const int diag = p.Skv - p.Sq;                       // row i sees keys j <= i + diag

  int kend = p.Skv;                                    // keys any row of the workgroup sees
  if (CAUSAL) kend = min(p.Skv, min(p.Sq, q0 + RT) + diag);
  const int ntiles = kend > 0 ? (kend + BCT - 1) / BCT : 0;

  FwdWave<D, CAUSAL> wv;
  const LaneGeom g = make_geom<D>(lane);
  const unsigned ring = lds_addr(smem);
#pragma unroll
  for (int st = 0; st < D / 16; ++st) wv.kb_[st] = ring + 2u * g.kbase[st];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) wv.vb_[db] = ring + R::kVBase + 2u * g.vbase[db];

  // Waves w and w + 4 of an eight-wave workgroup run on one SIMD. Under the causal mask the
  // 32-row blocks of a Q tile need 1 .. 8 units of the last 256 keys, so the SIMD pairs get
  // blocks (0, 7), (1, 6), (2, 5), (3, 4): nine units each, which the waves work through
  // without barriers once the last tiles are resident.
  const int wr = pack ? (w >> 2) : (NW == 8 && w >= 4) ? 11 - w : w;
  const int row_lo = q0 + 32 * wr;                     // first query row of this wave
  const int row_hi = min(row_lo + 31, p.Sq - 1);       // last real row of this wave
  // keys this wave needs, in 32-key units
  int kw = row_lo < p.Sq ? p.Skv : 0;
  if (CAUSAL && row_lo < p.Sq) kw = max(0, min(p.Skv, row_hi + diag + 1));
  wv.nu = (kw + 31) / 32;
  // units [0, umask) need no per-element mask (neither the causal diagonal nor the tail)
  int umask = p.Skv / 32;
  if (CAUSAL) umask = min(umask, row_lo + diag + 1 > 0 ? (row_lo + diag + 1) / 32 : 0);
  wv.umask = umask;

  // ---- Q^T operand, resident in registers --------------------------------------------
  // Rows past the end of the sequence (last Q tile only) load row Sq - 1 instead: finite
  // scores whose output is never stored. Loading without a per-row branch lets all the
  // loads of a lane go out together.
  const int qrow = row_lo + g.lr;
  u32x4 qraw[D / 16];
  {
    const uint16_t* qp = p.q + b * p.q_bstride + ((int64_t)min(qrow, p.Sq - 1) * p.Hq + h) * D + 8 * g.hh;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qraw[s] = *reinterpret_cast<const u32x4*>(qp + 16 * s);
  }
  // Unit u masks this lane's key offsets above tmask - 32u. At d = 64 the threshold is
  // recomputed from an opaque read of the lane index wherever the guarded paths need it,
  // so that it is not live through the hot loop: the kernel then fits 168 registers and
  // three waves per SIMD (+6% on the 2k prefill). At d = 128 the register allocation that
  // follows from the same change made the hot loop 7% slower, so the threshold stays live
  // there (one register, spilled outside the hot loop).
  auto lane_tmask = [&]() {
    if constexpr (D == 64) {
      const unsigned ln = opaque_lane();
      const int qr = row_lo + (int)(ln & 31u);
      const int lim = CAUSAL ? min(p.Skv - 1, qr + diag) : p.Skv - 1;
      return lim - 4 * (int)(ln >> 5);
    } else {
      return wv.tmask;
    }
  };
  wv.tmask = (CAUSAL ? min(p.Skv - 1, qrow + diag) : p.Skv - 1) - 4 * g.hh;

  const int64_t kv_stride = (int64_t)p.Hkv * D;
  const uint16_t* kb = p.k + b * p.kv_bstride + (int64_t)hk * D;
  const uint16_t* vb = p.v + b * p.kv_bstride + (int64_t)hk * D;
  KvDma<D, BCT, NW, NS> dma;
  dma.init(kv_stride, w, lane);

#pragma unroll
  for (int i = 0; i < D / 32; ++i) wv.o[i] = f32x16{};
  wv.m = -INFINITY;
  wv.lacc = f32x4{};
  wv.ones = rowsum_ones(lane);
  wv.alpha = 1.f;
  wv.c = p.c;

  // ---- prologue: tiles 0 .. DIST - 1 issued, 0 and 1 resident, then Q.K^T of units 0, 1
  // and softmax of 0
  // Iteration j reads V of tile j and K of tile j + 1 and issues the copy of tile j + DIST
  // into the stage of tile j - 1, which every wave has finished with at the barrier
  // closing iteration j - 1. That barrier follows a wait for this wave's copies of tile
  // j + 1 (the copies of later tiles may stay in flight). After iteration jl, which issues
  // the last tile, every tile is resident: jl ends with a full wait and a barrier, and the
  // iterations after it run with neither.
  // The Q loads and the copies of tiles 0 and 1 are waited for together (iteration 0 reads
  // K of tile 1 already); the copies of tiles 2 .. DIST - 1 go out after that wait, so the
  // wait the compiler places before the first use of the Q registers (it does not see the
  // copies, and waits for every outstanding load) finds nothing left to wait for.
  constexpr int NB = 2 * KvDma<D, BCT, NW, NS>::NPW;   // copies per wave and tile
  const int jl = ntiles - 1 - DIST;                      // last iteration that issues a copy
  if (ntiles > 0) dma.issue(kb, vb, kv_stride, 0, p.Skv, ring, w, lane);
  if (ntiles > 1) dma.issue(kb, vb, kv_stride, 1, p.Skv, ring, w, lane);
  wait_vmcnt<0>();
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    asm volatile("" : "+v"(qraw[s]));                   // the first use of Q stays after the wait
    wv.q[s] = (qraw[s] ^ p.qsign) & p.qmask;            // the sign of the scale is folded into Q
  }
#pragma unroll
  for (int t = 2; t < DIST; ++t)
    if (t < ntiles) dma.issue(kb, vb, kv_stride, t, p.Skv, ring, w, lane);
  if (jl < 0) wait_vmcnt<0>();                          // every tile issued: resident before the loop
  __syncthreads();
  auto tile_end = [&](int jj) {
    if (jj < jl) {
      wait_vmcnt<(DIST - 2) * NB>();
      __syncthreads();
    } else if (jj == jl) {
      wait_vmcnt<0>();
      __syncthreads();
    }
  };

  if (wv.nu > 0) {
    wv.s0 = qk_unit<D>(wv.kb_, 0, wv.q);
    if (wv.nu > 1) wv.s1 = qk_unit<D>(wv.kb_, 32 * D * 2, wv.q);
    wv.softmax_any(wv.s0, wv.p0, 0);    // o is zero here, so unit 0's factor needs no application
  }

  // ---- main loop: one tile (two units) per iteration ------------------------------
  // Tiles [0, jf) have all four pipeline units live and unmasked for this wave (and a
  // finite running max, set by unit 0) and run without guards; the rest run guarded.
  // Every wave passes the same number of barriers.
  int jf = min(wv.nu - 3, umask - 2);
  jf = jf > 0 ? min((jf + 1) / 2, ntiles) : 0;
  int j = 0;
  while (j < jf) {
    // hot loop: no guards, no max reductions, no accumulator rescale
    int stop = 0;
    for (; j < jf; ++j) {
      if (j <= jl) dma.issue(kb, vb, kv_stride, j + DIST, p.Skv, ring, w, lane);
      unsigned ka[D / 16], va[D / 32], kj[D / 16];
      wv.tile_addrs(j, ka, va, kj);
      if (!wv.fast_slot_a(ka, va)) { stop = 1; break; }
      if (!wv.fast_slot_b(ka, va)) { stop = 2; break; }
      tile_end(j);
    }
    if (stop == 0) break;
    // A row max jumped inside tile j: redo that unit, finish the tile, resume.
    wv.tmask = lane_tmask();
    unsigned ka[D / 16], va[D / 32], kj[D / 16];
    wv.tile_addrs(j, ka, va, kj);
    if (stop == 1) {
      wv.redo_unit(kj, 32 * D * 2, wv.p1);                    // unit 2j + 1
      if (!wv.fast_slot_b(ka, va)) wv.redo_unit(ka, 0, wv.p0);  // unit 2j + 2
    } else {
      wv.redo_unit(ka, 0, wv.p0);                             // unit 2j + 2
    }
    tile_end(j);
    ++j;
  }
  wv.tmask = lane_tmask();
  for (; j < ntiles; ++j) {
    if (j <= jl) dma.issue(kb, vb, kv_stride, j + DIST, p.Skv, ring, w, lane);
    wv.guarded_tile(j);
    tile_end(j);
  }

  // ---- epilogue: O = acc / l, LSE = ln2 * (m + log2 l) -------------------------------
  // the lane's row again from an opaque read of the lane index: no lane-dependent output
  // address stays live through the tile loop (at d = 128 that removed 20 of the 36 bytes per
  // lane of spills outside the loop, at a small gain)
  const unsigned lane_e = opaque_lane();
  const int hh_e = (int)(lane_e >> 5);
  const int qrow_e = row_lo + (int)(lane_e & 31u);
  const float lt = pair_sum(wv.lacc[0]);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (qrow_e < p.Sq) {
    const int64_t obase = b * p.o_bstride + ((int64_t)qrow_e * p.Hq + h) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int dim = 32 * db + 8 * i + 4 * hh_e;
        const float o0 = wv.o[db][4 * i + 0] * inv, o1 = wv.o[db][4 * i + 1] * inv;
        const float o2 = wv.o[db][4 * i + 2] * inv, o3 = wv.o[db][4 * i + 3] * inv;
        if (OUT_F32) {
          float4 v4 = make_float4(o0, o1, o2, o3);
          *reinterpret_cast<float4*>(static_cast<float*>(p.o) + obase + dim) = v4;
        } else {
          u32x2 v2 = {pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.o) + obase + dim) = v2;
        }
      }
    if (p.lse != nullptr && hh_e == 0)
      p.lse[(int64_t)(b * p.Hq + h) * p.Sq + qrow_e] = lt > 0.f ? (wv.m + fast_log2(lt)) * kLn2 : -INFINITY;
  }
}

// Workgroups of one launch: one per (batch, query head, Q tile), or with packed query heads
// one per (batch, KV head, 64-row Q tile) — never more than fwd_grid_size's count.
static long long fwd_launch_size(const FwdParams& p, int d) {
  if (fwd_packs_gqa(d, p.Hq, p.Hkv)) {
    const int RT = 8 * fwd_waves(d);
    return (long long)p.B * p.Hkv * ((p.Sq + RT - 1) / RT);
  }
  return fwd_grid_size(p.B, p.Hq, p.Sq, d);
}

template <int D, bool CAUSAL, bool OUT_F32>
static hipError_t launch_fwd_t(const FwdParams& p, hipStream_t stream) {
  const long long total = fwd_launch_size(p, D);
  hipLaunchKernelGGL((fa_fwd_kernel<D, CAUSAL, OUT_F32>), dim3((unsigned)total), dim3(fwd_waves(D) * 64), 0,
                     stream, p);
  return hipGetLastError();
}

long long fwd_grid_size(int B, int Hq, int Sq, int d) {
  const int BR = 32 * fwd_waves(d);
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
