// Backward pass of exact attention for gfx950 (CDNA4): dQ, dK and dV.
//
// The backward pass recomputes the attention probabilities from Q, K and the forward's
// log-sum-exp instead of storing the attention matrix ("Tracing Tiled QKV Data Movement
// in FlashAttention's Memory Hierarchy", Conclusion). With P_ij = exp(scale s_ij - LSE_i),
// D_i = dO_i . O_i and dS_ij = P_ij (dO_i . V_j - D_i) the gradients are
//     dV_j = sum_i P_ij dO_i,   dK_j = scale sum_i dS_ij Q_i,   dQ_i = scale sum_j dS_ij K_j.
//
// Two kernels, neither with atomics:
//   * fa_bwd_dq_kernel: one workgroup per (batch, query head, 256 query rows; 128 at
//     d = 64). Q and dO of the wave's 32 rows stay in registers; K and V tiles stream
//     through LDS. Per 32-key unit it forms S^T = K Q^T and dP^T = V dO^T (a lane owns
//     one query row), builds dS^T in registers and accumulates dQ^T += K^T dS^T. It also
//     writes D.
//   * fa_bwd_dkdv_kernel (d = 64): one workgroup per (batch, KV head, 128 keys). K and V
//     of the wave's 32 keys stay in registers; 128-row Q and dO tiles of every query head
//     of the group stream through a two-stage LDS ring with their LSE and D rows. Per
//     32-query unit it forms S = Q K^T and dP = dO V^T (a lane owns one key), and
//     accumulates dV^T += dO^T P and dK^T += Q^T dS.
//   * fa_bwd_dkdv_pair_kernel (d = 128): the same work unit, with the four products of a
//     32-query unit split over two waves of one SIMD (S, P and dV in one; dP, dS and dK
//     in the other, one tile later, with P passed through LDS), so that each wave's
//     accumulators and resident operands fit two waves per SIMD.
// Splitting dQ from dK/dV costs two extra products per tile (S and dP are formed in
// both kernels) but keeps every output written once by one workgroup.
//
// Tiles that are read both row-wise (MFMA A operand rows) and transposed
// (ds_read_b64_tr_b16) use one XOR swizzle that is free of bank conflicts in both modes.
#include "fa_bwd.hpp"
#include "fa_device.hpp"
#include "fa_dma.hpp"

namespace fa {

namespace {

constexpr int kBwdTile = 64;     // rows per streamed LDS tile (dQ kernel)
// LDS ring depth of the dQ kernel in tiles; copies run NS - 1 tiles ahead, and the last
// NS - 1 tiles of a workgroup are resident together, so its waves finish them without
// barriers. At d = 128 (one workgroup per CU) four tiles (128 KB) measured best: +1% on the
// causal 8k backward, +3.5% at 2k, against three; five (all 160 KB) was slower than four.
constexpr int bwd_dq_stages(int d) { return d == 128 ? 4 : 3; }
constexpr int kBwdDkvTile = 128; // Q / dO rows per dK/dV tile (two-stage ring)

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
using dma::lds_addr;
using dma::lds_ptr;
using dma::lds_u8;
using dma::wait_vmcnt;

// 16-byte chunk c of tile row r is stored at chunk c ^ bswz(r). Row reads: 16 lanes
// read 16 consecutive rows at one chunk, so bswz must permute 16 consecutive rows
// onto distinct chunks (mod 16 for d = 128, per row parity for d = 64). Transposing
// reads: 32 lanes read 4 consecutive rows x 64 contiguous bytes, so 4 consecutive
// rows must differ in the swizzle bits above the 64-byte group.
template <int D>
__device__ __forceinline__ int bswz(int r) {
  return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// Per-lane LDS byte offsets inside one tile.
template <int D>
struct BwdGeom {
  unsigned row[D / 16];   // A operand rows: tile row (lane % 32), chunk 2s + lane / 32
  unsigned tr0[D / 32];   // transposing read, dim block db: rows 4 (lane/32) + (lane/4)%4
  unsigned tr8[D / 32];   // the same rows + 8
};

template <int D>
__device__ __forceinline__ BwdGeom<D> make_bgeom(int lane) {
  BwdGeom<D> g;
  const int lr = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) g.row[s] = 2u * (lr * D + (((2 * s + hh) ^ bswz<D>(lr)) << 3));
  // ds_read_b64_tr_b16: in each group of 16 lanes, lane 4r+q fetches 4 consecutive
  // dims of row r; lane i of the group then receives dim i of rows 0..3.
  const int G = lane >> 4, r = (lane >> 2) & 3, q = lane & 3;
  const int row0 = 4 * hh + r;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const int dim0 = 32 * db + 16 * (G & 1) + 4 * q;
    g.tr0[db] = 2u * (row0 * D + (((dim0 >> 3) ^ bswz<D>(row0)) << 3) + (dim0 & 7));
    g.tr8[db] = 2u * ((row0 + 8) * D + (((dim0 >> 3) ^ bswz<D>(row0 + 8)) << 3) + (dim0 & 7));
  }
  return g;
}

// X B for 32 tile rows starting at LDS byte `base`: A = the rows (32 x 16 per step),
// B = a resident operand (16 x 32 per step). Row lane%32 of the result is tile row
// lane%32... in the accumulator layout each lane owns column lane % 32 of B.
template <int D>
__device__ __forceinline__ f32x16 mm_rows(unsigned base, const BwdGeom<D>& g, const u32x4 (&bop)[D / 16]) {
  f32x16 s = {};
#pragma unroll
  for (int st = 0; st < D / 16; ++st) {
    const u32x4 a = *reinterpret_cast<const lds_u32x4*>(lds_ptr(base + g.row[st]));
    s = mfma_32x32x16(a, bop[st], s);
  }
  return s;
}

// acc[db] += X^T(dims of block db, tile rows 16t..16t+15) * B, for every dim block.
// B is the bf16 operand built by p_operand from accumulator registers, whose row
// order matches the rows the transposing read gives each lane.
template <int D>
__device__ __forceinline__ void mm_tr(unsigned base, int t, const BwdGeom<D>& g, u32x4 pb, f32x16 (&acc)[D / 32]) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const unsigned off = base + (unsigned)(t * 16 * D * 2);
    const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds_ptr(off + g.tr0[db])));
    const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds_ptr(off + g.tr8[db])));
    const u32x2 a0 = __builtin_bit_cast(u32x2, r0), a1 = __builtin_bit_cast(u32x2, r1);
    const u32x4 a = {a0[0], a0[1], a1[0], a1[1]};
    acc[db] = mfma_32x32x16(a, pb, acc[db]);
  }
}

// The same two products with every LDS operand read issued before the first MFMA
// that uses it (the register room of one wave per SIMD hides the LDS latency).
template <int D>
struct RowOps {
  u32x4 a[D / 16];
};
template <int D>
__device__ __forceinline__ RowOps<D> load_rows(unsigned base, const BwdGeom<D>& g) {
  RowOps<D> r;
#pragma unroll
  for (int st = 0; st < D / 16; ++st) r.a[st] = *reinterpret_cast<const lds_u32x4*>(lds_ptr(base + g.row[st]));
  return r;
}
template <int D>
struct TrOps {
  u32x4 a[D / 32];
};
template <int D>
__device__ __forceinline__ TrOps<D> load_tr(unsigned base, int t, const BwdGeom<D>& g) {
  TrOps<D> r;
  const unsigned off = base + (unsigned)(t * 16 * D * 2);
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds_ptr(off + g.tr0[db])));
    const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds_ptr(off + g.tr8[db])));
    const u32x2 a0 = __builtin_bit_cast(u32x2, r0), a1 = __builtin_bit_cast(u32x2, r1);
    r.a[db] = u32x4{a0[0], a0[1], a1[0], a1[1]};
  }
  return r;
}
template <int D>
__device__ __forceinline__ void mm_tr_ops(const TrOps<D>& x, u32x4 pb, f32x16 (&acc)[D / 32]) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = mfma_32x32x16(x.a[db], pb, acc[db]);
}

// Per-lane global byte offsets for the wave-level tile copies: copy n of wave w fills
// tile rows KPI*(w + NW*n) ...; lane i takes row KPI*(w + NW*n) + i / CPR and fetches
// global chunk (i % CPR) ^ bswz(row), so LDS chunk c of the row holds chunk c ^ bswz.
template <int D, int NW, int BT = kBwdTile>
struct TileDma {
  static constexpr int CPR = D / 8;
  static constexpr int KPI = 64 / CPR;
  static constexpr int NI = BT / KPI;
  static constexpr int NPW = NI / NW;            // copies per wave and tensor
  static_assert(NI % NW == 0, "copies must split evenly over the waves");
  unsigned off[NPW];

  __device__ __forceinline__ static int row_of(int n, int w, int lane) { return KPI * (w + NW * n) + lane / CPR; }

  __device__ __forceinline__ void init(int64_t row_stride, int w, int lane) {
#pragma unroll
    for (int n = 0; n < NPW; ++n) {
      const int r = row_of(n, w, lane);
      off[n] = (unsigned)(r * row_stride * 2) + (((lane % CPR) ^ bswz<D>(r)) << 4);
    }
  }

  // Copy tile rows [r0, r0 + 64) of a (row-strided) tensor into LDS byte `dst`. Rows at
  // or past `rmax` re-read row rmax - 1 (finite data whose weight is masked to 0).
  __device__ __forceinline__ void copy(const uint16_t* base, int64_t row_stride, int r0, int rmax, unsigned dst,
                                       int w, int lane) const {
    const uint16_t* t = base + (int64_t)r0 * row_stride;
    if (r0 + BT <= rmax) {
#pragma unroll
      for (int n = 0; n < NPW; ++n) dma::copy16(t, off[n], dst + (w + NW * n) * 1024);
    } else {
#pragma unroll
      for (int n = 0; n < NPW; ++n) {
        const int r = row_of(n, w, lane);
        const unsigned ro = (unsigned)((int64_t)min(r, rmax - 1 - r0) * row_stride * 2);
        dma::copy16(t, ro + (((lane % CPR) ^ bswz<D>(r)) << 4), dst + (w + NW * n) * 1024);
      }
    }
  }
};

// One software-pipelined step of the dQ kernel at d = 128: the 16 products S^T, dP^T of the
// next unit (alternating, each reading its LDS A operand two products ahead) with one
// softmax-gradient element of the current unit per product; the element's exponent, its
// exponential and its product with (dP - D) fall on consecutive steps.
template <int D, bool MASK>
__device__ __forceinline__ void dq_pipe_step(bool next, unsigned kn, unsigned vn, const BwdGeom<D>& g,
                                             const u32x4 (&qop)[D / 16], const u32x4 (&dop)[D / 16],
                                             const f32x16& sc, const f32x16& dc, f32x16& sn, f32x16& dn,
                                             f32x16& ds, float c, float lse2, float dsum, int kbase, int lim) {
  constexpr int N = 2 * (D / 16);      // products of the next unit
  static_assert(N == 16, "one softmax element per product");
  u32x4 op[N];
  auto load = [&](int i) {
    const unsigned base = (i & 1) ? vn : kn;
    op[i] = *reinterpret_cast<const lds_u32x4*>(lds_ptr(base + g.row[i >> 1]));
  };
  float tx[16], pe[16];
  if (next) {
    load(0);
    load(1);
  }
  tx[0] = fmaf(sc[0], c, -lse2);
  __builtin_amdgcn_sched_barrier(0);
  f32x16 a = {}, b = {};
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (next) {
      if (i + 2 < N) load(i + 2);
      if (i & 1) b = mfma_32x32x16(op[i], dop[i >> 1], b);
      else a = mfma_32x32x16(op[i], qop[i >> 1], a);
    }
    pe[i] = fast_exp2(tx[i]);
    if (i + 1 < 16) tx[i + 1] = fmaf(sc[i + 1], c, -lse2);
    if (i >= 1) {
      const int e = i - 1;
      float pv = pe[e];
      if (MASK && kbase + 8 * (e >> 2) + (e & 3) > lim) pv = 0.f;
      ds[e] = pv * (dc[e] - dsum);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  {
    float pv = pe[15];
    if (MASK && kbase + 8 * 3 + 3 > lim) pv = 0.f;
    ds[15] = pv * (dc[15] - dsum);
  }
  sn = a;
  dn = b;
}

__device__ __forceinline__ float bf16_lo(unsigned x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(unsigned x) { return __uint_as_float(x & 0xffff0000u); }

// 4 consecutive fp32 values of an accumulator, scaled, to 4 bf16 at dst (8 bytes).
__device__ __forceinline__ void store4(uint16_t* dst, const f32x16& a, int i, float sc) {
  u32x2 v = {pack_bf16x2(a[4 * i] * sc, a[4 * i + 1] * sc), pack_bf16x2(a[4 * i + 2] * sc, a[4 * i + 3] * sc)};
  *reinterpret_cast<u32x2*>(dst) = v;
}

}  // namespace

// ---------------------------------------------------------------------------------------
// dQ (and D): one workgroup per (batch, query head, bwd_dq_rows(D) query rows).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(bwd_dq_waves(D) * 64) __attribute__((amdgpu_waves_per_eu(2)))
void fa_bwd_dq_kernel(BwdParams p) {
  constexpr int NW = bwd_dq_waves(D), BT = kBwdTile, NS = bwd_dq_stages(D), BR = bwd_dq_rows(D);
  constexpr int DIST = NS - 1;                           // copies run DIST tiles ahead
  constexpr unsigned TB = BT * D * 2;                    // bytes per tile
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * NS * TB];   // K stages, then V stages

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, hh = lane >> 5;

  // Workgroups go to the XCDs round-robin; head-major numbering keeps each head on one
  // XCD (when the head count is a multiple of 8) and issues the heaviest causal query
  // tiles first.
  const int n_qt = (p.Sq + BR - 1) / BR;
  const int heads = p.B * p.Hq;
  const int rr = blockIdx.x / heads, hl = blockIdx.x - rr * heads;
  const int qt = CAUSAL ? n_qt - 1 - rr : rr;
  const int b = hl / p.Hq, h = hl - b * p.Hq;
  const int hk = (h * p.Hkv) / p.Hq;
  const int q0 = qt * BR;
  const int diag = p.Skv - p.Sq;                         // row i sees keys j <= i + diag

  int kend = p.Skv;                                      // keys any row of the workgroup sees
  if (CAUSAL) kend = max(0, min(p.Skv, min(p.Sq, q0 + BR) + diag));
  const int ntiles = (kend + BT - 1) / BT;

  // Waves w and w + 4 of an eight-wave workgroup share a SIMD; under the causal mask they
  // take complementary 32-row blocks (0 and 7, 1 and 6, ...), which evens out the SIMDs'
  // work over the last tiles, where the waves run without barriers.
  const int wr = (NW == 8 && w >= 4) ? 11 - w : w;
  const int row = q0 + 32 * wr + lr;
  const bool valid = row < p.Sq;

  const BwdGeom<D> g = make_bgeom<D>(lane);
  const unsigned ring = lds_addr(smem);
  const int64_t kv_stride = (int64_t)p.Hkv * D;
  const uint16_t* kb = p.k + ((int64_t)b * p.Skv * p.Hkv + hk) * D;
  const uint16_t* vb = p.v + ((int64_t)b * p.Skv * p.Hkv + hk) * D;
  TileDma<D, NW> dma;
  dma.init(kv_stride, w, lane);
  constexpr int PER_TILE = 2 * TileDma<D, NW>::NPW;     // copies per wave and tile

  auto issue = [&](int t) {
    const unsigned st = (unsigned)(t % NS) * TB;
    dma.copy(kb, kv_stride, t * BT, p.Skv, ring + st, w, lane);
    dma.copy(vb, kv_stride, t * BT, p.Skv, ring + NS * TB + st, w, lane);
  };

  // ---- resident Q and dO rows; D = dO . O ---------------------------------------------
  // Rows past the end of the sequence load row Sq - 1 (no per-row branch, so all the loads
  // go out together) and get lse2 = +inf, which makes every p, and so their dS, exactly 0.
  // The row loads and the copies of tiles 0 and 1 are waited for together.
  u32x4 qop[D / 16], dop[D / 16], oop[D / 16];
  const int64_t srow = ((int64_t)b * p.Hq + h) * p.Sq + min(row, p.Sq - 1);
  {
    const int64_t off = ((int64_t)(b * p.Sq + min(row, p.Sq - 1)) * p.Hq + h) * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      qop[s] = *reinterpret_cast<const u32x4*>(p.q + off + 16 * s);
      dop[s] = *reinterpret_cast<const u32x4*>(p.dout + off + 16 * s);
      oop[s] = *reinterpret_cast<const u32x4*>(p.o + off + 16 * s);
    }
  }
  float lse2 = p.lse[srow];
  if (ntiles > 0) issue(0);
  if (ntiles > 1) issue(1);
  wait_vmcnt<0>();                                       // only tile copies are issued below
  float dsum = 0.f;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    asm volatile("" : "+v"(dop[s]), "+v"(oop[s]));      // the first use stays after the wait
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dsum += bf16_lo(dop[s][i]) * bf16_lo(oop[s][i]) + bf16_hi(dop[s][i]) * bf16_hi(oop[s][i]);
  }
  dsum = pair_sum(dsum);
  asm volatile("" : "+v"(lse2));
  lse2 = valid ? lse2 * kLog2e : INFINITY;
  if (valid && hh == 0) p.dsum[srow] = dsum;
  if (!(lse2 > -INFINITY)) lse2 = 0.f;                   // a row that sees no key: every p is masked

  // ---- this wave's key range -----------------------------------------------------------
  const int row_lo = q0 + 32 * wr;
  const int row_hi = min(row_lo + 31, p.Sq - 1);
  int kw = row_lo < p.Sq ? p.Skv : 0;
  if (CAUSAL && row_lo < p.Sq) kw = max(0, min(p.Skv, row_hi + diag + 1));
  const int nu = (kw + 31) / 32;                         // 32-key units this wave computes
  int umask = p.Skv / 32;                                // units below need no per-element mask
  if (CAUSAL) umask = min(umask, max(0, row_lo + diag + 1) / 32);
  const int lim = valid ? (CAUSAL ? min(p.Skv - 1, row + diag) : p.Skv - 1) : -1;
  const float c = p.c;

  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = f32x16{};

  // Tiles 2 .. DIST - 1 go out after the row loads are waited for. Iteration j waits for
  // tile j (later tiles may stay in flight) and, after the barrier, issues tile j + DIST
  // into the stage of tile j - 1. From iteration jw on nothing is left to issue: jw waits
  // for every copy and passes one barrier, and the iterations after it need neither.
#pragma unroll
  for (int t = 2; t < DIST; ++t)
    if (t < ntiles) issue(t);
  const int jw = max(0, ntiles - DIST);
  if constexpr (D == 128) {
    // Software-pipelined units: the products S^T, dP^T of unit U + 1 run under the softmax
    // gradient of unit U, then dQ^T += K^T dS^T of unit U. Iteration j therefore reads tiles
    // j and j + 1, and waits for both.
    __syncthreads();                                     // tiles 0 and 1 resident everywhere
    f32x16 sc = {}, dc = {};
    if (nu > 0) {
      sc = mm_rows<D>(ring, g, qop);
      dc = mm_rows<D>(ring + NS * TB, g, dop);
    }
    for (int j = 0; j < ntiles; ++j) {
      if (j < jw) {
        wait_vmcnt<(DIST - 2) * PER_TILE>();             // tiles j and j + 1 landed
        __syncthreads();                                 // every wave's share landed; tile j - 1 is free
        issue(j + DIST);
      } else if (j == jw) {
        wait_vmcnt<0>();
        __syncthreads();                                 // every remaining tile resident everywhere
      }
      const unsigned kst = ring + (unsigned)(j % NS) * TB;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int U = 2 * j + u;
        if (U < nu) {
          const bool next = U + 1 < nu;
          const int Un = U + 1;
          const unsigned kn = ring + (unsigned)((Un >> 1) % NS) * TB + (unsigned)(Un & 1) * 32 * D * 2;
          const unsigned vn = kn + NS * TB;
          f32x16 sn, dn, ds;
          if (U >= umask)
            dq_pipe_step<D, true>(next, kn, vn, g, qop, dop, sc, dc, sn, dn, ds, c, lse2, dsum, 32 * U + 4 * hh, lim);
          else
            dq_pipe_step<D, false>(next, kn, vn, g, qop, dop, sc, dc, sn, dn, ds, c, lse2, dsum, 0, 0);
          mm_tr<D>(kst, 2 * u, g, p_operand(ds, 0), acc);
          mm_tr<D>(kst, 2 * u + 1, g, p_operand(ds, 1), acc);
          sc = sn;
          dc = dn;
        }
      }
    }
  } else
  for (int j = 0; j < ntiles; ++j) {
    if (j < jw) {
      wait_vmcnt<(DIST - 1) * PER_TILE>();               // tile j landed; tiles j + 1 .. j + DIST - 1 may not have
      __syncthreads();                                   // every wave's share landed; tile j - 1 is free
      issue(j + DIST);
    } else if (j == jw) {
      wait_vmcnt<0>();
      __syncthreads();                                   // every remaining tile resident everywhere
    }
    const unsigned kst = ring + (unsigned)(j % NS) * TB;
    const unsigned vst = kst + NS * TB;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int U = 2 * j + u;
      if (U < nu) {
        const f32x16 s = mm_rows<D>(kst + u * 32 * D * 2, g, qop);   // S^T: keys x queries
        const f32x16 dp = mm_rows<D>(vst + u * 32 * D * 2, g, dop);  // dP^T
        const bool masked = U >= umask;
        f32x16 ds;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float pe = fast_exp2(fmaf(s[e], c, -lse2));
          if (masked && 32 * U + 8 * (e >> 2) + 4 * hh + (e & 3) > lim) pe = 0.f;
          ds[e] = pe * (dp[e] - dsum);
        }
        mm_tr<D>(kst, 2 * u, g, p_operand(ds, 0), acc);
        mm_tr<D>(kst, 2 * u + 1, g, p_operand(ds, 1), acc);
      }
    }
  }

  // ---- epilogue: dQ = scale * acc -------------------------------------------------------
  if (valid) {
    uint16_t* dst = p.dq + ((int64_t)(b * p.Sq + row) * p.Hq + h) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) store4(dst + 32 * db + 8 * i + 4 * hh, acc[db], i, p.scale);
  }
}

// ---------------------------------------------------------------------------------------
// dK, dV: one workgroup per (batch, KV head, kBwdDkvKeys keys), over every query head
// of the KV head's group.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdDkvWaves * 64) void fa_bwd_dkdv_kernel(BwdParams p) {
  constexpr int NW = kBwdDkvWaves, BT = kBwdDkvTile, NS = 2, BC = kBwdDkvKeys;
  constexpr unsigned TB = BT * D * 2;                    // bytes per Q / dO tile
  constexpr unsigned VB = BT * 4;                        // bytes per LSE / D tile
  // Q stages, dO stages, LSE stages, D stages
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * NS * TB + 2 * NS * VB];
  static_assert(NW == 4, "waves 0..3 copy LSE and D, 64 rows each");

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, hh = lane >> 5;

  // Low key tiles are seen by the most query rows under the causal mask; they come first.
  const int heads = p.B * p.Hkv;
  const int kt = blockIdx.x / heads, hl = blockIdx.x - kt * heads;
  const int b = hl / p.Hkv, hk = hl - b * p.Hkv;
  const int grp = p.Hq / p.Hkv;
  const int k0 = kt * BC;
  const int diag = p.Skv - p.Sq;

  // query tiles that see any key of the workgroup (row i sees keys j <= i + diag)
  const int nq_all = (p.Sq + BT - 1) / BT;
  int qt0 = 0;
  if (CAUSAL) qt0 = min(nq_all, max(0, k0 - diag) / BT);
  const int nqt = nq_all - qt0;
  const int n_it = nqt * grp;

  const int key = k0 + 32 * w + lr;
  const bool kvalid = key < p.Skv;
  const int kw_lo = k0 + 32 * w;                         // first key of this wave

  // ---- resident K and V rows -----------------------------------------------------------
  // Keys past the end load key Skv - 1 (no per-key branch): finite data whose dK, dV rows
  // are never stored. They are waited for together with the first tile copy, below.
  u32x4 kop[D / 16], vop[D / 16];
  {
    const int64_t off = ((int64_t)(b * p.Skv + min(key, p.Skv - 1)) * p.Hkv + hk) * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      kop[s] = *reinterpret_cast<const u32x4*>(p.k + off + 16 * s);
      vop[s] = *reinterpret_cast<const u32x4*>(p.v + off + 16 * s);
    }
  }
  const float c = p.c;

  const BwdGeom<D> g = make_bgeom<D>(lane);
  const unsigned ring = lds_addr(smem);
  const unsigned lse_ring = ring + 2 * NS * TB;
  const unsigned dsum_ring = lse_ring + NS * VB;
  const int64_t q_stride = (int64_t)p.Hq * D;
  TileDma<D, NW, BT> dma;
  dma.init(q_stride, w, lane);

  auto issue = [&](int it) {
    const int hq = hk * grp + it / nqt;
    const int r0 = (qt0 + it % nqt) * BT;
    const unsigned st = (unsigned)(it % NS);
    const int64_t hoff = ((int64_t)b * p.Sq * p.Hq + hq) * D;
    dma.copy(p.q + hoff, q_stride, r0, p.Sq, ring + st * TB, w, lane);
    dma.copy(p.dout + hoff, q_stride, r0, p.Sq, ring + (NS + st) * TB, w, lane);
    // LSE (even waves) and D (odd waves) rows of the tile, 64 rows per wave; rows past Sq
    // re-read row Sq - 1 (r0 < Sq, so the offset is never negative)
    const int64_t soff = ((int64_t)b * p.Hq + hq) * p.Sq + r0;
    const int half = w >> 1;
    const unsigned ro = (unsigned)min(64 * half + lane, p.Sq - 1 - r0) * 4u;
    if ((w & 1) == 0) dma::copy4(p.lse + soff, ro, lse_ring + st * VB + 256u * half);
    else dma::copy4(p.dsum + soff, ro, dsum_ring + st * VB + 256u * half);
  };

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    dk[i] = f32x16{};
    dv[i] = f32x16{};
  }

  if (n_it > 0) issue(0);
  wait_vmcnt<0>();                                       // K, V rows; only tile copies are issued below
  for (int it = 0; it < n_it; ++it) {
    wait_vmcnt<0>();                                     // tile it landed (the only copies in flight)
    __syncthreads();                                     // every wave's share landed; tile it - 1 is free
    if (it + 1 < n_it) issue(it + 1);
    const unsigned st = (unsigned)(it % NS);
    const unsigned qst = ring + st * TB, dst = ring + (NS + st) * TB;
    const unsigned lst = lse_ring + st * VB, sst = dsum_ring + st * VB;
    const int r0 = (qt0 + it % nqt) * BT;
    // One code path for every tile (no branch around the accumulator updates, so the
    // accumulators stay in place across iterations); masks are applied in place. The
    // four units run one after the other: prefetching the next unit's operands under the
    // current unit's products overflows the architected VGPRs and gains nothing.
#pragma unroll 1
    for (int u = 0; u < BT / 32; ++u) {
      const int qu0 = r0 + 32 * u;                       // first query row of the unit
      const RowOps<D> aq = load_rows<D>(qst + u * 32 * D * 2, g);
      const RowOps<D> ad = load_rows<D>(dst + u * 32 * D * 2, g);
      f32x16 s = {}, dp = {};
#pragma unroll
      for (int st = 0; st < D / 16; ++st) {
        s = mfma_32x32x16(aq.a[st], kop[st], s);        // S: queries x keys
        dp = mfma_32x32x16(ad.a[st], vop[st], dp);      // dP
      }
      const TrOps<D> tv0 = load_tr<D>(dst, 2 * u, g), tv1 = load_tr<D>(dst, 2 * u + 1, g);
      const TrOps<D> tq0 = load_tr<D>(qst, 2 * u, g), tq1 = load_tr<D>(qst, 2 * u + 1, g);
      f32x16 pr, ds;
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const unsigned ro = (unsigned)(32 * u + 8 * gq + 4 * hh) * 4u;
        const f32x4 l4 = *reinterpret_cast<const lds_f32x4*>(lds_ptr(lst + ro));
        const f32x4 d4 = *reinterpret_cast<const lds_f32x4*>(lds_ptr(sst + ro));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = 4 * gq + i;
          pr[e] = fast_exp2(fmaf(s[e], c, -l4[i] * kLog2e));
          ds[e] = pr[e] * (dp[e] - d4[i]);
        }
      }
      bool masked = qu0 + 31 >= p.Sq;
      if (CAUSAL) masked = masked || qu0 + diag < kw_lo + 31;
      if (masked) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int qi = qu0 + 8 * (e >> 2) + 4 * hh + (e & 3);
          const bool off = qi >= p.Sq || (CAUSAL && key > qi + diag);
          pr[e] = off ? 0.f : pr[e];
          ds[e] = off ? 0.f : ds[e];
        }
      }
      mm_tr_ops<D>(tv0, p_operand(pr, 0), dv);
      mm_tr_ops<D>(tv1, p_operand(pr, 1), dv);
      mm_tr_ops<D>(tq0, p_operand(ds, 0), dk);
      mm_tr_ops<D>(tq1, p_operand(ds, 1), dk);
    }
  }

  // ---- epilogue: dK = scale * acc, dV = acc ---------------------------------------------
  if (kvalid) {
    const int64_t obase = ((int64_t)(b * p.Skv + key) * p.Hkv + hk) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int dim = 32 * db + 8 * i + 4 * hh;
        store4(p.dk + obase + dim, dk[db], i, p.scale);
        store4(p.dv + obase + dim, dv[db], i, 1.f);
      }
  }
}

// ---------------------------------------------------------------------------------------
// dK, dV at two waves per SIMD: one workgroup of eight waves per (batch, KV head, 128
// keys). Waves w and w + 4 share the 32 keys k0 + 32 (w % 4) and one SIMD. The first
// (role 0) holds K and the dV accumulators: per 32-query unit it forms S = Q K^T, the
// probabilities P, hands P to its partner through LDS and accumulates dV^T += dO^T P.
// The second (role 1) holds V and the dK accumulators: one tile later it forms
// dP = dO V^T, reads P, builds dS = P (dP - D) and accumulates dK^T += Q^T dS. Each wave
// then keeps 64 accumulator and 32 operand registers instead of twice that, so two
// waves share a SIMD and one's LDS reads and exponentials run under the other's matrix
// products. Q/dO tiles of BT rows stream through a three-stage ring (a tile is read by
// role 0 in one iteration and by role 1 in the next); P goes through two slots.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdPairWaves * 64, 2) void fa_bwd_dkdv_pair_kernel(BwdParams p) {
  constexpr int NW = kBwdPairWaves, NS = 3, NPAIR = 4, BC = 32 * NPAIR, BT = kBwdPairTile, NU = BT / 32;
  constexpr unsigned TB = BT * D * 2;                    // bytes per Q / dO stage
  constexpr unsigned VB = BT * 4;                        // bytes per LSE / D stage
  constexpr unsigned PU = 2048u;                         // P bytes per wave and unit (bf16)
  constexpr unsigned PS = NPAIR * NU * PU;               // P bytes per slot
  // Q stages | dO stages | P slots | LSE stages | D stages
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * NS * TB + 2 * PS + 2 * NS * VB];
  static_assert(BC == kBwdDkvKeys, "grid assumes kBwdDkvKeys keys per workgroup");

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = w & 3, role = w >> 2;
  const int lr = lane & 31, hh = lane >> 5;

  const int heads = p.B * p.Hkv;
  const int kt = blockIdx.x / heads, hl = blockIdx.x - kt * heads;
  const int b = hl / p.Hkv, hk = hl - b * p.Hkv;
  const int grp = p.Hq / p.Hkv;
  const int k0 = kt * BC;
  const int diag = p.Skv - p.Sq;

  const int nq_all = (p.Sq + BT - 1) / BT;
  int qt0 = 0;
  if (CAUSAL) qt0 = min(nq_all, max(0, k0 - diag) / BT);
  const int nqt = nq_all - qt0;
  const int n_it = nqt * grp;

  const int key = k0 + 32 * pair + lr;
  const bool kvalid = key < p.Skv;
  const int kw_lo = k0 + 32 * pair;

  // ---- resident K (role 0) or V (role 1) rows ------------------------------------------
  // Keys past the end load key Skv - 1 (no per-key branch): finite data whose dK, dV rows
  // are never stored. They are waited for together with the first tile copy, below.
  u32x4 rop[D / 16];
  {
    const uint16_t* src = role == 0 ? p.k : p.v;
    const int64_t off = ((int64_t)(b * p.Skv + min(key, p.Skv - 1)) * p.Hkv + hk) * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) rop[s] = *reinterpret_cast<const u32x4*>(src + off + 16 * s);
  }
  const float c = p.c;

  const BwdGeom<D> g = make_bgeom<D>(lane);
  const unsigned ring = lds_addr(smem);
  const unsigned p_ring = ring + 2 * NS * TB;
  const unsigned lse_ring = p_ring + 2 * PS;
  const unsigned dsum_ring = lse_ring + NS * VB;
  const int64_t q_stride = (int64_t)p.Hq * D;
  TileDma<D, NW, BT> dma;
  dma.init(q_stride, w, lane);

  auto issue = [&](int it) {
    const int hq = hk * grp + it / nqt;
    const int r0 = (qt0 + it % nqt) * BT;
    const unsigned st = (unsigned)(it % NS);
    const int64_t hoff = ((int64_t)b * p.Sq * p.Hq + hq) * D;
    dma.copy(p.q + hoff, q_stride, r0, p.Sq, ring + st * TB, w, lane);
    dma.copy(p.dout + hoff, q_stride, r0, p.Sq, ring + (NS + st) * TB, w, lane);
    // LSE (wave 0) and D (wave 1) rows of the tile; rows past Sq re-read row Sq - 1
    if (w < 2 && lane < BT) {
      const int64_t soff = ((int64_t)b * p.Hq + hq) * p.Sq + r0;
      const unsigned ro = (unsigned)min(lane, p.Sq - 1 - r0) * 4u;
      if (w == 0) dma::copy4(p.lse + soff, ro, lse_ring + st * VB);
      else dma::copy4(p.dsum + soff, ro, dsum_ring + st * VB);
    }
  };

  // unit-level mask: some (query, key) pair of the unit is outside the tensor or causal range
  auto unit_masked = [&](int qu0) {
    bool m = qu0 + 31 >= p.Sq;
    if (CAUSAL) m = m || qu0 + diag < kw_lo + 31;
    return m;
  };
  auto elem_off = [&](int qu0, int e) {
    const int qi = qu0 + 8 * (e >> 2) + 4 * hh + (e & 3);
    return qi >= p.Sq || (CAUSAL && key > qi + diag);
  };

  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = f32x16{};

  if (n_it > 0) issue(0);
  if (role == 0) {
    for (int it = 0; it <= n_it; ++it) {
      wait_vmcnt<0>();                                   // tile it landed
      __syncthreads();                                   // tile it - 2's stage and P slot it % 2 are free
      if (it + 1 < n_it) issue(it + 1);
      if (it < n_it) {
        const unsigned st = (unsigned)(it % NS);
        const unsigned qst = ring + st * TB, dst = ring + (NS + st) * TB, lst = lse_ring + st * VB;
        const unsigned pslot = p_ring + (unsigned)(it & 1) * PS + (unsigned)(pair * NU) * PU;
        const int r0 = (qt0 + it % nqt) * BT;
#pragma unroll 1
        for (int u = 0; u < NU; ++u) {
          const int qu0 = r0 + 32 * u;
          const RowOps<D> aq = load_rows<D>(qst + u * 32 * D * 2, g);
          f32x16 s = {};
#pragma unroll
          for (int st2 = 0; st2 < D / 16; ++st2) s = mfma_32x32x16(aq.a[st2], rop[st2], s);   // S: queries x keys
          const TrOps<D> tv0 = load_tr<D>(dst, 2 * u, g), tv1 = load_tr<D>(dst, 2 * u + 1, g);
          f32x16 pr;
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const f32x4 l4 = *reinterpret_cast<const lds_f32x4*>(lds_ptr(lst + (unsigned)(32 * u + 8 * gq + 4 * hh) * 4u));
#pragma unroll
            for (int i = 0; i < 4; ++i) pr[4 * gq + i] = fast_exp2(fmaf(s[4 * gq + i], c, -l4[i] * kLog2e));
          }
          if (unit_masked(qu0)) {
#pragma unroll
            for (int e = 0; e < 16; ++e) pr[e] = elem_off(qu0, e) ? 0.f : pr[e];
          }
          const u32x4 p0 = p_operand(pr, 0), p1 = p_operand(pr, 1);
          const unsigned pu = pslot + (unsigned)u * PU + (unsigned)lane * 16u;
          *reinterpret_cast<lds_u32x4*>((lds_u8*)(uintptr_t)pu) = p0;
          *reinterpret_cast<lds_u32x4*>((lds_u8*)(uintptr_t)(pu + 1024u)) = p1;
          mm_tr_ops<D>(tv0, p0, acc);                    // dV^T += dO^T P
          mm_tr_ops<D>(tv1, p1, acc);
        }
      }
    }
  } else {
    for (int it = 0; it <= n_it; ++it) {
      wait_vmcnt<0>();
      __syncthreads();                                   // P of tile it - 1 is in slot (it - 1) % 2
      if (it + 1 < n_it) issue(it + 1);
      if (it > 0) {
        const int jt = it - 1;
        const unsigned st = (unsigned)(jt % NS);
        const unsigned qst = ring + st * TB, dst = ring + (NS + st) * TB, sst = dsum_ring + st * VB;
        const unsigned pslot = p_ring + (unsigned)(jt & 1) * PS + (unsigned)(pair * NU) * PU;
        const int r0 = (qt0 + jt % nqt) * BT;
#pragma unroll 1
        for (int u = 0; u < NU; ++u) {
          const int qu0 = r0 + 32 * u;
          const RowOps<D> ad = load_rows<D>(dst + u * 32 * D * 2, g);
          f32x16 dp = {};
#pragma unroll
          for (int st2 = 0; st2 < D / 16; ++st2) dp = mfma_32x32x16(ad.a[st2], rop[st2], dp);   // dP
          const TrOps<D> tq0 = load_tr<D>(qst, 2 * u, g), tq1 = load_tr<D>(qst, 2 * u + 1, g);
          const unsigned pu = pslot + (unsigned)u * PU + (unsigned)lane * 16u;
          f32x16 pr;                                     // P as rounded for the dV product
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const u32x4 x = *reinterpret_cast<const lds_u32x4*>(lds_ptr(pu + 1024u * h2));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              pr[8 * h2 + 2 * i] = bf16_lo(x[i]);
              pr[8 * h2 + 2 * i + 1] = bf16_hi(x[i]);
            }
          }
          f32x16 ds;
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const f32x4 d4 = *reinterpret_cast<const lds_f32x4*>(lds_ptr(sst + (unsigned)(32 * u + 8 * gq + 4 * hh) * 4u));
#pragma unroll
            for (int i = 0; i < 4; ++i) ds[4 * gq + i] = pr[4 * gq + i] * (dp[4 * gq + i] - d4[i]);
          }
          if (unit_masked(qu0)) {
#pragma unroll
            for (int e = 0; e < 16; ++e) ds[e] = elem_off(qu0, e) ? 0.f : ds[e];
          }
          mm_tr_ops<D>(tq0, p_operand(ds, 0), acc);      // dK^T += Q^T dS
          mm_tr_ops<D>(tq1, p_operand(ds, 1), acc);
        }
      }
    }
  }

  // ---- epilogue: dV = acc (role 0), dK = scale * acc (role 1) ----------------------------
  if (kvalid) {
    const int64_t obase = ((int64_t)(b * p.Skv + key) * p.Hkv + hk) * D;
    uint16_t* dst = (role == 0 ? p.dv : p.dk) + obase;
    const float sc = role == 0 ? 1.f : p.scale;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) store4(dst + 32 * db + 8 * i + 4 * hh, acc[db], i, sc);
  }
}

long long bwd_dq_grid(int B, int Hq, int Sq, int d) {
  return (long long)B * Hq * ((Sq + bwd_dq_rows(d) - 1) / bwd_dq_rows(d));
}
long long bwd_dkdv_grid(int B, int Hkv, int Skv) {
  return (long long)B * Hkv * ((Skv + kBwdDkvKeys - 1) / kBwdDkvKeys);
}

template <int D, bool CAUSAL>
static hipError_t launch_bwd_t(const BwdParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((fa_bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)bwd_dq_grid(p.B, p.Hq, p.Sq, D)),
                     dim3(bwd_dq_waves(D) * 64), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (D == 128)
    hipLaunchKernelGGL((fa_bwd_dkdv_pair_kernel<D, CAUSAL>), dim3((unsigned)bwd_dkdv_grid(p.B, p.Hkv, p.Skv)),
                       dim3(kBwdPairWaves * 64), 0, stream, p);
  else
    hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)bwd_dkdv_grid(p.B, p.Hkv, p.Skv)),
                       dim3(kBwdDkvWaves * 64), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdParams& p, bool causal, hipStream_t stream) {
  if (p.d == 128) return causal ? launch_bwd_t<128, true>(p, stream) : launch_bwd_t<128, false>(p, stream);
  return causal ? launch_bwd_t<64, true>(p, stream) : launch_bwd_t<64, false>(p, stream);
}

}  // namespace fa
