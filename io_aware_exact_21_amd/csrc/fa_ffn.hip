// Feed-forward GEMMs of the blockwise transformer layer on the bf16 matrix cores.
//
// The feed-forward network acts on every token on its own ("I/O-Aware Kernels", section
// Blockwise Parallel Transformers), so each of its two products is a dense GEMM over the
// rows of one query block:  C[m, n] = act(sum_k X[m, k] W[n, k] + bias[n]),
// with X the block's activations [M, K] and W a linear layer's weights [N, K] (both
// row-major, k contiguous), fp32 accumulation, the bias and the optional ReLU applied
// to the fp32 sum, and one bf16 rounding (round-to-nearest-even) at the store.
//
// One workgroup of four waves (one per SIMD) computes a 256 x 256 tile of C. Tiles of
// kBK k-columns of X and W stream through a two-stage LDS ring by direct global -> LDS
// copies. The products are formed transposed, C^T = W X^T, on v_mfma_f32_32x32x16_bf16:
// the W rows are the A operand and the X rows the B operand, so in the accumulator a lane
// owns one row m of C and 4 consecutive n per register group; the epilogue stages the
// rounded tile through LDS and stores whole 256-byte row segments (direct 8-byte stores
// from the accumulator layout doubled the bytes written and made the first GEMM 14%
// slower). Each wave owns 128 rows m x 128 columns n: 4 x 4 products per 16-wide k step,
// every LDS operand read feeding four products, with the 256 accumulator registers in the
// AGPR file. (Eight waves of 64 x 128, two per SIMD, read 1.5x the LDS bytes per product
// and ran the blockwise layer 9-13% slower; 32-wide k stages were slower still.)
//
// The schedule keeps the matrix cores fed across stage boundaries: the operands of the
// next k step are read, one 16-byte read between consecutive products, while the current
// step's products run, and the stage's barrier sits before its last k step, whose operands
// are already in registers. Past that barrier the last step's products overlap the reads
// of the next stage's first operands and the first half of the copies of the stage after
// it; the second half goes out during the next step. (With the barrier at the stage end
// and the compiler's own placement of the reads, each step waited for its operands and the
// matrix cores were busy 52% of the time; with all sixteen copies in one step, 64%.)
#include <type_traits>

#include "fa_bpt.hpp"
#include "fa_device.hpp"
#include "fa_dma.hpp"

namespace fa {

namespace {

constexpr int kBM = 256, kBN = 256;
constexpr int kBK = 64;                            // k columns per LDS stage
constexpr int kStages = 2;                         // LDS ring depth
constexpr int kGroupRows = 8;                      // row tiles per group of the tile order
constexpr int kWaves = 4;                          // kWaves / 2 along m x 2 along n
constexpr int kWavesM = kWaves / 2;
constexpr int kWaveRows = kBM / kWavesM;          // rows m per wave
constexpr int MB = kWaveRows / 32;
constexpr int kRowBytes = kBK * 2;                 // bytes per tile row
constexpr int kChunks = kRowBytes / 16;            // 16-byte chunks per tile row
constexpr int kRowsPerCopy = 1024 / kRowBytes;     // tile rows per wave-level copy (1 KiB)
constexpr int kCopiesPerWave = kBM / kRowsPerCopy / kWaves;   // per tile and wave
constexpr unsigned kTileBytes = kBM * kRowBytes;   // X tile; the W tile is the same size
constexpr unsigned kStageBytes = 2 * kTileBytes;
constexpr int kSwzShift = kChunks == 8 ? 1 : 2;    // rows per 256-byte bank window: 2 or 4
static_assert(kBK == 64, "tile depth: four 16-wide k steps per stage");
static_assert(kStages * kStageBytes <= 160 * 1024, "LDS ring");

typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;

// 16-byte chunk c of tile row r sits at chunk c ^ swz(r): sixteen consecutive rows read at
// one logical chunk then fall on sixteen distinct 16-byte bank groups of the 256-byte bank
// window (a row is half or a quarter of that window).
__device__ __forceinline__ int ffn_swz(int r) { return (r >> kSwzShift) & (kChunks - 1); }

// Per-lane byte offsets of the wave-level copies of one 256-row tile: copy i fills tile
// rows kRowsPerCopy i ...; lane l takes row kRowsPerCopy i + l / kChunks and fetches its
// global chunk (l % kChunks) ^ swz(row). Rows at or past `rows` (the ragged edge of the
// matrix) re-read the last row; their results are never stored.
struct TileCopy {
  unsigned off[kCopiesPerWave];

  __device__ __forceinline__ void init(int64_t row_stride_bytes, int rows, int w, int lane) {
#pragma unroll
    for (int j = 0; j < kCopiesPerWave; ++j) {
      const int r = kRowsPerCopy * (w + kWaves * j) + lane / kChunks;
      const int rg = min(r, rows - 1);
      off[j] = (unsigned)(rg * row_stride_bytes) + (unsigned)(((lane % kChunks) ^ ffn_swz(r)) << 4);
    }
  }
};

template <bool RELU>
__global__ __launch_bounds__(kWaves * 64, 1) void ffn_gemm_kernel(FfnGemmParams p) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kStages * kStageBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w % kWavesM, wn = w / kWavesM;   // wave position: 128-row slab m, 128-column slab n

  // ---- tile of this workgroup. Workgroups are dealt to the 8 XCDs round-robin; XCD x
  // (blockIdx % 8) takes the x-th contiguous share of a grouped tile order that walks
  // kGroupRows row tiles x every column tile, column by column, so the 32 workgroups an XCD
  // runs at once cover a compact 8 x 4 block of tiles and share X and W panels in its L2.
  const int mt = (p.M + kBM - 1) / kBM, nt = (p.N + kBN - 1) / kBN;
  int tm, tn;
  {
    const int L = blockIdx.x, T = mt * nt, x = L & 7;
    const int t = x * (T >> 3) + min(x, T & 7) + (L >> 3);   // XCD x owns the blockIdx = x mod 8
    const int g = t / (kGroupRows * nt), r = t - g * (kGroupRows * nt);
    const int gm = min(kGroupRows, mt - g * kGroupRows);      // rows in this (maybe ragged) group
    tm = g * kGroupRows + r % gm;
    tn = r / gm;
  }
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int64_t kb = (int64_t)p.K * 2;             // row stride in bytes (X and W)

  TileCopy cx, cw;
  cx.init(kb, p.M - m0, w, lane);
  cw.init(kb, p.N - n0, w, lane);
  const unsigned char* xbase = reinterpret_cast<const unsigned char*>(p.x + (int64_t)m0 * p.K);
  const unsigned char* wbase = reinterpret_cast<const unsigned char*>(p.w + (int64_t)n0 * p.K);
  const unsigned ring = dma::lds_addr(smem);

  // operand read offsets within a tile: row (lane % 32) of a 32-row block, chunk 2 ks + lane / 32
  constexpr int KS = kBK / 16;
  const int lr = lane & 31, hh = lane >> 5;
  unsigned opoff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) opoff[ks] = (unsigned)(lr * kRowBytes + (((2 * ks + hh) ^ ffn_swz(lr)) << 4));
  const unsigned xrow = (unsigned)(wm * kWaveRows) * kRowBytes;          // this wave's X rows in a tile
  const unsigned wrow = kTileBytes + (unsigned)(wn * 128) * kRowBytes;   // this wave's W rows

  f32x16 acc[4][MB];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = f32x16{};

  // ---- k loop over a two-stage ring. The barrier of stage kt sits before its last k step,
  // whose operands are already in registers: past it no wave reads slot kt any more and
  // stage kt + 1 is visible, so that step's products run while the operands of stage
  // kt + 1's first step are read. The sixteen copies of stage kt + 2 into slot kt go out in
  // two halves, one copy before every second product: the first half in that last step of
  // stage kt, the second in the first step of stage kt + 1 (slot kt is then still unread,
  // and both halves have landed by the wait before the barrier in stage kt + 1). Within a
  // step, one operand read of the next step goes between consecutive products of its first
  // half (a scheduling fence after each product keeps that order).
  static_assert(kStages == 2 && MB == 4 && 2 * kCopiesPerWave == 16, "eight copies per half stage");
  const int KT = p.K / kBK;
  auto copy_one = [&](int s, int j) {   // copy j (X then W) of stage s into its slot
    const unsigned slot = ring + (unsigned)(s & 1) * kStageBytes;
    if (j < kCopiesPerWave)
      dma::copy16(xbase + (int64_t)s * kRowBytes, cx.off[j], slot + (w + kWaves * j) * 1024);
    else
      dma::copy16(wbase + (int64_t)s * kRowBytes, cw.off[j - kCopiesPerWave],
                  slot + kTileBytes + (w + kWaves * (j - kCopiesPerWave)) * 1024);
  };
  auto read_one = [&](unsigned st, unsigned off, int i, u32x4 (&an)[4], u32x4 (&bn)[MB]) {
    if (i < 4) an[i] = *reinterpret_cast<const lds_u32x4*>(dma::lds_ptr(st + wrow + off) + i * 32 * kRowBytes);
    else bn[i - 4] = *reinterpret_cast<const lds_u32x4*>(dma::lds_ptr(st + xrow + off) + (i - 4) * 32 * kRowBytes);
  };
#pragma unroll
  for (int j = 0; j < 16; ++j) copy_one(0, j);
  if (KT > 1) {
#pragma unroll
    for (int j = 0; j < 8; ++j) copy_one(1, j);     // the second half goes out in stage 0
    dma::wait_vmcnt<8>();                             // stage 0 landed
  } else {
    dma::wait_vmcnt<0>();
  }
  __syncthreads();
  u32x4 a[2][4], b[2][MB];
#pragma unroll
  for (int i = 0; i < 8; ++i) read_one(ring, opoff[0], i, a[0], b[0]);

  // stage kt; NEXT: stage kt + 1 exists, COPY: stage kt + 2 exists (known at compile time)
  auto run_stage = [&](int kt, auto next_c, auto copy_c) {
    constexpr bool NEXT = decltype(next_c)::value, COPY = decltype(copy_c)::value;
    const unsigned st = ring + (unsigned)(kt & 1) * kStageBytes;
    const unsigned st1 = ring + (unsigned)((kt + 1) & 1) * kStageBytes;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int cur = ks & 1, nxt = cur ^ 1;
      if (NEXT && ks == KS - 1) {
        dma::wait_vmcnt<0>();                         // stage kt + 1 landed
        __syncthreads();
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (i < 8) {
          if (ks + 1 < KS) read_one(st, opoff[ks + 1], i, a[nxt], b[nxt]);
          else if (NEXT) read_one(st1, opoff[0], i, a[nxt], b[nxt]);
        }
        if ((i & 1) == 0) {
          if (COPY && ks == KS - 1) copy_one(kt + 2, i >> 1);       // first half of stage kt + 2
          if (NEXT && ks == 0) copy_one(kt + 1, 8 + (i >> 1));      // second half of stage kt + 1
        }
        acc[i / MB][i % MB] = mfma_32x32x16(a[cur][i / MB], b[cur][i % MB], acc[i / MB][i % MB]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  int kt = 0;
  for (; kt + 2 < KT; ++kt) run_stage(kt, std::true_type{}, std::true_type{});
  if (kt + 1 < KT) run_stage(kt++, std::true_type{}, std::false_type{});
  run_stage(kt, std::false_type{}, std::false_type{});
  __syncthreads();   // every wave is done with the ring before the epilogue stages through it

// ---- epilogue: bias, activation and bf16 rounding in registers, then the wave's
  // kWaveRows x 128 tile goes through LDS (the ring is free after the last barrier) so that
  // the global stores are whole 256-byte row segments, 16 lanes per row. In the registers
  // lane (lr, hh) holds row 32 mb + lr and columns 32 nb + 8 i + 4 hh + j of the wave's tile;
  // in LDS 16-byte chunk c of tile row r sits at chunk c ^ (r & 15) (conflict-free writes
  // down a column and reads along a row).
  static_assert(kWaves * kWaveRows * 256 <= kStages * kStageBytes, "epilogue staging fits the ring");
  const unsigned stage = ring + (unsigned)w * (unsigned)(kWaveRows * 256);
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int nblk = n0 + 128 * wn + 32 * nb;
    float bias[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x2 bb = {0u, 0u};
      if (nblk < p.N) bb = *reinterpret_cast<const u32x2*>(p.bias + nblk + 8 * i + 4 * hh);
      bias[4 * i + 0] = __uint_as_float(bb[0] << 16);
      bias[4 * i + 1] = __uint_as_float(bb[0] & 0xffff0000u);
      bias[4 * i + 2] = __uint_as_float(bb[1] << 16);
      bias[4 * i + 3] = __uint_as_float(bb[1] & 0xffff0000u);
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int r = 32 * mb + lr;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[j] = acc[nb][mb][4 * i + j] + bias[4 * i + j];
          if (RELU) v[j] = fmaxf(v[j], 0.f);
        }
        const u32x2 o = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        const unsigned a = stage + (unsigned)(r * 256) + ((unsigned)((4 * nb + i) ^ (r & 15)) << 4) + 8u * hh;
        *reinterpret_cast<lds_u32x2*>((dma::lds_u8*)(uintptr_t)a) = o;
      }
    }
  }
  __syncthreads();
  const int j = lane & 15;                         // 16-byte chunk: columns 8 j .. 8 j + 7
  const int n = n0 + 128 * wn + 8 * j;
#pragma unroll 4
  for (int it = 0; it < kWaveRows / 4; ++it) {
    const int r = 4 * it + (lane >> 4);
    const u32x4 val = *reinterpret_cast<const lds_u32x4*>(dma::lds_ptr(stage + (unsigned)(r * 256) + ((unsigned)(j ^ (r & 15)) << 4)));
    const int m = m0 + kWaveRows * wm + r;
    if (m < p.M && n < p.N) {
      const int64_t row = (int64_t)(m / p.group_rows) * p.group_stride + (m % p.group_rows);
      *reinterpret_cast<u32x4*>(p.c + row * p.ldc + n) = val;
    }
  }
}

}  // namespace

long long ffn_gemm_grid(int M, int N) { return (long long)((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN); }

hipError_t launch_ffn_gemm(const FfnGemmParams& p, bool relu, hipStream_t stream) {
  const unsigned grid = (unsigned)ffn_gemm_grid(p.M, p.N);
  if (relu)
    hipLaunchKernelGGL(ffn_gemm_kernel<true>, dim3(grid), dim3(kWaves * 64), 0, stream, p);
  else
    hipLaunchKernelGGL(ffn_gemm_kernel<false>, dim3(grid), dim3(kWaves * 64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace fa
