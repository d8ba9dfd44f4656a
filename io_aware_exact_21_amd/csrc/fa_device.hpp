// Device-side building blocks shared by the prefill and decode kernels (gfx950 / CDNA4).
//
// Data layout on chip (one K/V tile of BCT keys, head size D, bf16):
//   * K and V tiles are stored row-major in LDS (one key per row), with the 16-byte
//     chunks of each row XOR-swizzled by the key index so that the MFMA operand reads
//     below hit distinct LDS banks.
//   * Scores are formed transposed, S^T = K * Q^T, on v_mfma_f32_32x32x16_bf16: the K
//     tile is the A operand (32 keys x 16 dims per lane-row), Q^T is the B operand and
//     stays in registers for the whole kernel. In the accumulator each lane then holds
//     one query row (lane % 32) and 16 of its keys, so the softmax row statistics are
//     lane-local except for one exchange between lanes l and l ^ 32.
//   * The output is accumulated transposed too, O^T = V^T * P^T: P (rounded to bf16)
//     is the B operand straight from the score registers, and V^T is read from the
//     row-major V tile with ds_read_b64_tr_b16 (gfx950's transposing LDS read).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Lazy rescaling: the running max used for the exponentials is only moved when the
// true row max exceeds it by more than this many powers of two. Any reference value
// gives the same final result (it cancels in O = acc / l); bounding the gap keeps
// every p = 2^(t - m) <= 2^kRescaleGap, far inside fp32 and bf16 range.
constexpr float kRescaleGap = 8.0f;

__device__ __forceinline__ f32x16 mfma_32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Two fp32 -> packed bf16 pair, round-to-nearest-even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(unsigned, r);
}

// Max / sum over the lane pair (l, l ^ 32) that shares one query row.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// ---- LDS tile swizzles (16-byte chunk index XOR a function of the key row) --------
// K rows: 16 consecutive lanes read 16 consecutive keys at one chunk (S^T A operand).
template <int D> __device__ __forceinline__ int k_swz(int key) {
  return D == 128 ? (key & 15) : ((key >> 1) & 7);
}
// V rows: a transposing read gathers 4 keys x 32 contiguous bytes per 16 lanes.
template <int D> __device__ __forceinline__ int v_swz(int key) {
  return D == 128 ? ((key & 3) << 2) : ((key & 2) << 1);
}

// Cooperative global -> register -> LDS copy of one K tile and one V tile.
// Keys at or beyond `kmax` are filled with zeros (never read from memory), so a
// masked key can never inject a NaN through 0 * V. The decode reads every cache byte
// exactly once, so the loads are non-temporal (streaming): they do not displace other
// data from the caches, and a streaming read of HBM sustains more bandwidth this way.
__device__ __forceinline__ u32x4 stream_load16(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

template <int D, int BCT, int NT>
struct TileCopy {
  static constexpr int CPR = D / 8;            // 16-byte chunks per key row
  static constexpr int CHUNKS = BCT * CPR;     // chunks per tile and tensor
  static constexpr int PER_T = (CHUNKS + NT - 1) / NT;
  u32x4 kr[PER_T];
  u32x4 vr[PER_T];

  __device__ __forceinline__ void load(const uint16_t* __restrict__ kb, const uint16_t* __restrict__ vb,
                                       int64_t row_stride, int k0, int kmax, int tid) {
#pragma unroll
    for (int p = 0; p < PER_T; ++p) {
      const int cid = tid + p * NT;
      const int key = cid / CPR, c = cid % CPR;
      u32x4 zk = {0u, 0u, 0u, 0u}, zv = {0u, 0u, 0u, 0u};
      if ((CHUNKS % NT == 0 || cid < CHUNKS) && k0 + key < kmax) {
        const int64_t off = (int64_t)(k0 + key) * row_stride + c * 8;
        zk = stream_load16(kb + off);
        zv = stream_load16(vb + off);
      }
      kr[p] = zk;
      vr[p] = zv;
    }
  }

  __device__ __forceinline__ void store(uint16_t* ks, uint16_t* vs, int tid) const {
#pragma unroll
    for (int p = 0; p < PER_T; ++p) {
      const int cid = tid + p * NT;
      if (CHUNKS % NT == 0 || cid < CHUNKS) {
        const int key = cid / CPR, c = cid % CPR;
        *reinterpret_cast<u32x4*>(ks + key * D + ((c ^ k_swz<D>(key)) << 3)) = kr[p];
        *reinterpret_cast<u32x4*>(vs + key * D + ((c ^ v_swz<D>(key)) << 3)) = vr[p];
      }
    }
  }
};

// Per-lane LDS offsets (in bf16 elements) for the MFMA operand reads.
struct LaneGeom {
  int lr, hh;        // query column (lane % 32) and lane half (lane / 32)
  int kbase[8];      // K operand: row lr, chunk (2s + hh) swizzled, for s = 0..D/16-1
  int vbase[4];      // V^T operand (transposing read): per 32-dim block db
};

template <int D>
__device__ __forceinline__ LaneGeom make_geom(int lane) {
  LaneGeom g;
  g.lr = lane & 31;
  g.hh = lane >> 5;
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    g.kbase[s] = g.lr * D + (((2 * s + g.hh) ^ k_swz<D>(g.lr)) << 3);
  // ds_read_b64_tr_b16: in each group of 16 lanes, lane 4r+q fetches 4 consecutive
  // dims of key row r; lane i of the group then receives dim i of rows 0..3.
  const int G = lane >> 4, r = (lane >> 2) & 3, q = lane & 3;
  const int key_l = 4 * g.hh + r;                  // + 16t + 8u
  const int dim_l = 16 * (G & 1) + 4 * q;          // + 32db
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const int dim0 = 32 * db + dim_l;
    g.vbase[db] = key_l * D + ((((dim0 >> 3) ^ v_swz<D>(key_l))) << 3) + (dim0 & 7);
  }
  return g;
}

// S^T block (32 keys starting at tile row kr0) for this lane's query column.
template <int D>
__device__ __forceinline__ f32x16 scores_block(const uint16_t* ks, const LaneGeom& g, int kr0,
                                               const u32x4 (&qop)[D / 16]) {
  f32x16 s = {};
#pragma unroll
  for (int st = 0; st < D / 16; ++st) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(ks + kr0 * D + g.kbase[st]);
    s = mfma_32x32x16(a, qop[st], s);
  }
  return s;
}

// O^T += V^T(keys 16t..16t+15 of the tile) * P^T for every 32-dim block.
template <int D>
__device__ __forceinline__ void pv_step(const uint16_t* vs, const LaneGeom& g, int t, u32x4 pb,
                                        f32x16 (&O)[D / 32]) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const uint16_t* p0 = vs + (16 * t) * D + g.vbase[db];
    const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
    const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 8 * D));
    const u32x2 a0 = __builtin_bit_cast(u32x2, r0), a1 = __builtin_bit_cast(u32x2, r1);
    const u32x4 a = {a0[0], a0[1], a1[0], a1[1]};
    O[db] = mfma_32x32x16(a, pb, O[db]);
  }
}

// bf16 B operand for PV key step t (keys 16t..16t+15) from the score registers.
__device__ __forceinline__ u32x4 p_operand(const f32x16& s, int half) {
  const int b = 8 * half;
  u32x4 r = {pack_bf16x2(s[b + 0], s[b + 1]), pack_bf16x2(s[b + 2], s[b + 3]),
             pack_bf16x2(s[b + 4], s[b + 5]), pack_bf16x2(s[b + 6], s[b + 7])};
  return r;
}

}  // namespace fa
