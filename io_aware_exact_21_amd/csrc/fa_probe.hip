// Ceiling probes for the roofline: the sustained bf16 matrix-core rate and the sustained
// HBM read bandwidth that this chip reaches under load, measured next to the attention
// kernels. Built into a separate library (libfa_probe.so); the attention library does
// not depend on it.
//
//   fa_probe_mfma_bf16: one workgroup of eight waves per CU (two per SIMD, as in the
//     forward kernel; its LDS allocation keeps a second workgroup off the CU). Every wave
//     keeps eight random bf16 A operands and two B operands in registers and issues
//     `iters` rounds of eight v_mfma_f32_32x32x16_bf16 into four independent
//     accumulators. FLOPs per launch = blocks * 8 waves * iters * 8 * 32768.
//   fa_probe_hbm_read: workgroup b of 128 threads streams its own contiguous slice of the
//     buffer with non-temporal 16-byte loads, eight 2 KiB rounds in flight. Bytes per
//     launch = the buffer size.
// Both write one float per thread to `sink` so that no load or product is dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMfmaThreads = 512;
constexpr int kReadThreads = 128;
constexpr int kReadRounds = 8;
constexpr int kMfmaLdsBytes = 96 * 1024;   // > half the LDS of a CU: one workgroup per CU

__global__ __launch_bounds__(kMfmaThreads) void mfma_probe_kernel(const u32x4* __restrict__ in,
                                                                   float* __restrict__ sink, int iters) {
  __shared__ float occupancy_pad[kMfmaLdsBytes / 4];
  // an index the compiler cannot bound keeps the whole array allocated
  const int pad_slot = (int)(((unsigned)iters * 7919u) % (unsigned)(kMfmaLdsBytes / 4));
  const int64_t g = (int64_t)blockIdx.x * kMfmaThreads + threadIdx.x;
  if (threadIdx.x == 0) occupancy_pad[pad_slot] = 0.f;
  u32x4 a[8], b[2];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = in[g * 10 + i];
  b[0] = in[g * 10 + 8];
  b[1] = in[g * 10 + 9];
  f32x16 c[4] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      c[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[j]),
                                                         __builtin_bit_cast(bf16x8, b[j & 1]), c[j & 3], 0, 0, 0);
  }
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) r += c[i][e];
  __syncthreads();
  sink[g] = r + occupancy_pad[pad_slot];
}

__global__ __launch_bounds__(kReadThreads) void read_probe_kernel(const u32x4* __restrict__ buf, int64_t n16,
                                                                   float* __restrict__ sink) {
  // slice of this workgroup: [lo, hi) in 16-byte units
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t lo = (int64_t)blockIdx.x * per;
  const int64_t hi = lo + per < n16 ? lo + per : n16;
  constexpr int64_t kRound = kReadThreads;                 // 16-byte units per round
  unsigned acc = 0u;
  int64_t i = lo + threadIdx.x;
  for (; i + (kReadRounds - 1) * kRound < hi; i += kReadRounds * kRound) {
    u32x4 x[kReadRounds];
#pragma unroll
    for (int r = 0; r < kReadRounds; ++r) x[r] = __builtin_nontemporal_load(buf + i + r * kRound);
#pragma unroll
    for (int r = 0; r < kReadRounds; ++r) acc ^= x[r][0] ^ x[r][1] ^ x[r][2] ^ x[r][3];
  }
  for (; i < hi; i += kRound) {
    const u32x4 x = __builtin_nontemporal_load(buf + i);
    acc ^= x[0] ^ x[1] ^ x[2] ^ x[3];
  }
  sink[(int64_t)blockIdx.x * kReadThreads + threadIdx.x] = (float)(acc & 0xffu);
}

}  // namespace

extern "C" {

// operands: blocks * 512 * 10 * 16 bytes of random bf16 data; sink: blocks * 512 floats.
int fa_probe_mfma_bf16(const void* operands, float* sink, int blocks, int iters, void* stream) {
  if (!operands || !sink || blocks < 1 || iters < 1) return 1;
  (void)hipGetLastError();
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(kMfmaThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(operands), sink, iters);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

// buf: `bytes` bytes (a multiple of 16, 16-byte aligned); sink: blocks * 128 floats.
int fa_probe_hbm_read(const void* buf, size_t bytes, float* sink, int blocks, void* stream) {
  if (!buf || !sink || blocks < 1 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(buf) & 15u)) return 1;
  (void)hipGetLastError();
  hipLaunchKernelGGL(read_probe_kernel, dim3(blocks), dim3(kReadThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(buf), (int64_t)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

}  // extern "C"
