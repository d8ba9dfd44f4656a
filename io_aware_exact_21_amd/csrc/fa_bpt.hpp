// Internal interface of the feed-forward GEMMs of the blockwise transformer layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// C[map(m), n] = act(sum_k x[m, k] w[n, k] + bias[n]) for m < M, n < N; bf16 in and out,
// fp32 accumulation, act = ReLU or identity. x [M, K] and w [N, K] are row-major (k
// contiguous; w is a linear layer's [out, in] weight). Output row m goes to row
// map(m) = (m / group_rows) * group_stride + m % group_rows of c, rows ldc elements
// apart. Requirements (checked by the caller): K a multiple of 64, N a multiple of 32,
// 255 * K * 2 < 2^32, pointers 16-byte aligned, ldc a multiple of 8 (16-byte row stores).
struct FfnGemmParams {
  const uint16_t* x;
  const uint16_t* w;
  const uint16_t* bias;
  uint16_t* c;
  int M, N, K;
  int64_t ldc;
  int group_rows;
  int64_t group_stride;
};

long long ffn_gemm_grid(int M, int N);
hipError_t launch_ffn_gemm(const FfnGemmParams& p, bool relu, hipStream_t stream);

}  // namespace fa
