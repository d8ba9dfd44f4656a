// Internal interface of the feed-forward GEMMs of the blockwise transformer layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

// Bytes of device workspace one FFN GEMM may use (hipBLASLt's own scratch).
constexpr size_t kBptGemmWorkspace = size_t(32) << 20;

// Row-major D [M, N] = X [M, K] W [K, N] + bias [N], then ReLU if `relu`; bf16 in and out,
// fp32 accumulation (hipBLASLt, with the bias and ReLU in its epilogue). Returns 0 on
// success, a hipBLASLt status otherwise. Serialised by a process-wide lock; the
// hipBLASLt handle and per-shape plans are created on first use and kept.
int ffn_gemm(int M, int N, int K, const void* x, const void* w, const void* bias, void* d, bool relu,
             void* workspace, size_t workspace_bytes, hipStream_t stream);

}  // namespace fa
