// Feed-forward GEMMs of the blockwise transformer layer, on hipBLASLt.
//
// The feed-forward network of a transformer block acts on every token on its own
// ("I/O-Aware Kernels", section Blockwise Parallel Transformers), so its two products
// are plain dense GEMMs over the rows of one query block. They run on the library GEMM
// with the bias (and, for the first, the ReLU) applied in its epilogue; the blockwise
// schedule around them is in fa_api.hip (fa_bpt_layer).
//
// Row-major Y [M, N] = X [M, K] W [K, N] is the column-major product Y^T = W^T X^T:
// A = W as an N x K column-major matrix (leading dimension N), B = X as K x M (leading
// dimension K), D = Y as N x M (leading dimension N). The bias then has one entry per
// row of D, which is what the library's bias epilogue broadcasts.
#include <hipblaslt/hipblaslt.h>

#include <map>
#include <mutex>
#include <tuple>

#include "fa_bpt.hpp"

namespace fa {

namespace {

struct Plan {
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t a = nullptr, b = nullptr, d = nullptr;
  hipblasLtMatmulAlgo_t algo{};
  size_t ws = 0;
};

// hipBLASLt handles and plans belong to the device that was current when they were
// made: both are kept per device, created on first use, and used under one lock.
std::mutex g_mu;
std::map<int, hipblasLtHandle_t> g_handles;
std::map<std::tuple<int, int, int, int, bool, size_t>, Plan> g_plans;

void destroy_plan(Plan& p) {
  if (p.a) hipblasLtMatrixLayoutDestroy(p.a);
  if (p.b) hipblasLtMatrixLayoutDestroy(p.b);
  if (p.d) hipblasLtMatrixLayoutDestroy(p.d);
  if (p.desc) hipblasLtMatmulDescDestroy(p.desc);
  p = Plan{};
}

int make_plan(hipblasLtHandle_t handle, int M, int N, int K, bool relu, size_t ws_cap, Plan* out) {
  Plan p;
  const int st = [&]() -> int {
    hipblasStatus_t st = hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F);
    if (st != HIPBLAS_STATUS_SUCCESS) return (int)st;
    const hipblasOperation_t opn = HIPBLAS_OP_N;
    const hipblasLtEpilogue_t epi = relu ? HIPBLASLT_EPILOGUE_RELU_BIAS : HIPBLASLT_EPILOGUE_BIAS;
    const int32_t bias_type = HIP_R_16BF;
    if ((st = hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opn, sizeof(opn))) ||
        (st = hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opn, sizeof(opn))) ||
        (st = hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_EPILOGUE, &epi, sizeof(epi))) ||
        (st = hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_BIAS_DATA_TYPE, &bias_type,
                                              sizeof(bias_type))))
      return (int)st;
    if ((st = hipblasLtMatrixLayoutCreate(&p.a, HIP_R_16BF, N, K, N)) ||
        (st = hipblasLtMatrixLayoutCreate(&p.b, HIP_R_16BF, K, M, K)) ||
        (st = hipblasLtMatrixLayoutCreate(&p.d, HIP_R_16BF, N, M, N)))
      return (int)st;
    hipblasLtMatmulPreference_t pref = nullptr;
    if ((st = hipblasLtMatmulPreferenceCreate(&pref))) return (int)st;
    const uint64_t cap = ws_cap;
    hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &cap, sizeof(cap));
    hipblasLtMatmulHeuristicResult_t res[1];
    int found = 0;
    st = hipblasLtMatmulAlgoGetHeuristic(handle, p.desc, p.a, p.b, p.d, p.d, pref, 1, res, &found);
    hipblasLtMatmulPreferenceDestroy(pref);
    if (st != HIPBLAS_STATUS_SUCCESS) return (int)st;
    if (found < 1) return (int)HIPBLAS_STATUS_NOT_SUPPORTED;
    p.algo = res[0].algo;
    p.ws = res[0].workspaceSize;
    return 0;
  }();
  if (st != 0) {
    destroy_plan(p);                                     // a partly made plan is not kept
    return st;
  }
  *out = p;
  return 0;
}

}  // namespace

int ffn_gemm(int M, int N, int K, const void* x, const void* w, const void* bias, void* d, bool relu,
             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return (int)HIPBLAS_STATUS_NOT_INITIALIZED;
  std::lock_guard<std::mutex> lock(g_mu);
  hipblasLtHandle_t& handle = g_handles[dev];
  if (!handle) {
    hipblasStatus_t st = hipblasLtCreate(&handle);
    if (st != HIPBLAS_STATUS_SUCCESS) {
      handle = nullptr;
      return (int)st;
    }
  }
  const auto key = std::make_tuple(dev, M, N, K, relu, workspace_bytes);
  auto it = g_plans.find(key);
  if (it == g_plans.end()) {
    Plan p;
    const int st = make_plan(handle, M, N, K, relu, workspace_bytes, &p);
    if (st) return st;
    it = g_plans.emplace(key, p).first;
  }
  Plan& p = it->second;
  hipblasStatus_t st = hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_BIAS_POINTER, &bias,
                                                       sizeof(bias));
  if (st != HIPBLAS_STATUS_SUCCESS) return (int)st;
  const float alpha = 1.f, beta = 0.f;
  st = hipblasLtMatmul(handle, p.desc, &alpha, w, p.a, x, p.b, &beta, d, p.d, d, p.d, &p.algo, workspace,
                       workspace_bytes, stream);
  return (int)st;
}

}  // namespace fa
