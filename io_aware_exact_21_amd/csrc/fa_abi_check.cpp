// Host-only driver of the C ABI's argument validation, built with the address and
// undefined-behaviour sanitizers on the host side (see sanitize_build.py). Every call
// below must be refused before anything is launched; the driver never touches a GPU.
// Exit status 0 and "fa_abi_check: N calls refused as expected" on success.
#include <stdint.h>
#include <stdio.h>

#include <limits>

#include "fa.h"

namespace {

int failures = 0, calls = 0;

void expect(int got, int want, const char* what, int line) {
  ++calls;
  if (got != want) {
    ++failures;
    fprintf(stderr, "line %d: %s returned %d, expected %d\n", line, what, got, want);
  }
}
#define EXPECT(call, want) expect((call), (want), #call, __LINE__)

// Fake device addresses: never dereferenced, because validation fails first.
void* const A = reinterpret_cast<void*>(uintptr_t(1) << 20);
void* const A8 = reinterpret_cast<void*>((uintptr_t(1) << 20) + 8);
float* const F = static_cast<float*>(A);
const int* const I = static_cast<const int*>(A);
const int* const I2 = reinterpret_cast<const int*>((uintptr_t(1) << 20) + 2);     // not 4-byte aligned
const float* const F2 = reinterpret_cast<const float*>((uintptr_t(1) << 20) + 2);

}  // namespace

int main() {
  const float nan = std::numeric_limits<float>::quiet_NaN();
  const float inf = std::numeric_limits<float>::infinity();
  // ---- fa_fwd / fa_fwd_f32out
  EXPECT(fa_fwd(nullptr, A, A, A, nullptr, 1, 1, 1, 4, 4, 64, 0, 0.1f, nullptr), FA_ERR_NULL);
  EXPECT(fa_fwd(A, A, A, A, nullptr, 0, 1, 1, 4, 4, 64, 0, 0.1f, nullptr), FA_ERR_SHAPE);
  EXPECT(fa_fwd(A, A, A, A, nullptr, 1, 6, 4, 4, 4, 64, 0, 0.1f, nullptr), FA_ERR_SHAPE);
  EXPECT(fa_fwd(A, A, A, A, nullptr, 1, 1, 1, -5, 4, 64, 0, 0.1f, nullptr), FA_ERR_SHAPE);
  EXPECT(fa_fwd(A, A, A, A, nullptr, 1, 1, 1, 4, 4, 96, 0, 0.1f, nullptr), FA_ERR_UNSUPPORTED);
  EXPECT(fa_fwd(A, A, A, A, nullptr, 1, 1, 1, 4, 4, 64, 2, 0.1f, nullptr), FA_ERR_SHAPE);
  EXPECT(fa_fwd(A, A, A, A, nullptr, 1, 1, 1, 4, 4, 64, 0, nan, nullptr), FA_ERR_SHAPE);
  EXPECT(fa_fwd(A, A, A, A, nullptr, 1, 1, 1, 4, 4, 64, 0, inf, nullptr), FA_ERR_SHAPE);
  EXPECT(fa_fwd(A8, A, A, A, nullptr, 1, 1, 1, 4, 4, 64, 0, 0.1f, nullptr), FA_ERR_ALIGN);
  EXPECT(fa_fwd(A, A, A, A, F + 1, 1, 1, 1, 4, 4, 64, 0, 0.1f, nullptr), FA_ERR_ALIGN);
  // sizes whose products overflow 32-bit and 64-bit arithmetic
  EXPECT(fa_fwd(A, A, A, A, nullptr, 1 << 30, 1 << 30, 1 << 30, 1 << 30, 1 << 30, 128, 1, 0.1f, nullptr),
         FA_ERR_SHAPE);
  EXPECT(fa_fwd(A, A, A, A, nullptr, 1, 270000, 270000, 2, 2, 128, 0, 0.1f, nullptr), FA_ERR_SHAPE);
  EXPECT(fa_fwd(A, A, A, A, nullptr, 2147483647, 1, 1, 2147483647, 1, 64, 0, 0.1f, nullptr), FA_ERR_SHAPE);
  EXPECT(fa_fwd_f32out(A, A, A, F, nullptr, 1, 1, 1, 4, 4, 80, 0, 0.1f, nullptr), FA_ERR_UNSUPPORTED);
  // ---- decode
  const size_t need = fa_decode_workspace_bytes(2, 8, 128, 4);
  EXPECT((int)(fa_decode_workspace_bytes(-1, 8, 128, 4) == 0), 1);
  EXPECT((int)(fa_decode_workspace_bytes(2, 8, 128, 0) == 0), 1);
  EXPECT(fa_decode(A, A, A, A, nullptr, 2, 8, 2, 100, 128, 0.1f, 4, nullptr, need, nullptr), FA_ERR_WORKSPACE);
  EXPECT(fa_decode(A, A, A, A, nullptr, 2, 8, 2, 100, 128, 0.1f, 4, A, need - 1, nullptr), FA_ERR_WORKSPACE);
  EXPECT(fa_decode(A, A, A, A, nullptr, 2, 66, 2, 100, 128, 0.1f, 4, A, need, nullptr), FA_ERR_UNSUPPORTED);
  EXPECT(fa_decode(A, A, A, nullptr, nullptr, 2, 8, 2, 100, 128, 0.1f, 4, A, need, nullptr), FA_ERR_NULL);
  EXPECT(fa_decode(A, A, A, A, nullptr, 2, 8, 2, 0, 128, 0.1f, 4, A, need, nullptr), FA_ERR_SHAPE);
  EXPECT(fa_decode(A, A, A, A, nullptr, 2147483647, 8, 8, 100, 128, 0.1f, 64, A, need, nullptr), FA_ERR_SHAPE);
  EXPECT(fa_decode_partials(A, A, A, nullptr, F, 2, 8, 2, 100, 128, 0.1f, 4, nullptr), FA_ERR_NULL);
  EXPECT(fa_decode_partials(A, A, A, F, F, 2, 8, 2, 100, 128, 0.1f, 0, nullptr), FA_ERR_SHAPE);
  EXPECT(fa_decode_combine(F, F, nullptr, nullptr, 2, 8, 128, 4, nullptr), FA_ERR_NULL);
  EXPECT(fa_decode_combine(F, F, A, nullptr, 2, 8, 96, 4, nullptr), FA_ERR_UNSUPPORTED);
  EXPECT(fa_decode_noalloc(A, A, A, A, nullptr, 64, 32, 8, 64 * 40, 128, 0.1f, 40, nullptr), FA_ERR_WORKSPACE);
  EXPECT(fa_decode_noalloc(A, A, A, A8, nullptr, 2, 8, 2, 100, 128, 0.1f, 2, nullptr), FA_ERR_ALIGN);
  // ---- paged decode
  EXPECT(fa_decode_paged(A, A, A, I, I, A, nullptr, 2, 8, 2, 128, 24, 8, 32, 0.1f, 4, A, need, nullptr),
         FA_ERR_SHAPE);
  EXPECT(fa_decode_paged(A, A, A, I, I, A, nullptr, 2, 8, 2, 128, 1 << 30, 8, 32, 0.1f, 4, A, need, nullptr),
         FA_ERR_SHAPE);
  EXPECT(fa_decode_paged(A, A, A, I, I, A, nullptr, 2, 8, 2, 128, 16, 8, 32, 0.1f, 4, A, need - 256, nullptr),
         FA_ERR_WORKSPACE);
  EXPECT(fa_decode_paged(A, A, A, I2, I, A, nullptr, 2, 8, 2, 128, 16, 8, 32, 0.1f, 4, A, need, nullptr),
         FA_ERR_ALIGN);
  // ---- backward
  const size_t bneed = fa_bwd_workspace_bytes(2, 8, 100);
  EXPECT(fa_bwd(A, A, A, A, F, A, A, A, A, 2, 8, 2, 100, 90, 128, 1, 0.1f, A, bneed - 1, nullptr), FA_ERR_WORKSPACE);
  EXPECT(fa_bwd(A, A, A, A, nullptr, A, A, A, A, 2, 8, 2, 100, 90, 128, 1, 0.1f, A, bneed, nullptr), FA_ERR_NULL);
  EXPECT(fa_bwd(A, A, A, A, F, A, A, A, A, 2, 8, 2, 100, 90, 128, 1, nan, A, bneed, nullptr), FA_ERR_SHAPE);
  EXPECT(fa_bwd(A, A, A, A, F, A, A, A, A, 1, 131073, 1, 2, 2, 128, 0, 0.1f, A, 1 << 20, nullptr), FA_ERR_SHAPE);
  // ---- fp8 forward
  EXPECT(fa_fwd_fp8(A, A, A, F, F, F, A, nullptr, 2, 8, 2, 100, 90, 100, 128, 1, 0.1f, nullptr), FA_ERR_SHAPE);
  EXPECT(fa_fwd_fp8(A, A, A, F, F, F, A, nullptr, 2, 8, 2, 100, 90, 80, 128, 1, 0.1f, nullptr), FA_ERR_SHAPE);
  EXPECT(fa_fwd_fp8(A, A, A, F2, F, F, A, nullptr, 2, 8, 2, 100, 90, 96, 128, 1, 0.1f, nullptr), FA_ERR_ALIGN);
  EXPECT(fa_fwd_fp8(A, A, A, F, F, F, A, nullptr, 1, 1048577, 1048577, 2, 2, 16, 64, 0, 0.1f, nullptr), FA_ERR_SHAPE);
  // ---- blockwise layer
  const size_t pneed = fa_bpt_workspace_bytes(2, 100, 64, 4, 64, 1024);
  EXPECT(fa_bpt_layer(A, A, A, A, A, A, A, A, 2, 4, 2, 100, 64, 1024, 1, 0.1f, 128, A, pneed, nullptr),
         FA_ERR_WORKSPACE);
  EXPECT(fa_bpt_layer(A, A, A, A, A, A, A, A, 2, 4, 2, 100, 64, 0, 1, 0.1f, 64, A, pneed, nullptr), FA_ERR_SHAPE);
  EXPECT(fa_bpt_layer(A, A, A, A, A, A, A, A, 2, 4, 2, 100, 64, 1024, 1, 0.1f, 64, A8, pneed, nullptr),
         FA_ERR_ALIGN);
  EXPECT((int)(fa_bpt_workspace_bytes(0, 100, 64, 4, 64, 1024) == 0), 1);
  EXPECT(fa_bpt_layer(A, A, A, A, A, A, A, A, 2, 4, 2, 100, 64, 1000, 1, 0.1f, 64, A, pneed, nullptr), FA_ERR_SHAPE);
  // ---- status strings
  for (int st = -3; st < 10; ++st) EXPECT((int)(fa_status_string(st) != nullptr), 1);
  if (failures) {
    fprintf(stderr, "fa_abi_check: %d of %d checks failed\n", failures, calls);
    return 1;
  }
  printf("fa_abi_check: %d calls refused as expected\n", calls);
  return 0;
}
