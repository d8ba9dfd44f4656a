// Internal launch interface of the fp8 (OCP e4m3) forward.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

constexpr int kFp8Waves = 8;                 // 32 query rows per wave
// At d = 64 a workgroup has four waves (128 query rows) and two workgroups share a CU:
// the finer grain shortens the causal tail of the small-head shapes.
constexpr int fp8_waves(int d) { return d == 64 ? 4 : kFp8Waves; }
constexpr int fp8_rows(int d) { return 32 * fp8_waves(d); }   // query rows per workgroup

struct Fp8Params {
  const uint8_t* q;        // [B, Sq, Hq, d]   e4m3 codes
  const uint8_t* k;        // [B, Skv, Hkv, d] e4m3 codes
  const uint8_t* vt;       // [B, Hkv, d, ldv] e4m3 codes (V transposed)
  const float* q_scale;    // [B, Hq]  dequantisation scales
  const float* k_scale;    // [B, Hkv]
  const float* v_scale;    // [B, Hkv]
  uint16_t* o;             // [B, Sq, Hq, d]   bf16
  float* lse;              // [B, Hq, Sq] or null
  int B, Hq, Hkv, Sq, Skv, d, ldv;
  float c;                 // softmax scale * log2(e) (any sign); the per-head scales multiply in
};

long long fp8_grid_size(int B, int Hq, int Sq, int d);
hipError_t launch_fwd_fp8(const Fp8Params& p, bool causal, hipStream_t stream);

}  // namespace fa
