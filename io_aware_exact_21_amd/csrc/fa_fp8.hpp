// Internal launch interface of the fp8 (OCP e4m3) forward.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Four waves of 32 query rows per workgroup (128 rows), and the kernel is built for three
// waves per SIMD (at most 168 registers), so three workgroups share a CU: the vector-ALU
// bound softmax of one wave then hides behind the products of two others. At d = 128 this
// was 11% faster on the causal 8k prefill than eight-wave workgroups at two waves per SIMD
// (the kernel needs 174 registers unconstrained; the few it spills lie outside the tile
// loop's common path); at d = 64 it fits 168 registers without spills.
constexpr int kFp8Waves = 4;
constexpr int kFp8WavesPerSimd = 3;
constexpr int fp8_waves(int) { return kFp8Waves; }
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
