// Internal launch interface of the backward pass (dQ, dK, dV).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Waves per backward workgroup: the dQ kernel gives each wave 32 query rows (two
// waves per SIMD). At d = 64 the dK/dV kernel gives each wave 32 keys and both their
// accumulators (four waves); at d = 128 two waves share 32 keys,
// one holding K and dV, the other V and dK, so that two waves fit a SIMD.
constexpr int kBwdDqWaves = 8;
constexpr int kBwdDkvWaves = 4;
constexpr int kBwdPairWaves = 8;
constexpr int kBwdPairTile = 64;   // Q / dO rows per streamed tile of the d = 128 dK/dV kernel
// At d = 64 a dQ workgroup has four waves (128 query rows) and two share a CU: the finer
// grain shortens the causal tail of the small-head shapes.
constexpr int bwd_dq_waves(int d) { return d == 64 ? 4 : kBwdDqWaves; }
constexpr int bwd_dq_rows(int d) { return 32 * bwd_dq_waves(d); }   // query rows per dQ workgroup
constexpr int kBwdDkvKeys = 32 * kBwdDkvWaves;  // keys per dK/dV workgroup

struct BwdParams {
  const uint16_t* q;      // [B, Sq, Hq, d]
  const uint16_t* k;      // [B, Skv, Hkv, d]
  const uint16_t* v;      // [B, Skv, Hkv, d]
  const uint16_t* o;      // [B, Sq, Hq, d]   forward output
  const uint16_t* dout;   // [B, Sq, Hq, d]   loss gradient of o
  const float* lse;       // [B, Hq, Sq]      forward log-sum-exp (natural log)
  uint16_t* dq;           // [B, Sq, Hq, d]
  uint16_t* dk;           // [B, Skv, Hkv, d]
  uint16_t* dv;           // [B, Skv, Hkv, d]
  float* dsum;            // [B, Hq, Sq]      workspace: D_i = dO_i . O_i
  int B, Hq, Hkv, Sq, Skv, d;
  float c;                // scale * log2(e), any sign
  float scale;
};

long long bwd_dq_grid(int B, int Hq, int Sq, int d);
long long bwd_dkdv_grid(int B, int Hkv, int Skv);
// dQ kernel (which also writes dsum), then dK/dV kernel, on one stream.
hipError_t launch_bwd(const BwdParams& p, bool causal, hipStream_t stream);

}  // namespace fa
