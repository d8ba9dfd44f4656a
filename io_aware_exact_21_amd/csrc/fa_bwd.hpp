// Internal launch interface of the backward pass (dQ, dK, dV).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Waves per backward workgroup: the dQ kernel gives each wave 32 query rows, the
// dK/dV kernel 32 keys.
constexpr int kBwdWaves = 4;
constexpr int kBwdRows = 32 * kBwdWaves;   // query rows (dQ) or keys (dK/dV) per workgroup

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

long long bwd_dq_grid(int B, int Hq, int Sq);
long long bwd_dkdv_grid(int B, int Hkv, int Skv);
// dQ kernel (which also writes dsum), then dK/dV kernel, on one stream.
hipError_t launch_bwd(const BwdParams& p, bool causal, hipStream_t stream);

}  // namespace fa
