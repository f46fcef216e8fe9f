// Host-side launchers of the HIP kernels (internal to libfa.so).
// Arguments are already validated by the C ABI layer (fa_api.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct FwdArgs {
  const void *q, *k, *v;
  void *o;
  float *lse;
  int B, H, T, D;
  float scale;
  bool causal;
  hipStream_t stream;
};

struct BwdArgs {
  const void *q, *k, *v, *o, *dout;
  const float *lse;
  void *dq, *dk, *dv;
  float *delta;  // workspace: D_i (B*H*T fp32), then LSE_i * log2(e) (B*H*T fp32)
  int B, H, T, D;
  float scale;
  bool causal;
  hipStream_t stream;
};

hipError_t launch_fwd_bf16(const FwdArgs &a);
hipError_t launch_fwd_f32(const FwdArgs &a);
hipError_t launch_bwd_bf16(const BwdArgs &a);

}  // namespace fa
