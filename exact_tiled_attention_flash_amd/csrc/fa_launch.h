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

// General bf16 forward: grouped K/V heads (Hq = G * Hkv), queries and keys of different
// lengths, and packed variable-length batches. Dense: q, o are (B, Hq, Tq, D), k, v are
// (B, Hkv, Tk, D), lse is (B, Hq, Tq). Packed (cu_q, cu_k non-null, B + 1 entries each): q, o
// are (Tq, Hq, D) and k, v are (Tk, Hkv, D) with Tq, Tk the total rows, sequence b owning rows
// [cu_q[b], cu_q[b+1]) and [cu_k[b], cu_k[b+1]); lse is (Hq, Tq). Causal is aligned at the
// bottom right: query i of a sequence sees key j iff j <= i + (Tk_b - Tq_b).
struct FwdBf16Problem {
  const void *q, *k, *v;
  void *o;
  float *lse;
  const int *cu_q, *cu_k;
  int B, Hq, Hkv, D;
  int Tq, Tk;    // dense: lengths; packed: total rows
  int max_q;     // longest query sequence (dense: Tq)
  float scale;
  bool causal;
  hipStream_t stream;
  // E4M3 Q K^T (null: bf16 q and k): codes laid out like q / k, one byte an element, and block
  // scale bytes, one per 32 elements of a row; q and k are then ignored
  const void *q8 = nullptr, *q_scale = nullptr, *k8 = nullptr, *k_scale = nullptr;
};

// Split-K decode: q, o (B, Hq, Tq, D) with G * Tq <= 32 (G = Hq / Hkv), k, v (B, Hkv, Tk, D),
// lse (B, Hq, Tq); seqlens (B) or null gives the valid keys of each sequence (clamped into
// [0, Tk]); workspace holds B * Hkv * nsplit * G * Tq * (D + 4) floats. Causal is aligned at
// the bottom right of each sequence's valid keys.
struct DecodeBf16Problem {
  const void *q, *k, *v;
  void *o;
  float *lse;
  const int *seqlens;
  void *workspace;
  int B, Hq, Hkv, Tq, Tk, D, nsplit;
  float scale;
  bool causal;
  hipStream_t stream;
};

hipError_t launch_fwd_bf16(const FwdArgs &a);
hipError_t launch_fwd_bf16_general(const FwdBf16Problem &p);
hipError_t launch_fwd_f32(const FwdArgs &a);
hipError_t launch_bwd_bf16(const BwdArgs &a);
hipError_t launch_bwd_f32(const BwdArgs &a);
hipError_t launch_decode_bf16(const DecodeBf16Problem &p);
// Block-scaled E4M3 codes and scale bytes of `elems` bf16 values (elems a multiple of 32).
hipError_t launch_quantize_mxfp8(const void *x, void *codes, void *scales, int64_t elems,
                                 hipStream_t stream);
int decode_max_splits();
// Validation of every fa_bwd argument except the workspace (status codes of include/fa.h).
int check_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
              const float *lse, const void *dq, const void *dk, const void *dv, int B, int H,
              int T, int D, float scale, int causal, int dtype);

}  // namespace fa
