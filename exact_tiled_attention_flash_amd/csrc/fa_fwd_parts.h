// Pieces shared by the forward kernels: matrix-core products with explicit register files,
// wait-state fences, compile-time loops, cross-half row maxima and the kernel arguments.
#pragma once

#include "fa_common.h"

namespace fa {
namespace fwd {

constexpr int kBlockN = 64;    // keys per tile
// a row's reference max moves only when exceeded by more than 2^8 (in the exp2 domain)
constexpr float kRescaleLog2 = 8.0f;

// Matrix-core products with explicit register files. The O^T accumulators and the Q^T
// operands live in AGPRs, which no VALU instruction touches in the steady state; the S^T
// results and everything the VALU works on stay in VGPRs.
// Written as inline asm because the compiler's own register-class choice either spills or
// fails at this register pressure; the hazards the compiler would otherwise pad are
// covered by the fences below, placed before any VALU access to a product's result.
__device__ __forceinline__ void mfma_s_first(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_s(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_o(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
}

// 20 wait states (more than the result latency of a 32x32x16 product) between the last
// product writing x and y and any later instruction that uses them.
__device__ __forceinline__ void fence2(f32x16& x, f32x16& y) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(x), "+v"(y));
}
template <int N>
__device__ __forceinline__ void fence_acc(f32x16 (&a)[2][N]) {
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < N; ++db) asm volatile("" : "+a"(a[qb][db]));
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory");
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < N; ++db) asm volatile("" : "+a"(a[qb][db]));
}

template <bool B>
struct Flag {
  static constexpr bool value = B;
};
// compile-time integer and loop: every step of a phase is generated as straight-line code
template <int V>
struct IC {
  static constexpr int value = V;
};
template <int I, int N, class F>
__device__ __forceinline__ void static_for(const F& f) {
  if constexpr (I < N) {
    f(IC<I>{});
    static_for<I + 1, N>(f);
  }
}
// tile parity: selects the register buffers of a tile at compile time
template <int P>
struct Par {
  static constexpr int value = P;
};

// v_permlane32_swap_b32 x, y: lanes 32-63 of x trade places with lanes 0-31 of y, so x
// becomes [x_lo | y_lo] and y becomes [x_hi | y_hi]. Inline asm: with this toolchain the
// builtin returns its first result for both results. Both swaps sit in one block between
// s_nop padding: read before the VALU writes of its operands had reached every lane, the
// swap returned stale upper lanes.
__device__ __forceinline__ void permlane32_swap2(float& x, float& y, float& u, float& w) {
  asm volatile(
      "s_nop 7\n\tv_permlane32_swap_b32 %0, %1\n\tv_permlane32_swap_b32 %2, %3\n\ts_nop 7"
      : "+v"(x), "+v"(y), "+v"(u), "+v"(w));
}

// Full-row maxima of two rows held as key halves in lanes l and l ^ 32 (a: query block 0,
// b: query block 1): swap(a, b) puts row a's halves side by side in lanes 0-31 and row b's
// in lanes 32-63, swap(b, a) the other way round.
__device__ __forceinline__ void halves_max2(float& a, float& b, int h) {
  float x = a, y = b, u = b, w = a;
  permlane32_swap2(x, y, u, w);
  const float f = fmaxf(x, y);   // lanes 0-31: row a, lanes 32-63: row b
  const float g = fmaxf(u, w);   // lanes 0-31: row b, lanes 32-63: row a
  a = h ? g : f;
  b = h ? f : g;
}

// Item x of n items is done at step s0 + x (s1 - s0) / n of its window [s0, s1).
constexpr int win_step(int x, int n, int s0, int s1) { return s0 + x * (s1 - s0) / n; }

// Kernel arguments (element strides; the layouts are described with FwdBf16Problem).
struct FwdKArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const int* cu_q;   // null: dense
  const int* cu_k;
  int64_t q_bs, q_hs, kv_bs, kv_hs, lse_bs, lse_hs;   // batch and head strides
  int q_rs, kv_rs;   // row strides of q / o and of k / v
  int Tq, Tk;        // dense lengths, or total rows of the packed arrays
  int G;             // query heads per K/V head
  int HG;            // head groups per batch (Hq / heads per workgroup)
  int hpw_log2;      // log2 of the query heads per workgroup (1, 2 or 4 heads)
  int nbhg;          // B * HG
  int nq;            // query tiles per (batch, head group)
  float c;           // scale * log2(e)
  // E4M3 Q K^T: codes of q / k (same layout and strides as q / k, one byte an element) and
  // their block scales (one byte per 32 elements of a row: element offset / 32)
  const uint8_t *q8, *k8, *qs, *ks;
};

// fence_acc for the accumulators of one query block
template <int N>
__device__ __forceinline__ void fence_acc1(f32x16 (&a)[N]) {
#pragma unroll
  for (int db = 0; db < N; ++db) asm volatile("" : "+a"(a[db]));
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory");
#pragma unroll
  for (int db = 0; db < N; ++db) asm volatile("" : "+a"(a[db]));
}

// Full-row maximum of one row held as key halves in lanes l and l ^ 32: after the swap of
// two copies, x holds lanes 0-31 of the row's value in both halves and y lanes 32-63.
__device__ __forceinline__ float halves_max1(float a) {
  float x = a, y = a;
  asm volatile("s_nop 7\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 7" : "+v"(x), "+v"(y));
  return fmaxf(x, y);
}

}  // namespace fwd
}  // namespace fa
