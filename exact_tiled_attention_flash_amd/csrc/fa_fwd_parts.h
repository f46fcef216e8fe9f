// Pieces of the forward kernel: matrix-core products with explicit register files (bf16 and
// E4M3), the E4M3 tile layout and loader, wait-state fences, compile-time loops, the
// cross-half row maximum and the kernel arguments.
#pragma once

#include "fa_common.h"
#include "fa_swz.h"

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
  int grp;           // (batch, head group)s an XCD works through together (xcd_grid_item)
  int B;             // sequences (packed) or batch size
  int vsched;        // packed batch walked longest sequence first (varlen_item), else 0
  float c;           // scale * log2(e)
  // E4M3 Q K^T: codes of q / k (same layout and strides as q / k, one byte an element) and
  // their block scales (one byte per 32 elements of a row: element offset / 32)
  const uint8_t *q8, *k8, *qs, *ks;
};

// E4M3 variant of the S products: 32 x 32 x 64 with a power-of-two scale per 32 k-values.
// Lane l supplies row (A) / column (B) l % 32; its bytes 0-15 are k-values 16 (l / 32) + 0..15
// of the first 32-value block and bytes 16-31 the same positions of the second block; the
// scale of block q of a row comes from lane row + 32 q, byte BYTE of its scale register
// (op_sel carries bit 0 of BYTE, op_sel_hi bit 1).
typedef int i32x8 __attribute__((ext_vector_type(8)));
template <bool FIRST, int BYTE>
__device__ __forceinline__ void mfma8_s(f32x16& d, const i32x8& a, const i32x8& b, uint32_t sa,
                                        uint32_t sb) {
  static_assert(BYTE == 0 || BYTE == 2, "scale byte");
  if constexpr (FIRST && BYTE == 0)
    asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, 0, %3, %4"
                 : "=&v"(d) : "v"(a), "a"(b), "v"(sa), "v"(sb));
  else if constexpr (FIRST)
    asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, 0, %3, %4 op_sel_hi:[1,1,0]"
                 : "=&v"(d) : "v"(a), "a"(b), "v"(sa), "v"(sb));
  else if constexpr (BYTE == 0)
    asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4"
                 : "+v"(d) : "v"(a), "a"(b), "v"(sa), "v"(sb));
  else
    asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[1,1,0]"
                 : "+v"(d) : "v"(a), "a"(b), "v"(sa), "v"(sb));
}

// A [64 x D] E4M3 tile in LDS (D bytes a row, 16-byte chunks XOR-swizzled so that 8 (D = 128)
// or 4 (D = 64) consecutive rows reading one logical chunk hit distinct banks for 32 and for
// 64 banks), followed by its block-scale bytes: D / 32 per row, in one dword per row (a direct
// load to LDS of 1 or 2 bytes a lane writes a zero-extended dword a lane).
template <int D>
struct SwzTile8 {
  static constexpr int CH = D / 16;
  static constexpr int RB = D;
  static constexpr int SB = D / 32;     // scale bytes per row in HBM
  static constexpr int sc_offset = 64 * RB;
  static constexpr int loadsPerWave = 64 * CH / 256;
  __device__ static __forceinline__ int swz(int row) { return D == 128 ? (row & 7) : ((row >> 1) & 3); }
  __device__ static __forceinline__ int offset(int row, int lchunk) {
    return row * RB + ((lchunk ^ swz(row)) << 4);
  }
};

// Direct buffer -> LDS loads of a 64-row E4M3 tile and its scales by the 4 waves of a
// workgroup (the same lane-to-chunk rule as BufTileLoader; rows at or past T arrive as zeros);
// wave 0 also moves the 64 rows' scale bytes.
template <int D>
struct TileLoader8 {
  using Tl = SwzTile8<D>;
  uint32_t vofs[Tl::loadsPerWave];   // byte offset of the lane's i-th chunk from the tile's row 0
  int wave, lane;
  uint32_t rsb, srs;   // bytes between rows of the codes and of the scales
  __device__ __forceinline__ TileLoader8(int wave_, int lane_, int row_stride)
      : wave(wave_), lane(lane_), rsb((uint32_t)row_stride), srs((uint32_t)row_stride / 32u) {
#pragma unroll
    for (int i = 0; i < Tl::loadsPerWave; ++i) {
      const int u = (wave * Tl::loadsPerWave + i) * 64 + lane;
      const int row = u / Tl::CH;
      vofs[i] = (uint32_t)row * rsb + (uint32_t)(((u % Tl::CH) ^ Tl::swz(row)) * 16);
    }
  }
  // codes and scales come through buffer resources over the T rows (rows at or past T: zeros)
  __device__ __forceinline__ void issue(uint8_t* dst, const i32x4& rsrc, int row0, int T,
                                        int i) const {
    buf_lds_dma<16>(dst + (wave * Tl::loadsPerWave + i) * 1024, rsrc, vofs[i],
                    (uint32_t)min(row0, T) * rsb);
  }
  __device__ __forceinline__ void issue_scales(uint8_t* dst, const i32x4& srsrc, int row0,
                                               int T) const {
    if (wave == 0)
      buf_lds_dma<Tl::SB>(dst + Tl::sc_offset, srsrc, (uint32_t)lane * srs,
                          (uint32_t)min(row0, T) * srs);
  }
  __device__ __forceinline__ void issue_all(uint8_t* dst, const i32x4& rsrc, const i32x4& srsrc,
                                            int row0, int T) const {
#pragma unroll
    for (int i = 0; i < Tl::loadsPerWave; ++i) issue(dst, rsrc, row0, T, i);
    issue_scales(dst, srsrc, row0, T);
  }
};

// 20 wait states (more than the result latency of a 32x32x16 product) between the last
// product writing the accumulators and any later instruction that uses them.
template <int N>
__device__ __forceinline__ void fence_acc(f32x16 (&a)[N]) {
#pragma unroll
  for (int db = 0; db < N; ++db) asm volatile("" : "+a"(a[db]));
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory");
#pragma unroll
  for (int db = 0; db < N; ++db) asm volatile("" : "+a"(a[db]));
}

// Full-row maximum of one row held as key halves in lanes l and l ^ 32. v_permlane32_swap_b32
// x, y trades lanes 32-63 of x with lanes 0-31 of y; on two copies of the value, x then holds
// lanes 0-31 in both halves and y lanes 32-63. Inline asm: with this toolchain the builtin
// returns its first result for both results. The swap sits between s_nop padding: read before
// the VALU writes of its operands had reached every lane, it returned stale upper lanes.
__device__ __forceinline__ float halves_max1(float a) {
  float x = a, y = a;
  asm volatile("s_nop 7\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 7" : "+v"(x), "+v"(y));
  return fmaxf(x, y);
}

}  // namespace fwd
}  // namespace fa
