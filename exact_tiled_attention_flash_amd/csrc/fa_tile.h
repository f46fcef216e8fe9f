// Cooperative staging of a 64-row bf16 tile from HBM into LDS, row-major and/or transposed.
#pragma once

#include "fa_common.h"

namespace fa {

// 256 threads move a [64 x D] bf16 tile. Thread t owns 16-byte chunk (t % (D/8))
// of RPT consecutive rows starting at RPT * (t / (D/8)), so one thread holds the
// same d-range of RPT neighbouring rows: enough to write both the row-major copy
// (16-byte stores) and the transposed copy (RPT bf16 of one column per store).
template <int D>
struct RowTile {
  static constexpr int kRows = 64;
  static constexpr int kChunks = D / 8;
  static constexpr int RPT = kRows * kChunks / 256;  // 4 for D = 128, 2 for D = 64
  static_assert(RPT == 2 || RPT == 4, "row split");

  __device__ static __forceinline__ void load(const uint16_t* __restrict__ src, int row0, int T,
                                              int tid, u32x4 (&r)[RPT]) {
    const int ch = tid % kChunks;
    const int g = tid / kChunks;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int row = row0 + g * RPT + i;
      r[i] = row < T ? *reinterpret_cast<const u32x4*>(src + (size_t)row * D + ch * 8)
                     : u32x4{0u, 0u, 0u, 0u};
    }
  }

  // dst[row][d], pitch in bf16 elements (multiple of 8)
  __device__ static __forceinline__ void store_rows(uint16_t* dst, int pitch, int tid,
                                                    const u32x4 (&r)[RPT]) {
    const int ch = tid % kChunks;
    const int g = tid / kChunks;
#pragma unroll
    for (int i = 0; i < RPT; ++i)
      *reinterpret_cast<u32x4*>(dst + (g * RPT + i) * pitch + ch * 8) = r[i];
  }

  __device__ static __forceinline__ uint32_t elem(const u32x4& x, int e) {
    const uint32_t w = x[e >> 1];
    return (e & 1) ? (w >> 16) : (w & 0xffffu);
  }

  // dst[d][row], pitch in bf16 elements (multiple of 4)
  __device__ static __forceinline__ void store_cols(uint16_t* dst, int pitch, int tid,
                                                    const u32x4 (&r)[RPT]) {
    const int ch = tid % kChunks;
    const int g = tid / kChunks;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint16_t* p = dst + (ch * 8 + e) * pitch + g * RPT;
      if constexpr (RPT == 4) {
        u32x2 w = {elem(r[0], e) | (elem(r[1], e) << 16), elem(r[2], e) | (elem(r[3], e) << 16)};
        *reinterpret_cast<u32x2*>(p) = w;
      } else {
        *reinterpret_cast<uint32_t*>(p) = elem(r[0], e) | (elem(r[1], e) << 16);
      }
    }
  }
};

// A operand of a 32x32x16 product whose k index runs over 16 tile rows in the
// order the S^T / S accumulator lays them out: k-slot s of lane half h is row
// base + (s < 4 ? 4h + s : 8 + 4h + s - 4). Reads the transposed copy
// (row index contiguous) at column-row `crow`.
__device__ __forceinline__ bf16x8 load_perm_k(const uint16_t* t, int pitch, int crow, int base,
                                              int h) {
  const uint16_t* p = t + crow * pitch + base + 4 * h;
  const u32x2 lo = *reinterpret_cast<const u32x2*>(p);
  const u32x2 hi = *reinterpret_cast<const u32x2*>(p + 8);
  return as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
}

}  // namespace fa
