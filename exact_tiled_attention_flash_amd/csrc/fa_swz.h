// 64-row bf16 tiles in LDS, loaded directly from HBM (global_load_lds_dwordx4) and read as
// matrix-core operands, row-major or transposed (ds_read_b64_tr_b16).
#pragma once

#include "fa_common.h"

namespace fa {

typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

// A [64 x D] bf16 tile stored unpadded; the 16-byte chunks of a row are XOR-swizzled so that
// (a) 16 lanes reading one logical chunk of 16 consecutive rows, and (b) a transposing read
// covering 8 consecutive rows x 4 chunks, spread evenly over the LDS banks.
template <int D>
struct SwzTile {
  static constexpr int CH = D / 8;                     // 16-byte chunks per row
  static constexpr int RB = D * 2;                     // bytes per row
  static constexpr int bytes = 64 * RB;
  static constexpr int loadsPerWave = 64 * CH / 256;   // 16-byte loads per lane (4 waves)
  static_assert(loadsPerWave * 256 == 64 * CH, "tile split");
  __device__ static __forceinline__ int swz(int row) {
    return D == 128 ? (((row & 7) << 1) | ((row >> 3) & 1)) : ((row >> 1) & 7);
  }
  __device__ static __forceinline__ int offset(int row, int lchunk) {
    return row * RB + ((lchunk ^ swz(row)) << 4);
  }
};

// Direct HBM -> LDS load of rows [row0, row0 + 64) of a (rows x D) matrix by the 4 waves of
// a workgroup. Lane `lane` of load i of wave `wave` fills tile bytes [16 u, 16 u + 16),
// u = (wave * loadsPerWave + i) * 64 + lane, i.e. physical chunk u % CH of row u / CH, with
// the logical chunk the swizzle maps there. Rows at or beyond T are clamped to row T - 1;
// callers mask or never store whatever depends on them.
template <int D>
__device__ __forceinline__ void issue_tile(uint8_t* dst, const uint16_t* __restrict__ src, int row0,
                                           int T, int wave, int lane) {
  using Tl = SwzTile<D>;
#pragma unroll
  for (int i = 0; i < Tl::loadsPerWave; ++i) {
    const int slot = wave * Tl::loadsPerWave + i;
    const int u = slot * 64 + lane;
    const int row = u / Tl::CH;
    const int lc = (u % Tl::CH) ^ Tl::swz(row);
    // 32-bit byte offset from the wave-uniform base (one head is below 2^31 bytes)
    const uint32_t off = (uint32_t)(min(row0 + row, T - 1) * D + lc * 8) * 2u;
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint8_t*>(src) + off,
                                     (lds_void*)(dst + slot * 1024), 16, 0, 0);
  }
}

// 16-byte operand fragment: 8 bf16 of row `row`, logical chunk `lchunk`.
template <int D>
__device__ __forceinline__ bf16x8 row_operand(const uint8_t* tile, int row, int lchunk) {
  return as_bf16x8(*reinterpret_cast<const u32x4*>(tile + SwzTile<D>::offset(row, lchunk)));
}

// A operand whose rows are the tile's columns d in [32 db, 32 db + 32) (lane l: d = 32 db +
// l % 32) and whose k-slots are tile rows kbase + {4h..4h+3, 8+4h..8+4h+3} (h = l / 32): the
// order in which a 32x32 accumulator holds its rows, so such an accumulator converted to
// bf16 is the matching B operand. Two transposing reads: within each 16-lane group, lane i
// addresses row kbase + 4 (g/2) + i/4 (+8), columns 32 db + 16 (g%2) + 4 (i%4) .. +3, and
// lane j receives four consecutive rows of column 32 db + 16 (g%2) + j.
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const uint8_t* tile, int db, int kbase, int lane) {
  using Tl = SwzTile<D>;
  const int g = lane >> 4, i = lane & 15;
  const int row = kbase + 4 * (g >> 1) + (i >> 2);
  const int d0 = db * 32 + (g & 1) * 16 + 4 * (i & 3);
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(tile + Tl::offset(row, d0 >> 3) + (d0 & 7) * 2));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(tile + Tl::offset(row + 8, d0 >> 3) + (d0 & 7) * 2));
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Pack 8 consecutive accumulator registers (o .. o+7) to a bf16 B operand.
__device__ __forceinline__ bf16x8 pack8(const f32x16& s, int o) {
  u32x4 w = {pack_bf16x2(s[o + 0], s[o + 1]), pack_bf16x2(s[o + 2], s[o + 3]),
             pack_bf16x2(s[o + 4], s[o + 5]), pack_bf16x2(s[o + 6], s[o + 7])};
  return as_bf16x8(w);
}

}  // namespace fa
