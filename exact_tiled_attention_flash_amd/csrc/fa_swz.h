// 64-row bf16 tiles in LDS, loaded directly from HBM (buffer -> LDS loads) and read as
// matrix-core operands, row-major or transposed (ds_read_b64_tr_b16).
#pragma once

#include "fa_common.h"

namespace fa {

typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource over `bytes` bytes from `base` (raw: no stride, no format conversion). A
// load whose offset (voffset + soffset) lies at or past `bytes` returns zeros without touching
// memory, and a direct-to-LDS load writes those zeros, so tiles reaching past the last row of
// a matrix need no address clamping.
__device__ __forceinline__ i32x4 rows_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return i32x4{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xffffu), (int)bytes, 0x00020000};
}

// Direct buffer -> LDS load of BYTES (16, 4 or 2) bytes a lane from voff + soff, written as
// inline asm so that the compiler does not track it. (It models a direct-to-LDS load as an
// LDS access that may complete out of order with the LDS reads, and from then on waits for all
// outstanding LDS reads wherever it needs any one of them.) The hardware counts the load in
// vmcnt only: the caller waits with s_waitcnt vmcnt, and a barrier for the other waves, before
// the destination is read. Lane l writes 16 bytes (BYTES = 16) or one zero-extended dword at
// LDS byte lds + 16 l (or + 4 l); `lds`, `rsrc` and `soff` are wave-uniform. M0 carries the
// LDS address and is set inside the same statement.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <int BYTES>
__device__ __forceinline__ void buf_lds_dma(void* lds, const i32x4& rsrc, uint32_t voff,
                                            uint32_t soff) {
  const uint32_t a = (uint32_t)(uintptr_t)(lds_void*)lds;
  if constexpr (BYTES == 16)
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(a), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
  else if constexpr (BYTES == 4)
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                 :: "s"(a), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
  else {
    static_assert(BYTES == 2, "buf_lds_dma size");
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_ushort %1, %2, %3 offen lds"
                 :: "s"(a), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
  }
}
#pragma clang diagnostic pop

// A [64 x D] bf16 tile stored unpadded; the 16-byte chunks of a row are XOR-swizzled. Two
// read patterns must spread over the LDS banks: (a) a 16-byte read by lanes holding
// consecutive rows of one logical chunk (8 rows per LDS cycle with 32 four-byte banks, 16
// with 64), and (b) a transposing read, whose 16-lane groups cover 4 consecutive rows x 2
// adjacent chunks (x 4 chunks per cycle with 64 banks). For D = 128 the swizzle maps row bits
// (0, 1, 2, 1^3) to chunk bits (2, 3, 0, 1): any aligned 8 (16) rows land on distinct chunks
// modulo 8 (16), and any aligned 4 rows differ in chunk bits 1-2 and in bits 2-3, which
// keeps both patterns conflict-free for either bank count.
template <int D>
struct SwzTile {
  static constexpr int CH = D / 8;                     // 16-byte chunks per row
  static constexpr int RB = D * 2;                     // bytes per row
  static constexpr int bytes = 64 * RB;
  static constexpr int loadsPerWave = 64 * CH / 256;   // 16-byte loads per lane (4 waves)
  static_assert(loadsPerWave * 256 == 64 * CH, "tile split");
  __device__ static __forceinline__ int swz(int row) {
    return D == 128 ? (((row & 3) << 2) | ((((row >> 1) ^ (row >> 3)) & 1) << 1) | ((row >> 2) & 1))
                    : ((row >> 1) & 7);
  }
  __device__ static __forceinline__ int offset(int row, int lchunk) {
    return row * RB + ((lchunk ^ swz(row)) << 4);
  }
};

// The same tile with another swizzle (D = 128), for tiles read as 16-row operands and by
// transposing reads in which 16-lane group g (of 4) takes rows 4 g .. 4 g + 3 of an aligned 16
// and one pair of adjacent logical chunks. Row bits 0-1 go to chunk bits 1-2, row bit 2 to
// chunk bit 0 and (row bit 2 xor row bit 3) to chunk bit 3. Any aligned 16 rows reading one
// logical chunk land on 16 distinct chunks; in a transposing read, groups 0 and 3 fill one
// half of the 16 chunk positions and groups 1 and 2 the other, so whichever two groups the
// LDS serves together, their 64 lanes hit distinct banks (64 banks).
template <int D>
struct SwzTileT {
  static_assert(D == 128, "laid out for 16 chunks a row");
  static constexpr int CH = D / 8;
  static constexpr int RB = D * 2;
  static constexpr int bytes = 64 * RB;
  static constexpr int loadsPerWave = 64 * CH / 256;
  __device__ static __forceinline__ int swz(int row) {
    return ((row & 3) << 1) | ((row >> 2) & 1) | ((((row >> 2) ^ (row >> 3)) & 1) << 3);
  }
  __device__ static __forceinline__ int offset(int row, int lchunk) {
    return row * RB + ((lchunk ^ swz(row)) << 4);
  }
};

// Direct buffer -> LDS loads of 64-row tiles of a (rows x D) matrix by the 4 waves of a
// workgroup, through a buffer resource over the source's T rows (rows_rsrc). Lane `lane` of
// load i of wave `wave` fills tile bytes [16 u, 16 u + 16), u = (wave * loadsPerWave + i) * 64
// + lane, i.e. physical chunk u % CH of row u / CH, with the logical chunk the swizzle maps
// there. Each lane's offset within the tile is fixed, the tile's first row goes into the
// scalar offset, and rows at or past T arrive as zeros: no per-load vector arithmetic remains.
// `wave` must be wave-uniform (it selects the LDS destination); rows of the source are
// `row_stride` elements apart (D for a (rows x D) matrix, H*D for one head of a packed
// (rows, H, D) array), and rows up to T of one source stay below 2^31 bytes.
template <int D, class TileT = SwzTile<D>>
struct BufTileLoader {
  using Tl = TileT;
  uint32_t vofs[Tl::loadsPerWave];   // byte offset of the lane's i-th chunk from the tile's row 0
  int wave;
  uint32_t rsb;                      // bytes between consecutive rows of the source matrix
  __device__ __forceinline__ BufTileLoader(int wave_, int lane, int row_stride = D)
      : wave(wave_), rsb((uint32_t)row_stride * 2u) {
#pragma unroll
    for (int i = 0; i < Tl::loadsPerWave; ++i) {
      const int u = (wave * Tl::loadsPerWave + i) * 64 + lane;
      const int row = u / Tl::CH;
      vofs[i] = (uint32_t)row * rsb + (uint32_t)(((u % Tl::CH) ^ Tl::swz(row)) * 16);
    }
  }
  // load i of rows [row0, row0 + 64) of the resource's matrix (T rows) into the tile at dst
  __device__ __forceinline__ void issue(uint8_t* dst, const i32x4& rsrc, int row0, int T,
                                        int i) const {
    buf_lds_dma<16>(dst + (wave * Tl::loadsPerWave + i) * 1024, rsrc, vofs[i],
                    (uint32_t)min(row0, T) * rsb);
  }
  __device__ __forceinline__ void issue_all(uint8_t* dst, const i32x4& rsrc, int row0, int T) const {
#pragma unroll
    for (int i = 0; i < Tl::loadsPerWave; ++i) issue(dst, rsrc, row0, T, i);
  }
};

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
