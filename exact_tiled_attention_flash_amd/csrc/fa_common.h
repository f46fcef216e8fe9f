// Shared device-side types and helpers for the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// Work-item and workgroup index straight from the hardware registers. The threadIdx /
// blockIdx accessors go through device-library functions that are not inlined into code
// built with -mno-amdgpu-ieee (mismatched function attributes); as calls they return the
// workgroup index in a VGPR, so everything derived from it would be computed per lane.
__device__ __forceinline__ int lane_thread_id() { return (int)__builtin_amdgcn_workitem_id_x(); }
__device__ __forceinline__ int workgroup_id() { return (int)__builtin_amdgcn_workgroup_id_x(); }
// index of this wave in its workgroup, as a wave-uniform (scalar) value
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(lane_thread_id() >> 6);
}

// Grid order over units (a batch and head, or head group) and their tiles. The 8 XCDs are
// dealt workgroups round-robin (workgroup L to XCD L % 8), so unit r = x (mod 8) stays on XCD
// x and its K, V, Q, dO lines are shared through that XCD's L2. With grp > 0 an XCD works
// through its units grp at a time, tile index slowest within the group, so that the tiles
// of a unit run together and find its lines still in L2 (4 MB per XCD); grp = 0 takes all
// of the XCD's units at once (r = L % n_units, tile = L / n_units). grp > 0 needs n_units to
// be a multiple of 8 grp. Tile 0 comes first; callers reverse it where the heaviest is last.
__host__ __device__ constexpr int xcd_group(int n_units) { return n_units % 32 == 0 ? 4 : 0; }
__device__ __forceinline__ void xcd_grid_item(int L, int n_units, int n_tiles, int grp, int& r,
                                              int& tile) {
  if (grp > 0) {
    const int m = L >> 3, per = n_tiles * grp;
    const int gi = m / per, w = m - gi * per;
    tile = w / grp;
    r = (L & 7) + 8 * (gi * grp + w % grp);
  } else {
    r = L % n_units;
    tile = L / n_units;
  }
}

// 32x32x16 bf16 matrix-core product, fp32 accumulate: acc += A(32x16) * B(16x32).
// Operand lane layout: lane l supplies row/column (l % 32) and the 8 k-values of
// k-half (l / 32). Result: lane l holds column (l % 32), rows
// 8*(r/4) + 4*(l/32) + (r%4) for r = 0..15.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// fp32 -> bf16, round to nearest even, two at a time (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// Race-check build (compiled with -DFA_SYNC_CHECK=1 into a separate library): every stage
// that reads a tile from LDS is preceded by a wait for all outstanding loads and LDS accesses
// of the wave and a workgroup barrier, so no read can overtake the direct-to-LDS loads or
// another wave's accesses whatever the hand-placed waits do. Its results must equal the
// release build's bit for bit. Every wave of a workgroup passes the same number of these
// points. In the release build this is nothing.
#ifndef FA_SYNC_CHECK
#define FA_SYNC_CHECK 0
#endif
__device__ __forceinline__ void sync_check() {
  if constexpr (FA_SYNC_CHECK != 0) {
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
  }
}

// Exchange with the lane 32 away (the other k-half of an MFMA operand).
__device__ __forceinline__ float swap_halves(float x) {
  return __shfl_xor(x, 32, 64);
}

}  // namespace fa
