// Block-scaled E4M3 quantization of bf16 rows, for the FP8 Q K^T forward.
//
// Source: "Lab 06 - Attention kernels", "Stretch" list (E4M3 Q and K for the Q K^T product).
// The format and the scaling the pages leave open are fixed as follows. E4M3 is the OCP 8-bit
// format (sign, 4 exponent bits with bias 7, 3 mantissa bits, subnormals m/8 * 2^-6, largest
// finite 448). Every 32 consecutive elements of a row share one power-of-two scale: the block
// exponent e is the largest integer with amax * 2^e <= 448 (at most 127; 0 for an all-zero
// block), stored as the byte 127 - e; each element becomes the E4M3 value nearest to x * 2^e,
// ties to even, with the sign of x. Multiplying by 2^e is exact, so the codes depend on the
// inputs alone.
//
// gfx950 mapping: the kernel is bound by HBM (2 bytes read, 1 + 1/32 written per element).
// Each lane takes 8 consecutive elements (one 16-byte load, one 8-byte store); the 4 lanes of
// a block agree on its maximum with two exchanges. The rounding is integer work on the fp32
// bit pattern: no conversion instruction whose rounding or saturation could differ.

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kQThreads = 256;

// E4M3 code (without sign) of a in [0, 448], nearest value, ties to even.
__device__ __forceinline__ uint32_t e4m3_code(float a) {
  if (a < 0x1p-6f) return (uint32_t)__builtin_rintf(a * 512.f);   // subnormal grid 2^-9
  const uint32_t u = __float_as_uint(a);
  const uint32_t r = u + 0x7FFFFu + ((u >> 20) & 1u);             // round 23 -> 3 mantissa bits
  return (r >> 20) - 960u;                                         // rebias 127 -> 7
}

__global__ __launch_bounds__(kQThreads) void quantize_mxfp8_kernel(const uint16_t* __restrict__ x,
                                                                   uint8_t* __restrict__ codes,
                                                                   uint8_t* __restrict__ scales,
                                                                   int64_t n8) {
  const int64_t g = (int64_t)workgroup_id() * kQThreads + lane_thread_id();
  // groups of 4 lanes form a block: a lane past the end still takes part in the exchanges
  const bool live = g < n8;
  u32x4 w = {0u, 0u, 0u, 0u};
  if (live) w = *reinterpret_cast<const u32x4*>(x + 8 * g);
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  int e = 0;
  if (amax > 0.f) {
    // amax = mant * 2^p, mant in [0.5, 1): 448 = 0.875 * 2^9
    const int p = __builtin_amdgcn_frexp_expf(amax);
    const float mant = __builtin_amdgcn_frexp_mantf(amax);
    e = min((mant <= 0.875f ? 9 : 8) - p, 127);
  }
  uint32_t c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float y = __builtin_amdgcn_ldexpf(v[i], e);
    c[i] = e4m3_code(fminf(fabsf(y), 448.f)) | ((__float_as_uint(v[i]) >> 24) & 0x80u);
  }
  if (live) {
    const u32x2 out = {c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24),
                       c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24)};
    *reinterpret_cast<u32x2*>(codes + 8 * g) = out;
    if ((g & 3) == 0) scales[g >> 2] = (uint8_t)(127 - e);
  }
}

}  // namespace

hipError_t launch_quantize_mxfp8(const void* x, void* codes, void* scales, int64_t elems,
                                 hipStream_t stream) {
  const int64_t n8 = elems / 8;
  const int64_t blocks = (n8 + kQThreads - 1) / kQThreads;
  hipLaunchKernelGGL(quantize_mxfp8_kernel, dim3((unsigned)blocks), dim3(kQThreads), 0, stream,
                     static_cast<const uint16_t*>(x), static_cast<uint8_t*>(codes),
                     static_cast<uint8_t*>(scales), n8);
  return hipGetLastError();
}

}  // namespace fa
