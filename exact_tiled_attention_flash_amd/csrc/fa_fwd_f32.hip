// Attention forward in IEEE fp32 end to end: gfx950 kernel on the fp32 matrix cores.
//
// Same method and tiling as the bf16 kernel ("Lab 06 - Attention kernels",
// section 3: per key tile S, m' = max(m, rowmax S), P = exp(S - m'),
// acc <- acc exp(m - m') + P V, l <- l exp(m - m') + rowsum P; O = acc / l,
// LSE = m + log l). Products use v_mfma_f32_32x32x2_f32 (true fp32 inputs and
// accumulation, no reduced-precision path), and P stays fp32.
//
// Workgroup: 4 waves, 128 queries (32 per wave); key tiles of 32 through LDS,
// double-buffered. S^T = K Q^T puts one query per lane; for the P V product
// the S^T accumulator register r of lane l is exactly the B operand of k-step
// r, and the matching A operand is V[key(r, l/32)][d = l%32], read from a
// row-major V tile.

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kBlockM = 128;
constexpr int kBlockN = 32;

__device__ __forceinline__ f32x16 mfma32_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

template <int D>
struct TileF32 {
  static constexpr int pitch = D + 4;                        // floats per LDS row
  static constexpr int tileElems = kBlockN * pitch;
  static constexpr int stageElems = 2 * tileElems;           // K then V
  static constexpr int chunks = D / 4;                       // 16-byte chunks per row
  static constexpr int loads = kBlockN * chunks / kThreads;  // per thread, per tensor
  static_assert(loads * kThreads == kBlockN * chunks, "tile split");
};

template <int D>
__device__ __forceinline__ void load_kv(const float* __restrict__ Kh, const float* __restrict__ Vh,
                                        int k0, int T, int tid, f32x4 (&kr)[TileF32<D>::loads],
                                        f32x4 (&vr)[TileF32<D>::loads]) {
  using Tl = TileF32<D>;
#pragma unroll
  for (int i = 0; i < Tl::loads; ++i) {
    const int u = tid + i * kThreads;
    const int key = k0 + u / Tl::chunks;
    const size_t off = (size_t)key * D + (u % Tl::chunks) * 4;
    kr[i] = key < T ? *reinterpret_cast<const f32x4*>(Kh + off) : f32x4{};
    vr[i] = key < T ? *reinterpret_cast<const f32x4*>(Vh + off) : f32x4{};
  }
}

template <int D>
__device__ __forceinline__ void store_kv(float* __restrict__ stage, int tid,
                                         const f32x4 (&kr)[TileF32<D>::loads],
                                         const f32x4 (&vr)[TileF32<D>::loads]) {
  using Tl = TileF32<D>;
#pragma unroll
  for (int i = 0; i < Tl::loads; ++i) {
    const int u = tid + i * kThreads;
    const int off = (u / Tl::chunks) * Tl::pitch + (u % Tl::chunks) * 4;
    *reinterpret_cast<f32x4*>(stage + off) = kr[i];
    *reinterpret_cast<f32x4*>(stage + Tl::tileElems + off) = vr[i];
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int T, int BH, int nq, float c) {
  using Tl = TileF32<D>;
  constexpr int nD = D / 32;
  __shared__ __attribute__((aligned(16))) float smem[2 * Tl::stageElems];

  const int tid = lane_thread_id();
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int h = lane >> 5;

  const int L = workgroup_id();
  const int bh = L % BH;
  int qt = L / BH;
  if (CAUSAL) qt = nq - 1 - qt;
  const int q0 = qt * kBlockM;
  const int qw0 = q0 + wave * 32;
  const int qrow = qw0 + l32;

  const size_t base = (size_t)bh * T * D;
  const float* Kh = K + base;
  const float* Vh = V + base;

  // Q^T operand: lane holds Q[qrow][2*kk + h] for every k-step kk.
  float qf[D / 2];
#pragma unroll
  for (int kk = 0; kk < D / 2; ++kk)
    qf[kk] = qrow < T ? Q[base + (size_t)qrow * D + 2 * kk + h] : 0.f;

  const int kend = CAUSAL ? min(T, q0 + kBlockM) : T;
  const int ntiles = (kend + kBlockN - 1) / kBlockN;

  f32x16 acc[nD];
#pragma unroll
  for (int db = 0; db < nD; ++db) acc[db] = f32x16{};
  float m_run = kNegInf;
  float l_run = 0.f;

  f32x4 kr[Tl::loads], vr[Tl::loads];
  load_kv<D>(Kh, Vh, 0, T, tid, kr, vr);
  store_kv<D>(smem, tid, kr, vr);
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int k0 = j * kBlockN;
    const bool more = j + 1 < ntiles;
    if (more) load_kv<D>(Kh, Vh, k0 + kBlockN, T, tid, kr, vr);
    const float* Ks = smem + (j & 1) * Tl::stageElems;
    const float* Vs = Ks + Tl::tileElems;
    sync_check();

    if (!(CAUSAL && k0 > qw0 + 31)) {
      f32x16 s = f32x16{};
#pragma unroll
      for (int kk = 0; kk < D / 2; ++kk) s = mfma32_f32(Ks[l32 * Tl::pitch + 2 * kk + h], qf[kk], s);

      const bool need_mask = (k0 + kBlockN > T) || (CAUSAL && (k0 + kBlockN - 1 > qw0));
      uint32_t valid = 0xffffu;
      if (need_mask) {
        valid = 0u;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 8 * (r >> 2) + 4 * h + (r & 3);
          const bool v = key < T && (!CAUSAL || key <= qrow);
          valid |= (v ? 1u : 0u) << r;
          s[r] = v ? s[r] : kNegInf;
        }
      }
      float mx = kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
      mx = fmaxf(mx, swap_halves(mx));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = (m_run == kNegInf) ? 0.f : exp2_fast((m_run - m_use) * c);
      const float mc = m_use * c;
      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = exp2_fast(fmaf(s[r], c, -mc));
        if (need_mask) p = (valid >> r) & 1u ? p : 0.f;
        s[r] = p;
        psum += p;
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < nD; ++db) acc[db] *= alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r >> 2) + 4 * h + (r & 3);
#pragma unroll
        for (int db = 0; db < nD; ++db)
          acc[db] = mfma32_f32(Vs[key * Tl::pitch + db * 32 + l32], s[r], acc[db]);
      }
    }
    if (more) store_kv<D>(smem + ((j + 1) & 1) * Tl::stageElems, tid, kr, vr);
    __syncthreads();
  }

  const float l_tot = l_run + swap_halves(l_run);
  if (qrow < T) {
    const float inv = 1.0f / l_tot;
    float* orow = O + base + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < nD; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 w = {acc[db][4 * g] * inv, acc[db][4 * g + 1] * inv, acc[db][4 * g + 2] * inv,
                   acc[db][4 * g + 3] * inv};
        *reinterpret_cast<f32x4*>(orow + db * 32 + 8 * g + 4 * h) = w;
      }
    }
    if (h == 0) LSE[(size_t)bh * T + qrow] = (m_run * c + log2_fast(l_tot)) * kLn2;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a) {
  const int BH = a.B * a.H;
  const int nq = (a.T + kBlockM - 1) / kBlockM;
  const float c = a.scale * 1.44269504088896340736f;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3(nq * BH), dim3(kThreads), 0, a.stream,
                     static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                     static_cast<const float*>(a.v), static_cast<float*>(a.o), a.lse, a.T, BH,
                     nq, c);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a) {
  if (a.D == 64) return a.causal ? launch<64, true>(a) : launch<64, false>(a);
  return a.causal ? launch<128, true>(a) : launch<128, false>(a);
}

}  // namespace fa
