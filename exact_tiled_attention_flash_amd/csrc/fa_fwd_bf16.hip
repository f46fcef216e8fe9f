// Attention forward, bf16 storage, fp32 accumulation: hand-written gfx950 kernel.
//
// Method: "Lab 06 - Attention kernels", section 3 (per query tile keep the
// row max m, row sum l and accumulator acc; per key tile rescale by
// exp(m - m') and add exp(S - m') V; finish with O = acc / l and
// LSE = m + log l; causal tiles above the diagonal are never loaded and only
// diagonal tiles are masked element-wise) and section 5 (one program per
// (query tile, batch*head)). "Triton FlashAttention-2 forward", "The kernel"
// (queries outermost, P rounded to the input dtype before the P V product,
// row sums in fp32, masked loads read zeros beyond T).
//
// gfx950 mapping
//   * Workgroup: 256 threads = 4 waves; 128 queries (32 per wave) of one
//     (b, h). Key tiles of 64 are streamed through LDS, double-buffered: the
//     global loads of tile j+1 are in flight while tile j is computed.
//   * Each wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 so that
//     lane l owns query (l % 32): a row's 64 scores sit in 32 registers of
//     lane l and 32 of lane l^32, so the row max needs one cross-lane swap
//     and the row sum none until the end.
//   * The S^T accumulator layout is exactly the B-operand layout of
//     O^T += V^T P^T over 16-key chunks, so P never leaves registers; V is
//     stored transposed in LDS so the A operand is two 8-byte reads.
//   * exp(x) is evaluated as exp2(x * scale * log2 e) with one FMA.
//   * Causal grid order is heaviest query tile first; consecutive workgroup
//     ids walk the (b, h) index fastest, which keeps all tiles of one head on
//     one XCD (workgroups are dealt to the 8 XCDs round-robin) so K and V of
//     a head are shared through that XCD's L2.

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kBlockM = 128;
constexpr int kBlockN = 64;

template <int D>
struct FwdTile {
  static constexpr int kPitch = D + 8;          // LDS row pitch of K (bf16 elements)
  static constexpr int vPitch = kBlockN + 4;    // LDS row pitch of V^T
  static constexpr int kElems = kBlockN * kPitch;
  static constexpr int vElems = D * vPitch;
  static constexpr int stageElems = kElems + vElems;
  static constexpr int chunks = D / 8;                          // 16-byte chunks per row
  static constexpr int kLoads = kBlockN * chunks / kThreads;    // K chunks per thread
  static constexpr int vKeys = kBlockN * chunks / kThreads;     // keys per V unit
  static_assert(kLoads * kThreads == kBlockN * chunks, "K tile split");
  static_assert(vKeys == 2 || vKeys == 4, "V unit");
};

template <int D>
__device__ __forceinline__ void load_kv(const uint16_t* __restrict__ Kh,
                                        const uint16_t* __restrict__ Vh, int k0, int T,
                                        int tid, u32x4 (&kr)[FwdTile<D>::kLoads],
                                        u32x4 (&vr)[FwdTile<D>::vKeys]) {
  using Tl = FwdTile<D>;
#pragma unroll
  for (int i = 0; i < Tl::kLoads; ++i) {
    const int u = tid + i * kThreads;
    const int key = k0 + u / Tl::chunks;
    const int ch = u % Tl::chunks;
    kr[i] = key < T ? *reinterpret_cast<const u32x4*>(Kh + (size_t)key * D + ch * 8)
                    : u32x4{0u, 0u, 0u, 0u};
  }
  const int ch = tid % Tl::chunks;
  const int g = tid / Tl::chunks;
#pragma unroll
  for (int i = 0; i < Tl::vKeys; ++i) {
    const int key = k0 + g * Tl::vKeys + i;
    vr[i] = key < T ? *reinterpret_cast<const u32x4*>(Vh + (size_t)key * D + ch * 8)
                    : u32x4{0u, 0u, 0u, 0u};
  }
}

// bf16 element e (0..7) of a 16-byte chunk, moved to the low half of a dword.
__device__ __forceinline__ uint32_t elem_lo(const u32x4& x, int e) {
  const uint32_t w = x[e >> 1];
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

template <int D>
__device__ __forceinline__ void store_kv(uint16_t* __restrict__ stage, int tid,
                                         const u32x4 (&kr)[FwdTile<D>::kLoads],
                                         const u32x4 (&vr)[FwdTile<D>::vKeys]) {
  using Tl = FwdTile<D>;
  uint16_t* Ks = stage;
  uint16_t* Vt = stage + Tl::kElems;
#pragma unroll
  for (int i = 0; i < Tl::kLoads; ++i) {
    const int u = tid + i * kThreads;
    *reinterpret_cast<u32x4*>(Ks + (u / Tl::chunks) * Tl::kPitch + (u % Tl::chunks) * 8) = kr[i];
  }
  const int ch = tid % Tl::chunks;
  const int g = tid / Tl::chunks;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    uint16_t* dst = Vt + (ch * 8 + e) * Tl::vPitch + g * Tl::vKeys;
    if constexpr (Tl::vKeys == 4) {
      u32x2 w = {elem_lo(vr[0], e) | (elem_lo(vr[1], e) << 16),
                 elem_lo(vr[2], e) | (elem_lo(vr[3], e) << 16)};
      *reinterpret_cast<u32x2*>(dst) = w;
    } else {
      *reinterpret_cast<uint32_t*>(dst) = elem_lo(vr[0], e) | (elem_lo(vr[1], e) << 16);
    }
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE,
    int T, int BH, int nq, float c) {
  using Tl = FwdTile<D>;
  constexpr int nD = D / 32;   // 32-row blocks of O^T
  constexpr int nK = D / 16;   // k-steps of S^T
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * Tl::stageElems];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int h = lane >> 5;

  const int L = blockIdx.x;
  const int bh = L % BH;
  int qt = L / BH;
  if (CAUSAL) qt = nq - 1 - qt;
  const int q0 = qt * kBlockM;
  const int qw0 = q0 + wave * 32;
  const int qrow = qw0 + l32;

  const size_t base = (size_t)bh * T * D;
  const uint16_t* Qh = Q + base;
  const uint16_t* Kh = K + base;
  const uint16_t* Vh = V + base;

  // Q^T fragments stay in registers: lane holds query qrow, d = 16*kk + 8*h + 0..7.
  bf16x8 qf[nK];
#pragma unroll
  for (int kk = 0; kk < nK; ++kk) {
    u32x4 x = qrow < T ? *reinterpret_cast<const u32x4*>(Qh + (size_t)qrow * D + kk * 16 + h * 8)
                       : u32x4{0u, 0u, 0u, 0u};
    qf[kk] = as_bf16x8(x);
  }

  const int kend = CAUSAL ? min(T, q0 + kBlockM) : T;
  const int ntiles = (kend + kBlockN - 1) / kBlockN;

  f32x16 acc[nD];
#pragma unroll
  for (int db = 0; db < nD; ++db) acc[db] = f32x16{};
  float m_run = kNegInf;
  float l_run = 0.f;

  u32x4 kr[Tl::kLoads];
  u32x4 vr[Tl::vKeys];
  load_kv<D>(Kh, Vh, 0, T, tid, kr, vr);
  store_kv<D>(smem, tid, kr, vr);
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int k0 = j * kBlockN;
    const bool more = j + 1 < ntiles;
    if (more) load_kv<D>(Kh, Vh, k0 + kBlockN, T, tid, kr, vr);

    const uint16_t* Ks = smem + (j & 1) * Tl::stageElems;
    const uint16_t* Vt = Ks + Tl::kElems;
    const bool wave_skip = CAUSAL && (k0 > qw0 + 31);
    if (!wave_skip) {
      // S^T for keys k0 + [0, 32) and k0 + [32, 64)
      f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
      for (int kk = 0; kk < nK; ++kk) {
        const u32x4 a0 = *reinterpret_cast<const u32x4*>(Ks + l32 * Tl::kPitch + kk * 16 + h * 8);
        const u32x4 a1 =
            *reinterpret_cast<const u32x4*>(Ks + (32 + l32) * Tl::kPitch + kk * 16 + h * 8);
        s0 = mfma32(as_bf16x8(a0), qf[kk], s0);
        s1 = mfma32(as_bf16x8(a1), qf[kk], s1);
      }

      const bool need_mask = (k0 + kBlockN > T) || (CAUSAL && (k0 + kBlockN - 1 > qw0));
      uint32_t valid = 0xffffffffu;  // bit r: key of s0[r]; bit 16+r: key of s1[r]
      if (need_mask) {
        valid = 0u;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 8 * (r >> 2) + 4 * h + (r & 3);
          const bool v0 = key < T && (!CAUSAL || key <= qrow);
          const bool v1 = key + 32 < T && (!CAUSAL || key + 32 <= qrow);
          valid |= (v0 ? 1u : 0u) << r;
          valid |= (v1 ? 1u : 0u) << (16 + r);
          s0[r] = v0 ? s0[r] : kNegInf;
          s1[r] = v1 ? s1[r] : kNegInf;
        }
      }

      float mx = kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
      mx = fmaxf(mx, swap_halves(mx));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = (m_run == kNegInf) ? 0.f : exp2_fast((m_run - m_use) * c);
      const float mc = m_use * c;

      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s0[r] = exp2_fast(fmaf(s0[r], c, -mc));
        s1[r] = exp2_fast(fmaf(s1[r], c, -mc));
      }
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s0[r] = (valid >> r) & 1u ? s0[r] : 0.f;
          s1[r] = (valid >> (16 + r)) & 1u ? s1[r] : 0.f;
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) psum += s0[r] + s1[r];
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < nD; ++db) acc[db] *= alpha;

      // P^T in bf16: chunk cc covers keys k0 + 16*cc + {4h..4h+3, 8+4h..8+4h+3}
      bf16x8 p[4];
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const f32x16& s = (cc < 2) ? s0 : s1;
        const int o = (cc & 1) * 8;
        u32x4 w = {pack_bf16x2(s[o + 0], s[o + 1]), pack_bf16x2(s[o + 2], s[o + 3]),
                   pack_bf16x2(s[o + 4], s[o + 5]), pack_bf16x2(s[o + 6], s[o + 7])};
        p[cc] = as_bf16x8(w);
      }
#pragma unroll
      for (int db = 0; db < nD; ++db) {
        const uint16_t* vrow = Vt + (db * 32 + l32) * Tl::vPitch + 4 * h;
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + 16 * cc);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 16 * cc + 8);
          const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
          acc[db] = mfma32(as_bf16x8(a), p[cc], acc[db]);
        }
      }
    }

    if (more) store_kv<D>(smem + ((j + 1) & 1) * Tl::stageElems, tid, kr, vr);
    __syncthreads();
  }

  const float l_tot = l_run + swap_halves(l_run);
  if (qrow < T) {
    const float inv = 1.0f / l_tot;
    uint16_t* orow = O + base + (size_t)qrow * D;
#pragma unroll
    for (int db = 0; db < nD; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = db * 32 + 8 * g + 4 * h;
        u32x2 w = {pack_bf16x2(acc[db][4 * g] * inv, acc[db][4 * g + 1] * inv),
                   pack_bf16x2(acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + d0) = w;
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
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), dim3(nq * BH), dim3(kThreads), 0, a.stream,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.o), a.lse, a.T,
                     BH, nq, c);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a) {
  if (a.D == 64) return a.causal ? launch<64, true>(a) : launch<64, false>(a);
  return a.causal ? launch<128, true>(a) : launch<128, false>(a);
}

}  // namespace fa
