// Attention forward, bf16 storage, fp32 accumulation: hand-written gfx950 kernel.
//
// Method: "Lab 06 - Attention kernels", section 3 (per query tile keep the
// row max m, row sum l and accumulator acc; per key tile rescale by
// exp(m - m') and add exp(S - m') V; finish with O = acc / l and
// LSE = m + log l; causal tiles above the diagonal are never loaded and only
// diagonal tiles are masked element-wise) and section 5 (one program per
// (query tile, batch*head)). "Triton FlashAttention-2 forward", "The kernel"
// (queries outermost, P rounded to the input dtype before the P V product,
// row sums in fp32, masked loads read zeros beyond T). Section 2 of the lab
// page notes that subtracting any constant from the exponents and
// multiplying back is exact; this kernel uses that freedom (see "lazy
// rescale" below).
//
// gfx950 mapping
//   * Workgroup: 256 threads = 4 waves, one per SIMD; 256 queries of one
//     (b, h), 64 per wave as two 32-query blocks. Every K / V operand read
//     from LDS feeds two matrix-core products (one per query block), which
//     halves LDS traffic per flop compared with 32 queries per wave; LDS
//     bandwidth (128 B/clk/CU) is the limiter otherwise.
//   * Key tiles of 64 are double-buffered in LDS; the global loads of tile
//     j+1 are in flight while tile j is computed. K and V are stored
//     row-major with padded pitches chosen for conflict-free reads.
//   * S^T = K Q^T (v_mfma_f32_32x32x16_bf16) puts one query per lane: a
//     row's 64 scores sit in 32 registers of lane l and 32 of lane l^32.
//     The S^T accumulator layout is the B-operand layout of O^T += V^T P^T,
//     so P never leaves registers. The V^T A operand comes straight from the
//     row-major V tile through the transposing LDS read (ds_read_b64_tr_b16):
//     within each 16-lane group, lane i addresses V[key0 + i/4][d0 + 4(i%4)]
//     and lane j receives V[key0 .. key0+3][d0 + j].
//   * exp(x) is exp2(x * scale * log2 e): one FMA and one v_exp_f32.
//   * Lazy rescale: a row's reference max is only moved (and acc, l
//     rescaled) when the new tile max exceeds it by more than 2^8 in the
//     exponent; otherwise P <= 2^8 is accumulated against the stale
//     reference. acc / l is unchanged by the choice of reference, and the
//     bound keeps every fp32 value far from overflow. The branch is taken
//     on the first tile and rarely afterwards.
//   * The loop over key tiles is split: tiles that need no mask run in a
//     lean main loop; the causal diagonal tiles and the ragged last tile
//     run in a masked tail, where fully hidden 32-query blocks are skipped.
//   * Causal grid order is heaviest query tile first; consecutive workgroup
//     ids walk (b, h) fastest, which keeps all tiles of one head on one XCD
//     (workgroups are dealt to the 8 XCDs round-robin) so K and V of a head
//     are shared through that XCD's L2.

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kBlockM = 256;   // queries per workgroup
constexpr int kBlockN = 64;    // keys per tile

typedef short s16x4 __attribute__((ext_vector_type(4)));

template <int D>
struct FwdTile {
  static constexpr int CH = D / 8;                      // 16-byte chunks per row
  static constexpr int RB = D * 2;                      // bytes per row (unpadded)
  static constexpr int tileBytes = kBlockN * RB;        // one K or V tile
  static constexpr int stageBytes = 2 * tileBytes;      // K tile, then V tile
  static constexpr int loadsPerWave = kBlockN * CH / kThreads;  // 16-byte loads per lane per tensor
  static_assert(loadsPerWave * kThreads == kBlockN * CH, "tile split");
  // XOR swizzle of the 16-byte chunks of a row. For D = 128 the row's low three bits go to
  // chunk bits 1-3 and row bit 3 to chunk bit 0: 16 consecutive rows reading one logical
  // chunk (the K operand) hit 16 different chunk positions, and the 8 rows x 4 chunks of a
  // transposing V read cover every chunk position exactly twice.
  __device__ static __forceinline__ int swz(int row) {
    return D == 128 ? (((row & 7) << 1) | ((row >> 3) & 1)) : ((row >> 1) & 7);
  }
  __device__ static __forceinline__ int offset(int row, int lchunk) {
    return row * RB + ((lchunk ^ swz(row)) << 4);
  }
};

typedef __attribute__((address_space(3))) void lds_void;

// Issue the direct global->LDS loads of key tile k0 (K and V) into `stage`.
// Lane `lane` of load i of wave `wave` fills LDS bytes [16 u, 16 u + 16) of
// the tile, u = (wave * loadsPerWave + i) * 64 + lane, i.e. physical chunk
// u % CH of row u / CH; it fetches the logical chunk that the swizzle maps
// there. Rows at or beyond T are clamped to row T - 1: such keys are masked
// out of S and their V rows only ever meet P = 0.
template <int D>
__device__ __forceinline__ void issue_kv(uint8_t* stage, const uint16_t* __restrict__ Kh,
                                         const uint16_t* __restrict__ Vh, int k0, int T,
                                         int wave, int lane) {
  using Tl = FwdTile<D>;
#pragma unroll
  for (int i = 0; i < Tl::loadsPerWave; ++i) {
    const int slot = wave * Tl::loadsPerWave + i;
    const int u = slot * 64 + lane;
    const int row = u / Tl::CH;
    const int lc = (u % Tl::CH) ^ Tl::swz(row);
    const size_t g = (size_t)min(k0 + row, T - 1) * D + lc * 8;
    __builtin_amdgcn_global_load_lds(Kh + g, (lds_void*)(stage + slot * 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(Vh + g, (lds_void*)(stage + Tl::tileBytes + slot * 1024), 16,
                                     0, 0);
  }
}

// A operand of O^T += V^T P^T for d rows [32 db, 32 db + 32) and keys 16 cc + {4h..4h+3,
// 8+4h..8+4h+3}: two transposing reads from the row-major (swizzled) V tile.
template <int D>
__device__ __forceinline__ bf16x8 v_operand(const uint8_t* Vs, int db, int cc, int lane) {
  using Tl = FwdTile<D>;
  const int g = lane >> 4, i = lane & 15;
  const int key = 16 * cc + 4 * (g >> 1) + (i >> 2);
  const int d0 = db * 32 + (g & 1) * 16 + 4 * (i & 3);
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(Vs + Tl::offset(key, d0 >> 3) + (d0 & 7) * 2));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(Vs + Tl::offset(key + 8, d0 >> 3) + (d0 & 7) * 2));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE,
    int T, int BH, int nq, float c) {
  using Tl = FwdTile<D>;
  constexpr int nD = D / 32;   // 32-row blocks of O^T
  constexpr int nK = D / 16;   // k-steps of S^T
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * Tl::stageBytes];

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
  const int qw0 = q0 + wave * 64;

  const size_t base = (size_t)bh * T * D;
  const uint16_t* Qh = Q + base;
  const uint16_t* Kh = K + base;
  const uint16_t* Vh = V + base;

  // Q^T fragments stay in registers: query block qb, lane holds query qw0 + 32 qb + l32,
  // d = 16 kk + 8 h + 0..7.
  bf16x8 qf[2][nK];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qrow = qw0 + 32 * qb + l32;
#pragma unroll
    for (int kk = 0; kk < nK; ++kk) {
      u32x4 x = qrow < T ? *reinterpret_cast<const u32x4*>(Qh + (size_t)qrow * D + kk * 16 + h * 8)
                         : u32x4{0u, 0u, 0u, 0u};
      qf[qb][kk] = as_bf16x8(x);
    }
  }

  const int kend = CAUSAL ? min(T, q0 + kBlockM) : T;
  const int ntiles = (kend + kBlockN - 1) / kBlockN;
  // tiles [0, nfull) need no mask for any query of this workgroup
  int nfull = (CAUSAL ? min(q0, T) : T) / kBlockN;
  nfull = min(nfull, ntiles);

  f32x16 acc[2][nD];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < nD; ++db) acc[qb][db] = f32x16{};
  float m_ref[2] = {kNegInf, kNegInf};   // running row max (raw score units)
  float l_run[2] = {0.f, 0.f};           // partial row sums over this lane's key half

  issue_kv<D>(smem, Kh, Vh, 0, T, wave, lane);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // Scores -> probabilities for one 32-query block; returns P^T as 4 bf16 B operands.
  auto softmax_block = [&](f32x16 (&s)[2], int qb, bool masked, int k0, bf16x8 (&p)[4]) {
    const int qrow = qw0 + 32 * qb + l32;
    uint32_t valid = 0xffffffffu;
    if (masked) {
      valid = 0u;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
          const bool ok = key < T && (!CAUSAL || key <= qrow);
          valid |= (ok ? 1u : 0u) << (16 * kb + r);
          s[kb][r] = ok ? s[kb][r] : kNegInf;
        }
    }
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; r += 2)
      mx = fmaxf(mx, fmaxf(fmaxf(s[0][r], s[0][r + 1]), fmaxf(s[1][r], s[1][r + 1])));
    mx = fmaxf(mx, swap_halves(mx));
    const float m_old = m_ref[qb];
    const float m_new = fmaxf(m_old, mx);
    // alpha = exp(m_old - m_new) (1 when the max did not move, 0 on the row's first tile)
    const float alpha = (m_old == kNegInf) ? 0.f : exp2_fast((m_old - m_new) * c);
    m_ref[qb] = m_new;
    l_run[qb] *= alpha;
#pragma unroll
    for (int db = 0; db < nD; ++db) acc[qb][db] *= alpha;
    const float mc = (m_new == kNegInf ? 0.f : m_new) * c;
    float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float e = exp2_fast(fmaf(s[kb][r], c, -mc));
        if (masked) e = (valid >> (16 * kb + r)) & 1u ? e : 0.f;
        s[kb][r] = e;
      }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      ps0 += s[0][r];
      ps1 += s[1][r];
    }
    l_run[qb] += ps0 + ps1;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const f32x16& sv = s[cc >> 1];
      const int o = (cc & 1) * 8;
      u32x4 w = {pack_bf16x2(sv[o + 0], sv[o + 1]), pack_bf16x2(sv[o + 2], sv[o + 3]),
                 pack_bf16x2(sv[o + 4], sv[o + 5]), pack_bf16x2(sv[o + 6], sv[o + 7])};
      p[cc] = as_bf16x8(w);
    }
  };

  auto tile = [&](int j, bool masked) {
    const int k0 = j * kBlockN;
    const bool more = j + 1 < ntiles;
    if (more) issue_kv<D>(smem + ((j + 1) & 1) * Tl::stageBytes, Kh, Vh, k0 + kBlockN, T, wave, lane);
    const uint8_t* Ks = smem + (j & 1) * Tl::stageBytes;
    const uint8_t* Vs = Ks + Tl::tileBytes;
    // which 32-query blocks of this wave see any key of the tile
    const bool act0 = !masked || !CAUSAL || k0 <= qw0 + 31;
    const bool act1 = !masked || !CAUSAL || k0 <= qw0 + 63;
    if (act1) {
      f32x16 s0[2] = {f32x16{}, f32x16{}}, s1[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int kk = 0; kk < nK; ++kk) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 a = as_bf16x8(
              *reinterpret_cast<const u32x4*>(Ks + Tl::offset(kb * 32 + l32, 2 * kk + h)));
          if (act0) s0[kb] = mfma32(a, qf[0][kk], s0[kb]);
          s1[kb] = mfma32(a, qf[1][kk], s1[kb]);
        }
      }
      bf16x8 p0[4], p1[4];
      const bool mask0 = masked && (k0 + kBlockN > T || (CAUSAL && k0 + kBlockN - 1 > qw0));
      const bool mask1 = masked && (k0 + kBlockN > T || (CAUSAL && k0 + kBlockN - 1 > qw0 + 32));
      if (act0) softmax_block(s0, 0, mask0, k0, p0);
      softmax_block(s1, 1, mask1, k0, p1);
#pragma unroll
      for (int db = 0; db < nD; ++db) {
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          const bf16x8 a = v_operand<D>(Vs, db, cc, lane);
          if (act0) acc[0][db] = mfma32(a, p0[cc], acc[0][db]);
          acc[1][db] = mfma32(a, p1[cc], acc[1][db]);
        }
      }
    }
    // the next tile's loads (this wave's) have landed; the barrier makes every
    // wave's part visible and frees this stage for the loads of tile j + 2
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  for (int j = 0; j < nfull; ++j) tile(j, false);
  for (int j = nfull; j < ntiles; ++j) tile(j, true);

#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qrow = qw0 + 32 * qb + l32;
    const float l_tot = l_run[qb] + swap_halves(l_run[qb]);
    if (qrow < T) {
      const float inv = 1.0f / l_tot;
      uint16_t* orow = O + base + (size_t)qrow * D;
#pragma unroll
      for (int db = 0; db < nD; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = db * 32 + 8 * g + 4 * h;
          u32x2 w = {pack_bf16x2(acc[qb][db][4 * g] * inv, acc[qb][db][4 * g + 1] * inv),
                     pack_bf16x2(acc[qb][db][4 * g + 2] * inv, acc[qb][db][4 * g + 3] * inv)};
          *reinterpret_cast<u32x2*>(orow + d0) = w;
        }
      }
      if (h == 0) LSE[(size_t)bh * T + qrow] = (m_ref[qb] * c + log2_fast(l_tot)) * kLn2;
    }
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
