// Attention backward in IEEE fp32 end to end: three gfx950 kernels on the fp32 matrix cores.
//
// Method: "Lab 06 - Attention kernels", section 4: P = exp(S - LSE) recomputed per tile from
// the saved LSE, dV = P^T dO, dP = dO V^T, dS = P * (dP - D) with D_i = rowsum(dO * O)_i,
// dQ = dS K scale, dK = dS^T Q scale; the causal mask is applied before the exponential as in
// the forward. The same two-kernel split as the bf16 backward (the page's "Stretch" list):
// key tiles outer for dK and dV, query tiles outer for dQ, so there are no atomics and the
// result is deterministic. Products are v_mfma_f32_32x32x2_f32 (fp32 inputs, fp32
// accumulation); P and dS stay fp32 (no reduced-precision operand anywhere).
//
//   bwd_pre_f32_kernel   D_i and LSE_i * log2(e) into the workspace
//   bwd_dkdv_f32_kernel  workgroup = 128 keys (32 per wave) of one (b, h); K and V of the
//                        wave's keys stay in registers as B operands; loops over 32-query
//                        tiles of Q, dO, LSE, D staged in LDS. S = Q K^T and dP = dO V^T
//                        put one key per lane (lane l: key l % 32; register r: query
//                        8 (r / 4) + 4 (l / 32) + r % 4 of the tile), which is the B-operand
//                        layout of dV^T += dO^T P and dK^T += Q^T dS at k-step r: their A
//                        operands are single dO / Q values read from the LDS tile.
//   bwd_dq_f32_kernel    workgroup = 128 queries (32 per wave); Q and dO in registers;
//                        loops over 32-key tiles of K and V in LDS; S^T = K Q^T and
//                        dP^T = V dO^T put one query per lane, the B-operand layout of
//                        dQ^T += K^T dS^T.
// Tiles are loaded with plain 16-byte global loads into registers one tile ahead and written
// to LDS after the current tile's products (rows at or past T are written as zeros).

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 32;           // rows per staged tile (queries or keys)
constexpr int kRowsPerWG = 128;     // keys (dK/dV) or queries (dQ) per workgroup
constexpr float kLog2e = 1.44269504088896340736f;

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------------ D_i, LSE_i * log2(e)
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_pre_f32_kernel(const float* __restrict__ O,
                                                               const float* __restrict__ dO,
                                                               const float* __restrict__ LSE,
                                                               float* __restrict__ Dv,
                                                               float* __restrict__ L2,
                                                               int64_t rows) {
  constexpr int LPR = D / 4;             // lanes per row, one 16-byte chunk each
  constexpr int RPB = kThreads / LPR;    // rows per workgroup
  const int64_t row = (int64_t)workgroup_id() * RPB + lane_thread_id() / LPR;
  const int ch = lane_thread_id() % LPR;
  float s = 0.f;
  if (row < rows) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(O + row * D + ch * 4);
    const f32x4 b = *reinterpret_cast<const f32x4*>(dO + row * D + ch * 4);
    s = a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3];
  }
#pragma unroll
  for (int off = LPR / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  if (ch == 0 && row < rows) {
    Dv[row] = s;
    L2[row] = LSE[row] * kLog2e;
  }
}

// A [32 x D] fp32 tile in LDS with a row pitch of D + 2 floats: the 4-byte operand reads
// (lane l: row l % 32, column 2 kk + l / 32) fall on 64 distinct banks.
template <int D>
struct TileF32 {
  static constexpr int pitch = D + 2;
  static constexpr int elems = kTile * pitch;
  static constexpr int chunks = D / 4;                       // 16-byte chunks per row
  static constexpr int loads = kTile * chunks / kThreads;    // per thread
  static_assert(loads * kThreads == kTile * chunks, "tile split");
};

// rows [r0, r0 + 32) of a (T x D) matrix into registers; rows at or past T as zeros
template <int D>
__device__ __forceinline__ void load_tile(const float* __restrict__ src, int r0, int T, int tid,
                                          f32x4 (&x)[TileF32<D>::loads]) {
  using Tl = TileF32<D>;
#pragma unroll
  for (int i = 0; i < Tl::loads; ++i) {
    const int u = tid + i * kThreads;
    const int row = r0 + u / Tl::chunks;
    x[i] = row < T ? *reinterpret_cast<const f32x4*>(src + (size_t)row * D + (u % Tl::chunks) * 4)
                   : f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

template <int D>
__device__ __forceinline__ void store_tile(float* __restrict__ dst, int tid,
                                           const f32x4 (&x)[TileF32<D>::loads]) {
  using Tl = TileF32<D>;
#pragma unroll
  for (int i = 0; i < Tl::loads; ++i) {
    const int u = tid + i * kThreads;
    float* p = dst + (u / Tl::chunks) * Tl::pitch + (u % Tl::chunks) * 4;   // 8-byte aligned
    *reinterpret_cast<f32x2*>(p) = f32x2{x[i][0], x[i][1]};
    *reinterpret_cast<f32x2*>(p + 2) = f32x2{x[i][2], x[i][3]};
  }
}

// Store a [32 rows x D] block held as D/32 accumulators whose lane l holds row l % 32 and whose
// register r holds column 32 db + 8 (r / 4) + 4 (l / 32) + r % 4, times mul.
template <int D>
__device__ __forceinline__ void store_cols(float* __restrict__ dst_row, const f32x16 (&acc)[D / 32],
                                           float mul, int h) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 w = {acc[db][4 * g] * mul, acc[db][4 * g + 1] * mul, acc[db][4 * g + 2] * mul,
                       acc[db][4 * g + 3] * mul};
      *reinterpret_cast<f32x4*>(dst_row + db * 32 + 8 * g + 4 * h) = w;
    }
  }
}

// ------------------------------------------------------------------ dK, dV
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ Dv, const float* __restrict__ L2,
    float* __restrict__ dK, float* __restrict__ dV, int T, int BH, float c, float scale) {
  using Tl = TileF32<D>;
  constexpr int nD = D / 32;
  constexpr int nK = D / 2;                          // k-steps of S and dP
  constexpr int stage = 2 * Tl::elems + 2 * kTile;   // Q tile, dO tile, L2, D
  __shared__ __attribute__((aligned(16))) float smem[2 * stage];

  const int tid = lane_thread_id();
  const int wave = wave_id();
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int h = lane >> 5;

  const int L = workgroup_id();
  const int bh = L % BH;
  const int k0 = (L / BH) * kRowsPerWG;
  const int kw0 = k0 + wave * 32;
  const int key = kw0 + l32;
  const size_t base = (size_t)bh * T * D;
  const size_t rbase = (size_t)bh * T;

  // K^T and V^T B operands: lane holds K[key][2 kk + h] for every k-step kk
  float kf[nK], vf[nK];
#pragma unroll
  for (int kk = 0; kk < nK; ++kk) {
    kf[kk] = key < T ? K[base + (size_t)key * D + 2 * kk + h] : 0.f;
    vf[kk] = key < T ? V[base + (size_t)key * D + 2 * kk + h] : 0.f;
  }
  f32x16 dk[nD], dv[nD];
#pragma unroll
  for (int db = 0; db < nD; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  const int nqt = (T + kTile - 1) / kTile;
  const int qt0 = CAUSAL ? k0 / kTile : 0;
  f32x4 qr[Tl::loads], dr[Tl::loads];
  float l2r = 0.f, dvr = 0.f;
  auto fetch = [&](int qt) {
    load_tile<D>(Q + base, qt * kTile, T, tid, qr);
    load_tile<D>(dO + base, qt * kTile, T, tid, dr);
    if (tid < kTile) {
      const int q = qt * kTile + tid;
      l2r = q < T ? L2[rbase + q] : 0.f;
      dvr = q < T ? Dv[rbase + q] : 0.f;
    }
  };
  auto put = [&](float* st) {
    store_tile<D>(st, tid, qr);
    store_tile<D>(st + Tl::elems, tid, dr);
    if (tid < kTile) {
      st[2 * Tl::elems + tid] = l2r;
      st[2 * Tl::elems + kTile + tid] = dvr;
    }
  };
  if (qt0 < nqt) {
    fetch(qt0);
    put(smem);
  }
  __syncthreads();

  for (int qt = qt0; qt < nqt; ++qt) {
    const int it = qt - qt0;
    const bool more = qt + 1 < nqt;
    sync_check();
    if (more) fetch(qt + 1);
    const float* st = smem + (it & 1) * stage;
    const float* Qs = st;
    const float* dOs = st + Tl::elems;
    const float* l2s = st + 2 * Tl::elems;
    const float* dvs = l2s + kTile;
    const int q0 = qt * kTile;
    // a tile whose queries all come before this wave's keys contributes nothing (causal)
    if (!(CAUSAL && q0 + kTile - 1 < kw0)) {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int kk = 0; kk < nK; ++kk) {
        s = mfma_f32(Qs[l32 * Tl::pitch + 2 * kk + h], kf[kk], s);
        dp = mfma_f32(dOs[l32 * Tl::pitch + 2 * kk + h], vf[kk], dp);
      }
      // register r: query q0 + qr(r), qr(r) = 8 (r / 4) + 4 h + r % 4
      float p[16], ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = 8 * (r >> 2) + 4 * h + (r & 3);
        const int q = q0 + qi;
        const bool ok = q < T && (!CAUSAL || key <= q);
        const float pv = ok ? exp2_fast(fmaf(s[r], c, -l2s[qi])) : 0.f;
        p[r] = pv;
        ds[r] = pv * (dp[r] - dvs[qi]);
      }
      // dV^T[d][key] += sum_q dO[q][d] P[q][key], dK^T likewise with Q and dS; k-step r
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = 8 * (r >> 2) + 4 * h + (r & 3);
#pragma unroll
        for (int db = 0; db < nD; ++db) {
          dv[db] = mfma_f32(dOs[qi * Tl::pitch + db * 32 + l32], p[r], dv[db]);
          dk[db] = mfma_f32(Qs[qi * Tl::pitch + db * 32 + l32], ds[r], dk[db]);
        }
      }
    }
    if (more) put(smem + ((it + 1) & 1) * stage);
    __syncthreads();
  }

  // lane l holds key l % 32 and columns 32 db + 8 (r / 4) + 4 h + r % 4 of dK^T, dV^T
  if (key < T) {
    store_cols<D>(dV + base + (size_t)key * D, dv, 1.0f, h);
    store_cols<D>(dK + base + (size_t)key * D, dk, scale, h);
  }
}

// ------------------------------------------------------------------ dQ
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void bwd_dq_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ Dv, const float* __restrict__ L2,
    float* __restrict__ dQ, int T, int BH, int nq, float c, float scale) {
  using Tl = TileF32<D>;
  constexpr int nD = D / 32;
  constexpr int nK = D / 2;
  constexpr int stage = 2 * Tl::elems;   // K tile, then V tile
  __shared__ __attribute__((aligned(16))) float smem[2 * stage];

  const int tid = lane_thread_id();
  const int wave = wave_id();
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int h = lane >> 5;

  const int L = workgroup_id();
  const int bh = L % BH;
  int qt = L / BH;
  if (CAUSAL) qt = nq - 1 - qt;   // longest key range first
  const int q0 = qt * kRowsPerWG;
  const int qw0 = q0 + wave * 32;
  const int qrow = qw0 + l32;
  const size_t base = (size_t)bh * T * D;

  float qf[nK], df[nK];
#pragma unroll
  for (int kk = 0; kk < nK; ++kk) {
    qf[kk] = qrow < T ? Q[base + (size_t)qrow * D + 2 * kk + h] : 0.f;
    df[kk] = qrow < T ? dO[base + (size_t)qrow * D + 2 * kk + h] : 0.f;
  }
  const float l2 = qrow < T ? L2[(size_t)bh * T + qrow] : 0.f;
  const float dval = qrow < T ? Dv[(size_t)bh * T + qrow] : 0.f;
  f32x16 dq[nD];
#pragma unroll
  for (int db = 0; db < nD; ++db) dq[db] = f32x16{};

  const int kend = CAUSAL ? min(T, q0 + kRowsPerWG) : T;
  const int ntiles = (kend + kTile - 1) / kTile;
  f32x4 kr[Tl::loads], vr[Tl::loads];
  load_tile<D>(K + base, 0, T, tid, kr);
  load_tile<D>(V + base, 0, T, tid, vr);
  store_tile<D>(smem, tid, kr);
  store_tile<D>(smem + Tl::elems, tid, vr);
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const bool more = j + 1 < ntiles;
    sync_check();
    if (more) {
      load_tile<D>(K + base, (j + 1) * kTile, T, tid, kr);
      load_tile<D>(V + base, (j + 1) * kTile, T, tid, vr);
    }
    const float* Ks = smem + (j & 1) * stage;
    const float* Vs = Ks + Tl::elems;
    const int k0 = j * kTile;
    if (!(CAUSAL && k0 > qw0 + 31)) {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int kk = 0; kk < nK; ++kk) {
        s = mfma_f32(Ks[l32 * Tl::pitch + 2 * kk + h], qf[kk], s);
        dp = mfma_f32(Vs[l32 * Tl::pitch + 2 * kk + h], df[kk], dp);
      }
      // register r: key k0 + kr(r), kr(r) = 8 (r / 4) + 4 h + r % 4; lane: query qrow
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kj = k0 + 8 * (r >> 2) + 4 * h + (r & 3);
        const bool ok = kj < T && (!CAUSAL || kj <= qrow);
        const float pv = ok ? exp2_fast(fmaf(s[r], c, -l2)) : 0.f;
        ds[r] = pv * (dp[r] - dval);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ki = 8 * (r >> 2) + 4 * h + (r & 3);
#pragma unroll
        for (int db = 0; db < nD; ++db)
          dq[db] = mfma_f32(Ks[ki * Tl::pitch + db * 32 + l32], ds[r], dq[db]);
      }
    }
    if (more) {
      float* nx = smem + ((j + 1) & 1) * stage;
      store_tile<D>(nx, tid, kr);
      store_tile<D>(nx + Tl::elems, tid, vr);
    }
    __syncthreads();
  }

  if (qrow < T) store_cols<D>(dQ + base + (size_t)qrow * D, dq, scale, h);
}

template <int D, bool CAUSAL>
hipError_t launch(const BwdArgs& a) {
  const int BH = a.B * a.H;
  const float c = a.scale * kLog2e;
  const int64_t rows = (int64_t)BH * a.T;
  const float* q = static_cast<const float*>(a.q);
  const float* k = static_cast<const float*>(a.k);
  const float* v = static_cast<const float*>(a.v);
  const float* o = static_cast<const float*>(a.o);
  const float* dout = static_cast<const float*>(a.dout);
  float* dvec = a.delta;
  float* lse2 = a.delta + rows;
  constexpr int rpb = kThreads / (D / 4);
  hipLaunchKernelGGL((bwd_pre_f32_kernel<D>), dim3((unsigned)((rows + rpb - 1) / rpb)),
                     dim3(kThreads), 0, a.stream, o, dout, a.lse, dvec, lse2, rows);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  const int nk = (a.T + kRowsPerWG - 1) / kRowsPerWG;
  hipLaunchKernelGGL((bwd_dkdv_f32_kernel<D, CAUSAL>), dim3(nk * BH), dim3(kThreads), 0, a.stream,
                     q, k, v, dout, dvec, lse2, static_cast<float*>(a.dk),
                     static_cast<float*>(a.dv), a.T, BH, c, a.scale);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  const int nq = (a.T + kRowsPerWG - 1) / kRowsPerWG;
  hipLaunchKernelGGL((bwd_dq_f32_kernel<D, CAUSAL>), dim3(nq * BH), dim3(kThreads), 0, a.stream,
                     q, k, v, dout, dvec, lse2, static_cast<float*>(a.dq), a.T, BH, nq, c,
                     a.scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_f32(const BwdArgs& a) {
  if (a.D == 64) return a.causal ? launch<64, true>(a) : launch<64, false>(a);
  return a.causal ? launch<128, true>(a) : launch<128, false>(a);
}

}  // namespace fa
