// Attention backward, bf16 storage, fp32 accumulation: three hand-written gfx950 kernels.
//
// Method: "Lab 06 - Attention kernels", section 4: with P = exp(S - LSE) recomputed per tile
// from the saved LSE, dV = P^T dO, dP = dO V^T, dS = P * (dP - D) where D_i = rowsum(dO * O)_i
// (an O(T d) pass instead of a reduction over P), dQ = dS K scale and dK = dS^T Q scale; the
// causal mask is applied before the exponential exactly as in the forward ("Common bugs").
// Work split per the page's "Stretch" list: one kernel with key tiles outer (dK, dV
// accumulate in registers) and one with query tiles outer (dQ accumulates in registers), so
// no atomics are needed and the result is deterministic.
//
//   bwd_pre_kernel   D_i = sum_d dO_id O_id and LSE_i * log2(e), into the workspace (HBM-bound)
//   bwd_dkdv_kernel  workgroup = 128 keys (32 per wave) of one (b, h); loops over 64-query
//                    tiles from the diagonal down. Per wave: S = Q K^T and dP = dO V^T with
//                    K, V held in registers (lane = key), then dV^T += dO^T P and
//                    dK^T += Q^T dS, whose A operands are transposing LDS reads of the
//                    row-major Q and dO tiles. The tile's two 32-query blocks run as one
//                    pipelined body: one block's exponentials under the other's products.
//   bwd_dq_kernel    workgroup = 128 queries (32 per wave); loops over 64-key tiles up to
//                    the diagonal. Per wave: S^T = K Q^T and dP^T = V dO^T with Q, dO in
//                    registers (lane = query), then dQ^T += K^T dS^T with K^T a transposing
//                    read of the row-major K tile. Two workgroups per compute unit; the
//                    dK/dV kernel runs two at D = 64 (239 registers a wave) and one at
//                    D = 128 (384: K, V, dK, dV for 32 keys stay in registers).
// Tiles reach LDS by direct buffer -> LDS loads (no staging registers; rows past T arrive as
// zeros), double-buffered and written as inline asm the compiler does not track; the
// accumulator layout of S / S^T doubles as the B-operand layout of the following product
// (k-slots permuted the same way for both operands), so P and dS never leave registers.

#include "fa_common.h"
#include "fa_launch.h"
#include "fa_swz.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr float kLog2e = 1.44269504088896340736f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) {
  return __builtin_bit_cast(float, w & 0xffff0000u);
}

// ------------------------------------------------------------------ D_i, LSE_i * log2(e)
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_pre_kernel(const uint16_t* __restrict__ O,
                                                           const uint16_t* __restrict__ dO,
                                                           const float* __restrict__ LSE,
                                                           float* __restrict__ Dv,
                                                           float* __restrict__ L2, int64_t rows) {
  constexpr int LPR = D / 8;             // lanes per row, one 16-byte chunk each
  constexpr int RPB = kThreads / LPR;    // rows per workgroup
  const int64_t row = (int64_t)workgroup_id() * RPB + lane_thread_id() / LPR;
  const int ch = lane_thread_id() % LPR;
  float s = 0.f;
  if (row < rows) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(O + row * D + ch * 8);
    const u32x4 b = *reinterpret_cast<const u32x4*>(dO + row * D + ch * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) s += bf16_lo(a[i]) * bf16_lo(b[i]) + bf16_hi(a[i]) * bf16_hi(b[i]);
  }
#pragma unroll
  for (int off = LPR / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  if (ch == 0 && row < rows) {
    Dv[row] = s;
    L2[row] = LSE[row] * kLog2e;
  }
}

// Store a 32 x D block held as D/32 accumulators (lane = row, registers = d).
template <int D>
__device__ __forceinline__ void store_rows_bf16(uint16_t* __restrict__ dst, const f32x16 (&acc)[D / 32],
                                                float mul, int h) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 w = {pack_bf16x2(acc[db][4 * g] * mul, acc[db][4 * g + 1] * mul),
                 pack_bf16x2(acc[db][4 * g + 2] * mul, acc[db][4 * g + 3] * mul)};
      *reinterpret_cast<u32x2*>(dst + db * 32 + 8 * g + 4 * h) = w;
    }
  }
}

// 64 fp32 values of rows [row0, row0 + 64) straight into LDS (rows at or past T: zeros); one
// wave. rsrc covers the T values of one (b, h).
__device__ __forceinline__ void issue_stats(uint8_t* dst, const i32x4& rsrc, int row0, int T,
                                            int lane) {
  buf_lds_dma<4>(dst, rsrc, (uint32_t)lane * 4u, (uint32_t)min(row0, T) * 4u);
}

// Products of the D = 128 dK/dV kernel with explicit register files: S and dP in VGPRs (the
// vector unit works on them), K and V operands and the dK, dV accumulators in AGPRs, which no
// vector instruction touches inside the loop (left to itself the compiler parks three of the
// eight accumulators in VGPRs and copies them through AGPRs around every product; at D = 64
// the explicit split costs more registers than it saves moves). The compiler does not see
// these as products, so the waits it would insert are explicit: pad() before the vector unit
// reads a product's result or a product reads a value the vector unit just wrote.
__device__ __forceinline__ void mfma_sv_first(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_sv(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_acc(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
}
// 20 wait states (more than a 32x32x16 product's result latency) in program order after x's
// last writer
__device__ __forceinline__ void pad(f32x16& x, f32x16& y) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(x), "+v"(y));
}
__device__ __forceinline__ void pad_b(bf16x8& x, bf16x8& y) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(x), "+v"(y));
}

// ------------------------------------------------------------------ dK, dV
constexpr int kKeysPerWG = 128;
constexpr int kQTile = 64;

template <int D>
struct DkdvStage {
  static constexpr int q = 0;
  static constexpr int dO = SwzTile<D>::bytes;
  static constexpr int lse2 = 2 * SwzTile<D>::bytes;
  static constexpr int dvec = lse2 + 4 * kQTile;
  static constexpr int bytes = dvec + 4 * kQTile;
  static_assert(bytes % 256 == 0, "stage alignment (one full pass over the LDS banks)");
};

// Two workgroups per compute unit at D = 64 (at most 256 registers a wave), one at D = 128.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, D == 64 ? 2 : 1) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ Dv, const float* __restrict__ L2,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int T, int BH, int grp, float c,
    float scale) {
  using St = DkdvStage<D>;
  constexpr int nD = D / 32;
  constexpr int nK = D / 16;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * St::bytes];

  const int tid = lane_thread_id();
  const int wave = wave_id();
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int h = lane >> 5;

  const int L = workgroup_id();
  int bh, kt;
  xcd_grid_item(L, BH, (T + kKeysPerWG - 1) / kKeysPerWG, grp, bh, kt);
  const int k0 = kt * kKeysPerWG;   // key tile 0 (the heaviest when causal) first
  const int kw0 = k0 + wave * 32;
  const int key = kw0 + l32;
  const size_t base = (size_t)bh * T * D;
  const size_t rbase = (size_t)bh * T;

  bf16x8 kf[nK], vf[nK];
#pragma unroll
  for (int kk = 0; kk < nK; ++kk) {
    const size_t off = base + (size_t)key * D + kk * 16 + h * 8;
    kf[kk] = as_bf16x8(key < T ? *reinterpret_cast<const u32x4*>(K + off) : u32x4{0u, 0u, 0u, 0u});
    vf[kk] = as_bf16x8(key < T ? *reinterpret_cast<const u32x4*>(V + off) : u32x4{0u, 0u, 0u, 0u});
  }

  f32x16 dk[nD], dv[nD];
#pragma unroll
  for (int db = 0; db < nD; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }
  constexpr bool kAsm = D == 128;   // explicit-register products (see mfma_sv)
  if constexpr (kAsm) {
#pragma unroll
    for (int kk = 0; kk < nK; ++kk) asm volatile("" : "+a"(kf[kk]), "+a"(vf[kk]));
#pragma unroll
    for (int db = 0; db < nD; ++db) asm volatile("" : "+a"(dk[db]), "+a"(dv[db]));
    asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
  }

  const int nqt = (T + kQTile - 1) / kQTile;
  const int qt0 = CAUSAL ? k0 / kQTile : 0;

  // The tile loads are untracked inline asm (see buf_lds_dma): the wait + barrier closing each
  // iteration retires them before the stage is read, and retires the stage's readers before
  // it is refilled.
  const BufTileLoader<D> ld(wave, lane);
  const uint32_t tbytes = (uint32_t)T * (uint32_t)D * 2u;
  const i32x4 Qr = rows_rsrc(Q + base, tbytes), dOr = rows_rsrc(dO + base, tbytes);
  const i32x4 Lr = rows_rsrc(L2 + rbase, (uint32_t)T * 4u), Dr = rows_rsrc(Dv + rbase, (uint32_t)T * 4u);
  auto fetch = [&](int qt, uint8_t* st) {
    const int q0 = qt * kQTile;
    ld.issue_all(st + St::q, Qr, q0, T);
    ld.issue_all(st + St::dO, dOr, q0, T);
    if (wave == 0) issue_stats(st + St::lse2, Lr, q0, T, lane);
    if (wave == 1) issue_stats(st + St::dvec, Dr, q0, T, lane);
  };

  fetch(qt0, smem);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int qt = qt0; qt < nqt; ++qt) {
    const int it = qt - qt0;
    sync_check();
    if (qt + 1 < nqt) fetch(qt + 1, smem + ((it + 1) & 1) * St::bytes);
    const uint8_t* st = smem + (it & 1) * St::bytes;
    const uint8_t* Qs = st + St::q;
    const uint8_t* dOs = st + St::dO;
    const float* lse2 = reinterpret_cast<const float*>(st + St::lse2);
    const float* dvec = reinterpret_cast<const float*>(st + St::dvec);
    const int q0 = qt * kQTile;

    // Both 32-query blocks in one pipelined body: block 0's scores are worked through under
    // block 1's S and dP products, and block 1's under block 0's dV and dK products. A block
    // wholly before this wave's keys (causal) runs masked and contributes zeros.
    bool nm[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qb0 = q0 + qb * 32;
      nm[qb] = (CAUSAL && qb0 < kw0 + 31) || (qb0 + 32 > T);
    }
    // s / dp hold S and dP, then P and dS in place
    f32x16 s[2], dp[2];
    f32x4 l4[2][4], d4[2][4];
    bf16x8 pb[2][2], dsb[2][2];
    // LSE and D of 4 queries (group g of block qb). At D = 64 each group is read from LDS two
    // steps before the step whose scores first need it, so that only a few are live at a time
    // (the kernel then fits 256 registers without spilling: 8-20 % faster); at D = 128 a
    // block's four groups are read at once (measured even either way).
    constexpr bool kStatsPerGroup = D == 64;
    auto stat_group = [&](int qb, int g) {
      l4[qb][g] = *reinterpret_cast<const f32x4*>(lse2 + qb * 32 + 8 * g + 4 * h);
      d4[qb][g] = *reinterpret_cast<const f32x4*>(dvec + qb * 32 + 8 * g + 4 * h);
    };
    auto stats = [&](int qb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) stat_group(qb, g);
    };
    // one score of block qb: P = exp2(S c - LSE log2 e), dS = P (dP - D); lane = key, register
    // r = query q0 + 32 qb + 8 (r / 4) + 4 h + (r % 4)
    auto item = [&](int qb, int r) {
      const int g = r >> 2, i = r & 3;
      float pv = exp2_fast(fmaf(s[qb][r], c, -l4[qb][g][i]));
      if (__builtin_expect(nm[qb], 0)) {   // masked code out of line: no taken branch per score
        const int qi = q0 + 32 * qb + 8 * g + 4 * h + i;
        const bool ok = qi < T && (!CAUSAL || key <= qi);
        pv = ok ? pv : 0.f;
      }
      s[qb][r] = pv;
      dp[qb][r] = pv * (dp[qb][r] - d4[qb][g][i]);
    };
    auto pack = [&](int qb, int cc) {
      pb[qb][cc] = pack8(s[qb], 8 * cc);
      dsb[qb][cc] = pack8(dp[qb], 8 * cc);
    };
    // S and dP of both blocks, product f = nK qb + kk; operands read two products ahead (left
    // to itself the compiler reads each one just before its product and waits out the LDS
    // latency)
    constexpr int nF = 2 * nK;
    constexpr int nT = 2 * nD;
    // steps: x < nF the S / dP products, then nF + t the dV / dK products; block 0's scores are
    // worked through in steps [nK, nF), block 1's in [nF, nF + nT)
    if constexpr (!kStatsPerGroup) stats(0);
    auto prefetch_stats = [&](int x) {
      if constexpr (!kStatsPerGroup) {
        if (x == nK / 2 + 2) stats(1);
        return;
      }
      int qb = -1, r0 = 0;
      if (x >= nK && x < nF) qb = 0, r0 = ((x - nK) * 16) / nK;
      if (x >= nF && x < nF + nT) qb = 1, r0 = ((x - nF) * 16) / nT;
      if (qb >= 0 && r0 % 4 == 0) stat_group(qb, r0 / 4);
    };
    bf16x8 qa[nF], da[nF];
    auto rd = [&](int f) {
      qa[f] = row_operand<D>(Qs, (f / nK) * 32 + l32, 2 * (f % nK) + h);
      da[f] = row_operand<D>(dOs, (f / nK) * 32 + l32, 2 * (f % nK) + h);
    };
    rd(0);
    rd(1);
#pragma unroll
    for (int f = 0; f < nF; ++f) {
      const int qb = f / nK, kk = f % nK;
      if (f + 2 < nF) rd(f + 2);
      if constexpr (kAsm) {
        if (kk == 0) {
          mfma_sv_first(s[qb], qa[f], kf[kk]);
          mfma_sv_first(dp[qb], da[f], vf[kk]);
        } else {
          mfma_sv(s[qb], qa[f], kf[kk]);
          mfma_sv(dp[qb], da[f], vf[kk]);
        }
      } else {
        if (kk == 0) {
          s[qb] = f32x16{};
          dp[qb] = f32x16{};
        }
        s[qb] = mfma32(qa[f], kf[kk], s[qb]);
        dp[qb] = mfma32(da[f], vf[kk], dp[qb]);
      }
      __builtin_amdgcn_sched_barrier(0);
      prefetch_stats(f + 2);
      if (kAsm && f == nK) pad(s[0], dp[0]);   // block 0's last products were one step back
      if (qb == 1) {
#pragma unroll
        for (int r = (kk * 16) / nK; r < ((kk + 1) * 16) / nK; ++r) item(0, r);
        if (kk == nK / 2 - 1) pack(0, 0);
        if (kk == nK - 1) pack(0, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // dV and dK of both blocks, product t = nT qb + 2 db + cc, transposed operands read two
    // products ahead
    sync_check();
    bf16x8 ta[2 * nT], tb[2 * nT];
    auto rdt = [&](int t) {
      const int qb = t / nT, tt = t % nT;
      ta[t] = tr_operand<D>(dOs, tt / 2, qb * 32 + 16 * (tt % 2), lane);
      tb[t] = tr_operand<D>(Qs, tt / 2, qb * 32 + 16 * (tt % 2), lane);
    };
    rdt(0);
    rdt(1);
#pragma unroll
    for (int t = 0; t < 2 * nT; ++t) {
      const int qb = t / nT, tt = t % nT, db = tt / 2, cc = tt % 2;
      if (t + 2 < 2 * nT) rdt(t + 2);
      if constexpr (kAsm) {
        if (t == 1) pad_b(pb[0][1], dsb[0][1]);        // packed in the last S step
        if (t == nT + 1) pad_b(pb[1][1], dsb[1][1]);   // packed one step back
        mfma_acc(dv[db], ta[t], pb[qb][cc]);
        mfma_acc(dk[db], tb[t], dsb[qb][cc]);
      } else {
        dv[db] = mfma32(ta[t], pb[qb][cc], dv[db]);
        dk[db] = mfma32(tb[t], dsb[qb][cc], dk[db]);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (kAsm && t == 0) pad(s[1], dp[1]);   // block 1's last products were in the last S step
      prefetch_stats(nF + t + 2);
      if (qb == 0) {
#pragma unroll
        for (int r = (tt * 16) / nT; r < ((tt + 1) * 16) / nT; ++r) item(1, r);
        if (tt == nT / 2 - 1) pack(1, 0);
        if (tt == nT - 1) pack(1, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  if constexpr (kAsm) {
#pragma unroll
    for (int db = 0; db < nD; ++db)
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+a"(dk[db]), "+a"(dv[db]));
  }
  if (key < T) {
    store_rows_bf16<D>(dV + base + (size_t)key * D, dv, 1.0f, h);
    store_rows_bf16<D>(dK + base + (size_t)key * D, dk, scale, h);
  }
}

// ------------------------------------------------------------------ dQ
constexpr int kQueriesPerWG = 128;
constexpr int kKTile = 64;

// At most 256 registers a wave (the kernel fits them without spilling), so two workgroups
// share each compute unit and each SIMD runs one wave's products under the other's vector
// work, as in the forward; 64 KB of LDS a workgroup.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ Dv, const float* __restrict__ L2,
    uint16_t* __restrict__ dQ, int T, int BH, int nq, int grp, float c, float scale) {
  using Tl = SwzTile<D>;
  constexpr int nD = D / 32;
  constexpr int nK = D / 16;
  constexpr int stageBytes = 2 * Tl::bytes;   // K tile, then V tile
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * stageBytes];

  const int tid = lane_thread_id();
  const int wave = wave_id();
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int h = lane >> 5;

  const int L = workgroup_id();
  int bh, qt;
  xcd_grid_item(L, BH, nq, grp, bh, qt);
  if (CAUSAL) qt = nq - 1 - qt;  // longest key range first
  const int q0 = qt * kQueriesPerWG;
  const int qw0 = q0 + wave * 32;
  const int qrow = qw0 + l32;
  const size_t base = (size_t)bh * T * D;

  bf16x8 qf[nK], dof[nK];
#pragma unroll
  for (int kk = 0; kk < nK; ++kk) {
    const size_t off = base + (size_t)qrow * D + kk * 16 + h * 8;
    qf[kk] = as_bf16x8(qrow < T ? *reinterpret_cast<const u32x4*>(Q + off) : u32x4{0u, 0u, 0u, 0u});
    dof[kk] = as_bf16x8(qrow < T ? *reinterpret_cast<const u32x4*>(dO + off) : u32x4{0u, 0u, 0u, 0u});
  }
  const float lse2 = qrow < T ? L2[(size_t)bh * T + qrow] : 0.f;
  const float dval = qrow < T ? Dv[(size_t)bh * T + qrow] : 0.f;

  f32x16 dq[nD];
#pragma unroll
  for (int db = 0; db < nD; ++db) dq[db] = f32x16{};

  const int kend = CAUSAL ? min(T, q0 + kQueriesPerWG) : T;
  const int ntiles = (kend + kKTile - 1) / kKTile;

  // untracked tile loads, retired by the wait + barrier closing each iteration
  const BufTileLoader<D> ld(wave, lane);
  const uint32_t tbytes = (uint32_t)T * (uint32_t)D * 2u;
  const i32x4 Kr = rows_rsrc(K + base, tbytes), Vr = rows_rsrc(V + base, tbytes);
  auto fetch = [&](int j, uint8_t* st) {
    ld.issue_all(st, Kr, j * kKTile, T);
    ld.issue_all(st + Tl::bytes, Vr, j * kKTile, T);
  };
  fetch(0, smem);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // One tile's products. A causal wave computes only the tiles that start at or before its
  // last query; the tiles after them it only helps load, in a loop of its own, so that no
  // branch around the products makes the compiler copy the dQ accumulators at the join.
  auto tile = [&](int j) {
    const int k0 = j * kKTile;
    const uint8_t* Ks = smem + (j & 1) * stageBytes;
    const uint8_t* Vs = Ks + Tl::bytes;
    f32x16 s[2], dp[2];
    // operand fragments are read two products ahead (f = nK kb + kk)
    constexpr int nF = 2 * nK;
    bf16x8 ka[nF], va[nF];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      ka[f] = row_operand<D>(Ks, (f / nK) * 32 + l32, 2 * (f % nK) + h);
      va[f] = row_operand<D>(Vs, (f / nK) * 32 + l32, 2 * (f % nK) + h);
    }
#pragma unroll
    for (int f = 0; f < nF; ++f) {
      const int kb = f / nK, kk = f % nK;
      if (f + 2 < nF) {
        ka[f + 2] = row_operand<D>(Ks, ((f + 2) / nK) * 32 + l32, 2 * ((f + 2) % nK) + h);
        va[f + 2] = row_operand<D>(Vs, ((f + 2) / nK) * 32 + l32, 2 * ((f + 2) % nK) + h);
      }
      if (kk == 0) {
        s[kb] = f32x16{};
        dp[kb] = f32x16{};
      }
      s[kb] = mfma32(ka[f], qf[kk], s[kb]);
      dp[kb] = mfma32(va[f], dof[kk], dp[kb]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // the first transposed K operands load under the softmax work below
    sync_check();
    constexpr int nT = 4 * nD;   // (db, cc), cc fastest
    bf16x8 ta[nT];
    ta[0] = tr_operand<D>(Ks, 0, 0, lane);
    ta[1] = tr_operand<D>(Ks, 0, 16, lane);
    // lane = query; register r of block kb = key k0 + 32 kb + 8*(r/4) + 4h + (r%4)
    const bool need_mask = (k0 + kKTile > T) || (CAUSAL && (k0 + kKTile - 1 > qw0));
    bf16x8 dsb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 ds;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pv = exp2_fast(fmaf(s[kb][r], c, -lse2));
        if (__builtin_expect(need_mask, 0)) {
          const int kj = k0 + 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3);
          const bool ok = kj < T && (!CAUSAL || kj <= qrow);
          pv = ok ? pv : 0.f;
        }
        ds[r] = pv * (dp[kb][r] - dval);
      }
      dsb[2 * kb] = pack8(ds, 0);
      dsb[2 * kb + 1] = pack8(ds, 8);
    }
#pragma unroll
    for (int t = 0; t < nT; ++t) {
      if (t + 2 < nT) ta[t + 2] = tr_operand<D>(Ks, (t + 2) / 4, 16 * ((t + 2) % 4), lane);
      dq[t / 4] = mfma32(ta[t], dsb[t % 4], dq[t / 4]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  const int ntw = CAUSAL ? min(ntiles, (qw0 + 31) / kKTile + 1) : ntiles;
  // (each iteration of either loop passes two race-check points, so the waves of a
  // workgroup stay in step there too)
  for (int j = 0; j < ntw; ++j) {
    sync_check();
    if (j + 1 < ntiles) fetch(j + 1, smem + ((j + 1) & 1) * stageBytes);
    tile(j);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  for (int j = ntw; j < ntiles; ++j) {
    sync_check();
    sync_check();
    if (j + 1 < ntiles) fetch(j + 1, smem + ((j + 1) & 1) * stageBytes);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  if (qrow < T) store_rows_bf16<D>(dQ + base + (size_t)qrow * D, dq, scale, h);
}

template <int D, bool CAUSAL>
hipError_t launch(const BwdArgs& a) {
  const int BH = a.B * a.H;
  const float c = a.scale * kLog2e;
  const int64_t rows = (int64_t)BH * a.T;
  const uint16_t* q = static_cast<const uint16_t*>(a.q);
  const uint16_t* k = static_cast<const uint16_t*>(a.k);
  const uint16_t* v = static_cast<const uint16_t*>(a.v);
  const uint16_t* o = static_cast<const uint16_t*>(a.o);
  const uint16_t* dout = static_cast<const uint16_t*>(a.dout);
  float* dvec = a.delta;
  float* lse2 = a.delta + rows;
  constexpr int rpb = kThreads / (D / 8);
  hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)((rows + rpb - 1) / rpb)), dim3(kThreads),
                     0, a.stream, o, dout, a.lse, dvec, lse2, rows);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  const int nk = (a.T + kKeysPerWG - 1) / kKeysPerWG;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3(nk * BH), dim3(kThreads), 0, a.stream, q, k,
                     v, dout, dvec, lse2, static_cast<uint16_t*>(a.dk), static_cast<uint16_t*>(a.dv),
                     a.T, BH, xcd_group(BH), c, a.scale);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  const int nq = (a.T + kQueriesPerWG - 1) / kQueriesPerWG;
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3(nq * BH), dim3(kThreads), 0, a.stream, q, k,
                     v, dout, dvec, lse2, static_cast<uint16_t*>(a.dq), a.T, BH, nq, xcd_group(BH), c,
                     a.scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a) {
  if (a.D == 64) return a.causal ? launch<64, true>(a) : launch<64, false>(a);
  return a.causal ? launch<128, true>(a) : launch<128, false>(a);
}

}  // namespace fa
