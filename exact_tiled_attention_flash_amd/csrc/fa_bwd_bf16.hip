// Attention backward, bf16 storage, fp32 accumulation: two hand-written gfx950 kernels.
//
// Method: "Lab 06 - Attention kernels", section 4: with P = exp(S - LSE) recomputed per tile
// from the saved LSE, dV = P^T dO, dP = dO V^T, dS = P * (dP - D) where D_i = rowsum(dO * O)_i
// (an O(T d) pass instead of a reduction over P), dQ = dS K scale and dK = dS^T Q scale; the
// causal mask is applied before the exponential exactly as in the forward ("Common bugs").
// Work split per the page's "Stretch" list: one kernel with key tiles outer (dK, dV
// accumulate in registers) and one with query tiles outer (dQ accumulates in registers), so
// no atomics are needed and the result is deterministic.
//
//   bwd_dkdv_kernel  (D = 64) workgroup = 128 keys (32 per wave) of one (b, h); loops over
//                    64-query tiles from the diagonal down. Per wave: S = Q K^T and dP = dO V^T
//                    with K, V held in registers (lane = key), then dV^T += dO^T P and
//                    dK^T += Q^T dS, whose A operands are transposing LDS reads of the
//                    row-major Q and dO tiles. The tile's two 32-query blocks run as one
//                    pipelined body: one block's exponentials under the other's products.
//   bwd_dkdv16_kernel (D = 128) the same with 16 keys a wave on 16 x 16 x 32 products, 64 keys
//                    a workgroup: K, V and the dK, dV accumulators of 32 keys would not leave
//                    room for two waves on a SIMD at D = 128, those of 16 keys do.
//   bwd_dq_kernel    runs first. Workgroup = 128 queries (32 per wave); it computes its rows'
//                    D_i = sum_d dO_id O_id and LSE_i * log2(e) from the dO it holds and one
//                    read of O, and writes them to the workspace for the dK/dV kernel; then
//                    loops over 64-key tiles up to the diagonal. Per wave: S^T = K Q^T and
//                    dP^T = V dO^T with Q, dO in registers (lane = query), then
//                    dQ^T += K^T dS^T with K^T a transposing read of the row-major K tile.
//   All the gradient kernels run two workgroups per compute unit (at most 256 registers a
//   wave).
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

// D = 64 (D = 128 runs bwd_dkdv16_kernel below): two workgroups per compute unit, at most 256
// registers a wave.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void bwd_dkdv_kernel(
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
  static_assert(D == 64, "D = 128 runs bwd_dkdv16_kernel");

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
      if (kk == 0) {
        s[qb] = f32x16{};
        dp[qb] = f32x16{};
      }
      s[qb] = mfma32(qa[f], kf[kk], s[qb]);
      dp[qb] = mfma32(da[f], vf[kk], dp[qb]);
      __builtin_amdgcn_sched_barrier(0);
      prefetch_stats(f + 2);
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
      dv[db] = mfma32(ta[t], pb[qb][cc], dv[db]);
      dk[db] = mfma32(tb[t], dsb[qb][cc], dk[db]);
      __builtin_amdgcn_sched_barrier(0);
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

  if (key < T) {
    store_rows_bf16<D>(dV + base + (size_t)key * D, dv, 1.0f, h);
    store_rows_bf16<D>(dK + base + (size_t)key * D, dk, scale, h);
  }
}

// ------------------------------------------------------------------ dK, dV with 16 keys a wave
// D = 128: a wave owns 16 keys, so that K and V (B operands, 16 registers each) and the dK^T,
// dV^T accumulators (8 blocks of 16 x 16, 32 registers each) leave room for two waves on every
// SIMD (at most 256 registers a wave): one wave's softmax work runs under the other's products,
// as in the forward and dQ kernels. Products are v_mfma_f32_16x16x32_bf16 (16 x 16 output,
// k = 32): A lane l supplies row l % 16, B lane l column l % 16, both the 8 k-values of lane group
// l / 16; the result's lane l holds column l % 16, rows 4 (l / 16) + i in register i.
//   S = Q K^T and dP = dO V^T per 16-query block qb: A = 16 bytes of Q (dO) row 16 qb + l % 16,
//     logical chunk 4 kk + l / 16 of the LDS tile; B = K (V) of key l % 16, the same 8 d-values.
//     Result: lane = key, register i = query 16 qb + 4 (l / 16) + i.
//   dV^T += dO^T P and dK^T += Q^T dS per 32-query chunk c: B = P (dS) of blocks 2c and 2c + 1
//     packed to bf16, so lane group g holds queries 32 c + 4 g + (0..3) and 32 c + 16 + 4 g + (0..3);
//     A = the same queries of dO (Q) at column d = 16 db + l % 16, two transposing reads.
constexpr int kKeysPerWG16 = 64;

template <bool B>
struct MaskTag {
  static constexpr bool value = B;
};
template <int P>
struct StageTag {
  static constexpr int value = P;
};

template <int D>
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void bwd_dkdv16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ Dv, const float* __restrict__ L2,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int T, int BH, int grp, float c,
    float scale) {
  static_assert(D == 128, "the 16-keys-a-wave schedule is laid out for D = 128");
  using Tl = SwzTileT<D>;   // Q and dO tiles: see SwzTileT
  using St = DkdvStage<D>;
  constexpr int nD = D / 16;   // 16-wide d blocks of dK^T, dV^T
  constexpr int nK = D / 32;   // k-steps of S and dP
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * St::bytes];

  const int tid = lane_thread_id();
  const int wave = wave_id();
  const int lane = tid & 63;
  const int j16 = lane & 15;
  const int g = lane >> 4;

  const int L = workgroup_id();
  int bh, kt;
  xcd_grid_item(L, BH, (T + kKeysPerWG16 - 1) / kKeysPerWG16, grp, bh, kt);
  const int k0 = kt * kKeysPerWG16;   // key tile 0 (the heaviest when causal) first
  const int kw0 = k0 + wave * 16;
  const int key = kw0 + j16;
  const size_t base = (size_t)bh * T * D;
  const size_t rbase = (size_t)bh * T;

  // B operands: K and V of this lane's key, d = 32 kk + 8 g + 0..7
  bf16x8 kf[nK], vf[nK];
#pragma unroll
  for (int kk = 0; kk < nK; ++kk) {
    const size_t off = base + (size_t)key * D + kk * 32 + g * 8;
    kf[kk] = as_bf16x8(key < T ? *reinterpret_cast<const u32x4*>(K + off) : u32x4{0u, 0u, 0u, 0u});
    vf[kk] = as_bf16x8(key < T ? *reinterpret_cast<const u32x4*>(V + off) : u32x4{0u, 0u, 0u, 0u});
  }
  f32x4 dk[nD], dv[nD];
#pragma unroll
  for (int db = 0; db < nD; ++db) {
    dk[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    dv[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // per-lane LDS offsets. Row-operand reads: row 16 qb + j16, logical chunk 4 kk + g (the swizzle
  // depends on row bits 0-3 only, so 16 qb is a constant offset). Transposing reads: lane i of
  // group g addresses row 4 g + i / 4 (+ 32 c + 16 hi, constant offsets), columns 16 db + 4 (i % 4).
  uint32_t roff[nK], toff[nD];
#pragma unroll
  for (int kk = 0; kk < nK; ++kk) roff[kk] = (uint32_t)Tl::offset(j16, 4 * kk + g);
  {
    const int row = 4 * g + (j16 >> 2);
#pragma unroll
    for (int db = 0; db < nD; ++db) {
      const int d0 = 16 * db + 4 * (j16 & 3);
      toff[db] = (uint32_t)(Tl::offset(row, d0 >> 3) + (d0 & 7) * 2);
    }
  }
  auto rowop = [&](const uint8_t* tile, int qb, int kk) {
    return as_bf16x8(*reinterpret_cast<const u32x4*>(tile + qb * 16 * Tl::RB + roff[kk]));
  };
  auto trop = [&](const uint8_t* tile, int cc, int db) {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const uint8_t* b0 = tile + cc * 32 * Tl::RB + toff[db];
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)b0);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(b0 + 16 * Tl::RB));
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
  };

  const int nqt = (T + kQTile - 1) / kQTile;
  const int qt0 = CAUSAL ? k0 / kQTile : 0;
  const BufTileLoader<D, Tl> ld(wave, lane);
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

  // One query tile. Steps are pinned with sched_barrier; operands are read two steps ahead.
  //   phase 1, steps f = 4 qb + kk (16): S and dP products of block qb; block qb - 1's
  //     exponentials and dS (one query row i = kk of the block per step) run under them
  //   phase 2, steps t = 8 cc + db (16): dV and dK products of chunk cc; block 3's softmax
  //     runs under steps 0-3 and its chunk is packed at step 4 (first used at step 8)
  // MASK: the tile may hold a query before one of this wave's keys (causal) or past T.
  auto tile = [&](int qt, auto par_tag, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr int PAR = decltype(par_tag)::value;   // stage of this tile, known at compile time
    sync_check();
    // the load destination stays a run-time offset: with a constant one this toolchain emits an
    // illegal null check on the cast of the LDS pointer inside the load helper
    if (qt + 1 < nqt) fetch(qt + 1, smem + ((qt - qt0 + 1) & 1) * St::bytes);
    const uint8_t* st = smem + PAR * St::bytes;
    const uint8_t* Qs = st + St::q;
    const uint8_t* dOs = st + St::dO;
    const float* lse2 = reinterpret_cast<const float*>(st + St::lse2);
    const float* dvec = reinterpret_cast<const float*>(st + St::dvec);
    const int q0 = qt * kQTile;

    f32x4 s[4], dp[4], l4[4], d4[4];
    bf16x8 pb[2], dsb[2];
    auto stats = [&](int qb) {
      l4[qb] = *reinterpret_cast<const f32x4*>(lse2 + 16 * qb + 4 * g);
      d4[qb] = *reinterpret_cast<const f32x4*>(dvec + 16 * qb + 4 * g);
    };
    // P = exp2(S c - LSE log2 e) and dS = P (dP - D) of row i of block qb (query
    // q0 + 16 qb + 4 g + i), in place
    auto item = [&](int qb, int i) {
      float pv = exp2_fast(fmaf(s[qb][i], c, -l4[qb][i]));
      if constexpr (MASK) {
        const int qi = q0 + 16 * qb + 4 * g + i;
        pv = (qi < T && (!CAUSAL || key <= qi)) ? pv : 0.f;
      }
      s[qb][i] = pv;
      dp[qb][i] = pv * (dp[qb][i] - d4[qb][i]);
    };
    auto pack = [&](int cc) {
      pb[cc] = as_bf16x8(u32x4{pack_bf16x2(s[2 * cc][0], s[2 * cc][1]),
                               pack_bf16x2(s[2 * cc][2], s[2 * cc][3]),
                               pack_bf16x2(s[2 * cc + 1][0], s[2 * cc + 1][1]),
                               pack_bf16x2(s[2 * cc + 1][2], s[2 * cc + 1][3])});
      dsb[cc] = as_bf16x8(u32x4{pack_bf16x2(dp[2 * cc][0], dp[2 * cc][1]),
                                pack_bf16x2(dp[2 * cc][2], dp[2 * cc][3]),
                                pack_bf16x2(dp[2 * cc + 1][0], dp[2 * cc + 1][1]),
                                pack_bf16x2(dp[2 * cc + 1][2], dp[2 * cc + 1][3])});
    };

    bf16x8 qa[16], da[16];
    auto rd1 = [&](int f) {
      qa[f] = rowop(Qs, f / nK, f % nK);
      da[f] = rowop(dOs, f / nK, f % nK);
    };
    rd1(0);
    rd1(1);
    stats(0);
#pragma unroll
    for (int f = 0; f < 4 * nK; ++f) {
      const int qb = f / nK, kk = f % nK;
      if (f + 2 < 4 * nK) rd1(f + 2);
      if (kk == 0) {
        s[qb] = mfma16<D>(qa[f], kf[kk], f32x4{0.f, 0.f, 0.f, 0.f});
        dp[qb] = mfma16<D>(da[f], vf[kk], f32x4{0.f, 0.f, 0.f, 0.f});
      } else {
        s[qb] = mfma16<D>(qa[f], kf[kk], s[qb]);
        dp[qb] = mfma16<D>(da[f], vf[kk], dp[qb]);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (kk == 0 && qb < 3) stats(qb + 1);
      if (qb > 0) item(qb - 1, kk);
      if (f == 3 * nK - 1) pack(0);   // block 1's last row was just done: chunk 0 complete
      __builtin_amdgcn_sched_barrier(0);
    }

    sync_check();
    bf16x8 ta[16], tb[16];
    auto rd2 = [&](int t) {
      ta[t] = trop(dOs, t / nD, t % nD);
      tb[t] = trop(Qs, t / nD, t % nD);
    };
    rd2(0);
    rd2(1);
#pragma unroll
    for (int t = 0; t < 2 * nD; ++t) {
      const int cc = t / nD, db = t % nD;
      if (t + 2 < 2 * nD) rd2(t + 2);
      dv[db] = mfma16<D>(ta[t], pb[cc], dv[db]);
      dk[db] = mfma16<D>(tb[t], dsb[cc], dk[db]);
      __builtin_amdgcn_sched_barrier(0);
      if (t < 4) item(3, t);
      if (t == 4) pack(1);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  fetch(qt0, smem);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // masked: the first tile when causal (it holds the diagonal) and a ragged last tile. Tiles
  // go in pairs so that each one's LDS stage is a compile-time constant (the stage offsets then
  // fold into the reads' immediate offsets).
  const bool ragged = T % kQTile != 0;
  auto run = [&](int qt, auto par_tag) {
    const bool m = (CAUSAL && qt == qt0) || (ragged && qt == nqt - 1);
    if (m) tile(qt, par_tag, MaskTag<true>{});
    else tile(qt, par_tag, MaskTag<false>{});
  };
  int qt = qt0;
  for (; qt + 1 < nqt; qt += 2) {
    run(qt, StageTag<0>{});
    run(qt + 1, StageTag<1>{});
  }
  if (qt < nqt) run(qt, StageTag<0>{});

  // lane (g, j16) holds key kw0 + j16 and d = 16 db + 4 g + 0..3 of dK^T and dV^T
  if (key < T) {
    uint16_t* dvr = dV + base + (size_t)key * D;
    uint16_t* dkr = dK + base + (size_t)key * D;
#pragma unroll
    for (int db = 0; db < nD; ++db) {
      *reinterpret_cast<u32x2*>(dvr + 16 * db + 4 * g) =
          u32x2{pack_bf16x2(dv[db][0], dv[db][1]), pack_bf16x2(dv[db][2], dv[db][3])};
      *reinterpret_cast<u32x2*>(dkr + 16 * db + 4 * g) =
          u32x2{pack_bf16x2(dk[db][0] * scale, dk[db][1] * scale),
                pack_bf16x2(dk[db][2] * scale, dk[db][3] * scale)};
    }
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
    const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO, const float* __restrict__ LSE,
    float* __restrict__ Dv, float* __restrict__ L2, uint16_t* __restrict__ dQ, int T, int BH, int nq,
    int grp, float c, float scale) {
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
  // D_i = rowsum(dO * O) over this lane's half of the row's d values plus the other half's
  // (lane l ^ 32), and LSE_i log2 e; both go to the workspace for the dK/dV kernel, which runs
  // after this one
  float dsum = 0.f;
#pragma unroll
  for (int kk = 0; kk < nK; ++kk) {
    const size_t off = base + (size_t)qrow * D + kk * 16 + h * 8;
    const u32x4 ow = qrow < T ? *reinterpret_cast<const u32x4*>(O + off) : u32x4{0u, 0u, 0u, 0u};
    const u32x4 dw = __builtin_bit_cast(u32x4, dof[kk]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dsum += bf16_lo(ow[i]) * bf16_lo(dw[i]) + bf16_hi(ow[i]) * bf16_hi(dw[i]);
  }
  const float dval = dsum + swap_halves(dsum);
  const float lse2 = qrow < T ? LSE[(size_t)bh * T + qrow] * kLog2e : 0.f;
  if (h == 0 && qrow < T) {
    Dv[(size_t)bh * T + qrow] = dval;
    L2[(size_t)bh * T + qrow] = lse2;
  }

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
  // PAR: the tile's LDS stage as a compile-time constant (the stage offset folds into the
  // reads' immediate offsets); MASK: the tile may hold a key after one of the wave's queries
  // (causal) or past T, so its scores are masked.
  auto tile = [&](int j, auto par_tag, auto mask_tag) {
    constexpr int PAR = decltype(par_tag)::value;   // -1: stage j & 1 at run time
    constexpr bool MASK = decltype(mask_tag)::value;
    const int k0 = j * kKTile;
    const uint8_t* Ks = smem + (PAR < 0 ? (j & 1) : PAR) * stageBytes;
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
    bf16x8 dsb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 ds;
      // key kj = k0 + 32 kb + 4 h + e(r), e(r) = 8 (r / 4) + r % 4, is visible iff kj < T and
      // (causal) kj <= qrow: one compare of the constant e(r) with a per-lane limit
      const int elim = (CAUSAL ? min(qrow, T - 1) : T - 1) - (k0 + 32 * kb + 4 * h);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pv = exp2_fast(fmaf(s[kb][r], c, -lse2));
        if constexpr (MASK) pv = (8 * (r >> 2) + (r & 3)) <= elim ? pv : 0.f;
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
  // tiles [0, nu) need no mask: every key at or before the wave's first query, none past T
  const int nfull = T / kKTile;
  const int nu = CAUSAL ? min(nfull, qw0 >= kKTile - 1 ? (qw0 - (kKTile - 1)) / kKTile + 1 : 0)
                        : nfull;
  // Straight-line loops only (a branch around a tile body makes the compiler copy the dQ
  // accumulators at the join): unmasked tiles in pairs with compile-time stages, then the
  // rest of the wave's tiles with masks and a run-time stage, then the tiles it only helps
  // load. Each iteration of every loop passes two race-check points.
  int j = 0;
  for (; j + 1 < nu; j += 2) {
    sync_check();
    fetch(j + 1, smem + stageBytes);
    tile(j, StageTag<0>{}, MaskTag<false>{});
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    sync_check();
    // the load destination stays a run-time offset (see the dK/dV kernel)
    if (j + 2 < ntiles) fetch(j + 2, smem + ((j + 2) & 1) * stageBytes);
    tile(j + 1, StageTag<1>{}, MaskTag<false>{});
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  for (; j < ntw; ++j) {
    sync_check();
    if (j + 1 < ntiles) fetch(j + 1, smem + ((j + 1) & 1) * stageBytes);
    tile(j, StageTag<-1>{}, MaskTag<true>{});
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  for (; j < ntiles; ++j) {
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
  // the dQ kernel first: it also writes D_i and LSE_i log2 e, which the dK/dV kernel reads
  const int nq = (a.T + kQueriesPerWG - 1) / kQueriesPerWG;
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3(nq * BH), dim3(kThreads), 0, a.stream, q, k,
                     v, o, dout, a.lse, dvec, lse2, static_cast<uint16_t*>(a.dq), a.T, BH, nq,
                     xcd_group(BH), c, a.scale);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  if constexpr (D == 128) {
    const int nk = (a.T + kKeysPerWG16 - 1) / kKeysPerWG16;
    hipLaunchKernelGGL((bwd_dkdv16_kernel<D, CAUSAL>), dim3(nk * BH), dim3(kThreads), 0, a.stream,
                       q, k, v, dout, dvec, lse2, static_cast<uint16_t*>(a.dk),
                       static_cast<uint16_t*>(a.dv), a.T, BH, xcd_group(BH), c, a.scale);
  } else {
    const int nk = (a.T + kKeysPerWG - 1) / kKeysPerWG;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3(nk * BH), dim3(kThreads), 0, a.stream, q,
                       k, v, dout, dvec, lse2, static_cast<uint16_t*>(a.dk),
                       static_cast<uint16_t*>(a.dv), a.T, BH, xcd_group(BH), c, a.scale);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a) {
  if (a.D == 64) return a.causal ? launch<64, true>(a) : launch<64, false>(a);
  return a.causal ? launch<128, true>(a) : launch<128, false>(a);
}

}  // namespace fa
