// Split-K decode: a few new query rows against a long K/V cache, bf16 storage, fp32
// accumulation. Hand-written gfx950 kernels.
//
// Method: "Lab 06 - Attention kernels", "Check yourself" answers 2 and 7 and the stretch
// goals. With one query row per head the only parallelism of the forward's grid is batch x
// heads, far fewer workgroups than compute units, each walking every key. Here the keys of a
// sequence are split across workgroups; each computes the partial statistics of section 3
// (running max m, sum l, unnormalised accumulator acc) over its key range, and a second
// kernel merges the partials with the same rescaling rule (every partial scaled by
// exp(m_s - max_s m_s)). All query heads that share one K/V head (grouped-query attention)
// are stacked in the same product, so each K/V tile read from HBM serves all of them. The
// "Common bugs" list on the same page warns that key ranges visited out of order can leave a
// row with no visible key (max = -inf); both kernels guard it.
//
// gfx950 mapping
//   * One wave per workgroup, one workgroup per (b, K/V head, split); each streams 32-key
//     tiles of K and V through a ring of S LDS slots with direct HBM -> LDS loads (S - 1
//     tiles in flight while one is used). Workgroups of one wave let the LDS budget, not a
//     fixed wave count, set how many run per compute unit.
//   * The M = G * Tq query rows of the group (at most 32) are the columns of one
//     32 x 32 x 16 bf16 product: S^T = K Q^T puts one query row per lane (two lanes per row,
//     16 keys each); O^T += V^T P^T takes P straight from the S^T registers and V^T from a
//     transposing LDS read. The matrix cores are far from busy at these shapes; the kernel is
//     bound by HBM.
//   * The partials go to the workspace as fp32: acc [split][M][D] and (m, l, l_rounded) per
//     row, with m in the exp2 domain (scores times scale * log2 e). The merge kernel gives
//     each output row one workgroup of 256 threads, which read several splits at once.
//   * With per-sequence lengths (up to 64 sequences) the split slots of a K/V head are shared
//     out in proportion to the sequences' lengths (dec_plan), so that every split streams about
//     the same number of key tiles.
//   * As in the forward kernel, P is rounded to bf16 before the P V product; O is normalised
//     by the sum of the rounded P and LSE uses the fp32 sum of the unrounded exponentials.

#include <type_traits>

#include "fa_common.h"
#include "fa_launch.h"
#include "fa_swz.h"

namespace fa {
namespace {

constexpr int kKeys = 32;   // keys per tile

struct DecKArgs {
  const uint16_t *q, *k, *v;
  float* part;                // partial accumulators, then partial statistics
  const int* seqlens;         // (B) valid keys per sequence, or null for Tk
  int Hq, Hkv, G, Tq, Tk, M;  // M = G * Tq query rows per K/V head
  int nsplit, nwork;          // splits per (b, K/V head); nwork = B * Hkv * nsplit
  float c;                    // scale * log2(e)
  int causal;
  int B;
  int bal;                    // split slots shared out by length (dec_plan), else 0
};

constexpr int kMaxSplit = 1024;   // splits of one (b, K/V head) the merge can take

// Sum of x over the 64 lanes of the wave, as a wave-uniform value: DPP exchanges within each
// row of 16 lanes (pairs, quads, half-row mirror, row mirror), then the four row sums. Needs
// every lane active.
__device__ __forceinline__ int wave_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0xb1, 0xf, 0xf, false);    // quad_perm [1,0,3,2]
  x += __builtin_amdgcn_update_dpp(0, x, 0x4e, 0xf, 0xf, false);    // quad_perm [2,3,0,1]
  x += __builtin_amdgcn_update_dpp(0, x, 0x141, 0xf, 0xf, false);   // row_half_mirror
  x += __builtin_amdgcn_update_dpp(0, x, 0x140, 0xf, 0xf, false);   // row_mirror
  return __builtin_amdgcn_readlane(x, 0) + __builtin_amdgcn_readlane(x, 16) +
         __builtin_amdgcn_readlane(x, 32) + __builtin_amdgcn_readlane(x, 48);
}

// Split plan of a batch with per-sequence lengths (at most 64 sequences, lane b holds sequence
// b). With one split count for every sequence, the splits of a short sequence are short and
// the long sequences' splits run on alone at the end. Here the B * nsplit split slots of each
// K/V head are shared out in proportion to the sequences' key tiles: sequence b gets
// ns = 1 + (B * nsplit - B) * nt_b / (sum of nt) slots (at most kMaxSplit), the slots
// first .. first + ns - 1 in sequence order, so every split walks about the same number of
// tiles and the slots left over run nothing. Both kernels compute the same plan from the
// lengths. Needs every lane active.
struct DecPlan {
  int nt, ns, first;   // this lane's sequence: key tiles, splits, first slot
};
__device__ __forceinline__ DecPlan dec_plan(const int* seqlens, int B, int Tk, int nsplit) {
  const int b = lane_thread_id() & 63;
  DecPlan p{0, 0, 0};
  if (b < B) p.nt = (min(max(seqlens[b], 0), Tk) + kKeys - 1) / kKeys;
  const int tot = wave_sum(p.nt);
  if (b < B)
    p.ns = min(1 + (tot > 0 ? (int)((int64_t)(B * nsplit - B) * p.nt / tot) : 0), kMaxSplit);
  for (int b2 = 0; b2 < B; ++b2) {
    const int n2 = __builtin_amdgcn_readlane(p.ns, b2);
    p.first += b2 < b ? n2 : 0;
  }
  return p;
}

// Direct HBM -> LDS loads of one 32-row tile of a (rows x D) matrix by a single wave, into the
// swizzled layout of SwzTile (rows 0..31). Lane `lane` of load i fills tile bytes [16 u,
// 16 u + 16), u = 64 i + lane: physical chunk u % CH of row u / CH. Rows at or beyond T are
// clamped to T - 1.
template <int D>
struct WaveTileLoader {
  using Tl = SwzTile<D>;
  static constexpr int N = kKeys * Tl::CH / 64;   // 16-byte loads per lane per tile
  int row[N];
  uint32_t cofs[N];
  __device__ __forceinline__ explicit WaveTileLoader(int lane) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int u = i * 64 + lane;
      row[i] = u / Tl::CH;
      cofs[i] = (uint32_t)(((u % Tl::CH) ^ Tl::swz(row[i])) * 16);
    }
  }
  __device__ __forceinline__ void issue(uint8_t* dst, const uint16_t* __restrict__ src, int row0,
                                        int T) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const uint32_t off = (uint32_t)min(row0 + row[i], T - 1) * (uint32_t)Tl::RB + cofs[i];
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint8_t*>(src) + off,
                                       (lds_void*)(dst + i * 1024), 16, 0, 0);
    }
  }
};

// LDS reads of the K / V tiles as inline asm. The compiler's own wait analysis cannot always
// tell which slot of the ring a read touches and then waits for every outstanding HBM -> LDS
// load, which would empty the ring; here the kernel waits for exactly the loads of the slot
// it reads (s_waitcnt vmcnt) and for the reads themselves with lds_fence, whose register
// operands make every use of the fragments depend on the wait.
typedef __attribute__((address_space(3))) uint8_t lds_u8;
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return (uint32_t)(uintptr_t)(const lds_u8*)p;
}
__device__ __forceinline__ u32x4 lds_read_b128(uint32_t addr) {
  u32x4 x;
  asm volatile("ds_read_b128 %0, %1" : "=v"(x) : "v"(addr));
  return x;
}
__device__ __forceinline__ u32x2 lds_read_tr(uint32_t addr) {
  u32x2 x;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(x) : "v"(addr));
  return x;
}
template <int N>
__device__ __forceinline__ void lds_fence(u32x4 (&x)[N]) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(x[i]));
}

template <int I, int N, class F>
__device__ __forceinline__ void dec_static_for(const F& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    dec_static_for<I + 1, N>(f);
  }
}

template <int D, int S>
__global__ __launch_bounds__(64) void decode_bf16_kernel(const DecKArgs a) {
  using Tl = SwzTile<D>;
  constexpr int TB = kKeys * Tl::RB;   // bytes of one 32-row tile
  constexpr int nK = D / 16;           // k-steps of S^T
  constexpr int nD = D / 32;           // 32-row blocks of O^T
  constexpr int LPT = 2 * WaveTileLoader<D>::N;   // loads per tile (K and V)
  static_assert(S >= 2 && S <= 4, "2 to 4 slots");
  static_assert((S - 1) * LPT <= 63, "loads in flight must fit the vmcnt counter");
  // one LDS object per slot: with the slot known at compile time the compiler can tell the
  // slot being read from the ones still being filled
  __shared__ __attribute__((aligned(1024))) uint8_t k0[TB], k1[TB], k2[S > 2 ? TB : 16],
      k3[S > 3 ? TB : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t v0[TB], v1[TB], v2[S > 2 ? TB : 16],
      v3[S > 3 ? TB : 16];
  auto kslot = [&](auto sc) -> uint8_t* {
    constexpr int s = decltype(sc)::value;
    if constexpr (s == 0) return k0;
    else if constexpr (s == 1) return k1;
    else if constexpr (s == 2) return k2;
    else return k3;
  };
  auto vslot = [&](auto sc) -> uint8_t* {
    constexpr int s = decltype(sc)::value;
    if constexpr (s == 0) return v0;
    else if constexpr (s == 1) return v1;
    else if constexpr (s == 2) return v2;
    else return v3;
  };

  const int lane = lane_thread_id();
  const int l32 = lane & 31, h = lane >> 5;
  const int gw = workgroup_id();
  if (gw >= a.nwork) return;
  int b, kvh, split, nsp, L = a.Tk;
  if (a.bal) {
    // slot j of K/V head kvh belongs to the sequence whose range of slots holds it
    const int per = a.nwork / a.Hkv;   // B * nsplit slots a K/V head
    kvh = gw / per;
    const int j = gw - kvh * per;
    const DecPlan pl = dec_plan(a.seqlens, a.B, a.Tk, a.nsplit);
    const uint64_t own = __builtin_amdgcn_ballot_w64(pl.ns > 0 && pl.first <= j && j < pl.first + pl.ns);
    if (own == 0) return;   // a slot left over: no partial, the merge does not read it
    b = (int)__builtin_ctzll(own);
    split = j - __builtin_amdgcn_readlane(pl.first, b);
    nsp = __builtin_amdgcn_readlane(pl.ns, b);
    L = __builtin_amdgcn_readfirstlane(min(max(a.seqlens[b], 0), a.Tk));
  } else {
    split = gw % a.nsplit;
    const int bh0 = gw / a.nsplit;   // b * Hkv + K/V head
    b = bh0 / a.Hkv;
    kvh = bh0 % a.Hkv;
    nsp = a.nsplit;
    if (a.seqlens) L = __builtin_amdgcn_readfirstlane(min(max(a.seqlens[b], 0), a.Tk));
  }
  const int bh = b * a.Hkv + kvh;
  const int nt = (L + kKeys - 1) / kKeys;
  const int t0 = (int)((int64_t)split * nt / nsp);
  const int t1 = (int)((int64_t)(split + 1) * nt / nsp);

  const int64_t kv_off = (int64_t)bh * a.Tk * D;
  const uint16_t* Kh = a.k + kv_off;
  const uint16_t* Vh = a.v + kv_off;
  const WaveTileLoader<D> ld(lane);
  const int last = max(t1 - 1, t0);
  auto issue = [&](auto sc, int t) __attribute__((always_inline)) {
    const int tt = min(t, last) * kKeys;   // past the split: reload its last tile, never read
    ld.issue(kslot(sc), Kh, tt, L);
    ld.issue(vslot(sc), Vh, tt, L);
  };

  // Query row of this lane's column: n = g * Tq + i (head kvh * G + g, position i). Columns
  // n >= M are zero padding and are never stored.
  const int n = l32;
  const bool live = n < a.M;
  const int g = n / a.Tq, qi = n % a.Tq;
  // keys this column may see: j < L, and causally j <= qi + L - Tq (bottom-right aligned)
  const int lim = a.causal ? qi + L - a.Tq : L - 1;
  bf16x8 qf[nK];
  {
    const uint16_t* Qr = a.q + (((int64_t)b * a.Hq + kvh * a.G + g) * a.Tq + qi) * D;
#pragma unroll
    for (int kk = 0; kk < nK; ++kk) {
      u32x4 x = live ? *reinterpret_cast<const u32x4*>(Qr + kk * 16 + h * 8) : u32x4{0, 0, 0, 0};
      qf[kk] = as_bf16x8(x);
    }
  }

  f32x16 acc[nD];
#pragma unroll
  for (int db = 0; db < nD; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  float m = kNegInf, l = 0.f, lr = 0.f;   // m in the exp2 domain; l, lr over this lane's keys
  const float c = a.c;
  // last key every column sees: tiles ending at or before it need no mask
  const int lim_min = a.causal ? L - a.Tq : L - 1;

  // Per-lane LDS byte offsets of the tile operands (the same in every slot): the S^T A
  // operand of k-step kk is 16 bytes of key row l32, logical chunk 2 kk + h; the V^T A operand
  // of key step cc and d-block db is two transposing 8-byte reads (rows r0 and r0 + 8).
  uint32_t kofs[nK], vofs[2][nD][2];
#pragma unroll
  for (int kk = 0; kk < nK; ++kk) kofs[kk] = (uint32_t)Tl::offset(l32, 2 * kk + h);
  {
    const int g4 = lane >> 4, i16 = lane & 15;
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int db = 0; db < nD; ++db) {
        const int row = 16 * cc + 4 * (g4 >> 1) + (i16 >> 2);
        const int d0 = db * 32 + (g4 & 1) * 16 + 4 * (i16 & 3);
        vofs[cc][db][0] = (uint32_t)(Tl::offset(row, d0 >> 3) + (d0 & 7) * 2);
        vofs[cc][db][1] = (uint32_t)(Tl::offset(row + 8, d0 >> 3) + (d0 & 7) * 2);
      }
  }

  auto tile = [&](auto sc, int t) __attribute__((always_inline)) {
    sync_check();
    const uint32_t Kb = lds_addr(kslot(sc));
    const uint32_t Vb = lds_addr(vslot(sc));
    u32x4 kf[nK];
#pragma unroll
    for (int kk = 0; kk < nK; ++kk) kf[kk] = lds_read_b128(Kb + kofs[kk]);
    lds_fence(kf);
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < nK; ++kk) s = mfma32(as_bf16x8(kf[kk]), qf[kk], s);
    // the V operands load while the VALU works on the scores
    u32x4 vf[2 * nD];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int db = 0; db < nD; ++db) {
        const u32x2 lo = lds_read_tr(Vb + vofs[cc][db][0]);
        const u32x2 hi = lds_read_tr(Vb + vofs[cc][db][1]);
        vf[cc * nD + db] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
    // scores to the exp2 domain; lane holds keys 32 t + 8 (r / 4) + 4 h + r % 4
    const int kb = t * kKeys + 4 * h;
    float x[16];
    if (t * kKeys + kKeys - 1 <= lim_min) {
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = s[r] * c;
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = kb + 8 * (r >> 2) + (r & 3);
        x[r] = j <= lim ? s[r] * c : kNegInf;
      }
    }
    float mt = x[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = fmaxf(mt, x[r]);
    mt = fmaxf(mt, swap_halves(mt));
    const float m_new = fmaxf(m, mt);
    if (__builtin_amdgcn_ballot_w64(m_new > m)) {
      // exp2(-inf) = 0 clears the (still empty) sums of a column seeing its first key
      const float alpha = m_new > m ? exp2_fast(m - m_new) : 1.f;
      l *= alpha;
      lr *= alpha;
#pragma unroll
      for (int db = 0; db < nD; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
      m = m_new;
    }
    // a column with no visible key so far keeps m = -inf: subtract 0 so its exponentials are 0
    const float mu = m == kNegInf ? 0.f : m;
    uint32_t pw[8];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = exp2_fast(x[r] - mu), p1 = exp2_fast(x[r + 1] - mu);
      l += p0 + p1;
      const uint32_t w = pack_bf16x2(p0, p1);
      pw[r / 2] = w;
      lr += __uint_as_float(w << 16) + __uint_as_float(w & 0xffff0000u);
    }
    lds_fence(vf);
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const u32x4 pb = {pw[4 * cc], pw[4 * cc + 1], pw[4 * cc + 2], pw[4 * cc + 3]};
#pragma unroll
      for (int db = 0; db < nD; ++db)
        acc[db] = mfma32(as_bf16x8(vf[cc * nD + db]), as_bf16x8(pb), acc[db]);
    }
  };

  // ring of S slots: tile t lives in slot (t - t0) % S. Whole groups of S tiles run with
  // every step unconditional, so the waits are known at compile time: S - 1 tiles stay in
  // flight while one is used. The last (fewer than S) tiles are already loading when the
  // groups end; they wait once and run.
  if (t1 > t0) {
    dec_static_for<0, S - 1>([&](auto sc) { issue(sc, t0 + decltype(sc)::value); });
    int t = t0;
    for (; t + S <= t1; t += S) {
      dec_static_for<0, S>([&](auto sc) {
        constexpr int s = decltype(sc)::value;
        issue(std::integral_constant<int, (s + S - 1) % S>{}, t + s + S - 1);
        // tile t + s's loads are older than the (S - 1) * LPT issued after them
        __builtin_amdgcn_s_waitcnt((((S - 1) * LPT) & 15) | ((((S - 1) * LPT) >> 4) << 14) |
                                   (0x7 << 4) | (0xF << 8));
        tile(sc, t + s);
      });
    }
    __builtin_amdgcn_s_waitcnt(0);
    dec_static_for<0, S - 1>([&](auto sc) {
      if (t + decltype(sc)::value < t1) tile(sc, t + decltype(sc)::value);
    });
  }

  // ---- partials: this lane's half of column n, summed with the other half ----------------
  l += swap_halves(l);
  lr += swap_halves(lr);
  if (live) {
    const int64_t row = (int64_t)gw * a.M + n;
    float* P = a.part + row * D;
#pragma unroll
    for (int db = 0; db < nD; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 w = {acc[db][4 * q4], acc[db][4 * q4 + 1], acc[db][4 * q4 + 2],
                         acc[db][4 * q4 + 3]};
        *reinterpret_cast<f32x4*>(P + 32 * db + 8 * q4 + 4 * h) = w;
      }
    if (h == 0) {
      float* St = a.part + (int64_t)a.nwork * a.M * D + row * 4;
      *reinterpret_cast<f32x4*>(St) = f32x4{m, l, lr, 0.f};
    }
  }
}

// ---- merge: one workgroup per output row -------------------------------------------------
// 256 threads: thread t reads columns 4 (t % (D / 4)) .. +3 of every (256 / (D / 4))-th split,
// so the splits of a row are read in parallel with 16-byte loads; the split weights and the
// per-group sums meet in LDS.
struct MergeKArgs {
  const float* part;
  uint16_t* o;
  float* lse;
  int Hq, Hkv, G, Tq, M, nsplit, nwork, rows;   // rows = B * Hq * Tq
  const int* seqlens;                           // with bal: the split plan's lengths
  int B, Tk, bal;
};

constexpr int kMergeThreads = 256;

template <int D>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(const MergeKArgs a) {
  constexpr int C4 = D / 4;                  // float4 columns of a row
  constexpr int NG = kMergeThreads / C4;     // splits read in parallel
  __shared__ float wsh[kMaxSplit];
  __shared__ float red[3][kMergeThreads / 64];
  __shared__ f32x4 part_o[NG][C4];
  const int tid = lane_thread_id();
  const int lane = tid & 63, wave = tid >> 6;
  const int R = workgroup_id();
  const int qi = R % a.Tq;
  const int hq = (R / a.Tq) % a.Hq;
  const int b = R / (a.Tq * a.Hq);
  const int kvh = hq / a.G, g = hq % a.G;
  const int r = g * a.Tq + qi;                                   // row within the K/V group
  int64_t w0 = ((int64_t)b * a.Hkv + kvh) * a.nsplit;           // first split's work index
  int nsp = a.nsplit;
  if (a.bal) {   // this sequence's slots of the split plan
    const DecPlan pl = dec_plan(a.seqlens, a.B, a.Tk, a.nsplit);
    w0 = (int64_t)kvh * (a.nwork / a.Hkv) + __builtin_amdgcn_readlane(pl.first, b);
    nsp = __builtin_amdgcn_readlane(pl.ns, b);
  }
  const float* St = a.part + (int64_t)a.nwork * a.M * D;

  // global max of the splits' m (exp2 domain)
  float mx = kNegInf;
  for (int s = tid; s < nsp; s += kMergeThreads) mx = fmaxf(mx, St[((w0 + s) * a.M + r) * 4]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  if (lane == 0) red[0][wave] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
  // weights; a split that saw no key (m = -inf) weighs 0, and so does every split of a row
  // that saw none (then O = 0, LSE = -inf)
  float sl = 0.f, slr = 0.f;
  for (int s = tid; s < nsp; s += kMergeThreads) {
    const f32x4 st = *reinterpret_cast<const f32x4*>(St + ((w0 + s) * a.M + r) * 4);
    const float w = st[0] == kNegInf ? 0.f : exp2_fast(st[0] - mx);
    wsh[s] = w;
    sl += w * st[1];
    slr += w * st[2];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    sl += __shfl_xor(sl, o, 64);
    slr += __shfl_xor(slr, o, 64);
  }
  __syncthreads();   // wsh complete; red[0] read by everyone
  if (lane == 0) {
    red[1][wave] = sl;
    red[2][wave] = slr;
  }
  const int c4 = tid % C4, sg = tid / C4;
  const float* A = a.part + (w0 * a.M + r) * D + c4 * 4;
  const int64_t stride = (int64_t)a.M * D;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  int s = sg;
  for (; s + 3 * NG < nsp; s += 4 * NG) {
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(A + s * stride);
    const f32x4 x1 = *reinterpret_cast<const f32x4*>(A + (s + NG) * stride);
    const f32x4 x2 = *reinterpret_cast<const f32x4*>(A + (s + 2 * NG) * stride);
    const f32x4 x3 = *reinterpret_cast<const f32x4*>(A + (s + 3 * NG) * stride);
    acc += wsh[s] * x0 + wsh[s + NG] * x1 + wsh[s + 2 * NG] * x2 + wsh[s + 3 * NG] * x3;
  }
  for (; s < nsp; s += NG) acc += wsh[s] * *reinterpret_cast<const f32x4*>(A + s * stride);
  part_o[sg][c4] = acc;
  __syncthreads();
  if (tid < C4) {
    f32x4 o = part_o[0][tid];
#pragma unroll
    for (int k = 1; k < NG; ++k) o += part_o[k][tid];
    const float lr_tot = red[2][0] + red[2][1] + red[2][2] + red[2][3];
    const float inv = lr_tot > 0.f ? 1.f / lr_tot : 0.f;
    const u32x2 w = {pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv)};
    *reinterpret_cast<u32x2*>(a.o + (int64_t)R * D + tid * 4) = w;
    if (tid == 0) {
      const float l_tot = red[1][0] + red[1][1] + red[1][2] + red[1][3];
      a.lse[R] = l_tot > 0.f ? (mx + log2_fast(l_tot)) * kLn2 : kNegInf;
    }
  }
}

constexpr int kSlots = 2;

template <int D>
hipError_t launch_decode_d(const DecodeBf16Problem& p) {
  const int G = p.Hq / p.Hkv;
  const int M = G * p.Tq;
  const int nwork = p.B * p.Hkv * p.nsplit;
  DecKArgs ka{static_cast<const uint16_t*>(p.q), static_cast<const uint16_t*>(p.k),
              static_cast<const uint16_t*>(p.v), static_cast<float*>(p.workspace), p.seqlens,
              p.Hq, p.Hkv, G, p.Tq, p.Tk, M, p.nsplit, nwork, p.scale * 1.4426950408889634f,
              p.causal ? 1 : 0, p.B, 0};
  // per-sequence lengths, at most 64 sequences: split slots shared out by length (dec_plan)
  const int bal = p.seqlens && p.B <= 64 ? 1 : 0;
  ka.bal = bal;
  hipLaunchKernelGGL((decode_bf16_kernel<D, kSlots>), dim3(nwork), dim3(64), 0, p.stream, ka);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows = p.B * p.Hq * p.Tq;
  MergeKArgs ma{static_cast<const float*>(p.workspace), static_cast<uint16_t*>(p.o), p.lse, p.Hq,
                p.Hkv, G, p.Tq, M, p.nsplit, nwork, rows, p.seqlens, p.B, p.Tk, bal};
  hipLaunchKernelGGL(decode_merge_kernel<D>, dim3(rows), dim3(kMergeThreads), 0, p.stream, ma);
  return hipGetLastError();
}

}  // namespace

int decode_max_splits() { return kMaxSplit; }

hipError_t launch_decode_bf16(const DecodeBf16Problem& p) {
  return p.D == 64 ? launch_decode_d<64>(p) : launch_decode_d<128>(p);
}

}  // namespace fa
