// Attention forward, bf16 storage (or E4M3 Q and K), fp32 accumulation: hand-written gfx950
// kernel with one 32-query block per wave and two workgroups on every compute unit.
//
// Method: "Lab 06 - Attention kernels", section 3 (per query tile keep the row max m, row
// sum l and accumulator acc; per key tile rescale by exp(m - m') and add exp(S - m') V;
// finish with O = acc / l and LSE = m + log l; causal tiles above the diagonal are never
// loaded, diagonal tiles are masked element-wise) and section 5 (one program per
// (query tile, batch*head)). "Triton FlashAttention-2 forward", "The kernel" (P rounded to
// the input dtype before the P V product, masked loads read zeros beyond T). Section 2 of
// the lab page: subtracting any constant from the exponents and dividing it back out is
// exact, which the lazy reference relies on. The E4M3 Q K^T variant follows the same page's
// "Stretch" list; the format and block scaling are described with the quantizer.
//
// gfx950 mapping
//   * A wave issues a 32x32x16 product in about 12 cycles of its own time and the product
//     occupies the matrix core for 32, so a single wave per SIMD leaves the matrix core idle
//     while it works through the softmax. Every wave here holds one block of 32 queries (O^T
//     in 64 AGPRs, Q^T in 32), a wave needs at most 256 registers, and two workgroups of 4
//     waves share each compute unit: the SIMD runs one wave's products while the other
//     wave's vector instructions issue.
//   * Workgroup: 4 waves, 128 queries of one (b, h) (or 128 / hpw queries of hpw heads that
//     share a K/V head, so every K/V tile loaded serves all of them). Causal grid order is
//     heaviest query tile first; consecutive workgroup ids walk (b, head group) fastest,
//     which keeps a head's tiles on one XCD (workgroups are dealt to the 8 XCDs round-robin)
//     so its K and V are shared through that XCD's L2; each XCD takes its heads four at a
//     time, so that the query tiles reading one head's K and V run together.
//   * K and V tiles (64 keys) reach LDS by direct buffer -> LDS loads into XOR-swizzled
//     row-major tiles, two slots each (64 KB a workgroup); K runs one tile ahead of V. The
//     buffer resource ends at the last key row, so rows past it arrive as zeros and a load
//     costs no vector arithmetic. The loads are inline asm, out of the compiler's sight: it
//     would otherwise wait for every outstanding LDS read wherever it needs one of them.
//   * S^T = K Q^T (v_mfma_f32_32x32x16_bf16, or v_mfma_scale_f32_32x32x64_f8f6f4 for E4M3)
//     puts one query per lane; a row's 64 scores of a tile sit in two 16-register blocks
//     (key halves kb = 0, 1) of lanes l and l ^ 32. The S^T accumulator layout is the
//     B-operand layout of O^T += V^T P^T, so P never leaves registers; the V^T A operand is
//     a transposing LDS read (ds_read_b64_tr_b16) of the row-major tile.
//   * exp(x) is exp2(x * scale * log2 e): one FMA and one v_exp_f32.
//   * Lazy reference: a row's reference max m_ref moves only when a tile max exceeds it by
//     more than 2^8 in the exp2 domain (and on the first tile), so P <= 2^8 and the O^T
//     accumulators are rescaled in a rare wave-uniform branch, never in the steady state.
//     O is normalised by the sum of the bf16-rounded P that actually multiplied V, so a
//     dominant key's rounding cancels between numerator and denominator; LSE uses the fp32
//     sum of the unrounded exponentials.
//   * Software pipeline across key tiles: phase X of iteration j runs the S products of tile
//     j+1 while the VALU finishes key half 1 of tile j (exponentials, fp32 and rounded sums,
//     packing) and takes the max over key half 0 of tile j+1; phase Y runs tile j's P V
//     products while the VALU takes the max over key half 1 of tile j+1, moves the
//     references and works through key half 0 of tile j+1. Each step of a phase holds one
//     product followed by a fixed share of the VALU work, fenced with sched_barrier. The
//     E4M3 products (4 a tile for D = 128, each four times the work of a bf16 one) sit on
//     every fourth step of the same schedule; at D = 128 the first six P V products of tile j
//     (key half 0's chunks, finished in the previous phase Y) move into phase X, on two of the
//     three steps between E4M3 products, so phase X is not left with a quarter of the products
//     under all of its VALU work.

#include "fa_common.h"
#include "fa_launch.h"
#include "fa_swz.h"
#include "fa_fwd_parts.h"

namespace fa {
namespace {

using namespace fwd;

constexpr int kThreads = 256;
constexpr int kBlockM = 128;   // queries per workgroup, 32 per wave

// 20 wait states between the last product writing x and any later instruction that uses it.
__device__ __forceinline__ void fence1(f32x16& x) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(x));
}
// The same ordering point with only N + 1 wait states of padding (N = -1: none), where the
// schedule already places that many instructions after the product: the vector reads of x
// cannot move above it. The assembly check of the build verifies the total.
template <int N>
__device__ __forceinline__ void fence_n(f32x16& x) {
  if constexpr (N < 0) asm volatile("" : "+v"(x));
  else asm volatile("s_nop %1" : "+v"(x) : "i"(N));
}

// m = max(m, v[0], v[1], ..., v[2C - 1]) as C dependent v_max3_f32 in one asm statement: the
// compiler pads the reader of an inline-asm result as if the asm were a transcendental, so a
// chain of one-instruction statements costs a wait state per link, one statement does not
template <int C>
__device__ __forceinline__ void max3_chain(float& m, const float* v) {
  static_assert(C >= 1 && C <= 4, "one to four links");
  if constexpr (C == 1)
    asm volatile("v_max3_f32 %0, %0, %1, %2" : "+v"(m) : "v"(v[0]), "v"(v[1]));
  else if constexpr (C == 2)
    asm volatile("v_max3_f32 %0, %0, %1, %2\n\tv_max3_f32 %0, %0, %3, %4"
                 : "+v"(m) : "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]));
  else if constexpr (C == 3)
    asm volatile("v_max3_f32 %0, %0, %1, %2\n\tv_max3_f32 %0, %0, %3, %4\n\t"
                 "v_max3_f32 %0, %0, %5, %6"
                 : "+v"(m) : "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]));
  else
    asm volatile("v_max3_f32 %0, %0, %1, %2\n\tv_max3_f32 %0, %0, %3, %4\n\t"
                 "v_max3_f32 %0, %0, %5, %6\n\tv_max3_f32 %0, %0, %7, %8"
                 : "+v"(m)
                 : "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]),
                   "v"(v[7]));
}

// ---- per-step work assignment (all compile-time) --------------------------------------
// Items of one tile: 32 score elements per lane, v = 16 kb + r; 4 chunks of 8 (v / 8 = ch,
// the B operand P[ch] of keys 16 ch .. 16 ch + 15); 8 max items per key half (pairs of
// elements). Key half 0 of a tile is finished in phase Y of the iteration before the one
// that multiplies it, key half 1 in phase X of that iteration.
template <int D, int NPX = 0>
struct Sched1 {
  static constexpr int nK = D / 16, nD = D / 32;
  static constexpr int NX = 2 * nK;   // phase X steps (S products, f = nK kb + kk)
  // the first NPX P V products of a tile (g = 0 .. NPX - 1, key half 0's chunks) run in phase
  // X, on the steps i with i % 4 = 2 or 3 (the E4M3 S products take the steps i % 4 = 0)
  static constexpr int NY = 4 * nD - NPX;   // phase Y steps (P V products g = NPX + i)
  static constexpr int pvx(int i) {
    int k = 0;
    for (int t = 0; t < NX; ++t)
      if (t % 4 >= 2 && k < NPX) {
        if (t == i) return k;
        ++k;
      }
    return -1;
  }
  static constexpr int XE0 = 0, XE1 = NX - 3, XS0 = 1, XS1 = NX - 1;
  static constexpr int XM0 = nK + 2, XM1 = NX;
  static constexpr int YM0 = 2, YM1 = 3, YR = YM1, YE0 = YR + 1, YE1 = NY - 1;
  static constexpr int YS0 = YE0 + 1, YS1 = NY;
  static constexpr int x_exp(int v) { return win_step(v - 16, 16, XE0, XE1); }   // v in [16, 32)
  static constexpr int x_sum(int v) { return win_step(v - 16, 16, XS0, XS1); }
  static constexpr int x_pack(int ch) { return x_exp(8 * ch + 7) + 1; }            // ch = 2, 3
  static constexpr int XF = (x_sum(31) > x_pack(3) ? x_sum(31) : x_pack(3)) + 1;
  static constexpr int x_max(int t) { return win_step(t, 8, XM0, XM1); }           // kb = 0
  static constexpr int y_max(int t) { return win_step(t, 8, YM0, YM1); }           // kb = 1
  // the max items of a step are consecutive: the first one and how many
  static constexpr int max_first(bool y, int i) {
    for (int t = 0; t < 8; ++t)
      if ((y ? y_max(t) : x_max(t)) == i) return t;
    return 0;
  }
  static constexpr int max_count(bool y, int i) {
    int n = 0;
    for (int t = 0; t < 8; ++t) n += (y ? y_max(t) : x_max(t)) == i;
    return n;
  }
  static constexpr int y_exp(int v) { return win_step(v, 16, YE0, YE1); }          // v in [0, 16)
  static constexpr int y_sum(int v) { return win_step(v, 16, YS0, YS1); }
  // chunk ch (0, 1) of the next tile overwrites P[ch] one step after this tile's last product
  // that reads it (g = nD ch + nD - 1, phase Y step g - NPX; none in Y when g < NPX)
  static constexpr int y_pack(int ch) {
    return y_exp(8 * ch + 7) + 1 > nD * (ch + 1) + 1 - NPX ? y_exp(8 * ch + 7) + 1
                                                            : nD * (ch + 1) + 1 - NPX;
  }
  static constexpr bool valid() {
    for (int v = 0; v < 16; ++v)
      if (y_sum(v) <= y_exp(v) || y_sum(v) >= NY) return false;
    for (int v = 16; v < 32; ++v)
      if (x_sum(v) <= x_exp(v) || x_sum(v) >= NX) return false;
    return YR < YE0 && XF < NX && y_max(7) < YR && y_pack(1) < NY && x_pack(3) < NX &&
           XM0 > nK && x_max(7) < NX;
  }
};
static_assert(Sched1<128>::valid() && Sched1<64>::valid() && Sched1<128, 6>::valid(),
              "pipeline schedule order");
static_assert(Sched1<128, 6>::pvx(2) == 0 && Sched1<128, 6>::pvx(11) == 5 &&
              Sched1<128, 6>::pvx(14) == -1 && Sched1<128, 6>::pvx(4) == -1, "P V steps in X");

// Grid order of a skewed packed batch of at most 64 sequences whose head-group count is a
// multiple of 8 (the host picks it; see the launch). As in xcd_grid_item, unit r = b HG + hg
// stays on XCD r % 8 (workgroup L runs on XCD L % 8), so every XCD holds HG / 8 units of every
// sequence. Within an XCD the sequences go in
// order of decreasing work (query tiles times keys; ties by index), a sequence's tiles heaviest
// first with its units fastest, so the longest causal tiles start first and the short
// sequences fill the end of the launch. The items of an XCD are numbered without gaps, so the
// grid needs only HG * (sum of the tile counts) workgroups instead of B * HG * (tiles of the
// longest sequence). Every wave computes the same item from the offsets: lane b holds
// sequence b, and each lane adds up the items of the sequences ordered before its own. False
// when the index lies past the XCD's last item (the grid is sized on the host from total_q,
// which bounds the tile count when the offsets do not decrease). Also returns the chosen
// sequence's first query and key rows and its lengths (clamped as for the other grid order).
__device__ __forceinline__ bool varlen_item(const FwdKArgs& a, int L, int qrows, int& r, int& qt,
                                            int& qs, int& tq, int& ks, int& tk) {
  const int b = lane_thread_id() & 63;
  int nt = 0, q0 = 0, lq = 0, k0 = 0, lk = 0;
  if (b < a.B) {
    q0 = min(max(a.cu_q[b], 0), a.Tq);
    lq = min(max(a.cu_q[b + 1], q0), a.Tq) - q0;
    k0 = min(max(a.cu_k[b], 0), a.Tk);
    lk = min(max(a.cu_k[b + 1], k0), a.Tk) - k0;
    nt = min((lq + qrows - 1) / qrows, a.nq);
  }
  // units of a sequence on XCD x: head groups x, x + 8, ... (HG is a multiple of 8)
  const int cnt = a.HG >> 3, items = cnt * nt;
  // order key: the work estimate (query tiles x keys; a non-negative float, so its bits order
  // as integers) with its low 6 bits replaced by 63 - b, so that every key differs and near
  // ties go by index; branch-free, a few instructions per sequence
  const float work = (float)nt * (float)(lk + 1);
  const uint32_t key = (__builtin_bit_cast(uint32_t, work) & ~63u) | (uint32_t)(63 - b);
  int before = 0;
  for (int b2 = 0; b2 < a.B; ++b2) {
    const uint32_t k2 = (uint32_t)__builtin_amdgcn_readlane((int)key, b2);
    const int i2 = __builtin_amdgcn_readlane(items, b2);
    before += k2 > key ? i2 : 0;
  }
  const int m = L >> 3;
  const uint64_t own = __builtin_amdgcn_ballot_w64(items > 0 && before <= m && m < before + items);
  if (own == 0) return false;
  const int bs = (int)__builtin_ctzll(own);
  const int w = m - __builtin_amdgcn_readlane(before, bs);
  const int lvl = w / cnt;
  qt = __builtin_amdgcn_readlane(nt, bs) - 1 - lvl;
  r = bs * a.HG + (L & 7) + 8 * (w - lvl * cnt);
  qs = __builtin_amdgcn_readlane(q0, bs);
  tq = __builtin_amdgcn_readlane(lq, bs);
  ks = __builtin_amdgcn_readlane(k0, bs);
  tk = __builtin_amdgcn_readlane(lk, bs);
  return true;
}

template <int D, bool CAUSAL, bool QK8>
__global__ __launch_bounds__(kThreads, 2) void fwd_q32_kernel(const FwdKArgs args) {
  using Tl = SwzTile<D>;
  using Tl8 = SwzTile8<D>;
  // E4M3: the S products take a quarter of phase X's steps, so part of P V moves there
  using S = Sched1<D, (QK8 && D == 128) ? 6 : 0>;
  constexpr int NPX = (QK8 && D == 128) ? 6 : 0;
  // padding before the max reads of the next tile's scores: in phase X they come three steps
  // (three products and their vector work) after the last product of key half 0, enough on
  // their own; in phase Y two products after the last one of key half 1, which needs 8 more
  constexpr int FX = -1, FY = 7;
  constexpr int nD = D / 32;      // 32-row blocks of O^T
  constexpr int nK = D / 16;      // k-steps of S^T = K Q^T (bf16)
  constexpr int nK8 = D / 64;     // k-steps of the E4M3 products
  constexpr int nKF8 = 2 * nK8;   // E4M3 K fragments per tile: f = nK8 kb + kk
  constexpr int NX = S::NX, NY = S::NY;
  // odd steps of phase X that issue K loads (E4M3: the codes, then one for the scales)
  constexpr int LK = QK8 ? Tl8::loadsPerWave + 1 : Tl::loadsPerWave;
  static_assert(LK + Tl::loadsPerWave <= NX / 2, "tile loads fit the odd steps of phase X");
  __shared__ __attribute__((aligned(1024))) uint8_t ks0[Tl::bytes], ks1[Tl::bytes];
  __shared__ __attribute__((aligned(1024))) uint8_t vs0[Tl::bytes], vs1[Tl::bytes];

  const int tid = lane_thread_id();
  const int wave = wave_id();
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int h = lane >> 5;

  // scale = 0 gives uniform weights over the visible keys; the kernel computes it as Q = 0
  // with a positive c (every score is then exactly 0), so that c > 0 everywhere below and a
  // masked score (-inf) always gives exp2(-inf * c - mc) = 0 with no select
  const bool zero_scale = args.c == 0.f;
  const float c = zero_scale ? 1.0f : args.c;
  // Workgroup -> (query tile, batch, head group) = (qt, r), hpw query heads sharing one K/V
  // head, 128 / hpw consecutive queries each; heaviest causal tile first. Within an XCD's
  // group of r the tiles walk the same keys at about the same time and share each K/V line.
  const int L = workgroup_id();
  const int qrows = kBlockM >> args.hpw_log2;
  int r, qt;
  int qs = 0, Tq = args.Tq, ks = 0, Tk = args.Tk;
  if (args.vsched) {
    if (!varlen_item(args, L, qrows, r, qt, qs, Tq, ks, Tk)) return;   // uniform per workgroup
  } else {
    xcd_grid_item(L, args.nbhg, args.nq, args.grp, r, qt);
    if (CAUSAL) qt = args.nq - 1 - qt;
  }
  const int b = r / args.HG, hg = r % args.HG;
  const int hpw = 1 << args.hpw_log2;
  const int h0 = hg * hpw;
  const int hq = h0 + (wave & (hpw - 1));   // this wave's query head
  const int kvh = h0 / args.G;
  if (args.cu_q && !args.vsched) {
    qs = min(max(args.cu_q[b], 0), args.Tq);
    Tq = min(max(args.cu_q[b + 1], qs), args.Tq) - qs;
    ks = min(max(args.cu_k[b], 0), args.Tk);
    Tk = min(max(args.cu_k[b + 1], ks), args.Tk) - ks;
    qs = __builtin_amdgcn_readfirstlane(qs);
    Tq = __builtin_amdgcn_readfirstlane(Tq);
    ks = __builtin_amdgcn_readfirstlane(ks);
    Tk = __builtin_amdgcn_readfirstlane(Tk);
  }
  const int q0 = qt * qrows;
  if (q0 >= Tq) return;   // uniform per workgroup
  const int qw0 = q0 + (wave >> args.hpw_log2) * 32;   // this wave's first query
  const int shift = CAUSAL ? Tk - Tq : 0;              // bottom-right alignment
  const int qrow = qw0 + l32;                          // this lane's query

  const uint16_t* Qh = args.q + b * args.q_bs + (int64_t)qs * args.q_rs + hq * args.q_hs;
  uint16_t* Oh = args.o + b * args.q_bs + (int64_t)qs * args.q_rs + hq * args.q_hs;
  float* Lh = args.lse + b * args.lse_bs + hq * args.lse_hs + qs;
  const uint16_t* Kh = args.k + b * args.kv_bs + (int64_t)ks * args.kv_rs + kvh * args.kv_hs;
  const uint16_t* Vh = args.v + b * args.kv_bs + (int64_t)ks * args.kv_rs + kvh * args.kv_hs;
  const int T = Tk;
  auto kslot = [&](int t) -> uint8_t* { return (t & 1) ? ks1 : ks0; };
  auto vslot = [&](int t) -> uint8_t* { return (t & 1) ? vs1 : vs0; };
  auto kslot_p = [&](auto jp, int j, int d) -> uint8_t* {
    constexpr int P = decltype(jp)::value;
    if constexpr (P < 0) return kslot(j + d);
    else return ((P + d) & 1) ? ks1 : ks0;
  };
  auto vslot_p = [&](auto jp, int j, int d) -> uint8_t* {
    constexpr int P = decltype(jp)::value;
    if constexpr (P < 0) return vslot(j + d);
    else return ((P + d) & 1) ? vs1 : vs0;
  };
  const BufTileLoader<D> ld(wave, lane, args.kv_rs);
  const TileLoader8<D> ld8(wave, lane, args.kv_rs);
  // buffer resources over this head's T key rows (one head stays below 2^31 bytes)
  const uint32_t kv_bytes = (uint32_t)T * (uint32_t)args.kv_rs * 2u;
  const i32x4 Kr = rows_rsrc(Kh, kv_bytes), Vr = rows_rsrc(Vh, kv_bytes);
  i32x4 Kr8 = Kr, Ksr = Kr;
  if constexpr (QK8) {
    const int64_t ko = b * args.kv_bs + (int64_t)ks * args.kv_rs + kvh * args.kv_hs;
    Kr8 = rows_rsrc(args.k8 + ko, kv_bytes / 2u);
    Ksr = rows_rsrc(args.ks + ko / 32, kv_bytes / 64u);
  }

  // keys seen by the workgroup's last query, and by all of its queries
  const int kend = CAUSAL ? min(Tk, q0 + qrows + shift) : Tk;
  const int ntiles = kend > 0 ? (kend + kBlockN - 1) / kBlockN : 0;
  const int kall = CAUSAL ? min(Tk, q0 + shift + 1) : Tk;
  const int nfull = kall > 0 ? min(kall / kBlockN, ntiles) : 0;

  if (ntiles == 0) {   // no query of this workgroup sees a key
    if (qrow < Tq) {
      uint16_t* orow = Oh + (int64_t)qrow * args.q_rs;
#pragma unroll
      for (int d0 = 0; d0 < D; d0 += 8)
        if ((d0 / 8) % 2 == h) *reinterpret_cast<u32x4*>(orow + d0) = u32x4{0u, 0u, 0u, 0u};
      if (h == 0) Lh[qrow] = kNegInf;
    }
    return;
  }

  // the first tiles' loads go out before the Q loads, so that the two latencies overlap
  if constexpr (!QK8) {
    ld.issue_all(kslot(0), Kr, 0, T);
    if (ntiles > 1) ld.issue_all(kslot(1), Kr, kBlockN, T);
  } else {
    ld8.issue_all(kslot(0), Kr8, Ksr, 0, T);
    if (ntiles > 1) ld8.issue_all(kslot(1), Kr8, Ksr, kBlockN, T);
  }
  ld.issue_all(vslot(0), Vr, 0, T);

  // Q^T fragments, moved into AGPRs: lane holds query qrow, d = 16 kk + 8 h + 0..7. E4M3: codes
  // of k-step kk at d = 64 kk + 16 h + 0..15 and 64 kk + 32 + 16 h + 0..15, and the row's scale
  // bytes shifted so that byte 2 kk is block 2 kk + h (the block whose scale this lane half
  // supplies).
  bf16x8 qf[QK8 ? 1 : nK];
  i32x8 qf8[QK8 ? nK8 : 1];
  uint32_t qsc = 0u;
  if constexpr (!QK8) {
#pragma unroll
    for (int kk = 0; kk < nK; ++kk) {
      u32x4 x = qrow < Tq && !zero_scale
                    ? *reinterpret_cast<const u32x4*>(Qh + (int64_t)qrow * args.q_rs + kk * 16 + h * 8)
                    : u32x4{0u, 0u, 0u, 0u};
      qf[kk] = as_bf16x8(x);
    }
#pragma unroll
    for (int kk = 0; kk < nK; ++kk) asm volatile("" : "+a"(qf[kk]));
    asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int kk = 0; kk < nK; ++kk) asm volatile("" : "+a"(qf[kk]));
  } else {
    const int64_t qe = b * args.q_bs + (int64_t)(qs + qrow) * args.q_rs + hq * args.q_hs;
    const uint8_t* Qr = args.q8 + qe;
#pragma unroll
    for (int kk = 0; kk < nK8; ++kk) {
      u32x4 x0 = {0u, 0u, 0u, 0u}, x1 = {0u, 0u, 0u, 0u};
      if (qrow < Tq && !zero_scale) {
        x0 = *reinterpret_cast<const u32x4*>(Qr + 64 * kk + 16 * h);
        x1 = *reinterpret_cast<const u32x4*>(Qr + 64 * kk + 32 + 16 * h);
      }
      qf8[kk] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                      (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
    }
    uint32_t sc = 0x7f7f7f7fu;
    if (qrow < Tq) {
      const uint8_t* Qs = args.qs + qe / 32;
      sc = D == 128 ? *reinterpret_cast<const uint32_t*>(Qs) : *reinterpret_cast<const uint16_t*>(Qs);
    }
    qsc = sc >> (8 * h);
#pragma unroll
    for (int kk = 0; kk < nK8; ++kk) asm volatile("" : "+a"(qf8[kk]));
    asm volatile("" : "+v"(qsc));
    asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int kk = 0; kk < nK8; ++kk) asm volatile("" : "+a"(qf8[kk]));
    asm volatile("" : "+v"(qsc));
  }


  f32x16 acc[nD];
#pragma unroll
  for (int db = 0; db < nD; ++db) acc[db] = f32x16{};
  float m_ref, mc;                  // reference max (raw score units) and m_ref * c
  // row sums per key half: fp32 exponentials (l) and bf16-rounded P (r, two chains), for the
  // tiles already folded in (lp, rp) and for the tile in progress (tl, tr)
  float lp[2] = {0.f, 0.f}, rp[2] = {0.f, 0.f}, tl[2] = {0.f, 0.f}, tr[2] = {0.f, 0.f};
  float pm[2];                      // partial row maxima of the next tile, per key half
  // scores: key half 0 (one buffer) and key half 1 (two, by tile parity); P chunks 0-3
  f32x16 s0, s1a, s1b;
  bf16x8 p[4];
  auto sblk = [&](auto par, int kb) -> f32x16& {
    if constexpr (decltype(par)::value == 0) return kb ? s1a : s0;
    else return kb ? s1b : s0;
  };
  const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3f803f80u);

  // element r of key half kb is key 32 kb + 8 (r / 4) + (r % 4) + 4 h of the tile; it is
  // valid iff that local index is below the returned limit
  auto tile_lim = [&](int t) {
    const int k0 = t * kBlockN;
    int l = Tk - k0;
    if (CAUSAL) l = min(l, qrow + shift - k0 + 1);
    return l - 4 * h;
  };

  // ---- work items ------------------------------------------------------------------------
  auto max_item = [&](auto par, int kb, int t, bool masked, int lim) {
    f32x16& x = sblk(par, kb);
    float a = x[2 * t], b2 = x[2 * t + 1];
    if (masked) {
      const int kla = 32 * kb + 8 * (t >> 1) + 2 * (t & 1);
      a = kla < lim ? a : kNegInf;
      b2 = kla + 1 < lim ? b2 : kNegInf;
      x[2 * t] = a;
      x[2 * t + 1] = b2;
    }
    float m = pm[kb];
    asm volatile("v_max3_f32 %0, %0, %1, %2" : "+v"(m) : "v"(a), "v"(b2));
    pm[kb] = m;
  };
  // max items t0 .. t0 + n - 1 of key half kb (masks as in max_item), chained in statements of
  // up to four links
  auto max_items = [&](auto par, int kb, auto t0c, auto nc, bool masked, int lim) {
    constexpr int t0 = decltype(t0c)::value, n = decltype(nc)::value;
    f32x16& x = sblk(par, kb);
    float v[2 * n];
#pragma unroll
    for (int k = 0; k < n; ++k) {
      const int t = t0 + k;
      float a = x[2 * t], b2 = x[2 * t + 1];
      if (masked) {
        const int kla = 32 * kb + 8 * (t >> 1) + 2 * (t & 1);
        a = kla < lim ? a : kNegInf;
        b2 = kla + 1 < lim ? b2 : kNegInf;
        x[2 * t] = a;
        x[2 * t + 1] = b2;
      }
      v[2 * k] = a;
      v[2 * k + 1] = b2;
    }
    float m = pm[kb];
    static_for<0, (n + 3) / 4>([&](auto gc) {
      constexpr int g = decltype(gc)::value;
      max3_chain<(n - 4 * g < 4 ? n - 4 * g : 4)>(m, v + 8 * g);
    });
    pm[kb] = m;
  };
  auto exp_item = [&](auto par, int v) {
    const int kb = v >> 4, rr = v & 15;
    f32x16& blk = sblk(par, kb);
    const float x = blk[rr];
    // masked scores are -inf and mc is finite (0 while a row has seen no key), so they give 0
    float e = exp2_fast(fmaf(x, c, -mc));
    asm volatile("" : "+v"(e));   // keeps the exponential at its step
    blk[rr] = e;
  };
  auto sum_item = [&](auto par, int v) {
    const int kb = v >> 4, rr = v & 15;
    tl[kb] += sblk(par, kb)[rr];
    asm volatile("" : "+v"(tl[kb]));
  };
  // pack chunk ch to the bf16 B operand P[ch] and add the rounded values
  auto pack_item = [&](auto par, int ch) {
    const int kb = ch >> 1, o = (ch & 1) * 8;
    const f32x16& sv = sblk(par, kb);
    const uint32_t w0 = pack_bf16x2(sv[o + 0], sv[o + 1]), w1 = pack_bf16x2(sv[o + 2], sv[o + 3]);
    const uint32_t w2 = pack_bf16x2(sv[o + 4], sv[o + 5]), w3 = pack_bf16x2(sv[o + 6], sv[o + 7]);
    tr[0] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w0), ones, tr[0], false);
    tr[1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w1), ones, tr[1], false);
    tr[0] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w2), ones, tr[0], false);
    tr[1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w3), ones, tr[1], false);
    asm volatile("" : "+v"(tr[0]), "+v"(tr[1]));
    p[ch] = as_bf16x8(u32x4{w0, w1, w2, w3});
  };
  auto fold = [&]() {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      lp[i] += tl[i];
      rp[i] += tr[i];
      tl[i] = 0.f;
      tr[i] = 0.f;
    }
  };
  // moves the references (every row of the wave, when any row's next tile exceeds its
  // reference by more than the margin) and says whether a rescale is due. A row's maximum
  // beats the reference by the margin iff one of its two key halves (lanes l and l ^ 32) does,
  // and the ballot covers both halves, so the decision needs no cross-half exchange; the
  // full-row maximum is formed only when the reference moves (wave-uniform, rare after the
  // first tile).
  auto reduce = [&](float& m_old) {
    const float ah = fmaxf(pm[0], pm[1]);
    m_old = m_ref;
    if constexpr (D == 128) {
      // a row that has seen no key yet (m_ref = -inf) needs the move as soon as it sees one
      // (ah finite: the difference is +inf); while it still sees none (ah = -inf too) it has
      // nothing to move, and the comparison of the undefined difference is false
      const bool need = (ah - m_ref) * c > kRescaleLog2;
      const bool any = __builtin_amdgcn_ballot_w64(need) != 0;
      if (__builtin_expect(any, 0)) {   // out of line: the common path falls through
        m_ref = fmaxf(m_ref, halves_max1(ah));
        mc = m_ref == kNegInf ? 0.f : m_ref * c;
      }
      return any;
    } else {
      // D = 64 has half the steps per tile to hide a branch in: the full-row maximum every
      // tile, no branch (measured faster there)
      const float a = halves_max1(ah);
      const bool need = (a - m_ref) * c > kRescaleLog2;   // no-key rows: as for D = 128
      const bool any = __builtin_amdgcn_ballot_w64(need) != 0;
      m_ref = any ? fmaxf(m_ref, a) : m_ref;
      mc = m_ref == kNegInf ? 0.f : m_ref * c;
      return any;
    }
  };
  auto rescale = [&](float m_old) {
    const float alpha = m_old == m_ref ? 1.f : exp2_fast((m_old - m_ref) * c);
#pragma unroll
    for (int db = 0; db < nD; ++db) acc[db] *= alpha;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      lp[i] *= alpha;
      rp[i] *= alpha;
    }
  };
  // Operand reads from a tile: only the in-row part of an address depends on the lane and the
  // k-step, so it is kept per k-step (koff) or per 32-column block of V (voff); the key-half
  // and 16-key chunk steps (32 and 16 rows) leave the swizzle unchanged and become constant
  // offsets. K fragment f = nK kb + kk: 8 bf16 of key row 32 kb + l32, logical chunk 2 kk + h.
  // V^T fragment g = nD cc + db: as tr_operand with kbase = 16 cc.
  uint32_t koff[nK], voff[nD][2];
#pragma unroll
  for (int kk = 0; kk < nK; ++kk) koff[kk] = (uint32_t)Tl::offset(l32, 2 * kk + h);
  {
    const int g4 = lane >> 4, i16 = lane & 15;
    const int row = 4 * (g4 >> 1) + (i16 >> 2);
#pragma unroll
    for (int db = 0; db < nD; ++db) {
      const int d0 = db * 32 + (g4 & 1) * 16 + 4 * (i16 & 3);
      voff[db][0] = (uint32_t)(Tl::offset(row, d0 >> 3) + (d0 & 7) * 2);
      voff[db][1] = (uint32_t)(Tl::offset(row + 8, d0 >> 3) + (d0 & 7) * 2);
    }
  }
  auto k_frag = [&](const uint8_t* Ks, int f) {
    return as_bf16x8(*reinterpret_cast<const u32x4*>(Ks + (f / nK) * 32 * Tl::RB + koff[f % nK]));
  };
  // E4M3 K fragment f = nK8 kb + kk: key row 32 kb + l32, the two 16-byte chunks of this lane
  // half in k-step kk; and the row's scale bytes, shifted like the Q scales
  auto k_frag8 = [&](const uint8_t* Ks, int f) {
    const int row = (f / nK8) * 32 + l32, kk = f % nK8;
    const u32x4 x0 = *reinterpret_cast<const u32x4*>(Ks + Tl8::offset(row, 4 * kk + h));
    const u32x4 x1 = *reinterpret_cast<const u32x4*>(Ks + Tl8::offset(row, 4 * kk + 2 + h));
    return i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                 (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
  };
  auto k_scale = [&](const uint8_t* Ks, int kb) -> uint32_t {
    const uint32_t sc = *reinterpret_cast<const uint32_t*>(Ks + Tl8::sc_offset + (32 * kb + l32) * 4);
    return sc >> (8 * h);
  };
  auto v_frag = [&](const uint8_t* Vs, int g) {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const uint8_t* base = Vs + (g / nD) * 16 * Tl::RB;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + voff[g % nD][0]));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + voff[g % nD][1]));
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
  };

  // ---- one pipelined iteration: tile j finishes, tile j+1 starts --------------------------
  // On entry: key half 0 of tile j is exponentiated, summed and packed (P[0], P[1]); cur holds
  // key half 1's scores; tile j+1's K is in kslot(j+1), tile j's V in vslot(j).
  auto iteration = [&](auto cur, auto nxt, int j, auto mask_tag, auto jp) {
    constexpr bool MASK = decltype(mask_tag)::value;   // tile j+1 may need masks
    const int lim = MASK ? tile_lim(j + 1) : 0;
    const uint8_t* Kn = kslot_p(jp, j, 1);
    const uint8_t* Vs = vslot_p(jp, j, 0);
    pm[0] = pm[1] = kNegInf;
    sync_check();

    // phase X: S of tile j+1 | key half 1 of tile j
    bf16x8 kf[QK8 ? 1 : NX];
    i32x8 kf8[QK8 ? nKF8 : 1];
    uint32_t ksc[2] = {0u, 0u};
    if constexpr (!QK8) {
      kf[0] = k_frag(Kn, 0);
      kf[1] = k_frag(Kn, 1);
    } else {
      kf8[0] = k_frag8(Kn, 0);
      kf8[1] = k_frag8(Kn, 1);
      ksc[0] = k_scale(Kn, 0);
      ksc[1] = k_scale(Kn, 1);
      // the products read the scales a few instructions after the VALU shift wrote them
      asm volatile("s_nop 4" : "+v"(ksc[0]), "+v"(ksc[1]));
    }
    bf16x8 vf[4 * nD];
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, NX>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      constexpr int kb = i / nK, kk = i % nK;
      if constexpr (!QK8 && i + 2 < NX) kf[i + 2] = k_frag(Kn, i + 2);
      // loads of K j+2 and V j+1, one per odd step (past the last tile, K j+2 loads zeros
      // into a slot nobody reads any more)
      if constexpr ((i & 1) && (i >> 1) < LK) {
        if constexpr (!QK8) ld.issue(kslot_p(jp, j, 2), Kr, (j + 2) * kBlockN, T, i >> 1);
        else if constexpr ((i >> 1) < Tl8::loadsPerWave)
          ld8.issue(kslot_p(jp, j, 2), Kr8, (j + 2) * kBlockN, T, i >> 1);
        else ld8.issue_scales(kslot_p(jp, j, 2), Ksr, (j + 2) * kBlockN, T);
      }
      if constexpr ((i & 1) && (i >> 1) >= LK && (i >> 1) < LK + Tl::loadsPerWave)
        ld.issue(vslot_p(jp, j, 1), Vr, (j + 1) * kBlockN, T, (i >> 1) - LK);
      if constexpr (i + 2 < NX && S::pvx(i + 2) >= 0) vf[S::pvx(i + 2)] = v_frag(Vs, S::pvx(i + 2));
      if constexpr (i == NX - 2) {
        vf[NPX] = v_frag(Vs, NPX);
        vf[NPX + 1] = v_frag(Vs, NPX + 1);
      }
      if constexpr (!QK8) {
        if constexpr (kk == 0) mfma_s_first(sblk(nxt, kb), kf[i], qf[kk]);
        else mfma_s(sblk(nxt, kb), kf[i], qf[kk]);
      } else if constexpr (i % 4 == 0) {
        // one E4M3 product every fourth step: fragment m = i / 4
        constexpr int m = i / 4, kb8 = m / nK8, kk8 = m % nK8;
        if constexpr (m + 2 < nKF8) kf8[m + 2] = k_frag8(Kn, m + 2);
        mfma8_s<kk8 == 0, 2 * kk8>(sblk(nxt, kb8), kf8[m], qf8[kk8], ksc[kb8], qsc);
      }
      if constexpr (S::pvx(i) >= 0) {
        constexpr int g = S::pvx(i);
        mfma_o(acc[g % nD], vf[g], p[g / nD]);
      }
      // the step's VALU work follows its product, so consecutive products are evenly spaced
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (i == S::XM0) fence_n<FX>(sblk(nxt, 0));
      static_for<16, 32>([&](auto vc) {
        constexpr int v = decltype(vc)::value;
        if constexpr (S::x_exp(v) == i) exp_item(cur, v);
        if constexpr (S::x_sum(v) == i) sum_item(cur, v);
      });
      static_for<2, 4>([&](auto cc_) {
        constexpr int ch = decltype(cc_)::value;
        if constexpr (S::x_pack(ch) == i) pack_item(cur, ch);
      });
      if constexpr (i == S::XF) fold();
      if constexpr (S::max_count(false, i) > 0)
        max_items(nxt, 0, IC<S::max_first(false, i)>{}, IC<S::max_count(false, i)>{}, MASK, lim);
      __builtin_amdgcn_sched_barrier(0);
    });

    // phase Y: P V of tile j | max, reference update and key half 0 of tile j+1
    sync_check();
    float m_old = 0.f;
    bool any = false;
    static_for<0, NY>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      constexpr int g = NPX + i, cc = g / nD, db = g % nD;
      if constexpr (i + 2 < NY) vf[g + 2] = v_frag(Vs, g + 2);
      mfma_o(acc[db], vf[g], p[cc]);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (i == S::YM0) fence_n<FY>(sblk(nxt, 1));
      if constexpr (S::max_count(true, i) > 0)
        max_items(nxt, 1, IC<S::max_first(true, i)>{}, IC<S::max_count(true, i)>{}, MASK, lim);
      if constexpr (i == S::YR) any = reduce(m_old);
      static_for<0, 16>([&](auto vc) {
        constexpr int v = decltype(vc)::value;
        if constexpr (S::y_exp(v) == i) exp_item(nxt, v);
        if constexpr (S::y_sum(v) == i) sum_item(nxt, v);
      });
      static_for<0, 2>([&](auto cc_) {
        constexpr int ch = decltype(cc_)::value;
        if constexpr (S::y_pack(ch) == i) pack_item(nxt, ch);
      });
      __builtin_amdgcn_sched_barrier(0);
    });
    if (any) {
      fence_acc(acc);
      rescale(m_old);
    }
    // this wave's loads of K j+2 and V j+1 have landed; the barrier publishes every wave's
    // part and retires kslot(j+1) and vslot(j)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  // ---- last tile: finish key half 1 and multiply (no next tile) ----------------------------
  auto last = [&](auto cur, int j) {
    sync_check();
    const uint8_t* Vs = vslot(j);
#pragma unroll
    for (int v = 16; v < 32; ++v) exp_item(cur, v);
#pragma unroll
    for (int v = 16; v < 32; ++v) sum_item(cur, v);
    pack_item(cur, 2);
    pack_item(cur, 3);
    fold();
    // the products below read P right after the VALU wrote it
    asm volatile("s_nop 7\n\ts_nop 7" : "+v"(p[2]), "+v"(p[3]));
#pragma unroll
    for (int g = 0; g < 4 * nD; ++g) mfma_o(acc[g % nD], v_frag(Vs, g), p[g / nD]);
    // the products are inline asm, whose latency the compiler does not see: the padding sits
    // here, right after them, so that no register copy the compiler places where the callers'
    // paths join can read an accumulator before its product has written it
    fence_acc(acc);
  };

  // ---- prologue: tile 0's scores, max and key half 0 -------------------------------------
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  sync_check();
  {
    const uint8_t* K0 = kslot(0);
    if constexpr (!QK8) {
#pragma unroll
      for (int f = 0; f < NX; ++f) {
        const bf16x8 a = k_frag(K0, f);
        const int kb = f / nK, kk = f % nK;
        f32x16& dst = kb ? s1a : s0;
        if (kk == 0) mfma_s_first(dst, a, qf[kk]);
        else mfma_s(dst, a, qf[kk]);
      }
    } else {
      uint32_t ksc0[2] = {k_scale(K0, 0), k_scale(K0, 1)};
      asm volatile("s_nop 4" : "+v"(ksc0[0]), "+v"(ksc0[1]));
      static_for<0, nKF8>([&](auto fc) {
        constexpr int f = decltype(fc)::value, kb = f / nK8, kk = f % nK8;
        const i32x8 a = k_frag8(K0, f);
        mfma8_s<kk == 0, 2 * kk>(kb ? s1a : s0, a, qf8[kk], ksc0[kb], qsc);
      });
    }
    fence1(s0);
    fence1(s1a);
    const bool masked = nfull == 0;
    const int lim = tile_lim(0);
    pm[0] = pm[1] = kNegInf;
#pragma unroll
    for (int u = 0; u < 16; ++u) max_item(Par<0>{}, u >> 3, u & 7, masked, lim);
    // a row that sees no key of tile 0 keeps -inf here; its exponentials are all masked to 0
    m_ref = halves_max1(fmaxf(pm[0], pm[1]));
    mc = m_ref == kNegInf ? 0.f : m_ref * c;
#pragma unroll
    for (int v = 0; v < 16; ++v) exp_item(Par<0>{}, v);
#pragma unroll
    for (int v = 0; v < 16; ++v) sum_item(Par<0>{}, v);
    pack_item(Par<0>{}, 0);
    pack_item(Par<0>{}, 1);
  }
  // every wave is done with kslot(0) before iteration 0 refills it
  __syncthreads();

  int j = 0;
  for (; j + 2 < nfull; j += 2) {
    iteration(Par<0>{}, Par<1>{}, j, Flag<false>{}, IC<0>{});
    iteration(Par<1>{}, Par<0>{}, j + 1, Flag<false>{}, IC<1>{});
  }
  // one more unmasked iteration when tile j + 1 needs no mask, after which tile j + 1's key
  // half 1 moves to the even buffer the masked tail expects
  if (j + 1 < nfull) {
    iteration(Par<0>{}, Par<1>{}, j, Flag<false>{}, IC<0>{});
    s1a = s1b;
    ++j;
  }
  // masked tail (at most the diagonal tiles): one body, the next tile's key half 1 moved into
  // the even buffer after each iteration so the roles never alternate. A wave none of whose
  // queries sees a key of the last tile (causal: the first waves of the workgroup) stops one
  // tile early: it finishes tile ntiles - 2 on its own, issues its share of the last tile's V
  // loads (the other waves read them) and meets the barrier that iteration would have held.
  const bool dead = CAUSAL && ntiles >= 2 && qw0 + 31 + shift < (ntiles - 1) * kBlockN;
  for (; j + 1 < ntiles; ++j) {
    if (dead && j + 2 == ntiles) break;
    iteration(Par<0>{}, Par<1>{}, j, Flag<true>{}, IC<-1>{});
    s1a = s1b;
  }
  // one call of the last-tile body on both paths, so that the accumulators stay in the same
  // registers (two calls made the compiler copy them between register blocks at the join)
  const bool early = dead && j + 2 == ntiles;
  if (early) {
#pragma unroll
    for (int i = 0; i < Tl::loadsPerWave; ++i) ld.issue(vslot(j + 1), Vr, (j + 1) * kBlockN, T, i);
  }
  last(Par<0>{}, j);
  if (early) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  const float l_half = lp[0] + lp[1];
  const float r_half = rp[0] + rp[1];
  const float l_tot = l_half + swap_halves(l_half);
  const float r_tot = r_half + swap_halves(r_half);
  if (qrow < Tq) {
    // a row that sees no key at all (causal, fewer keys than queries) gets O = 0, LSE = -inf
    const float inv = r_tot > 0.f ? 1.0f / r_tot : 0.f;
    uint16_t* orow = Oh + (int64_t)qrow * args.q_rs;
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
    if (h == 0) Lh[qrow] = l_tot > 0.f ? (m_ref * c + log2_fast(l_tot)) * kLn2 : kNegInf;
  }
}

template <int D, bool CAUSAL, bool QK8>
hipError_t launch(const FwdBf16Problem& p) {
  FwdKArgs k{};
  k.q8 = static_cast<const uint8_t*>(p.q8);
  k.k8 = static_cast<const uint8_t*>(p.k8);
  k.qs = static_cast<const uint8_t*>(p.q_scale);
  k.ks = static_cast<const uint8_t*>(p.k_scale);
  k.q = static_cast<const uint16_t*>(p.q);
  k.k = static_cast<const uint16_t*>(p.k);
  k.v = static_cast<const uint16_t*>(p.v);
  k.o = static_cast<uint16_t*>(p.o);
  k.lse = p.lse;
  k.cu_q = p.cu_q;
  k.cu_k = p.cu_k;
  k.G = p.Hq / p.Hkv;
  k.hpw_log2 = k.G % 4 == 0 ? 2 : (k.G % 2 == 0 ? 1 : 0);
  k.HG = p.Hq >> k.hpw_log2;
  k.nbhg = p.B * k.HG;
  k.nq = (p.max_q + (kBlockM >> k.hpw_log2) - 1) / (kBlockM >> k.hpw_log2);
  // four (batch, head group)s at a time on each XCD: their K and V (2 MB each at T = 4096,
  // D = 128) stay about within the XCD's 4 MB L2 while all their query tiles read them
  k.grp = xcd_group(k.nbhg);
  k.Tq = p.Tq;
  k.Tk = p.Tk;
  if (p.cu_q) {   // packed (rows, heads, D)
    k.q_rs = p.Hq * D;
    k.kv_rs = p.Hkv * D;
    k.q_bs = k.kv_bs = 0;
    k.q_hs = D;
    k.kv_hs = D;
    k.lse_bs = 0;
    k.lse_hs = p.Tq;
  } else {        // (B, heads, rows, D)
    k.q_rs = k.kv_rs = D;
    k.q_hs = (int64_t)p.Tq * D;
    k.kv_hs = (int64_t)p.Tk * D;
    k.q_bs = (int64_t)p.Hq * k.q_hs;
    k.kv_bs = (int64_t)p.Hkv * k.kv_hs;
    k.lse_hs = p.Tq;
    k.lse_bs = (int64_t)p.Hq * p.Tq;
  }
  k.c = p.scale * 1.44269504088896340736f;
  k.B = p.B;
  int64_t grid = (int64_t)k.nq * k.nbhg;
  // skewed packed batches (the longest sequence at least 2048 rows and at least 2.5 times the
  // mean length) of up to 64 sequences (one per lane) with whole XCD shares of head groups:
  // longest sequence first, no workgroups for tiles past a sequence's end (varlen_item). Batches
  // of even or short lengths keep the grouped order, which measured faster for them.
  if (p.cu_q && p.B <= 64 && k.HG % 8 == 0 && p.max_q >= 2048 &&
      (int64_t)p.Tq * 5 <= (int64_t)p.B * p.max_q * 2) {
    const int64_t qr = kBlockM >> k.hpw_log2;
    const int64_t tiles = ((int64_t)p.Tq + (int64_t)p.B * (qr - 1)) / qr;   // >= sum of tile counts
    k.vsched = 1;
    grid = (int64_t)k.HG * (tiles < (int64_t)p.B * k.nq ? tiles : (int64_t)p.B * k.nq);
  }
  hipLaunchKernelGGL((fwd_q32_kernel<D, CAUSAL, QK8>), dim3((unsigned)grid), dim3(kThreads), 0, p.stream, k);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16_general(const FwdBf16Problem& p) {
  if (p.q8) {
    if (p.D == 64) return p.causal ? launch<64, true, true>(p) : launch<64, false, true>(p);
    return p.causal ? launch<128, true, true>(p) : launch<128, false, true>(p);
  }
  if (p.D == 64) return p.causal ? launch<64, true, false>(p) : launch<64, false, false>(p);
  return p.causal ? launch<128, true, false>(p) : launch<128, false, false>(p);
}

hipError_t launch_fwd_bf16(const FwdArgs& a) {
  const FwdBf16Problem p{a.q, a.k, a.v, a.o, a.lse, nullptr, nullptr, a.B, a.H, a.H, a.D,
                         a.T, a.T, a.T, a.scale, a.causal, a.stream};
  return launch_fwd_bf16_general(p);
}

}  // namespace fa
