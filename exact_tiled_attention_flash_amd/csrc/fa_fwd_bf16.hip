// Attention forward, bf16 storage, fp32 accumulation: hand-written gfx950 kernel with two
// 32-query blocks per wave and one wave per SIMD. It runs the E4M3 Q K^T variant; with bf16 Q
// and K the forward runs fwd_q32_kernel (one block per wave, two workgroups per compute unit),
// which has the same arithmetic, and the QK8 = false code below is not instantiated.
//
// Method: "Lab 06 - Attention kernels", section 3 (per query tile keep the row max m, row
// sum l and accumulator acc; per key tile rescale by exp(m - m') and add exp(S - m') V;
// finish with O = acc / l and LSE = m + log l; causal tiles above the diagonal are never
// loaded, diagonal tiles are masked element-wise) and section 5 (one program per
// (query tile, batch*head)). "Triton FlashAttention-2 forward", "The kernel" (queries
// outermost, P rounded to the input dtype before the P V product, masked loads read zeros
// beyond T). Section 2 of the lab page: subtracting any constant from the exponents and
// dividing it back out is exact, which the lazy reference below relies on.
//
// gfx950 mapping
//   * Workgroup: 256 threads = 4 waves, one per SIMD; 256 queries of one (b, h), 64 per
//     wave as two 32-query blocks. Every K / V operand read from LDS feeds two
//     matrix-core products (one per query block), which halves LDS traffic per flop
//     compared with 32 queries per wave.
//   * S^T = K Q^T (v_mfma_f32_32x32x16_bf16) puts one query per lane: a row's 64 scores of
//     a tile sit in 32 registers of lane l and 32 of lane l ^ 32. The S^T accumulator
//     layout is the B-operand layout of O^T += V^T P^T, so P never leaves registers; the
//     V^T A operand is a transposing LDS read (ds_read_b64_tr_b16) of the row-major tile.
//   * K and V tiles (64 keys) reach LDS by direct buffer -> LDS loads into XOR-swizzled
//     row-major tiles, two slots each; K runs one tile ahead of V (see the pipeline). The
//     buffer resource ends at the last key row, so rows past it arrive as zeros and a load
//     costs no vector arithmetic. The loads are inline asm, out of the compiler's sight:
//     it would otherwise wait for every outstanding LDS read wherever it needs one of them.
//   * exp(x) is exp2(x * scale * log2 e): one FMA and one v_exp_f32.
//   * Lazy reference: a row's reference max m_ref moves only when a tile max exceeds it by
//     more than 2^8 in the exp2 domain (and on the first tile), so P <= 2^8 and the O^T
//     accumulators are rescaled in a rare wave-uniform branch, never in the steady state.
//     O is normalised by the sum of the bf16-rounded P that actually multiplied V, so a
//     dominant key's rounding cancels between numerator and denominator; LSE uses the
//     fp32 sum of the unrounded exponentials.
//   * Software pipeline across key tiles, one wave: phase X of iteration j runs the S
//     products of tile j+1 on the matrix cores while the VALU finishes tile j (the last
//     exponentials, fp32 and rounded row sums, bf16 packing); phase Y runs tile j's
//     P V products while the VALU takes tile j+1's row max, moves the references and
//     starts its exponentials. Each step of a phase holds one matrix-core product and a
//     fixed share of the VALU work, fenced with sched_barrier so the compiler keeps the
//     interleaving.
//   * Causal grid order is heaviest query tile first; consecutive workgroup ids walk
//     (b, h) fastest, which keeps all tiles of one head on one XCD (workgroups are dealt
//     to the 8 XCDs round-robin) so K and V of a head are shared through that XCD's L2.

#include "fa_common.h"
#include "fa_launch.h"
#include "fa_swz.h"
#include "fa_fwd_parts.h"

namespace fa {
namespace {

using namespace fwd;

constexpr int kThreads = 256;
constexpr int kBlockM = 256;   // queries per workgroup

// E4M3 variant of the S products: 32 x 32 x 64 with a power-of-two scale per 32 k-values.
// Lane l supplies row (A) / column (B) l % 32; its bytes 0-15 are k-values 16 (l / 32) + 0..15
// of the first 32-value block and bytes 16-31 the same positions of the second block; the
// scale of block q of a row comes from lane row + 32 q, byte BYTE of its scale register
// (op_sel carries bit 0 of BYTE, op_sel_hi bit 1).
typedef int i32x8 __attribute__((ext_vector_type(8)));
template <bool FIRST, int BYTE>
__device__ __forceinline__ void mfma8_s(f32x16& d, const i32x8& a, const i32x8& b, uint32_t sa,
                                        uint32_t sb) {
  static_assert(BYTE == 0 || BYTE == 2, "scale byte");
  if constexpr (FIRST && BYTE == 0)
    asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, 0, %3, %4"
                 : "=&v"(d) : "v"(a), "a"(b), "v"(sa), "v"(sb));
  else if constexpr (FIRST)
    asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, 0, %3, %4 op_sel_hi:[1,1,0]"
                 : "=&v"(d) : "v"(a), "a"(b), "v"(sa), "v"(sb));
  else if constexpr (BYTE == 0)
    asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4"
                 : "+v"(d) : "v"(a), "a"(b), "v"(sa), "v"(sb));
  else
    asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[1,1,0]"
                 : "+v"(d) : "v"(a), "a"(b), "v"(sa), "v"(sb));
}

// A [64 x D] E4M3 tile in LDS (D bytes a row, 16-byte chunks XOR-swizzled so that 8 (D = 128)
// or 4 (D = 64) consecutive rows reading one logical chunk hit distinct banks for 32 and for
// 64 banks), followed by its block-scale bytes: D / 32 per row, in one dword per row (a direct
// HBM -> LDS load of 1 or 2 bytes a lane writes a zero-extended dword a lane).
template <int D>
struct SwzTile8 {
  static constexpr int CH = D / 16;
  static constexpr int RB = D;
  static constexpr int SB = D / 32;     // scale bytes per row in HBM
  static constexpr int sc_offset = 64 * RB;
  static constexpr int loadsPerWave = 64 * CH / 256;
  __device__ static __forceinline__ int swz(int row) { return D == 128 ? (row & 7) : ((row >> 1) & 3); }
  __device__ static __forceinline__ int offset(int row, int lchunk) {
    return row * RB + ((lchunk ^ swz(row)) << 4);
  }
};

// Direct HBM -> LDS loads of a 64-row E4M3 tile and its scales by the 4 waves of a workgroup
// (the same lane-to-chunk rule as TileLoader); wave 0 also moves the 64 rows' scale bytes.
template <int D>
struct TileLoader8 {
  using Tl = SwzTile8<D>;
  uint32_t vofs[Tl::loadsPerWave];   // byte offset of the lane's i-th chunk from the tile's row 0
  int wave, lane;
  uint32_t rsb, srs;   // bytes between rows of the codes and of the scales
  __device__ __forceinline__ TileLoader8(int wave_, int lane_, int row_stride)
      : wave(wave_), lane(lane_), rsb((uint32_t)row_stride), srs((uint32_t)row_stride / 32u) {
#pragma unroll
    for (int i = 0; i < Tl::loadsPerWave; ++i) {
      const int u = (wave * Tl::loadsPerWave + i) * 64 + lane;
      const int row = u / Tl::CH;
      vofs[i] = (uint32_t)row * rsb + (uint32_t)(((u % Tl::CH) ^ Tl::swz(row)) * 16);
    }
  }
  // codes and scales come through buffer resources over the T rows (rows at or past T: zeros)
  __device__ __forceinline__ void issue(uint8_t* dst, const i32x4& rsrc, int row0, int T,
                                        int i) const {
    buf_lds_dma<16>(dst + (wave * Tl::loadsPerWave + i) * 1024, rsrc, vofs[i],
                    (uint32_t)min(row0, T) * rsb);
  }
  __device__ __forceinline__ void issue_scales(uint8_t* dst, const i32x4& srsrc, int row0,
                                               int T) const {
    if (wave == 0)
      buf_lds_dma<Tl::SB>(dst + Tl::sc_offset, srsrc, (uint32_t)lane * srs,
                          (uint32_t)min(row0, T) * srs);
  }
  __device__ __forceinline__ void issue_all(uint8_t* dst, const i32x4& rsrc, const i32x4& srsrc,
                                            int row0, int T) const {
#pragma unroll
    for (int i = 0; i < Tl::loadsPerWave; ++i) issue(dst, rsrc, row0, T, i);
    issue_scales(dst, srsrc, row0, T);
  }
};


// ---- per-step work assignment (all compile-time) --------------------------------------
// Items of one tile: 64 score elements per lane, v = 32 qb + 16 kb + r; 8 chunks of 8
// (v / 8 = 4 qb + cc, the B operand P[qb][cc]); 16 max items per key half (pairs of
// elements). Query block 0 of a tile is finished in phase Y of the iteration before it is
// used, query block 1 in phase X of its own iteration.

template <int D>
struct Sched {
  static constexpr int nK = D / 16, nD = D / 32;
  static constexpr int NX = 4 * nK;                  // phase X steps (S products)
  static constexpr int NY = 8 * nD;                  // phase Y steps (P V products)
  // phase Y: max over key half kb = 1, reference update, then query block 0's
  // exponentials, sums and packing
  static constexpr int YM0 = 2, YM1 = 2 + NY / 4, YR = YM1, YE0 = YR + 1, YE1 = NY - NY / 8;
  static constexpr int YS0 = YE0 + 1, YS1 = NY;
  // phase X: query block 1's exponentials, sums and packing, then the fold of the tile's
  // sums; max over key half kb = 0 of the next tile once its products are done
  static constexpr int XE0 = 0, XE1 = NX / 2, XS0 = 1, XS1 = NX / 2 + 4;
  static constexpr int XM0 = NX / 2 + 2, XM1 = NX;
  static constexpr int y_exp(int v) { return win_step(v, 32, YE0, YE1); }
  static constexpr int y_sum(int v) { return win_step(v, 32, YS0, YS1); }
  static constexpr int x_exp(int v) { return win_step(v - 32, 32, XE0, XE1); }
  static constexpr int x_sum(int v) { return win_step(v - 32, 32, XS0, XS1); }
  // a chunk is packed one step after its last exponential
  static constexpr int y_pack(int ch) { return y_exp(8 * ch + 7) + 1; }
  static constexpr int x_pack(int ch) { return x_exp(8 * ch + 7) + 1; }
  static constexpr int XF = (x_sum(63) > x_pack(7) ? x_sum(63) : x_pack(7)) + 1;
  static constexpr int x_max(int u) { return win_step(u, 16, XM0, XM1); }   // kb = 0
  static constexpr int y_max(int u) { return win_step(u, 16, YM0, YM1); }   // kb = 1
  // every sum and pack comes after the exponentials it reads, within its phase
  static constexpr bool valid() {
    for (int v = 0; v < 32; ++v)
      if (y_sum(v) <= y_exp(v) || y_sum(v) >= NY || y_pack(v / 8) >= NY) return false;
    for (int v = 32; v < 64; ++v)
      if (x_sum(v) <= x_exp(v) || x_sum(v) >= NX) return false;
    return YR < YE0 && XE1 <= NX && XF < NX && y_max(15) < YR;
  }
};
static_assert(Sched<128>::valid() && Sched<64>::valid(), "pipeline schedule order");


template <int D, bool CAUSAL, bool QK8>
__global__ __launch_bounds__(kThreads, 1) void fwd_bf16_kernel(const FwdKArgs args) {
  using Tl = SwzTile<D>;
  using S = Sched<D>;
  constexpr int nD = D / 32;   // 32-row blocks of O^T
  constexpr int nK = D / 16;   // k-steps of S^T
  constexpr int nKF = 2 * nK;  // K operand fragments per tile: f = nK kb + kk
  constexpr int nVF = 4 * nD;  // V operand fragments per tile: g = nD cc + db
  using Tl8 = SwzTile8<D>;
  constexpr int nK8 = D / 64;    // k-steps of an E4M3 S product
  constexpr int nKF8 = 2 * nK8;  // E4M3 K fragments per tile: f = nK8 kb + kk
  // odd steps of phase X that issue K loads (E4M3: the codes, then one for the scales)
  constexpr int LK = QK8 ? Tl8::loadsPerWave + 1 : Tl::loadsPerWave;
  // Two slots per tensor, each its own LDS object: where the slot parity is known at compile
  // time the compiler can tell a slot being refilled by DMA from the one being read, and
  // need not wait for the DMA before every LDS read.
  __shared__ __attribute__((aligned(1024))) uint8_t ks0[Tl::bytes], ks1[Tl::bytes];
  __shared__ __attribute__((aligned(1024))) uint8_t vs0[Tl::bytes], vs1[Tl::bytes];

  const int tid = lane_thread_id();
  const int wave = wave_id();
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int h = lane >> 5;

  const float c = args.c;
  // Workgroup -> (query tile, batch, head group): heaviest causal tiles first, (batch, head
  // group) fastest. A workgroup serves hpw query heads that share one K/V head, each with
  // 256 / hpw consecutive queries (64 per wave), so every K/V tile it loads feeds all of them.
  const int L = workgroup_id();
  const int r = L % args.nbhg;
  int qt = L / args.nbhg;
  if (CAUSAL) qt = args.nq - 1 - qt;
  const int b = r / args.HG, hg = r % args.HG;
  const int hpw = 1 << args.hpw_log2;
  const int h0 = hg * hpw;
  const int hq = h0 + (wave & (hpw - 1));             // this wave's query head
  const int kvh = h0 / args.G;                            // the workgroup's K/V head
  const int qrows = kBlockM >> args.hpw_log2;             // queries per head in this workgroup
  // sequence bounds (packed batches: clamped into the arrays whatever the offsets hold)
  int qs = 0, Tq = args.Tq, ks = 0, Tk = args.Tk;
  if (args.cu_q) {
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
  if (q0 >= Tq) return;   // past this sequence's queries (packed batches); uniform per workgroup
  const int qw0 = q0 + (wave >> args.hpw_log2) * 64;
  const int shift = CAUSAL ? Tk - Tq : 0;   // bottom-right alignment: 0 when Tq == Tk

  const uint16_t* Qh = args.q + b * args.q_bs + (int64_t)qs * args.q_rs + hq * args.q_hs;
  uint16_t* Oh = args.o + b * args.q_bs + (int64_t)qs * args.q_rs + hq * args.q_hs;
  float* Lh = args.lse + b * args.lse_bs + hq * args.lse_hs + qs;
  const uint16_t* Kh = args.k + b * args.kv_bs + (int64_t)ks * args.kv_rs + kvh * args.kv_hs;
  const uint16_t* Vh = args.v + b * args.kv_bs + (int64_t)ks * args.kv_rs + kvh * args.kv_hs;
  const int T = Tk;   // key rows of this sequence (tile rows at or past T load as zeros)
  auto kslot = [&](int t) -> uint8_t* { return (t & 1) ? ks1 : ks0; };
  auto vslot = [&](int t) -> uint8_t* { return (t & 1) ? vs1 : vs0; };
  // jp: parity of j as IC<0> / IC<1>, or IC<-1> when only known at run time
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

  // Q^T fragments stay in registers: query block qb, lane holds query qw0 + 32 qb + l32,
  // d = 16 kk + 8 h + 0..7. E4M3: codes of k-step kk at d = 64 kk + 16 h + 0..15 and
  // 64 kk + 32 + 16 h + 0..15, and the row's scale bytes shifted so that byte 2 kk is block
  // 2 kk + h (the block whose scale this lane half supplies).
  bf16x8 qf[2][QK8 ? 1 : nK];
  i32x8 qf8[2][QK8 ? nK8 : 1];
  uint32_t qsc[2] = {0u, 0u};
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qrow = qw0 + 32 * qb + l32;
    if constexpr (!QK8) {
#pragma unroll
      for (int kk = 0; kk < nK; ++kk) {
        u32x4 x = qrow < Tq
                      ? *reinterpret_cast<const u32x4*>(Qh + (int64_t)qrow * args.q_rs + kk * 16 + h * 8)
                      : u32x4{0u, 0u, 0u, 0u};
        qf[qb][kk] = as_bf16x8(x);
      }
    } else {
      const int64_t qe = b * args.q_bs + (int64_t)(qs + qrow) * args.q_rs + hq * args.q_hs;
      const uint8_t* Qr = args.q8 + qe;
#pragma unroll
      for (int kk = 0; kk < nK8; ++kk) {
        u32x4 x0 = {0u, 0u, 0u, 0u}, x1 = {0u, 0u, 0u, 0u};
        if (qrow < Tq) {
          x0 = *reinterpret_cast<const u32x4*>(Qr + 64 * kk + 16 * h);
          x1 = *reinterpret_cast<const u32x4*>(Qr + 64 * kk + 32 + 16 * h);
        }
        qf8[qb][kk] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                            (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
      }
      uint32_t sc = 0x7f7f7f7fu;
      if (qrow < Tq) {
        const uint8_t* Qs = args.qs + qe / 32;
        sc = D == 128 ? *reinterpret_cast<const uint32_t*>(Qs) : *reinterpret_cast<const uint16_t*>(Qs);
      }
      qsc[qb] = sc >> (8 * h);
    }
  }
  // Move Q^T into AGPRs now and pad the accumulator writes before any product reads them.
  if constexpr (!QK8) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int kk = 0; kk < nK; ++kk) asm volatile("" : "+a"(qf[qb][kk]));
    asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int kk = 0; kk < nK; ++kk) asm volatile("" : "+a"(qf[qb][kk]));
  } else {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int kk = 0; kk < nK8; ++kk) asm volatile("" : "+a"(qf8[qb][kk]));
      asm volatile("" : "+v"(qsc[qb]));
    }
    asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int kk = 0; kk < nK8; ++kk) asm volatile("" : "+a"(qf8[qb][kk]));
      asm volatile("" : "+v"(qsc[qb]));
    }
  }

  // keys seen by the workgroup's last query, and by all of its queries
  const int kend = CAUSAL ? min(Tk, q0 + qrows + shift) : Tk;
  const int ntiles = kend > 0 ? (kend + kBlockN - 1) / kBlockN : 0;
  const int kall = CAUSAL ? min(Tk, q0 + shift + 1) : Tk;
  // tiles [0, nfull) need no mask for any query of this workgroup
  const int nfull = kall > 0 ? min(kall / kBlockN, ntiles) : 0;

  if (ntiles == 0) {   // no query of this workgroup sees a key (uniform per workgroup)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qrow = qw0 + 32 * qb + l32;
      if (qrow < Tq) {
        uint16_t* orow = Oh + (int64_t)qrow * args.q_rs;
#pragma unroll
        for (int d0 = 0; d0 < D; d0 += 8)
          if ((d0 / 8) % 2 == h) *reinterpret_cast<u32x4*>(orow + d0) = u32x4{0u, 0u, 0u, 0u};
        if (h == 0) Lh[qrow] = kNegInf;
      }
    }
    return;
  }

  f32x16 acc[2][nD];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < nD; ++db) acc[qb][db] = f32x16{};
  float m_ref[2], mc[2];            // reference max (raw score units) and m_ref * c
  // row sums per (qb, key half kb): fp32 exponentials (l) and bf16-rounded P (r), for the
  // tiles already folded in (lp, rp) and for the tile in progress (tl, tr), which may
  // already use a newer reference
  float lp[2][2] = {{0.f, 0.f}, {0.f, 0.f}}, rp[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
  float tl[2][2] = {{0.f, 0.f}, {0.f, 0.f}}, tr[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
  float pm[2][2];                   // partial row maxima of the next tile, per (qb, kb)
  // Scores -> exponentials and the bf16 P of a tile, per query block. Query block 0 of a
  // tile is finished in the iteration before the tile's own, so its buffers are free again
  // when the next tile's products start: one score buffer for block 0, two for block 1
  // (tile parity); P of block 0 is double-buffered, P of block 1 single.
  f32x16 s0[2], s1a[2], s1b[2];
  bf16x8 p0a[4], p0b[4], p1[4];
  // buffers of a tile of parity par: score block (qb, kb), P operand (qb, cc)
  auto sblk = [&](auto par, int qb, int kb) -> f32x16& {
    if constexpr (decltype(par)::value == 0) return qb ? s1a[kb] : s0[kb];
    else return qb ? s1b[kb] : s0[kb];
  };
  auto pop = [&](auto par, int qb, int cc) -> bf16x8& {
    if constexpr (decltype(par)::value == 0) return qb ? p1[cc] : p0a[cc];
    else return qb ? p1[cc] : p0b[cc];
  };
  const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3f803f80u);

  // element (kb, r) of a lane is key 32 kb + 8 (r / 4) + (r % 4) + 4 h of the tile; it is
  // valid for query block qb iff that local index is below lim[qb]
  auto tile_lim = [&](int t, int (&lim)[2]) {
    const int k0 = t * kBlockN;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      int l = Tk - k0;
      if (CAUSAL) l = min(l, qw0 + 32 * qb + l32 + shift - k0 + 1);
      lim[qb] = l - 4 * h;
    }
  };

  // ---- work items ------------------------------------------------------------------------
  auto max_item = [&](auto par, int qb, int kb, int t, bool masked, const int (&lim)[2]) {
    f32x16& x = sblk(par, qb, kb);
    float a = x[2 * t], b = x[2 * t + 1];
    if (masked) {
      const int kla = 32 * kb + 8 * (t >> 1) + 2 * (t & 1);
      a = kla < lim[qb] ? a : kNegInf;
      b = kla + 1 < lim[qb] ? b : kNegInf;
      x[2 * t] = a;
      x[2 * t + 1] = b;
    }
    // one v_max3 per pair (left to itself the compiler reassociates the chain into a tree
    // of twice as many instructions); the scores' producers are fenced before the first item
    float m = pm[qb][kb];
    asm volatile("v_max3_f32 %0, %0, %1, %2" : "+v"(m) : "v"(a), "v"(b));
    pm[qb][kb] = m;
  };
  auto exp_item = [&](auto par, int v, bool masked) {
    const int qb = v >> 5, kb = (v >> 4) & 1, r = v & 15;
    f32x16& blk = sblk(par, qb, kb);
    const float x = blk[r];
    const float e = exp2_fast(fmaf(x, c, -mc[qb]));
    blk[r] = (masked && x == kNegInf) ? 0.f : e;
  };
  // The sums are pinned to their step with an empty asm that takes them as operands:
  // otherwise the compiler sinks the whole chain of additions to the end of the iteration,
  // where it runs as one block with no product to hide under.
  auto sum_item = [&](auto par, int v) {
    const int qb = v >> 5, kb = (v >> 4) & 1, r = v & 15;
    tl[qb][kb] += sblk(par, qb, kb)[r];
    asm volatile("" : "+v"(tl[qb][kb]));
  };
  // Pack chunk ch to the bf16 B operand and add the rounded values. The words are summed
  // before they are gathered into the operand vector: with this toolchain,
  // v_dot2c_f32_bf16 applied to an element of a 4-vector reads the vector's first register
  // for the second element too.
  auto pack_item = [&](auto spar, auto ppar, int ch) {
    const int qb = ch >> 2, cc = ch & 3, kb = cc >> 1, o = (cc & 1) * 8;
    const f32x16& sv = sblk(spar, qb, kb);
    const uint32_t w0 = pack_bf16x2(sv[o + 0], sv[o + 1]), w1 = pack_bf16x2(sv[o + 2], sv[o + 3]);
    const uint32_t w2 = pack_bf16x2(sv[o + 4], sv[o + 5]), w3 = pack_bf16x2(sv[o + 6], sv[o + 7]);
    tr[qb][0] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w0), ones, tr[qb][0], false);
    tr[qb][1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w1), ones, tr[qb][1], false);
    tr[qb][0] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w2), ones, tr[qb][0], false);
    tr[qb][1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w3), ones, tr[qb][1], false);
    asm volatile("" : "+v"(tr[qb][0]), "+v"(tr[qb][1]));
    pop(ppar, qb, cc) = as_bf16x8(u32x4{w0, w1, w2, w3});
  };
  // the finished tile's sums join the running sums (same reference by now)
  auto fold = [&]() {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        lp[qb][kb] += tl[qb][kb];
        rp[qb][kb] += tr[qb][kb];
        tl[qb][kb] = 0.f;
        tr[qb][kb] = 0.f;
      }
  };
  // Full-row maxima of the next tile; moves the references (all rows of the wave together,
  // when any row exceeds its reference by more than the margin) and returns whether the
  // folded sums and the accumulators need the rescale by exp(m_old - m_ref).
  auto reduce = [&](float (&m_old)[2]) {
    float a = fmaxf(pm[0][0], pm[0][1]), b = fmaxf(pm[1][0], pm[1][1]);
    halves_max2(a, b, h);
    // (a reference still at -inf belongs to a row that has not seen a key yet)
    const bool need = (a - m_ref[0]) * c > kRescaleLog2 || (b - m_ref[1]) * c > kRescaleLog2 ||
                      m_ref[0] == kNegInf || m_ref[1] == kNegInf;
    const bool any = __builtin_amdgcn_ballot_w64(need) != 0;
    m_old[0] = m_ref[0];
    m_old[1] = m_ref[1];
    m_ref[0] = any ? fmaxf(m_ref[0], a) : m_ref[0];
    m_ref[1] = any ? fmaxf(m_ref[1], b) : m_ref[1];
    mc[0] = m_ref[0] * c;
    mc[1] = m_ref[1] * c;
    return any;
  };
  auto rescale = [&](const float (&m_old)[2]) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float alpha = m_old[qb] == m_ref[qb] ? 1.f : exp2_fast((m_old[qb] - m_ref[qb]) * c);
#pragma unroll
      for (int db = 0; db < nD; ++db) acc[qb][db] *= alpha;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        lp[qb][kb] *= alpha;
        rp[qb][kb] *= alpha;
      }
    }
  };
  auto reset_max = [&]() {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) pm[qb][0] = pm[qb][1] = kNegInf;
  };
  auto k_frag = [&](const uint8_t* Ks, int f) {
    return row_operand<D>(Ks, (f / nK) * 32 + l32, 2 * (f % nK) + h);
  };
  auto v_frag = [&](const uint8_t* Vs, int g) { return tr_operand<D>(Vs, g % nD, 16 * (g / nD), lane); };
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

  // ---- one pipelined iteration: tile j finishes, tile j+1 starts --------------------------
  // On entry: query block 0 of tile j is exponentiated, summed (tl, tr) and packed (pc);
  // cur holds query block 1's scores; tile j+1's K is in kslot(j+1), tile j's V in vslot(j).
  // cur / nxt: parity tags of tile j and tile j+1
  auto iteration = [&](auto cur, auto nxt, int j, auto mask_tag, auto jp) {
    constexpr bool MASK = decltype(mask_tag)::value;   // tile j or j+1 may need masks
    int lim[2];
    if (MASK) tile_lim(j + 1, lim);
    const uint8_t* Kn = kslot_p(jp, j, 1);
    const uint8_t* Vs = vslot_p(jp, j, 0);
    reset_max();

    // phase X: S of tile j+1 | query block 1 of tile j
    bf16x8 kf[QK8 ? 1 : nKF];
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
    bf16x8 vf[nVF];
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, S::NX>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      constexpr int f = i >> 1, qb = i & 1, kb = f / nK, kk = f % nK;
      if constexpr (!QK8 && qb == 0 && f + 2 < nKF) kf[f + 2] = k_frag(Kn, f + 2);
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
      if constexpr (i == S::NX - 2) {
        vf[0] = v_frag(Vs, 0);
        vf[1] = v_frag(Vs, 1);
      }
      if constexpr (!QK8) {
        if constexpr (kk == 0) mfma_s_first(sblk(nxt, qb, kb), kf[f], qf[qb][kk]);
        else mfma_s(sblk(nxt, qb, kb), kf[f], qf[qb][kk]);
      } else if constexpr (i % 4 == 0) {
        // one E4M3 product every fourth step: m = i / 4 -> query block m % 2, fragment m / 2
        constexpr int m = i / 4, qb8 = m & 1, f8 = m >> 1, kb8 = f8 / nK8, kk8 = f8 % nK8;
        if constexpr (qb8 == 0 && f8 + 2 < nKF8) kf8[f8 + 2] = k_frag8(Kn, f8 + 2);
        mfma8_s<kk8 == 0, 2 * kk8>(sblk(nxt, qb8, kb8), kf8[f8], qf8[qb8][kk8], ksc[kb8], qsc[qb8]);
      }
      if constexpr (i == S::XM0) fence2(sblk(nxt, 0, 0), sblk(nxt, 1, 0));
      static_for<32, 64>([&](auto vc) {
        constexpr int v = decltype(vc)::value;
        if constexpr (S::x_exp(v) == i) exp_item(cur, v, MASK);
        if constexpr (S::x_sum(v) == i) sum_item(cur, v);
      });
      static_for<4, 8>([&](auto cc_) {
        constexpr int ch = decltype(cc_)::value;
        if constexpr (S::x_pack(ch) == i) pack_item(cur, cur, ch);
      });
      if constexpr (i == S::XF) fold();
      static_for<0, 16>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        if constexpr (S::x_max(u) == i) max_item(nxt, u >> 3, 0, u & 7, MASK, lim);
      });
      __builtin_amdgcn_sched_barrier(0);
    });

    // phase Y: P V of tile j | max, reference update and query block 0 of tile j+1
    float m_old[2];
    bool any = false;
    static_for<0, S::NY>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      constexpr int g = i >> 1, qb = i & 1, cc = g / nD, db = g % nD;
      if constexpr (qb == 0 && g + 2 < nVF) vf[g + 2] = v_frag(Vs, g + 2);
      mfma_o(acc[qb][db], vf[g], pop(cur, qb, cc));
      if constexpr (i == S::YM0) fence2(sblk(nxt, 0, 1), sblk(nxt, 1, 1));
      static_for<0, 16>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        if constexpr (S::y_max(u) == i) max_item(nxt, u >> 3, 1, u & 7, MASK, lim);
      });
      if constexpr (i == S::YR) any = reduce(m_old);
      static_for<0, 32>([&](auto vc) {
        constexpr int v = decltype(vc)::value;
        if constexpr (S::y_exp(v) == i) exp_item(nxt, v, MASK);
        if constexpr (S::y_sum(v) == i) sum_item(nxt, v);
      });
      static_for<0, 4>([&](auto cc_) {
        constexpr int ch = decltype(cc_)::value;
        if constexpr (S::y_pack(ch) == i) pack_item(nxt, nxt, ch);
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

  // ---- last tile: finish query block 1 and multiply (no next tile) -------------------------
  auto last = [&](auto cur, int j) {
    const uint8_t* Vs = vslot(j);
#pragma unroll
    for (int v = 32; v < 64; ++v) exp_item(cur, v, true);
#pragma unroll
    for (int v = 32; v < 64; ++v) sum_item(cur, v);
#pragma unroll
    for (int ch = 4; ch < 8; ++ch) pack_item(cur, cur, ch);
    fold();
    // the products below read P right after the VALU wrote it
    asm volatile("s_nop 7\n\ts_nop 7" : "+v"(p1[0]), "+v"(p1[1]), "+v"(p1[2]), "+v"(p1[3]));
#pragma unroll
    for (int g = 0; g < nVF; ++g) {
      const bf16x8 a = v_frag(Vs, g);
      const int cc = g / nD, db = g % nD;
      mfma_o(acc[0][db], a, pop(cur, 0, cc));
      mfma_o(acc[1][db], a, pop(cur, 1, cc));
    }
  };

  // ---- prologue: tile 0's scores, max and query block 0 ---------------------------------
  if constexpr (!QK8) {
    ld.issue_all(kslot(0), Kr, 0, T);
    ld.issue_all(vslot(0), Vr, 0, T);
    if (ntiles > 1) ld.issue_all(kslot(1), Kr, kBlockN, T);
  } else {
    ld8.issue_all(kslot(0), Kr8, Ksr, 0, T);
    ld.issue_all(vslot(0), Vr, 0, T);
    if (ntiles > 1) ld8.issue_all(kslot(1), Kr8, Ksr, kBlockN, T);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  {
    const uint8_t* K0 = kslot(0);
    if constexpr (!QK8) {
#pragma unroll
      for (int f = 0; f < nKF; ++f) {
        const bf16x8 a = k_frag(K0, f);
        const int kb = f / nK, kk = f % nK;
        if (kk == 0) {
          mfma_s_first(s0[kb], a, qf[0][kk]);
          mfma_s_first(s1a[kb], a, qf[1][kk]);
        } else {
          mfma_s(s0[kb], a, qf[0][kk]);
          mfma_s(s1a[kb], a, qf[1][kk]);
        }
      }
    } else {
      uint32_t ksc0[2] = {k_scale(K0, 0), k_scale(K0, 1)};
      asm volatile("s_nop 4" : "+v"(ksc0[0]), "+v"(ksc0[1]));
      static_for<0, nKF8>([&](auto fc) {
        constexpr int f = decltype(fc)::value, kb = f / nK8, kk = f % nK8;
        const i32x8 a = k_frag8(K0, f);
        mfma8_s<kk == 0, 2 * kk>(s0[kb], a, qf8[0][kk], ksc0[kb], qsc[0]);
        mfma8_s<kk == 0, 2 * kk>(s1a[kb], a, qf8[1][kk], ksc0[kb], qsc[1]);
      });
    }
    fence2(s0[0], s1a[0]);
    fence2(s0[1], s1a[1]);
    const bool masked = nfull == 0;
    int lim[2];
    tile_lim(0, lim);
    reset_max();
#pragma unroll
    for (int u = 0; u < 32; ++u) max_item(Par<0>{}, u >> 4, (u >> 3) & 1, u & 7, masked, lim);
    float a = fmaxf(pm[0][0], pm[0][1]), b = fmaxf(pm[1][0], pm[1][1]);
    halves_max2(a, b, h);
    // a row that sees no key of tile 0 keeps -inf here; its exponentials are all masked to 0
    m_ref[0] = a;
    m_ref[1] = b;
    mc[0] = a * c;
    mc[1] = b * c;
#pragma unroll
    for (int v = 0; v < 32; ++v) exp_item(Par<0>{}, v, masked);
#pragma unroll
    for (int v = 0; v < 32; ++v) sum_item(Par<0>{}, v);
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) pack_item(Par<0>{}, Par<0>{}, ch);
  }
  // every wave is done with kslot(0) before iteration 0 refills it
  __syncthreads();

  int j = 0;
  for (; j + 2 < nfull; j += 2) {
    iteration(Par<0>{}, Par<1>{}, j, Flag<false>{}, IC<0>{});
    iteration(Par<1>{}, Par<0>{}, j + 1, Flag<false>{}, IC<1>{});
  }
  // tile j + 1 may still need no mask (the pairs above stop one tile early): one more unmasked
  // iteration, after which tile j + 1's buffers move to the even set the masked tail expects
  if (j + 1 < nfull) {
    iteration(Par<0>{}, Par<1>{}, j, Flag<false>{}, IC<0>{});
    s1a[0] = s1b[0];
    s1a[1] = s1b[1];
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) p0a[cc] = p0b[cc];
    ++j;
  }
  // masked tail (at most four tiles): one body, the next tile's block-1 scores and block-0
  // P are moved into the even buffers after each iteration so the roles never alternate
  for (; j + 1 < ntiles; ++j) {
    iteration(Par<0>{}, Par<1>{}, j, Flag<true>{}, IC<-1>{});
    s1a[0] = s1b[0];
    s1a[1] = s1b[1];
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) p0a[cc] = p0b[cc];
  }
  last(Par<0>{}, j);

  fence_acc(acc);
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qrow = qw0 + 32 * qb + l32;
    const float l_half = lp[qb][0] + lp[qb][1];
    const float r_half = rp[qb][0] + rp[qb][1];
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
          u32x2 w = {pack_bf16x2(acc[qb][db][4 * g] * inv, acc[qb][db][4 * g + 1] * inv),
                     pack_bf16x2(acc[qb][db][4 * g + 2] * inv, acc[qb][db][4 * g + 3] * inv)};
          *reinterpret_cast<u32x2*>(orow + d0) = w;
        }
      }
      if (h == 0) Lh[qrow] = l_tot > 0.f ? (m_ref[qb] * c + log2_fast(l_tot)) * kLn2 : kNegInf;
    }
  }
}

template <int D, bool CAUSAL, bool QK8>
hipError_t launch(const FwdBf16Problem& p) {
  FwdKArgs k;
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
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, QK8>), dim3(k.nq * k.nbhg), dim3(kThreads), 0, p.stream, k);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16_general(const FwdBf16Problem& p) {
  if (p.q8) {
    if (p.D == 64) return p.causal ? launch<64, true, true>(p) : launch<64, false, true>(p);
    return p.causal ? launch<128, true, true>(p) : launch<128, false, true>(p);
  }
  return launch_fwd_bf16_q32(p);
}

hipError_t launch_fwd_bf16(const FwdArgs& a) {
  const FwdBf16Problem p{a.q, a.k, a.v, a.o, a.lse, nullptr, nullptr, a.B, a.H, a.H, a.D,
                         a.T, a.T, a.T, a.scale, a.causal, a.stream};
  return launch_fwd_bf16_general(p);
}

}  // namespace fa
