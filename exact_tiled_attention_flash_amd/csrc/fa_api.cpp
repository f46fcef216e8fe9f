// C ABI of libfa.so: argument validation and kernel dispatch (declared in include/fa.h).
//
// Every check runs on the host before anything is enqueued, so a rejected
// call leaves all outputs untouched and makes no HIP runtime call at all.

#include <math.h>
#include <stdint.h>

#include "../../include/fa.h"
#include "fa_launch.h"

namespace {

constexpr int64_t kMaxElems = int64_t(1) << 40;   // per tensor; keeps every offset in range
constexpr int64_t kMaxBlocks = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxHeadBytes = (int64_t(1) << 31) - 1;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_sizes(int B, int H, int T, int D) {
  if (B < 1 || H < 1 || T < 1) return FA_ERR_SHAPE;
  if (D != 64 && D != 128) return FA_ERR_HEADDIM;
  const int64_t bh = int64_t(B) * H;
  if (bh > INT32_MAX) return FA_ERR_SHAPE;
  if (bh * T * D > kMaxElems) return FA_ERR_SHAPE;
  // one head of one tensor stays below 2^31 bytes: in-head offsets are 32-bit
  if (int64_t(T) * D * 2 > kMaxHeadBytes) return FA_ERR_SHAPE;
  // the largest grid: one workgroup per 64 rows of every (b, h)
  if (bh * ((int64_t(T) + 63) / 64) > kMaxBlocks) return FA_ERR_SHAPE;
  return FA_OK;
}

// Sizes of the grouped / cross-length / packed forward: Hq = G * Hkv, and the rows of one
// head of every tensor (Tq or Tk rows of `rs` elements) below 2^31 bytes.
int check_sizes_general(int B, int Hq, int Hkv, int Tq, int Tk, int D, int q_rs, int kv_rs) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Tq < 1 || Tk < 1) return FA_ERR_SHAPE;
  if (Hq % Hkv != 0) return FA_ERR_SHAPE;
  if (D != 64 && D != 128) return FA_ERR_HEADDIM;
  if (int64_t(B) * Hq * Tq * D > kMaxElems || int64_t(B) * Hkv * Tk * D > kMaxElems) return FA_ERR_SHAPE;
  if (int64_t(Tq) * q_rs * 2 > kMaxHeadBytes || int64_t(Tk) * kv_rs * 2 > kMaxHeadBytes) return FA_ERR_SHAPE;
  if (int64_t(B) * Hq * ((int64_t(Tq) + 63) / 64) > kMaxBlocks) return FA_ERR_SHAPE;
  return FA_OK;
}

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Query rows of one K/V head's group that one decode product holds.
constexpr int kDecodeMaxRows = 32;
constexpr int kDecodeKeys = 32;      // keys per decode tile
// Splits x (b, K/V head) aimed at: 2 workgroups per compute unit of 256 when every sequence
// has Tk keys (measured best from 4k to 128k keys and 1 to 128 (b, K/V head)s: longer splits
// pay each workgroup's first-load latency and the merge fewer times), 4 per compute unit when
// lengths may differ (the splits of short sequences end early; more, shorter splits balance
// the long ones).
constexpr int kDecodeTargetDense = 512;
constexpr int kDecodeTargetLens = 1024;

// Split count of the decode: the caller's (clamped to the key tiles), or enough splits that
// B * Hkv * splits is about the target for dense or per-sequence lengths.
int decode_splits(int B, int Hkv, int Tk, int num_splits, bool seqlens) {
  const int nt = (Tk + kDecodeKeys - 1) / kDecodeKeys;
  const int64_t target = seqlens ? kDecodeTargetLens : kDecodeTargetDense;
  int64_t s = num_splits > 0 ? num_splits
                             : (target + int64_t(B) * Hkv - 1) / (int64_t(B) * Hkv);
  if (s > nt) s = nt;
  if (s > fa::decode_max_splits()) s = fa::decode_max_splits();
  return s < 1 ? 1 : int(s);
}

int check_decode(int B, int Hq, int Hkv, int Tq, int Tk, int D, int num_splits) {
  if (int rc = check_sizes_general(B, Hq, Hkv, Tq, Tk, D, D, D)) return rc;
  if (int64_t(Hq / Hkv) * Tq > kDecodeMaxRows) return FA_ERR_SHAPE;
  if (num_splits < 0) return FA_ERR_ARG;
  return FA_OK;
}

int check_scale(float scale) {
  if (!isfinite(scale) || scale < 0.f) return FA_ERR_SCALE;
  return FA_OK;
}

}  // namespace

namespace fa {

// Every argument of the backward except its workspace.
int check_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
              const float* lse, const void* dq, const void* dk, const void* dv, int B, int H,
              int T, int D, float scale, int causal, int dtype) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_NULL;
  if (int rc = check_sizes(B, H, T, D)) return rc;
  if (dtype != FA_F32 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (int rc = check_scale(scale)) return rc;
  for (const void* p : {q, k, v, o, dout, static_cast<const void*>(lse), dq, dk, dv})
    if (!aligned16(p)) return FA_ERR_ALIGN;
  return FA_OK;
}

}  // namespace fa

extern "C" {

int fa_abi_version(void) { return FA_ABI_VERSION; }

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "null pointer argument";
    case FA_ERR_SHAPE: return "invalid shape (B, H, T must be >= 1 and sizes must fit the index range)";
    case FA_ERR_HEADDIM: return "unsupported head dimension (D must be 64 or 128)";
    case FA_ERR_DTYPE: return "unsupported dtype for this call";
    case FA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case FA_ERR_SCALE: return "scale must be finite and >= 0";
    case FA_ERR_ARG: return "invalid argument";
    case FA_ERR_HIP: return "HIP runtime rejected a kernel launch";
    case FA_ERR_SCRATCH: return "sizes exceed the library's fixed scratch buffer (fa_bwd_noalloc_max_bytes)";
    default: return "unknown status";
  }
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int T,
           int D, float scale, int causal, int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (int rc = check_sizes(B, H, T, D)) return rc;
  if (dtype != FA_F32 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (int rc = check_scale(scale)) return rc;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;

  fa::FwdArgs a{q, k, v, o, lse, B, H, T, D, scale, causal != 0,
                static_cast<hipStream_t>(stream)};
  const hipError_t e = dtype == FA_BF16 ? fa::launch_fwd_bf16(a) : fa::launch_fwd_f32(a);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
               int Hkv, int Tq, int Tk, int D, float scale, int causal, int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (int rc = check_sizes_general(B, Hq, Hkv, Tq, Tk, D, D, D)) return rc;
  if (dtype != FA_BF16) return FA_ERR_DTYPE;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (int rc = check_scale(scale)) return rc;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;
  const fa::FwdBf16Problem p{q, k, v, o, lse, nullptr, nullptr, B, Hq, Hkv, D, Tq, Tk, Tq,
                             scale, causal != 0, static_cast<hipStream_t>(stream)};
  return fa::launch_fwd_bf16_general(p) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                  const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int Hq, int Hkv,
                  int total_q, int total_k, int max_seqlen_q, int D, float scale, int causal,
                  int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse || !cu_seqlens_q || !cu_seqlens_k) return FA_ERR_NULL;
  if (max_seqlen_q < 1 || max_seqlen_q > total_q) return FA_ERR_SHAPE;
  if (int rc = check_sizes_general(1, Hq, Hkv, total_q, total_k, D, Hq * D, Hkv * D)) return rc;
  if (B < 1 || int64_t(B) * Hq * ((int64_t(max_seqlen_q) + 63) / 64) > kMaxBlocks) return FA_ERR_SHAPE;
  if (dtype != FA_BF16) return FA_ERR_DTYPE;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (int rc = check_scale(scale)) return rc;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      !aligned4(cu_seqlens_q) || !aligned4(cu_seqlens_k))
    return FA_ERR_ALIGN;
  const fa::FwdBf16Problem p{q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, D, total_q,
                             total_k, max_seqlen_q, scale, causal != 0,
                             static_cast<hipStream_t>(stream)};
  return fa::launch_fwd_bf16_general(p) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_quantize_mxfp8(const void* x, void* codes, void* scales, int rows, int D, int dtype,
                      void* stream) {
  if (!x || !codes || !scales) return FA_ERR_NULL;
  if (rows < 1 || D < 32 || D % 32 != 0) return FA_ERR_SHAPE;
  if (int64_t(rows) * D > kMaxElems) return FA_ERR_SHAPE;
  if (dtype != FA_BF16) return FA_ERR_DTYPE;
  if (!aligned16(x) || !aligned16(codes) || !aligned4(scales)) return FA_ERR_ALIGN;
  return fa::launch_quantize_mxfp8(x, codes, scales, int64_t(rows) * D,
                                   static_cast<hipStream_t>(stream)) == hipSuccess
             ? FA_OK
             : FA_ERR_HIP;
}

int fa_fwd_fp8qk(const void* q8, const void* q_scale, const void* k8, const void* k_scale,
                 const void* v, void* o, float* lse, int B, int Hq, int Hkv, int Tq, int Tk, int D,
                 float scale, int causal, void* stream) {
  if (!q8 || !q_scale || !k8 || !k_scale || !v || !o || !lse) return FA_ERR_NULL;
  if (int rc = check_sizes_general(B, Hq, Hkv, Tq, Tk, D, D, D)) return rc;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (int rc = check_scale(scale)) return rc;
  if (!aligned16(q8) || !aligned16(k8) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      !aligned4(q_scale) || !aligned4(k_scale))
    return FA_ERR_ALIGN;
  fa::FwdBf16Problem p{q8, k8, v, o, lse, nullptr, nullptr, B, Hq, Hkv, D, Tq, Tk, Tq,
                       scale, causal != 0, static_cast<hipStream_t>(stream)};
  p.q8 = q8;
  p.q_scale = q_scale;
  p.k8 = k8;
  p.k_scale = k_scale;
  return fa::launch_fwd_bf16_general(p) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_decode_workspace_bytes(int B, int Hq, int Hkv, int Tq, int Tk, int D, int num_splits) {
  if (check_decode(B, Hq, Hkv, Tq, Tk, D, num_splits) != FA_OK) return 0;
  // the automatic count with per-sequence lengths is never below the dense one: size for it
  const size_t s = decode_splits(B, Hkv, Tk, num_splits, true);
  return sizeof(float) * size_t(B) * size_t(Hq) * size_t(Tq) * s * size_t(D + 4);
}

int fa_fwd_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                  const int* cache_seqlens, void* workspace, size_t workspace_bytes, int B, int Hq,
                  int Hkv, int Tq, int Tk, int D, int num_splits, float scale, int causal, int dtype,
                  void* stream) {
  if (!q || !k || !v || !o || !lse || !workspace) return FA_ERR_NULL;
  if (int rc = check_decode(B, Hq, Hkv, Tq, Tk, D, num_splits)) return rc;
  if (dtype != FA_BF16) return FA_ERR_DTYPE;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (int rc = check_scale(scale)) return rc;
  if (workspace_bytes < fa_decode_workspace_bytes(B, Hq, Hkv, Tq, Tk, D, num_splits)) return FA_ERR_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      !aligned16(workspace) || (cache_seqlens && !aligned4(cache_seqlens)))
    return FA_ERR_ALIGN;
  const fa::DecodeBf16Problem p{q, k, v, o, lse, cache_seqlens, workspace, B, Hq, Hkv, Tq, Tk, D,
                                decode_splits(B, Hkv, Tk, num_splits, cache_seqlens != nullptr),
                                scale, causal != 0,
                                static_cast<hipStream_t>(stream)};
  return fa::launch_decode_bf16(p) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_bwd_workspace_bytes(int B, int H, int T, int D) {
  if (check_sizes(B, H, T, D) != FA_OK) return 0;
  return 2 * sizeof(float) * size_t(B) * size_t(H) * size_t(T);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
           int B, int H, int T, int D, float scale, int causal, int dtype, void* stream) {
  if (int rc = fa::check_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, T, D, scale, causal, dtype))
    return rc;
  if (!workspace) return FA_ERR_NULL;
  if (workspace_bytes < fa_bwd_workspace_bytes(B, H, T, D)) return FA_ERR_ARG;
  if (!aligned16(workspace)) return FA_ERR_ALIGN;
  fa::BwdArgs a{q, k, v, o, dout, lse, dq, dk, dv, static_cast<float*>(workspace), B, H, T, D,
                scale, causal != 0, static_cast<hipStream_t>(stream)};
  const hipError_t e = dtype == FA_BF16 ? fa::launch_bwd_bf16(a) : fa::launch_bwd_f32(a);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"
