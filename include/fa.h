/*
 * fa.h - C ABI of the MI355X (gfx950) exact tiled attention library, libfa.so.
 *
 * The operation is exact softmax attention,
 *     S = scale * Q K^T,   P = softmax_rows(S),   O = P V,
 *     LSE_i = log sum_j exp(S_ij)           (natural log, one value per row),
 * computed by the online-softmax tile recurrence so the T x T matrix never
 * reaches device memory, and its gradient computed from the saved LSE with
 * D_i = rowsum(dO * O) and per-tile recomputation of P.
 * Sources:
 *   "Lab 06 - Attention kernels: online softmax -> FlashAttention -> Triton",
 *     section 2 (online softmax), section 3 (forward recurrence, causal tile
 *     skipping, O = acc / l and LSE = m + log l), section 4 (backward with
 *     D = rowsum(dO * O), dQ = dS K scale, dK = dS^T Q scale), section 5
 *     (one program per (query tile, batch*head); contiguous (B, H, T, D)).
 *   "Triton FlashAttention-2 forward", "The kernel" (launcher layout, scale
 *     1/sqrt(D) by default, fp32 accumulation, output cast to input dtype).
 *   "Flash Attention and Kernel Optimization", "Output and saved state" (the
 *     saved LSE row statistic used by the backward).
 *
 * Conventions shared by every call
 *   Layout     q, k, v, o, dout, dq, dk, dv are contiguous row-major
 *              (B, H, T, D) arrays: element (b, h, t, d) sits at
 *              ((b*H + h)*T + t)*D + d. lse and the backward workspace hold
 *              (B, H, T) float32 values at (b*H + h)*T + t.
 *   Types      dtype FA_BF16: tensors hold bfloat16 (products in bf16 on the
 *              matrix cores, accumulation and all softmax statistics in fp32,
 *              outputs rounded to nearest-even). dtype FA_F32: everything is
 *              IEEE fp32. lse is always float32.
 *   Masking    causal != 0: key j is visible to query i iff j <= i; one
 *              length T shared by queries and keys.
 *   Scale      finite and >= 0 (0 gives uniform weights over visible keys);
 *              callers usually pass 1/sqrt(D).
 *   Memory     every pointer is device memory owned by the caller and must be
 *              16-byte aligned. The library never allocates, frees or
 *              synchronises: each call validates its arguments on the host,
 *              enqueues kernels on `stream` (a hipStream_t; NULL = the null
 *              stream) and returns. Results are ready when the stream is.
 *   Errors     calls return FA_OK (0) or a negative fa_status. On any
 *              validation error nothing is enqueued and no output is
 *              touched. FA_ERR_HIP means a kernel launch was rejected by the
 *              runtime; outputs are then unspecified.
 *   Threads    calls are reentrant; concurrent calls on different streams
 *              must not share output buffers.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_ABI_VERSION 5

enum fa_dtype {
    FA_F32 = 0,
    FA_BF16 = 1
};

enum fa_status {
    FA_OK = 0,
    FA_ERR_NULL = -1,      /* a required pointer is NULL */
    FA_ERR_SHAPE = -2,     /* B, H or T < 1, the sizes overflow the index range, or one
                              head of one tensor (T * D elements) reaches 2^31 bytes */
    FA_ERR_HEADDIM = -3,   /* D is not 64 or 128 */
    FA_ERR_DTYPE = -4,     /* dtype is not a supported fa_dtype for this call */
    FA_ERR_ALIGN = -5,     /* a pointer is not 16-byte aligned */
    FA_ERR_SCALE = -6,     /* scale is negative, NaN or infinite */
    FA_ERR_ARG = -7,       /* any other bad argument (causal not 0/1, workspace too small) */
    FA_ERR_HIP = -8,       /* the HIP runtime rejected a launch */
    FA_ERR_SCRATCH = -9    /* the sizes need more than the library's fixed scratch buffer */
};

/* Version of this ABI (FA_ABI_VERSION). */
int fa_abi_version(void);

/* Static text for a status code ("ok", "null pointer", ...). Never NULL. */
const char *fa_status_string(int status);

/*
 * Forward: o = softmax(scale * q k^T [causal mask]) v and lse per row.
 *   q, k, v  in:  (B, H, T, D) of dtype
 *   o        out: (B, H, T, D) of dtype
 *   lse      out: (B, H, T) float32, natural-log log-sum-exp of each row of
 *                 scale * q k^T over the visible keys
 * Source: "Lab 06 - Attention kernels", section 3 (the (m, l, acc)
 * recurrence; O = acc / l; LSE = m + log l) and section 5 (launch layout).
 */
int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
           int B, int H, int T, int D, float scale, int causal, int dtype,
           void *stream);

/*
 * Forward with grouped K/V heads and separate query and key lengths (FA_BF16 only).
 *   q      in:  (B, Hq, Tq, D) bf16
 *   k, v   in:  (B, Hkv, Tk, D) bf16; Hq must be a multiple G of Hkv and query
 *               head h attends with K/V head h / G
 *   o      out: (B, Hq, Tq, D) bf16
 *   lse    out: (B, Hq, Tq) float32
 * Causal masking is aligned at the bottom right: query i sees key j iff
 * j <= i + (Tk - Tq) (the top-left rule of fa_fwd when Tq == Tk). A query that
 * sees no key (possible when Tk < Tq) gets o = 0 and lse = -inf.
 * One workgroup serves up to four query heads of a group, so every K/V tile it
 * loads feeds all of them. Tq, Tk >= 1; the rows of one head of any tensor stay
 * below 2^31 bytes (FA_ERR_SHAPE otherwise).
 * Source: "Lab 06 - Attention kernels", "Check yourself" question 7 and its
 * answer (GQA: map the program to a K/V head so a tile loaded once serves the
 * query heads sharing it), and the build-order table, step 2 (query and key
 * lengths may differ).
 */
int fa_fwd_gqa(const void *q, const void *k, const void *v, void *o, float *lse,
               int B, int Hq, int Hkv, int Tq, int Tk, int D, float scale,
               int causal, int dtype, void *stream);

/*
 * Forward over a packed batch of B variable-length sequences (FA_BF16 only).
 *   cu_seqlens_q, cu_seqlens_k  in: device int32 arrays of B + 1 offsets (4-byte
 *               aligned): sequence b owns query rows [cu_seqlens_q[b],
 *               cu_seqlens_q[b+1]) and key rows [cu_seqlens_k[b],
 *               cu_seqlens_k[b+1]). The kernels clamp the offsets into
 *               [0, total] and treat a decreasing pair as an empty sequence, so
 *               no access leaves the arrays whatever they hold.
 *   q      in:  (total_q, Hq, D) bf16;  k, v in: (total_k, Hkv, D) bf16
 *   o      out: (total_q, Hq, D) bf16;  lse out: (Hq, total_q) float32
 *   max_seqlen_q  bound on every query length (sizes the grid; rows of a
 *               longer sequence beyond it are left unwritten)
 * Heads and masking as fa_fwd_gqa, per sequence. Rows not covered by any
 * sequence are left unwritten. The offsets are expected not to decrease: for a
 * skewed batch (max_seqlen_q >= 2048 and at least 2.5 times total_q / B) of up to
 * 64 sequences with a multiple of 8 query-head groups (Hq, or Hq / 2 or Hq / 4
 * when Hq / Hkv is a multiple of 2 or 4) the grid is sized from total_q, and
 * sequences that overlap may then leave some of their rows unwritten.
 * Source: "Triton FlashAttention-2 forward", "Exercises" (a cu_seqlens index
 * tensor packs requests of different lengths into one launch).
 */
int fa_fwd_varlen(const void *q, const void *k, const void *v, void *o, float *lse,
                  const int *cu_seqlens_q, const int *cu_seqlens_k, int B, int Hq,
                  int Hkv, int total_q, int total_k, int max_seqlen_q, int D,
                  float scale, int causal, int dtype, void *stream);

/*
 * Block-scaled E4M3 quantization (FA_BF16 input only), the input of fa_fwd_fp8qk.
 *   x       in:  rows x D bf16, contiguous (16-byte aligned); D a positive multiple of 32
 *   codes   out: rows x D bytes (16-byte aligned), OCP E4M3: sign, 4 exponent bits (bias 7),
 *                3 mantissa bits, subnormals m/8 * 2^-6, largest finite 448
 *   scales  out: rows x (D / 32) bytes (4-byte aligned): for each block of 32 consecutive
 *                elements of a row, 127 - e where e is the largest integer with
 *                amax * 2^e <= 448 (amax the block's largest magnitude; e at most 127, and
 *                0 for an all-zero block)
 * Each element becomes the E4M3 value nearest to x * 2^e (ties to even) with the sign of x;
 * the block's values are then code value * 2^(scale - 127). Inputs must be finite.
 * A (B, H, T, D) tensor is rows = B * H * T.
 * Source: "Lab 06 - Attention kernels", "Stretch" list (E4M3 Q and K for the Q K^T
 * product); the format details and the power-of-two block scaling are this library's
 * reading of what the page leaves open.
 */
int fa_quantize_mxfp8(const void *x, void *codes, void *scales, int rows, int D, int dtype,
                      void *stream);

/*
 * Forward with E4M3 Q and K for the Q K^T product (bf16 V, P and output, fp32 statistics).
 *   q8, q_scale  in: codes (B, Hq, Tq, D) bytes and scales (B, Hq, Tq, D / 32) bytes of Q,
 *                as fa_quantize_mxfp8 writes them (codes 16-byte, scales 4-byte aligned)
 *   k8, k_scale  in: the same for K, (B, Hkv, Tk, D) and (B, Hkv, Tk, D / 32)
 *   v      in:  (B, Hkv, Tk, D) bf16
 *   o      out: (B, Hq, Tq, D) bf16;  lse out: (B, Hq, Tq) float32
 * S = scale * sum over blocks of (Q codes . K codes) * 2^(q scale - 127) * 2^(k scale - 127),
 * on the gfx950 matrix cores' scaled E4M3 products with fp32 accumulation; everything after
 * S is the bf16 forward's (heads, masking and lengths as fa_fwd_gqa).
 * Source: "Lab 06 - Attention kernels", "Stretch" list (FP8 E4M3 Q and K for Q K^T,
 * accuracy measured against speed).
 */
int fa_fwd_fp8qk(const void *q8, const void *q_scale, const void *k8, const void *k_scale,
                 const void *v, void *o, float *lse, int B, int Hq, int Hkv, int Tq, int Tk,
                 int D, float scale, int causal, void *stream);

/*
 * Bytes of device workspace fa_fwd_decode needs for these sizes and this
 * num_splits (0 = the automatic choice): 4 * B * Hq * Tq * splits * (D + 4),
 * where splits is num_splits clamped to [1, min(ceil(Tk / 32), 1024)], or with
 * num_splits = 0 the smallest count that gives about 1024 (b, K/V head, split)
 * workgroups, within the same bounds (the most the automatic choice of
 * fa_fwd_decode takes). Returns 0 if the sizes are invalid.
 */
size_t fa_decode_workspace_bytes(int B, int Hq, int Hkv, int Tq, int Tk, int D,
                                 int num_splits);

/*
 * Split-K decode: a few new query rows per sequence against a long K/V cache
 * (FA_BF16 only). The same result as fa_fwd_gqa on the valid keys, computed
 * with the keys of every (b, K/V head) split across workgroups.
 *   q      in:  (B, Hq, Tq, D) bf16; (Hq / Hkv) * Tq must be <= 32
 *   k, v   in:  (B, Hkv, Tk, D) bf16, the cache; query head h uses K/V head
 *               h / (Hq / Hkv)
 *   cache_seqlens in: NULL (every sequence has Tk valid keys) or a device int32
 *               array of B counts (4-byte aligned); sequence b attends to keys
 *               [0, cache_seqlens[b]), the count clamped into [0, Tk] on the
 *               device
 *   o      out: (B, Hq, Tq, D) bf16;  lse out: (B, Hq, Tq) float32
 *   workspace   at least fa_decode_workspace_bytes(...) bytes owned by the
 *               caller; partial results, contents on return unspecified
 *   num_splits  key splits per (b, K/V head); 0 = automatic: the smallest
 *               count that gives about 512 (b, K/V head, split) workgroups
 *               when cache_seqlens is NULL and about 1024 when it is given,
 *               within the bounds above. With cache_seqlens and B <= 64 the
 *               B * splits workgroups of each K/V head are shared out among
 *               the sequences in proportion to their valid keys (at least one
 *               each), so a long sequence gets more of them than a short one
 * Causal masking is aligned at the bottom right of each sequence's valid keys
 * L: query i sees key j iff j <= i + (L - Tq). A query that sees no key gets
 * o = 0 and lse = -inf. Two kernels: the splits write their partial (max, sum,
 * accumulator); the second merges them.
 * Source: "Lab 06 - Attention kernels", "Check yourself" answer 2 (split-K:
 * partition the keys, a partial (m, l, acc) per program, merge with the same
 * rescaling rule), answer 7 (one program per K/V head serving the query heads
 * that share it), and the "Stretch" list (FlashDecoding with a second merge
 * kernel, measured at T_q = 1 against T_k = 32k).
 */
int fa_fwd_decode(const void *q, const void *k, const void *v, void *o, float *lse,
                  const int *cache_seqlens, void *workspace, size_t workspace_bytes,
                  int B, int Hq, int Hkv, int Tq, int Tk, int D, int num_splits,
                  float scale, int causal, int dtype, void *stream);

/*
 * Bytes of device workspace fa_bwd needs for these sizes: 8*B*H*T (the
 * row vectors D_i = rowsum(dout * o) and LSE_i * log2(e), fp32 each, for
 * either dtype). Returns 0 if the sizes are invalid.
 * Source: "Lab 06 - Attention kernels", section 4 (the backward's O(T d)
 * preprocessing pass computes D_i = rowsum(dO * O) once per row, so the
 * gradient kernels read one value per query instead of reducing over P)
 * and "Check yourself" answer 6.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int T, int D);

/*
 * Backward: given dout = dL/do, compute dq, dk, dv.
 *   q, k, v, o  in:  as passed to / returned by fa_fwd (o must be that
 *                    forward's output for the same q, k, v, scale, causal)
 *   dout        in:  (B, H, T, D) of dtype
 *   lse         in:  (B, H, T) float32 from that fa_fwd call
 *   dq, dk, dv  out: (B, H, T, D) of dtype
 *   workspace   scratch of at least fa_bwd_workspace_bytes(B, H, T, D)
 *               bytes, owned by the caller; contents on return unspecified
 * Kernels (FA_BF16): dq with query tiles outer, which also computes its rows'
 * D_i = rowsum(dout * o) into the workspace; then dk, dv with key tiles outer
 * and query tiles inner. FA_F32: a D_i pass, then dk, dv, then dq. P =
 * exp(S - LSE) is recomputed per tile with the same mask as the forward. No
 * atomics: the
 * result is deterministic. dtype FA_BF16: bf16 tensors, fp32 accumulation,
 * P and dS rounded to bf16 for the matrix-core products, gradients rounded
 * to nearest-even. dtype FA_F32: fp32 tensors, fp32 products with P and dS
 * kept in fp32.
 * Source: "Lab 06 - Attention kernels", section 4 and the "Stretch" list
 * (two backward kernels: dK/dV with key tiles outer, dQ with query tiles
 * outer).
 */
int fa_bwd(const void *q, const void *k, const void *v, const void *o,
           const void *dout, const float *lse, void *dq, void *dk, void *dv,
           void *workspace, size_t workspace_bytes,
           int B, int H, int T, int D, float scale, int causal, int dtype,
           void *stream);

/*
 * Backward that allocates nothing and takes no workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation. Arguments, results, dtypes and errors as fa_bwd, whose kernels it runs; the
 * D_i and LSE_i * log2(e) rows live instead in a fixed device array of this library,
 * fa_bwd_noalloc_max_bytes() bytes (16 MiB: B * H * T up to 2^21 rows), which every GPU the
 * library runs on holds until the process ends. Sizes that need more return FA_ERR_SCRATCH
 * and touch nothing. The array's device address is looked up once per device (on the first
 * call with that device current); no call allocates or frees memory. Every call on one GPU
 * uses that GPU's array: calls that overlap on one GPU (different streams, or another
 * thread) race and must be serialised by the caller; a call may reuse the array as soon as
 * the previous call's work has been enqueued on the same stream.
 */
size_t fa_bwd_noalloc_max_bytes(void);
int fa_bwd_noalloc(const void *q, const void *k, const void *v, const void *o,
                   const void *dout, const float *lse, void *dq, void *dk, void *dv,
                   int B, int H, int T, int D, float scale, int causal, int dtype,
                   void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
