"""CPU float64 oracle for exact attention (forward and backward).

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
link this module: only the tests, the smoke check and the CPU-baseline leg of
the benchmark use it. It shares no code with the HIP path; its inputs are
plain numpy arrays (callers upcast bf16/fp32 storage to float64 exactly).

Sources (page titles; sections named after each function):
  [Lab06]  "Lab 06 - Attention kernels: online softmax -> FlashAttention -> Triton"
  [FA2nb]  "Triton FlashAttention-2 forward" (notebook)
  [FAopt]  "Flash Attention and Kernel Optimization" (llm-from-scratch docs)

Conventions (the plainest reading the pages support):
  * Layout (B, H, T, D); one sequence length T shared by queries and keys.
  * S = scale * Q K^T; the scale is inside the softmax, hence inside LSE.
  * causal: key j is visible to query i iff j <= i (top-left aligned).
  * LSE is the natural-log log-sum-exp of each row of S, with no epsilon.
  * Output dtype handling is the caller's business: this module returns
    float64 everywhere.

Every function here is pinned by the not-gpu tests against something other
than itself (closed forms, brute force, torch float64 CPU routines, finite
differences); see tests/test_oracle.py.
"""
from __future__ import annotations

import numpy as np

_ROW_CHUNK = 2048  # rows of S materialised at once (bounds memory at long T)


def _check_qkv(q, k, v):
    for name, x in (("q", q), ("k", k), ("v", v)):
        if x.dtype != np.float64:
            raise TypeError(f"oracle expects float64 arrays, {name} is {x.dtype}")
        if x.ndim != 4:
            raise ValueError(f"{name} must be (B, H, T, D), got shape {x.shape}")
    if q.shape != k.shape or q.shape != v.shape:
        raise ValueError(f"q/k/v shapes differ: {q.shape} {k.shape} {v.shape}")


def scores(q_bh: np.ndarray, k_bh: np.ndarray, scale: float, causal: bool,
           rows: np.ndarray | None = None) -> np.ndarray:
    """Scaled, masked score rows S[i, :] = scale * q_i . k_j for one (b, h).

    [Lab06] section 3 (S = Q K^T * scale per tile); [FA2nb] "The kernel" (the
    causal rule keeps key n for query m when m >= n). Masked entries are -inf.
    `rows` selects query indices (default: all).
    """
    T = k_bh.shape[0]
    if rows is None:
        rows = np.arange(q_bh.shape[0])
    s = (q_bh[rows] @ k_bh.T) * scale
    if causal:
        keys = np.arange(T)
        s = np.where(keys[None, :] <= rows[:, None], s, -np.inf)
    return s


def softmax_stats(s: np.ndarray):
    """Row max m, row sum l = sum_j exp(S_ij - m_i) and LSE = m + ln l.

    [Lab06] section 2: logsumexp equals m + log l. Two-pass definition (max
    first, then the shifted sum), not the online recurrence.
    """
    m = np.max(s, axis=-1)
    l = np.sum(np.exp(s - m[..., None]), axis=-1)
    return m, l, m + np.log(l)


def attention_rows(q_bh, k_bh, v_bh, scale: float, causal: bool, rows: np.ndarray):
    """O and LSE for selected query rows of one (b, h), by the definition.

    O_i = sum_j softmax(S_i)_j V_j with S materialised for those rows only.
    [Lab06] section 1 (the dense computation the method reproduces exactly)
    and section 3 (O and LSE are what the tiled method returns).
    """
    rows = np.asarray(rows, dtype=np.int64)
    k_bh, v_bh = np.ascontiguousarray(k_bh), np.ascontiguousarray(v_bh)
    s = scores(q_bh, k_bh, scale, causal, rows)
    _, _, lse = softmax_stats(s)
    p = np.exp(s - lse[:, None])
    return p @ v_bh, lse


def attention_forward(q, k, v, scale: float, causal: bool):
    """Exact attention forward for every (b, h): returns (O, LSE) in float64.

    O has shape (B, H, T, D), LSE has shape (B, H, T). S is materialised one
    (b, h) at a time in chunks of query rows, with a two-pass softmax.
    """
    _check_qkv(q, k, v)
    B, H, T, D = q.shape
    o = np.empty_like(q)
    lse = np.empty((B, H, T), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, T, _ROW_CHUNK):
                rows = np.arange(r0, min(T, r0 + _ROW_CHUNK))
                o[b, h, rows], lse[b, h, rows] = attention_rows(
                    q[b, h], k[b, h], v[b, h], scale, causal, rows)
    return o, lse


def online_softmax_stats(x: np.ndarray, block: int):
    """Online (streaming) max and shifted sum over the last axis.

    [Lab06] section 2 (Milakov & Gimelshein): visit the values block by block,
    keep the running max m and l = sum exp(x - m); when a block raises the max
    to m', multiply l by exp(m - m') before adding the block's own terms.
    Returns (m, l, m + ln l). The first block starts from m = -inf, l = 0, and
    the exp(m - m') factor is taken as 0 while m is still -inf.
    """
    x = np.asarray(x, dtype=np.float64)
    m = np.full(x.shape[:-1], -np.inf)
    l = np.zeros(x.shape[:-1])
    n = x.shape[-1]
    for j0 in range(0, n, block):
        blk = x[..., j0:j0 + block]
        m_new = np.maximum(m, np.max(blk, axis=-1))
        safe = np.where(np.isneginf(m_new), 0.0, m_new)
        alpha = np.where(np.isneginf(m), 0.0, np.exp(m - safe))
        l = l * alpha + np.sum(np.exp(blk - safe[..., None]), axis=-1)
        m = m_new
    return m, l, m + np.log(l)


def attention_forward_online(q, k, v, scale: float, causal: bool,
                             block_m: int, block_n: int):
    """The tiled FlashAttention forward recurrence, in float64.

    [Lab06] section 3; [FA2nb] "The kernel"; [FAopt] "Running softmax state".
    For each query tile keep (m, l, acc) per row; for each key tile: S tile,
    m' = max(m, rowmax S), P~ = exp(S - m'), acc <- acc*exp(m - m') + P~ V,
    l <- l*exp(m - m') + rowsum P~. Finish with O = acc / l and
    LSE = m + ln l. Causal: key tiles that lie wholly after the tile's last
    query are not visited ([Lab06] section 3 figure and "Common bugs": the
    last needed key tile is the one holding query i1 - 1); the diagonal tile
    is masked element-wise. Block sizes need not divide T.

    Exists to show that the recurrence reaches the two-pass result; the GPU
    parity tests compare against attention_forward / attention_rows.
    """
    _check_qkv(q, k, v)
    B, H, T, D = q.shape
    o = np.empty_like(q)
    lse = np.empty((B, H, T))
    for b in range(B):
        for h in range(H):
            for i0 in range(0, T, block_m):
                i1 = min(T, i0 + block_m)
                qi = q[b, h, i0:i1]
                m = np.full(i1 - i0, -np.inf)
                l = np.zeros(i1 - i0)
                acc = np.zeros((i1 - i0, D))
                j_end = i1 if causal else T          # keys [0, j_end) can be visible
                for j0 in range(0, j_end, block_n):
                    j1 = min(T, j0 + block_n)
                    s = (qi @ k[b, h, j0:j1].T) * scale
                    if causal:
                        qi_idx = np.arange(i0, i1)[:, None]
                        kj_idx = np.arange(j0, j1)[None, :]
                        s = np.where(kj_idx <= qi_idx, s, -np.inf)
                    m_new = np.maximum(m, np.max(s, axis=1))
                    safe = np.where(np.isneginf(m_new), 0.0, m_new)
                    alpha = np.where(np.isneginf(m), 0.0, np.exp(m - safe))
                    p = np.exp(s - safe[:, None])
                    acc = acc * alpha[:, None] + p @ v[b, h, j0:j1]
                    l = l * alpha + np.sum(p, axis=1)
                    m = m_new
                o[b, h, i0:i1] = acc / l[:, None]
                lse[b, h, i0:i1] = m + np.log(l)
    return o, lse


def attention_backward(q, k, v, o, do, lse, scale: float, causal: bool):
    """Exact attention backward, dense, for every (b, h).

    [Lab06] section 4: P = exp(S - LSE) recomputed from the saved LSE;
    dV = P^T dO; dP = dO V^T; D_i = rowsum(dO * O)_i; dS = P * (dP - D);
    dQ = scale * dS K; dK = scale * dS^T Q. [FAopt] "Autograd Wrapper and
    Backward Path" lists the same dense steps (rebuild S, mask, softmax, then
    the five gradients). The mask is applied before the exponential, as in
    the forward ([Lab06] "Common bugs"). o and lse must be the oracle's own
    forward outputs (or exact equivalents).
    Returns (dQ, dK, dV) in float64.
    """
    _check_qkv(q, k, v)
    B, H, T, D = q.shape
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    for b in range(B):
        for h in range(H):
            s = scores(q[b, h], k[b, h], scale, causal)
            p = np.exp(s - lse[b, h][:, None])
            dv[b, h] = p.T @ do[b, h]
            dp = do[b, h] @ v[b, h].T
            dvec = np.sum(do[b, h] * o[b, h], axis=1)
            ds = p * (dp - dvec[:, None])
            dq[b, h] = scale * (ds @ k[b, h])
            dk[b, h] = scale * (ds.T @ q[b, h])
    return dq, dk, dv


def backward_delta(o, do):
    """D_i = sum_d dO_id * O_id ([Lab06] section 4 and "Check yourself" answer 6)."""
    return np.sum(o * do, axis=-1)


def attention_backward_rows(q_bh, k_bh, v_bh, do_bh, scale: float, causal: bool,
                            rows: np.ndarray):
    """dQ of selected query rows of one (b, h), by the definition.

    [Lab06] section 4 restricted to rows i: dQ_i = scale * sum_j dS_ij K_j with
    dS_ij = P_ij (dP_ij - D_i), P_i the softmax of row i of S, dP_i = dO_i V^T and
    D_i = dO_i . O_i. Every quantity of row i needs row i of S only, so long
    sequences can be checked on a sample of rows. Returns (len(rows), D) float64.
    """
    rows = np.asarray(rows, dtype=np.int64)
    o_r, lse_r = attention_rows(q_bh, k_bh, v_bh, scale, causal, rows)
    s = scores(q_bh, k_bh, scale, causal, rows)
    p = np.exp(s - lse_r[:, None])
    dp = do_bh[rows] @ v_bh.T
    dvec = np.sum(do_bh[rows] * o_r, axis=1)
    ds = p * (dp - dvec[:, None])
    return scale * (ds @ k_bh)


def attention_backward_key_tail(q_bh, k_bh, v_bh, do_bh, scale: float, r0: int):
    """Causal: dK and dV of keys r0 .. T-1 of one (b, h), by the definition.

    Under the causal rule key j is seen only by queries i >= j, so the gradients
    of the keys from r0 on need P, dP and D of query rows r0 .. T-1 only
    ([Lab06] section 4: dV_j = sum_i P_ij dO_i, dK_j = scale * sum_i dS_ij Q_i);
    each of those rows' LSE and O still comes from its whole row of S.
    Returns (dK, dV), each (T - r0, D) float64.
    """
    T = k_bh.shape[0]
    rows = np.arange(r0, T)
    o_r, lse_r = attention_rows(q_bh, k_bh, v_bh, scale, True, rows)
    s = scores(q_bh, k_bh, scale, True, rows)[:, r0:]
    p = np.exp(s - lse_r[:, None])
    dv = p.T @ do_bh[rows]
    dp = do_bh[rows] @ v_bh[r0:].T
    dvec = np.sum(do_bh[rows] * o_r, axis=1)
    ds = p * (dp - dvec[:, None])
    return scale * (ds.T @ q_bh[rows]), dv


def attention_cross(q_h, k_h, v_h, scale: float, causal: bool):
    """One head with Tq query rows against Tk key rows: (O, LSE) in float64.

    [Lab06] the build-order table, step 2: query and key lengths may differ.
    The pages fix no causal rule for Tq != Tk; the reading taken is the
    bottom-right one: query i sees key j iff j <= i + (Tk - Tq), which is the
    top-left rule of `scores` when Tq == Tk. A row that sees no key at all
    (only possible when Tk < Tq) gets O = 0 and LSE = -inf. S is materialised
    in chunks of query rows, softmax in two passes.
    """
    # head slices of packed (rows, H, D) arrays are strided; numpy's products on them are
    # an order of magnitude slower than on a contiguous copy (same values)
    q_h, k_h, v_h = (np.ascontiguousarray(x) for x in (q_h, k_h, v_h))
    Tq, Tk = q_h.shape[0], k_h.shape[0]
    o = np.zeros((Tq, v_h.shape[1]), dtype=np.float64)
    lse = np.full(Tq, -np.inf)
    keys = np.arange(Tk)
    for r0 in range(0, Tq, _ROW_CHUNK):
        rows = np.arange(r0, min(Tq, r0 + _ROW_CHUNK))
        s = (q_h[rows] @ k_h.T) * scale
        if causal:
            s = np.where(keys[None, :] <= rows[:, None] + (Tk - Tq), s, -np.inf)
        seen = np.isfinite(s).any(axis=1)
        if seen.any():
            _, _, row_lse = softmax_stats(s[seen])
            p = np.exp(s[seen] - row_lse[:, None])
            o[rows[seen]] = p @ v_h
            lse[rows[seen]] = row_lse
    return o, lse


def attention_forward_gqa(q, k, v, scale: float, causal: bool):
    """Grouped K/V heads: q (B, Hq, Tq, D), k and v (B, Hkv, Tk, D), Hq = G * Hkv.

    [Lab06] "Check yourself" question 7 and its answer: the query heads of a
    group share one K/V head; query head h uses K/V head h // G. Every (b, h)
    is `attention_cross` on its own K/V head. Returns O (B, Hq, Tq, D) and
    LSE (B, Hq, Tq).
    """
    for name, x in (("q", q), ("k", k), ("v", v)):
        if x.dtype != np.float64 or x.ndim != 4:
            raise ValueError(f"{name} must be a float64 (B, H, T, D) array")
    B, Hq, Tq, D = q.shape
    Hkv = k.shape[1]
    if k.shape != v.shape or Hq % Hkv or k.shape[0] != B or k.shape[3] != D:
        raise ValueError(f"bad grouped shapes {q.shape} {k.shape} {v.shape}")
    G = Hq // Hkv
    o = np.empty_like(q)
    lse = np.empty((B, Hq, Tq))
    for b in range(B):
        for h in range(Hq):
            o[b, h], lse[b, h] = attention_cross(q[b, h], k[b, h // G], v[b, h // G], scale, causal)
    return o, lse


def attention_forward_varlen(q, k, v, cu_q, cu_k, scale: float, causal: bool):
    """A packed batch: q (total_q, Hq, D), k and v (total_k, Hkv, D).

    [FA2nb] "Exercises": a cu_seqlens index tensor packs requests of different
    lengths into one launch. Sequence b owns query rows [cu_q[b], cu_q[b+1])
    and key rows [cu_k[b], cu_k[b+1]); each sequence is grouped attention on
    its own rows (`attention_cross` per head). Returns O (total_q, Hq, D),
    zero on rows no sequence covers, and LSE (Hq, total_q), -inf there.
    """
    total_q, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    o = np.zeros_like(q)
    lse = np.full((Hq, total_q), -np.inf)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        if q1 <= q0:
            continue
        for h in range(Hq):
            ob, lb = attention_cross(q[q0:q1, h], k[k0:k1, h // G], v[k0:k1, h // G], scale, causal)
            o[q0:q1, h] = ob
            lse[h, q0:q1] = lb
    return o, lse


def attention_decode(q, k, v, cache_seqlens, scale: float, causal: bool):
    """New query rows against a K/V cache: q (B, Hq, Tq, D), k and v (B, Hkv, Tk, D).

    [Lab06] "Check yourself" question 2 and the "Stretch" list (decoding against
    a long K/V cache). Sequence b attends to its first cache_seqlens[b] keys
    (all Tk when cache_seqlens is None; counts clamped into [0, Tk]); the
    result is the definition, `attention_cross` on those keys with the grouped
    head mapping of `attention_forward_gqa` (bottom-right causal alignment, so
    the last query row sees every valid key). Returns O (B, Hq, Tq, D) and
    LSE (B, Hq, Tq).
    """
    B, Hq, Tq, D = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    o = np.zeros_like(q)
    lse = np.full((B, Hq, Tq), -np.inf)
    for b in range(B):
        L = Tk if cache_seqlens is None else int(min(max(int(cache_seqlens[b]), 0), Tk))
        if L == 0:
            continue
        for h in range(Hq):
            o[b, h], lse[b, h] = attention_cross(q[b, h], k[b, h // G, :L], v[b, h // G, :L],
                                                 scale, causal)
    return o, lse


def split_partial(q_h, k_h, v_h, scale: float, key_lo: int, key_hi: int, limits):
    """Partial softmax state of query rows over the keys [key_lo, key_hi).

    [Lab06] "Check yourself" answer 2: each program of a split-K decode keeps
    its own (m, l, acc) over its share of the keys. `limits[i]` is the last key
    row i may see (masking); keys outside the range or beyond the limit do not
    count. A row that sees no key of the range has m = -inf, l = 0, acc = 0
    (the guard the page's "Common bugs" list asks for when key ranges are
    visited out of order). Returns (m, l, acc) in the natural-log domain.
    """
    q_h, k_h, v_h = (np.ascontiguousarray(x) for x in (q_h, k_h, v_h))
    Tq = q_h.shape[0]
    keys = np.arange(key_lo, key_hi)
    s = (q_h @ k_h[key_lo:key_hi].T) * scale
    s = np.where(keys[None, :] <= np.asarray(limits)[:, None], s, -np.inf)
    m = np.max(s, axis=1) if key_hi > key_lo else np.full(Tq, -np.inf)
    safe = np.where(np.isneginf(m), 0.0, m)
    p = np.exp(s - safe[:, None])
    return m, np.sum(p, axis=1), p @ v_h[key_lo:key_hi]


def merge_partials(ms, ls, accs):
    """Merge split-K partial states: [Lab06] "Check yourself" answer 2 (the same
    rescaling rule as the online recurrence). With m* = max_s m_s, every partial
    is weighted by exp(m_s - m*) (0 for an empty partial); O = sum w acc / sum w l
    and LSE = m* + ln(sum w l). Rows with no key in any partial: O = 0,
    LSE = -inf. Inputs are lists over splits of (rows,), (rows,), (rows, D).
    """
    ms, ls, accs = np.stack(ms), np.stack(ls), np.stack(accs)
    m_star = np.max(ms, axis=0)
    seen = ~np.isneginf(m_star)
    safe = np.where(seen, m_star, 0.0)
    w = np.where(np.isneginf(ms), 0.0, np.exp(ms - safe[None, :]))
    l = np.sum(w * ls, axis=0)
    acc = np.sum(w[:, :, None] * accs, axis=0)
    o = np.zeros(acc.shape)
    o[seen] = acc[seen] / l[seen, None]
    lse = np.full(m_star.shape, -np.inf)
    lse[seen] = m_star[seen] + np.log(l[seen])
    return o, lse


def attention_split_k(q_h, k_h, v_h, scale: float, causal: bool, bounds):
    """One head by split-K: partial states over the key ranges [bounds[s],
    bounds[s+1]) ([Lab06] "Stretch": FlashDecoding), merged by `merge_partials`.
    Same masking convention as `attention_cross` (bottom-right causal). Exists to
    show that split-and-merge reaches the definition, including empty ranges and
    ranges a row cannot see.
    """
    Tq, Tk = q_h.shape[0], k_h.shape[0]
    limits = np.arange(Tq) + (Tk - Tq) if causal else np.full(Tq, Tk - 1)
    parts = [split_partial(q_h, k_h, v_h, scale, int(bounds[s]), int(bounds[s + 1]), limits)
             for s in range(len(bounds) - 1)]
    return merge_partials(*zip(*parts))
