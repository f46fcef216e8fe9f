"""Workload bookkeeping for the benchmark: metric FLOPs, algorithmic bytes, peaks.

FLOP count of one attention forward: two T x T x D products per (b, h), two
flops per multiply-add, so 4*B*H*T^2*D; a causal mask halves it ("Triton
FlashAttention-2 forward", smoke check of the shape algebra; "Lab 06 -
Attention kernels", the causal FLOP prediction before the benchmark).
Algorithmic bytes: Q, K and V read once and O written once (same smoke
check), plus the fp32 LSE row statistic this library also writes.
"""
from __future__ import annotations

# MI355X published dense peaks (TFLOP/s) and HBM bandwidth (GB/s)
PEAK_TFLOPS = {"bf16": 2516.6, "f32": 157.3}
PEAK_HBM_GBS = 8000.0


def fwd_flops(B: int, H: int, T: int, D: int, causal: bool) -> float:
    f = 4.0 * B * H * T * T * D
    return f / 2.0 if causal else f


def bwd_flops(B: int, H: int, T: int, D: int, causal: bool) -> float:
    """Five T x T x D products (dV, dP, dQ, dK plus the recomputed S): 10*B*H*T^2*D, causal halved."""
    f = 10.0 * B * H * T * T * D
    return f / 2.0 if causal else f


def fwd_bytes(B: int, H: int, T: int, D: int, elem_bytes: int, with_lse: bool = True) -> int:
    n = elem_bytes * B * H * D * (T + 2 * T + T)
    return n + (4 * B * H * T if with_lse else 0)


def bwd_bytes(B: int, H: int, T: int, D: int, elem_bytes: int) -> int:
    """Read Q, K, V, O, dO, LSE; write dQ, dK, dV; the D_i row vector written and read once."""
    return elem_bytes * B * H * T * D * 8 + 4 * B * H * T * 3


def score_matrix_bytes(B: int, H: int, T: int, elem_bytes: int) -> int:
    """Bytes of the T x T score matrix a naive implementation would write."""
    return elem_bytes * B * H * T * T


def gqa_flops(B: int, Hq: int, Tq: int, Tk: int, D: int, causal: bool) -> float:
    """Two Tq x Tk x D products per query head; a causal mask halves the count (the
    convention above, exact in the limit Tq = Tk)."""
    f = 4.0 * B * Hq * Tq * Tk * D
    return f / 2.0 if causal else f


def gqa_bytes(B: int, Hq: int, Hkv: int, Tq: int, Tk: int, D: int, elem_bytes: int) -> int:
    """Q read and O written per query head, K and V read once per K/V head, fp32 LSE."""
    return elem_bytes * B * D * (2 * Hq * Tq + 2 * Hkv * Tk) + 4 * B * Hq * Tq


def varlen_flops(lens_q, lens_k, Hq: int, D: int, causal: bool) -> float:
    """Sum of the per-sequence forward counts."""
    return sum(gqa_flops(1, Hq, int(a), int(b), D, causal) for a, b in zip(lens_q, lens_k))


def varlen_bytes(total_q: int, total_k: int, Hq: int, Hkv: int, D: int, elem_bytes: int) -> int:
    return elem_bytes * D * (2 * Hq * total_q + 2 * Hkv * total_k) + 4 * Hq * total_q


def decode_bytes(B: int, Hq: int, Hkv: int, Tq: int, D: int, valid_keys: int, elem_bytes: int) -> int:
    """K and V rows read once per K/V head (valid_keys summed over the batch), Q read and O
    written once, fp32 LSE. The split partials are not algorithmic traffic."""
    return elem_bytes * D * (2 * Hkv * valid_keys + 2 * B * Hq * Tq) + 4 * B * Hq * Tq
