"""Seeded synthetic attention inputs.

Every tensor is drawn from ``numpy.random.default_rng(seed)`` (PCG64) as
float32 standard normals, in the order Q, K, V, dO, and then (only for the
spiky long-context workload) the set of key positions whose rows are scaled.
bf16 tensors are produced from those float32 draws by round-to-nearest-even
on the bit pattern and are returned as ``uint16`` bit arrays, so the same
values can be uploaded to the GPU and upcast exactly to float64 for the
oracle.

Workloads follow the shapes the pages use for their checks and benchmarks
(random normal tensors of layout (B, H, T, D)); no dataset is involved.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic attention workload, contiguous (B, H, T, D) layout."""

    name: str
    B: int
    H: int
    T: int
    D: int
    dtype: str            # "f32" or "bf16"
    causal: bool
    backward: bool = False
    spike_frac: float = 0.0  # fraction of key positions whose K rows are scaled
    spike_scale: float = 8.0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)


WORKLOADS = {
    w.name: w
    for w in [
        # small fp32 case, non-causal
        Workload("fwd_f32_b1h2t128d64", 1, 2, 128, 64, "f32", False),
        # bf16, mid-size, both mask modes
        Workload("fwd_bf16_b1h8t1024d64", 1, 8, 1024, 64, "bf16", False),
        Workload("fwd_bf16_b1h8t1024d64_causal", 1, 8, 1024, 64, "bf16", True),
        # headline causal forward
        Workload("fwd_bf16_b4h16t4096d128_causal", 4, 16, 4096, 128, "bf16", True),
        # long, ragged, with 1% of key rows scaled by 8
        Workload("fwd_bf16_b1h32t16381d128_causal_spiky", 1, 32, 16381, 128, "bf16", True,
                 spike_frac=0.01, spike_scale=8.0),
        # causal backward
        Workload("bwd_bf16_b2h16t4096d128_causal", 2, 16, 4096, 128, "bf16", True, backward=True),
    ]
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = ((u[nan] >> 16).astype(np.uint16)) | np.uint16(0x40)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    return bf16_bits_to_f32(b).astype(np.float64)


def spike_positions(rng: np.random.Generator, T: int, frac: float) -> np.ndarray:
    """round(frac*T) distinct key positions in [0, T), sorted."""
    n = int(round(frac * T))
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(rng.choice(T, size=n, replace=False)).astype(np.int64)


def make_inputs(B: int, H: int, T: int, D: int, dtype: str = "bf16", seed: int = 0,
                with_do: bool = False, spike_frac: float = 0.0,
                spike_scale: float = 8.0) -> dict:
    """Draw Q, K, V (and dO) for one workload.

    Returns a dict with keys "q", "k", "v" (and "do", and "spikes" when
    spike_frac > 0). For dtype "bf16" the arrays are uint16 bit patterns; for
    "f32" they are float32. The draw order is fixed: Q, K, V, dO, spikes.
    """
    if dtype not in ("bf16", "f32"):
        raise ValueError(f"unknown dtype {dtype!r}")
    rng = np.random.default_rng(seed)
    shape = (B, H, T, D)
    out = {}
    names = ["q", "k", "v"] + (["do"] if with_do else [])
    for name in names:
        out[name] = rng.standard_normal(shape, dtype=np.float32)
    if spike_frac > 0.0:
        pos = spike_positions(rng, T, spike_frac)
        out["k"][:, :, pos, :] *= np.float32(spike_scale)
        out["spikes"] = pos
    if dtype == "bf16":
        for name in names:
            out[name] = f32_to_bf16_bits(out[name])
    return out


def make_workload_inputs(w: Workload, seed: int = 0) -> dict:
    return make_inputs(w.B, w.H, w.T, w.D, w.dtype, seed=seed, with_do=w.backward,
                       spike_frac=w.spike_frac, spike_scale=w.spike_scale)


@dataclasses.dataclass(frozen=True)
class GqaWorkload:
    """Grouped K/V heads: Q (B, Hq, Tq, D), K and V (B, Hkv, Tk, D), Hkv dividing Hq."""

    name: str
    B: int
    Hq: int
    Hkv: int
    Tq: int
    Tk: int
    D: int
    causal: bool

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)


@dataclasses.dataclass(frozen=True)
class VarlenWorkload:
    """A packed batch of n_seq sequences whose lengths are drawn log-uniformly from
    [min_len, max_len]; Q (total, Hq, D), K and V (total, Hkv, D), the same lengths for
    queries and keys (self-attention)."""

    name: str
    n_seq: int
    min_len: int
    max_len: int
    Hq: int
    Hkv: int
    D: int
    causal: bool

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)


GQA_WORKLOADS = {
    w.name: w
    for w in [
        # 32 query heads sharing 8 K/V heads, headline length
        GqaWorkload("gqa_bf16_b4hq32hkv8t4096d128_causal", 4, 32, 8, 4096, 4096, 128, True),
    ]
}

# one new query row per head against a long K/V cache (split-K decode), and the same cache
# read by a batch of 8 sequences whose valid lengths are drawn log-uniformly in [1024, 32768]
DECODE_WORKLOADS = {
    w.name: w
    for w in [
        GqaWorkload("decode_bf16_b1hq32hkv8tk32768d128", 1, 32, 8, 1, 32768, 128, True),
        GqaWorkload("decode_bf16_b8hq32hkv8tk32768d128_lens", 8, 32, 8, 1, 32768, 128, True),
    ]
}


def decode_lengths(w: GqaWorkload, seed: int = 0) -> np.ndarray:
    """Valid cache lengths of a decode batch: the full cache for one sequence, else drawn
    log-uniformly in [Tk / 32, Tk] (a generator of its own, after the tensors' draws)."""
    if w.B == 1:
        return np.array([w.Tk], dtype=np.int32)
    rng = np.random.default_rng(seed + 1)
    return varlen_lengths(rng, w.B, max(1, w.Tk // 32), w.Tk).astype(np.int32)


VARLEN_WORKLOADS = {
    w.name: w
    for w in [
        # 32 sequences of 64 .. 8192 tokens, 16 heads
        VarlenWorkload("varlen_bf16_n32l64to8192h16d128_causal", 32, 64, 8192, 16, 16, 128, True),
    ]
}


def make_gqa_inputs(w: GqaWorkload, seed: int = 0) -> dict:
    """bf16 bits of Q (B, Hq, Tq, D), then K and V (B, Hkv, Tk, D), drawn in that order."""
    rng = np.random.default_rng(seed)
    out = {"q": rng.standard_normal((w.B, w.Hq, w.Tq, w.D), dtype=np.float32)}
    for name in ("k", "v"):
        out[name] = rng.standard_normal((w.B, w.Hkv, w.Tk, w.D), dtype=np.float32)
    return {n: f32_to_bf16_bits(a) for n, a in out.items()}


def varlen_lengths(rng: np.random.Generator, n: int, lo: int, hi: int) -> np.ndarray:
    """n lengths, log-uniform on [lo, hi], rounded to integers."""
    x = np.exp(rng.uniform(math.log(lo), math.log(hi), n))
    return np.clip(np.rint(x), lo, hi).astype(np.int64)


def make_varlen_inputs(w: VarlenWorkload, seed: int = 0) -> dict:
    """Lengths first, then bf16 bits of packed Q, K, V; cu_seqlens int32 (n_seq + 1)."""
    rng = np.random.default_rng(seed)
    lens = varlen_lengths(rng, w.n_seq, w.min_len, w.max_len)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    total = int(cu[-1])
    out = {"lens": lens, "cu": cu,
           "q": f32_to_bf16_bits(rng.standard_normal((total, w.Hq, w.D), dtype=np.float32))}
    for name in ("k", "v"):
        out[name] = f32_to_bf16_bits(rng.standard_normal((total, w.Hkv, w.D), dtype=np.float32))
    return out
