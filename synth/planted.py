"""Seeded inputs with planted score structure: rows whose maximum moves between key tiles.

The online-softmax recurrence rescales its accumulator by exp(m - m') whenever a key tile
raises a row's maximum ("Lab 06 - Attention kernels", section 2, and "What to implement"
item 1: a maximum that jumps from -40 to 1000 across tiles; "Common bugs": the case where the
first tile already holds the row maximum). With N(0,1) inputs at scale 1/sqrt(D) the scores
are about N(0,1), so a later tile practically never beats an earlier one by much; these
inputs make it happen on purpose.

Construction (float32 draws, then round-to-nearest-even to bf16 like every other input):
  * Q, K, V are standard normals from numpy PCG64 with the given seed, drawn in that order.
  * Query coordinate 0 is set to 1 for rows that "see" the planted offsets and to 0 for the
    others (all rows, or every other row when `mixed`).
  * Key coordinate 0 is set to offset_j / scale, so that row i's score with key j is
    sees_i * offset_j plus the usual N(0, about 1) remainder of the other coordinates.
  * "Exact" keys also have coordinates 1.. zeroed, so their score is sees_i * offset_j alone
    (up to the bf16 rounding of offset_j / scale).

Scenarios (offsets in natural-log score units; positions relative to one sequence of T keys):
  jump            keys before p score about -40, key p scores 1000 (exact), later keys 0
  first_tile_max  keys 0..3 score 50 (exact), every other key 0: the first tile holds the max
  staircase       one exact key per 64-key tile t scores 12 t: each tile raises the max by
                  more than 2^8 in the exp2 domain (about 5.5 natural units)
  below_margin    the same staircase at 4 per tile: the maximum rises by less than that
  spiky           1 % of the keys score 8x their N(0,1) value (the long ragged workload's K
                  rows x 8), no planted offsets

This module draws numbers and places them; it computes nothing of attention.
"""
from __future__ import annotations

import math

import numpy as np

from .inputs import f32_to_bf16_bits, spike_positions

SCENARIOS = ("jump", "first_tile_max", "staircase", "below_margin")


def key_offsets(T: int, scenario: str, p: int | None = None):
    """(offset per key, mask of exact keys) for one sequence of T keys."""
    off = np.zeros(T, dtype=np.float64)
    exact = np.zeros(T, dtype=bool)
    if scenario == "jump":
        p = (3 * T) // 4 if p is None else min(max(p, 0), T - 1)
        off[:p] = -40.0
        off[p] = 1000.0
        exact[p] = True
    elif scenario == "first_tile_max":
        n = min(4, T)
        off[:n] = 50.0
        exact[:n] = True
    elif scenario in ("staircase", "below_margin"):
        step = 12.0 if scenario == "staircase" else 4.0
        for t in range(0, (T + 63) // 64):
            j = min(64 * t + 17, T - 1)
            off[j] = step * t
            exact[j] = True
    else:
        raise ValueError(f"unknown scenario {scenario!r}")
    return off, exact


def plant(q: np.ndarray, k: np.ndarray, scale: float, scenario: str, mixed: bool = False,
          p: int | None = None, row_axis: int = -2):
    """Place the scenario into float32 arrays q (..., Tq, D) and k (..., Tk, D) in place.
    Rows / keys run along `row_axis` (-2 for (B, H, T, D), -3 for packed (T, H, D))."""
    Tq, Tk = q.shape[row_axis], k.shape[row_axis]
    off, exact = key_offsets(Tk, scenario, p)
    qm = np.moveaxis(q, row_axis, 0)
    km = np.moveaxis(k, row_axis, 0)
    sees = np.ones(Tq, dtype=np.float32)
    if mixed:
        sees[1::2] = 0.0
    qm[..., 0] = sees.reshape((Tq,) + (1,) * (qm.ndim - 2))
    km[..., 0] = (off / scale).astype(np.float32).reshape((Tk,) + (1,) * (km.ndim - 2))
    km[exact, ..., 1:] = 0.0


def make_planted(B: int, Hq: int, Hkv: int, Tq: int, Tk: int, D: int, scenario: str,
                 seed: int = 0, mixed: bool = False, p: int | None = None) -> dict:
    """bf16 bits of Q (B, Hq, Tq, D), K and V (B, Hkv, Tk, D) with the scenario planted."""
    rng = np.random.default_rng(seed)
    scale = 1.0 / math.sqrt(D)
    q = rng.standard_normal((B, Hq, Tq, D), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, Tk, D), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, Tk, D), dtype=np.float32)
    plant(q, k, scale, scenario, mixed, p)
    return {"q": f32_to_bf16_bits(q), "k": f32_to_bf16_bits(k), "v": f32_to_bf16_bits(v),
            "scale": scale}


def make_planted_varlen(lens, Hq: int, Hkv: int, D: int, scenario: str, seed: int = 0,
                        mixed: bool = False) -> dict:
    """A packed batch (total, H, D) whose every sequence carries the scenario at its own
    positions (the jump at three quarters of each sequence); cu_seqlens int32."""
    rng = np.random.default_rng(seed)
    scale = 1.0 / math.sqrt(D)
    lens = np.asarray(lens, dtype=np.int64)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    total = int(cu[-1])
    q = rng.standard_normal((total, Hq, D), dtype=np.float32)
    k = rng.standard_normal((total, Hkv, D), dtype=np.float32)
    v = rng.standard_normal((total, Hkv, D), dtype=np.float32)
    for b in range(len(lens)):
        a, e = int(cu[b]), int(cu[b + 1])
        if e > a:
            plant(q[a:e], k[a:e], scale, scenario, mixed, row_axis=0)
    return {"q": f32_to_bf16_bits(q), "k": f32_to_bf16_bits(k), "v": f32_to_bf16_bits(v),
            "cu": cu, "lens": lens, "scale": scale}


def make_spiky(B: int, H: int, T: int, D: int, seed: int = 0, with_do: bool = True) -> dict:
    """Q, K, V (, dO) standard normals, then 1 % of the key positions (shared by all (b, h))
    scaled by 8, the long ragged workload's recipe at another size."""
    rng = np.random.default_rng(seed)
    out = {n: rng.standard_normal((B, H, T, D), dtype=np.float32)
           for n in (["q", "k", "v"] + (["do"] if with_do else []))}
    pos = spike_positions(rng, T, 0.01)
    out["k"][:, :, pos, :] *= np.float32(8.0)
    res = {n: f32_to_bf16_bits(a) for n, a in out.items()}
    res["spikes"] = pos
    return res
