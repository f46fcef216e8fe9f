"""The planted-score inputs (synth/planted.py) do what the rescale tests need them to do.

The bf16 forward keeps one reference maximum per row and moves it (rescaling the
accumulator by exp(m - m'), "Lab 06 - Attention kernels", section 2) only when some row of a
32-row wave sees a 64-key tile whose maximum beats its reference by more than 2^8 in the exp2
domain. These CPU tests replay that decision on the exact scores of the planted inputs and
check that the GPU tests built on them take the branch in a tile after the first (or, for the
first-tile-maximum case, never do), so that the GPU rescale tests cannot pass vacuously.
"""
import math

import numpy as np
import pytest

import oracle
from synth import bf16_bits_to_f64, planted

MARGIN_LOG2 = 8.0
LOG2E = 1.0 / math.log(2.0)


def late_rescales(q, k, scale, causal, block_m=128, wave_rows=32, block_n=64):
    """Number of (wave, key tile after the first) pairs that move the reference maximum of at
    least one row, for one (b, h) with Tq == Tk."""
    T = q.shape[0]
    s = oracle.scores(q, k, scale, causal)
    events = 0
    for w0 in range(0, T, wave_rows):
        rows = np.arange(w0, min(T, w0 + wave_rows))
        q0 = (w0 // block_m) * block_m
        kend = min(T, q0 + block_m) if causal else T
        ntiles = (kend + block_n - 1) // block_n
        ref = np.max(s[rows, :block_n], axis=1)
        for t in range(1, ntiles):
            a = np.max(s[rows, t * block_n:(t + 1) * block_n], axis=1)
            need = ((a - ref) * LOG2E > MARGIN_LOG2) | (np.isneginf(ref) & ~np.isneginf(a))
            if need.any():
                events += 1
                ref = np.maximum(ref, a)
    return events


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("scenario,mixed,p", [("jump", False, None), ("jump", True, None),
                                              ("jump", False, 70), ("staircase", False, None),
                                              ("staircase", True, None)])
def test_planted_scores_move_the_reference(scenario, mixed, p, causal, D):
    d = planted.make_planted(1, 1, 1, 1000, 1000, D, scenario, seed=D + 3, mixed=mixed, p=p)
    q, k = bf16_bits_to_f64(d["q"][0, 0]), bf16_bits_to_f64(d["k"][0, 0])
    n = late_rescales(q, k, d["scale"], causal)
    assert n >= (1 if scenario == "jump" else 4), n


@pytest.mark.parametrize("causal", [False, True])
def test_first_tile_maximum_never_moves(causal):
    d = planted.make_planted(1, 1, 1, 1000, 1000, 128, "first_tile_max", seed=1)
    q, k = bf16_bits_to_f64(d["q"][0, 0]), bf16_bits_to_f64(d["k"][0, 0])
    assert late_rescales(q, k, d["scale"], causal) == 0


def test_plain_normal_inputs_rarely_move_it():
    # why the planted inputs are needed: N(0,1) at scale 1/sqrt(D) gives no late move
    rng = np.random.default_rng(0)
    q = bf16_bits_to_f64(planted.f32_to_bf16_bits(rng.standard_normal((1000, 128), np.float32)))
    k = bf16_bits_to_f64(planted.f32_to_bf16_bits(rng.standard_normal((1000, 128), np.float32)))
    assert late_rescales(q, k, 128 ** -0.5, True) == 0


def test_planted_scores_have_the_stated_values():
    D = 128
    d = planted.make_planted(1, 1, 1, 1000, 1000, D, "jump", seed=0, p=600)
    s = oracle.scores(bf16_bits_to_f64(d["q"][0, 0]), bf16_bits_to_f64(d["k"][0, 0]), d["scale"],
                      False)
    assert abs(s[0, 600] - 1000.0) < 2.0 and np.all(s[:, 600] == s[0, 600])
    assert abs(np.median(s[:, :600]) + 40.0) < 1.0 and abs(np.median(s[:, 601:])) < 0.5
    m = planted.make_planted(1, 1, 1, 64, 64, D, "jump", seed=0, mixed=True, p=40)
    sm = oracle.scores(bf16_bits_to_f64(m["q"][0, 0]), bf16_bits_to_f64(m["k"][0, 0]), m["scale"],
                       False)
    assert np.all(sm[0::2, 40] > 900) and np.all(np.abs(sm[1::2, 40]) < 1e-9)


def test_planted_varlen_places_each_sequence():
    d = planted.make_planted_varlen([5, 0, 300], 2, 1, 64, "jump", seed=0)
    q, k = bf16_bits_to_f64(d["q"]), bf16_bits_to_f64(d["k"])
    a, e = int(d["cu"][2]), int(d["cu"][3])
    s = oracle.scores(q[a:e, 0], k[a:e, 0], d["scale"], False)
    assert abs(s[0, 225] - 1000.0) < 2.0
