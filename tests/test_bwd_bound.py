"""The derived error bound of the bf16 backward (tests/gpu_util.py, bwd_rounding_bound) on the
CPU: an emulation of the backward's bf16 roundings stays inside it, and plausible mistakes in a
backward do not.

The emulation takes the exact float64 forward, rounds O to bf16 before D_i = rowsum(dO * O)
("Lab 06 - Attention kernels", section 4), rounds dS and P to bf16 before the products and
rounds the gradients to bf16: the roundings the GPU backward performs. The planted mistakes are
the ones the page's "Common bugs" list warns about or that an index slip produces.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from gpu_util import bwd_rounding_bound
from synth import planted


def _rb(x):
    return synth.bf16_bits_to_f64(synth.f32_to_bf16_bits(np.asarray(x, dtype=np.float32)))


def _emulate(q, k, v, do, o, lse, scale, causal, mistake=None):
    s = oracle.scores(q, k, scale, causal if mistake != "no_mask" else False)
    p = np.exp(s - lse[:, None])
    if mistake == "no_mask":
        p = np.exp(oracle.scores(q, k, scale, False) - lse[:, None])
    dp = do @ v.T
    dvec = np.sum(do * _rb(o), axis=1)
    if mistake == "no_delta":
        dvec = 0 * dvec
    ds = _rb(p * (dp - dvec[:, None]))
    pb = _rb(p)
    kk = k.copy()
    if mistake == "drop_tile":
        kk[64:128] = 0.0
    sc = scale if mistake != "no_scale" else 1.0
    return _rb(sc * ds @ kk), _rb(sc * ds.T @ q), _rb(pb.T @ do)


@pytest.fixture(scope="module", params=[(64, False), (64, True), (128, True)])
def case(request):
    D, causal = request.param
    T = 300
    d = planted.make_spiky(1, 1, T, D, seed=D)
    q, k, v, do = (synth.bf16_bits_to_f64(d[n][0, 0]) for n in ("q", "k", "v", "do"))
    scale = 1 / math.sqrt(D)
    o, lse = oracle.attention_forward(*(x[None, None] for x in (q, k, v)), scale, causal)
    o, lse = o[0, 0], lse[0, 0]
    ref = oracle.attention_backward(*(x[None, None] for x in (q, k, v, o, do)), lse[None, None],
                                    scale, causal)
    ref = [r[0, 0] for r in ref]
    bounds = bwd_rounding_bound(q, k, v, do, o, lse, scale, causal)
    return q, k, v, do, o, lse, scale, causal, ref, bounds


def test_emulated_backward_inside_bound(case):
    q, k, v, do, o, lse, scale, causal, ref, bounds = case
    for g, r, b in zip(_emulate(q, k, v, do, o, lse, scale, causal), ref, bounds):
        assert np.all(np.abs(g - r) <= b)


@pytest.mark.parametrize("mistake", ["no_delta", "no_scale", "drop_tile", "no_mask"])
def test_planted_mistakes_exceed_bound(case, mistake):
    q, k, v, do, o, lse, scale, causal, ref, bounds = case
    if mistake == "no_mask" and not causal:
        pytest.skip("no mask to drop")
    out = _emulate(q, k, v, do, o, lse, scale, causal, mistake)
    assert any(np.any(np.abs(g - r) > b) for g, r, b in zip(out, ref, bounds)), mistake


def test_flat_tolerance_holds_for_plain_inputs():
    # at N(0,1) inputs (the backward workload's recipe) the same roundings stay inside the flat
    # 2e-2 that the sweep and full-size backward tests hold the GPU to; only inputs with large,
    # cancelling terms (scaled keys) need the derived bound
    d = synth.make_inputs(1, 1, 256, 128, "bf16", seed=3, with_do=True)
    q, k, v, do = (synth.bf16_bits_to_f64(d[n][0, 0]) for n in ("q", "k", "v", "do"))
    scale = 128 ** -0.5
    o, lse = oracle.attention_forward(*(x[None, None] for x in (q, k, v)), scale, True)
    ref = oracle.attention_backward(*(x[None, None] for x in (q, k, v)), o, do[None, None],
                                    lse, scale, True)
    out = _emulate(q, k, v, do, o[0, 0], lse[0, 0], scale, True)
    for g, r in zip(out, ref):
        assert np.max(np.abs(g - r[0, 0])) <= 2e-2
