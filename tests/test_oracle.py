"""Pins for the CPU float64 oracle (runs without a GPU).

Each check ties the oracle to something other than its own code: textbook or
library routines (scipy's logsumexp, torch's float64 CPU attention and
autograd), closed forms that follow from the definition, brute-force finite
differences, and the identities the pages state. The mutation tests at the
end plant plausible mistakes into the oracle (on the CPU) and confirm that at
least one pin catches each.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle
from oracle import attention as oattn


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------- online softmax
@pytest.mark.parametrize("n", [1, 37, 128, 1000])
@pytest.mark.parametrize("block", [7, 11, 16, 32])
def test_online_softmax_matches_logsumexp(n, block):
    x = _rand((5, n), seed=n * 31 + block) * 4.0
    m, l, lse = oracle.online_softmax_stats(x, block)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(x, axis=-1), rtol=0, atol=1e-12)
    np.testing.assert_array_equal(m, x.max(axis=-1))
    # l is the shifted sum at the final max: it lies in [1, n]
    assert np.all(l >= 1.0) and np.all(l <= n)


def test_online_softmax_handles_growing_max():
    # The maximum jumps from -40 to 1000 between blocks (Lab 06, "What to implement" item 1).
    x = np.full((1, 64), -40.0)
    x[0, 50] = 1000.0
    for block in (7, 11, 16, 32):
        m, l, lse = oracle.online_softmax_stats(x, block)
        # closed form: 1000 + ln(1 + 63 e^{-1040}) == 1000 in float64
        assert m[0] == 1000.0
        assert l[0] == 1.0
        assert lse[0] == 1000.0
    # a gentler jump where every term still matters
    y = np.concatenate([np.full(10, -40.0), np.full(10, 2.0)])[None]
    expect = 2.0 + math.log(10.0 + 10.0 * math.exp(-42.0))
    for block in (3, 7, 10, 11):
        assert abs(oracle.online_softmax_stats(y, block)[2][0] - expect) < 1e-13


def test_softmax_stats_two_pass_matches_scipy():
    x = _rand((7, 333), seed=3) * 10
    m, l, lse = oracle.softmax_stats(x)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(x, axis=-1), atol=1e-12, rtol=0)
    # masked entries (-inf) contribute nothing
    x[:, 100:] = -np.inf
    np.testing.assert_allclose(oracle.softmax_stats(x)[2],
                               scipy.special.logsumexp(x[:, :100], axis=-1), atol=1e-12, rtol=0)


# ---------------------------------------------------------------- forward vs torch
def _torch_attention(q, k, v, scale, causal):
    tq, tk, tv = (torch.from_numpy(a) for a in (q, k, v))
    o = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    s = torch.matmul(tq, tk.transpose(-1, -2).contiguous()) * scale
    if causal:
        T = q.shape[2]
        mask = torch.ones(T, T, dtype=torch.bool).tril()
        s = s.masked_fill(~mask, float("-inf"))
    return o.numpy(), torch.logsumexp(s, dim=-1).numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 33, 8), (2, 3, 37, 16), (1, 1, 130, 64), (1, 1, 1, 4)])
def test_forward_matches_torch_float64(shape, causal):
    q, k, v = (_rand(shape, seed=i + 10 * shape[2]) for i in range(3))
    scale = 1.0 / math.sqrt(shape[3])
    o, lse = oracle.attention_forward(q, k, v, scale, causal)
    o_t, lse_t = _torch_attention(q, k, v, scale, causal)
    np.testing.assert_allclose(o, o_t, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, lse_t, atol=1e-12, rtol=0)


def test_forward_row_chunking_at_long_t(monkeypatch):
    # row chunks must not change the result (a chunk boundary inside T)
    monkeypatch.setattr(oattn, "_ROW_CHUNK", 13)
    shape = (1, 1, 50, 8)
    q, k, v = (_rand(shape, seed=70 + i) for i in range(3))
    for causal in (False, True):
        o, lse = oracle.attention_forward(q, k, v, 0.3, causal)
        o_t, lse_t = _torch_attention(q, k, v, 0.3, causal)
        np.testing.assert_allclose(o, o_t, atol=1e-12, rtol=0)
        np.testing.assert_allclose(lse, lse_t, atol=1e-12, rtol=0)


def test_rows_match_full_forward():
    shape = (1, 1, 200, 32)
    q, k, v = (_rand(shape, seed=90 + i) for i in range(3))
    rows = np.array([0, 1, 63, 64, 127, 199])
    for causal in (False, True):
        o, lse = oracle.attention_forward(q, k, v, 0.2, causal)
        o_r, lse_r = oracle.attention_rows(q[0, 0], k[0, 0], v[0, 0], 0.2, causal, rows)
        # BLAS may block a subset of rows differently: agree to rounding
        np.testing.assert_allclose(o_r, o[0, 0, rows], atol=1e-14, rtol=0)
        np.testing.assert_allclose(lse_r, lse[0, 0, rows], atol=1e-14, rtol=0)


# ---------------------------------------------------------------- online tiled = two-pass
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("T", [1, 16, 33, 37, 64])
@pytest.mark.parametrize("blocks", [(7, 11), (11, 7), (16, 32), (32, 16), (16, 16)])
def test_online_tiled_matches_two_pass(T, blocks, causal):
    shape = (1, 2, T, 8)
    q, k, v = (_rand(shape, seed=i + 100 * T) for i in range(3))
    o2, lse2 = oracle.attention_forward(q, k, v, 0.5, causal)
    o1, lse1 = oracle.attention_forward_online(q, k, v, 0.5, causal, *blocks)
    np.testing.assert_allclose(o1, o2, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse1, lse2, atol=1e-12, rtol=0)


def test_online_tiled_causal_skip_regression_shape():
    # T=33 with query blocks of 7 and key blocks of 11: skipping one key tile
    # too many would drop keys of the last rows of a query tile.
    shape = (1, 1, 33, 4)
    q, k, v = (_rand(shape, seed=500 + i) for i in range(3))
    o1, lse1 = oracle.attention_forward_online(q, k, v, 1.0, True, 7, 11)
    o_t, lse_t = _torch_attention(q, k, v, 1.0, True)
    np.testing.assert_allclose(o1, o_t, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse1, lse_t, atol=1e-12, rtol=0)


def test_online_tiled_rescale_when_max_is_late():
    # The largest scores sit in the last key tile, so acc must be rescaled.
    T, D = 40, 4
    q = np.ones((1, 1, T, D))
    k = _rand((1, 1, T, D), seed=1) * 0.1
    k[0, 0, -3:] = 5.0
    v = _rand((1, 1, T, D), seed=2)
    o1, lse1 = oracle.attention_forward_online(q, k, v, 1.0, False, 8, 8)
    o_t, lse_t = _torch_attention(q, k, v, 1.0, False)
    np.testing.assert_allclose(o1, o_t, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse1, lse_t, atol=1e-12, rtol=0)


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("T", [1, 5, 64, 129])
def test_uniform_scores_closed_form(T):
    # Q = 0 makes every visible score equal: O is a mean of V rows and
    # LSE = ln(number of visible keys).
    D = 8
    q = np.zeros((1, 1, T, D))
    k = _rand((1, 1, T, D), seed=7)
    v = _rand((1, 1, T, D), seed=8)
    o, lse = oracle.attention_forward(q, k, v, 0.7, False)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0, 0].mean(axis=0), (T, D)), atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], np.full(T, math.log(T)), atol=1e-13)
    o, lse = oracle.attention_forward(q, k, v, 0.7, True)
    prefix = np.cumsum(v[0, 0], axis=0) / np.arange(1, T + 1)[:, None]
    np.testing.assert_allclose(o[0, 0], prefix, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], np.log(np.arange(1, T + 1)), atol=1e-13)
    # scale = 0 has the same effect with arbitrary Q
    q2 = _rand((1, 1, T, D), seed=9)
    o, lse = oracle.attention_forward(q2, k, v, 0.0, True)
    np.testing.assert_allclose(o[0, 0], prefix, atol=1e-13)


def test_single_key_closed_form():
    # T = 1: O = V and LSE = scale * q.k
    q, k, v = (_rand((2, 3, 1, 16), seed=20 + i) for i in range(3))
    for causal in (False, True):
        o, lse = oracle.attention_forward(q, k, v, 0.25, causal)
        np.testing.assert_array_equal(o, v)
        np.testing.assert_allclose(lse, 0.25 * np.sum(q * k, axis=-1), atol=1e-14)


def test_causal_row_zero_is_v0():
    q, k, v = (_rand((2, 2, 50, 16), seed=30 + i) for i in range(3))
    o, lse = oracle.attention_forward(q, k, v, 0.25, True)
    np.testing.assert_array_equal(o[:, :, 0], v[:, :, 0])
    np.testing.assert_allclose(lse[:, :, 0], 0.25 * np.sum(q[:, :, 0] * k[:, :, 0], axis=-1),
                               atol=1e-14)


def test_two_key_hand_example():
    # D = 1, T = 2, scale = 1: q = (1, 2), k = (0, 1), v = (3, 5).
    # Row 0 scores (0, 1): weights (1, e)/(1+e); row 1 scores (0, 2): (1, e^2)/(1+e^2).
    q = np.array([1.0, 2.0]).reshape(1, 1, 2, 1)
    k = np.array([0.0, 1.0]).reshape(1, 1, 2, 1)
    v = np.array([3.0, 5.0]).reshape(1, 1, 2, 1)
    e = math.e
    o, lse = oracle.attention_forward(q, k, v, 1.0, False)
    assert abs(o[0, 0, 0, 0] - (3 + 5 * e) / (1 + e)) < 1e-14
    assert abs(o[0, 0, 1, 0] - (3 + 5 * e * e) / (1 + e * e)) < 1e-14
    assert abs(lse[0, 0, 0] - math.log(1 + e)) < 1e-14
    assert abs(lse[0, 0, 1] - math.log(1 + e * e)) < 1e-14
    o, lse = oracle.attention_forward(q, k, v, 1.0, True)
    assert o[0, 0, 0, 0] == 3.0 and lse[0, 0, 0] == 0.0
    assert abs(o[0, 0, 1, 0] - (3 + 5 * e * e) / (1 + e * e)) < 1e-14


@pytest.mark.parametrize("causal", [False, True])
def test_probability_rows_sum_to_one(causal):
    q, k, v = (_rand((1, 2, 70, 8), seed=40 + i) * 3 for i in range(3))
    _, lse = oracle.attention_forward(q, k, v, 0.5, causal)
    for h in range(2):
        s = oracle.scores(q[0, h], k[0, h], 0.5, causal)
        np.testing.assert_allclose(np.exp(s - lse[0, h][:, None]).sum(axis=1), 1.0, atol=1e-12)


def test_spiky_keys_match_torch():
    # Long-context workload shape in miniature: 1% of key rows scaled by 8.
    import synth
    d = synth.make_inputs(1, 2, 301, 16, "bf16", seed=5, spike_frac=0.01)
    assert len(d["spikes"]) == 3
    q, k, v = (synth.bf16_bits_to_f64(d[n]) for n in "qkv")
    o, lse = oracle.attention_forward(q, k, v, 0.25, True)
    o_t, lse_t = _torch_attention(q, k, v, 0.25, True)
    np.testing.assert_allclose(o, o_t, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, lse_t, atol=1e-12, rtol=0)


# ---------------------------------------------------------------- backward
def _loss(q, k, v, do, scale, causal):
    o, _ = oracle.attention_forward(q, k, v, scale, causal)
    return float(np.sum(o * do))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 1, 5, 3), (1, 1, 9, 4), (1, 1, 2, 2)])
def test_backward_matches_finite_differences(shape, causal):
    q, k, v, do = (_rand(shape, seed=60 + i) for i in range(4))
    scale = 0.6
    o, lse = oracle.attention_forward(q, k, v, scale, causal)
    dq, dk, dv = oracle.attention_backward(q, k, v, o, do, lse, scale, causal)
    h = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss(q, k, v, do, scale, causal)
            x[idx] = old - h
            lm = _loss(q, k, v, do, scale, causal)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_torch_autograd(causal):
    shape = (2, 2, 45, 16)
    q, k, v, do = (_rand(shape, seed=80 + i) for i in range(4))
    scale = 0.25
    o, lse = oracle.attention_forward(q, k, v, scale, causal)
    dq, dk, dv = oracle.attention_backward(q, k, v, o, do, lse, scale, causal)
    tq, tk, tv = (torch.from_numpy(a.copy()).requires_grad_(True) for a in (q, k, v))
    to = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    to.backward(torch.from_numpy(do))
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12, rtol=0)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12, rtol=0)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12, rtol=0)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_rows_match_torch_autograd(causal):
    # dQ of a sample of rows, for sequences too long for the dense backward
    shape = (1, 1, 53, 16)
    q, k, v, do = (_rand(shape, seed=300 + i) for i in range(4))
    scale = 0.3
    tq, tk, tv = (torch.from_numpy(a.copy()).requires_grad_(True) for a in (q, k, v))
    to = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    to.backward(torch.from_numpy(do))
    rows = np.array([0, 1, 17, 52])
    dq = oracle.attention_backward_rows(q[0, 0], k[0, 0], v[0, 0], do[0, 0], scale, causal, rows)
    np.testing.assert_allclose(dq, tq.grad.numpy()[0, 0, rows], atol=1e-12, rtol=0)


@pytest.mark.parametrize("r0", [0, 1, 30, 52])
def test_backward_key_tail_matches_torch_autograd(r0):
    # causal dK, dV of the keys from r0 on, from the query rows that see them
    shape = (1, 1, 53, 16)
    q, k, v, do = (_rand(shape, seed=310 + i) for i in range(4))
    scale = 0.3
    tq, tk, tv = (torch.from_numpy(a.copy()).requires_grad_(True) for a in (q, k, v))
    to = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale)
    to.backward(torch.from_numpy(do))
    dk, dv = oracle.attention_backward_key_tail(q[0, 0], k[0, 0], v[0, 0], do[0, 0], scale, r0)
    np.testing.assert_allclose(dk, tk.grad.numpy()[0, 0, r0:], atol=1e-12, rtol=0)
    np.testing.assert_allclose(dv, tv.grad.numpy()[0, 0, r0:], atol=1e-12, rtol=0)


def test_backward_delta_identity():
    # sum_j P_ij dP_ij == rowsum(dO * O)  (Lab 06 section 4)
    shape = (1, 1, 33, 8)
    q, k, v, do = (_rand(shape, seed=95 + i) for i in range(4))
    for causal in (False, True):
        o, lse = oracle.attention_forward(q, k, v, 0.4, causal)
        s = oracle.scores(q[0, 0], k[0, 0], 0.4, causal)
        p = np.exp(s - lse[0, 0][:, None])
        dp = do[0, 0] @ v[0, 0].T
        np.testing.assert_allclose(np.sum(p * dp, axis=1), oracle.backward_delta(o, do)[0, 0],
                                   atol=1e-12)


# ---------------------------------------------------------------- planted mistakes
def _forward_pins_pass():
    shape = (1, 2, 33, 8)
    q, k, v = (_rand(shape, seed=200 + i) for i in range(3))
    ok = True
    for causal in (False, True):
        o, lse = oracle.attention_forward(q, k, v, 0.3, causal)
        o_t, lse_t = _torch_attention(q, k, v, 0.3, causal)
        ok &= np.allclose(o, o_t, atol=1e-10, rtol=0) and np.allclose(lse, lse_t, atol=1e-10, rtol=0)
    return ok


def test_planted_forward_mistakes_are_caught(monkeypatch):
    assert _forward_pins_pass()
    real_scores = oattn.scores

    def flipped_mask(q_bh, k_bh, scale, causal, rows=None):
        s = real_scores(q_bh, k_bh, scale, False, rows)
        if causal:
            r = np.arange(q_bh.shape[0]) if rows is None else rows
            s = np.where(np.arange(k_bh.shape[0])[None, :] >= r[:, None], s, -np.inf)
        return s

    def dropped_scale(q_bh, k_bh, scale, causal, rows=None):
        return real_scores(q_bh, k_bh, 1.0, causal, rows)

    def off_by_one_mask(q_bh, k_bh, scale, causal, rows=None):
        s = real_scores(q_bh, k_bh, scale, False, rows)
        if causal:
            r = np.arange(q_bh.shape[0]) if rows is None else rows
            s = np.where(np.arange(k_bh.shape[0])[None, :] < r[:, None], s, -np.inf)
            s[:, 0] = np.where(np.isneginf(s[:, 0]), 0.0, s[:, 0])
        return s

    for bad in (flipped_mask, dropped_scale, off_by_one_mask):
        monkeypatch.setattr(oattn, "scores", bad)
        assert not _forward_pins_pass(), bad.__name__
        monkeypatch.setattr(oattn, "scores", real_scores)

    real_stats = oattn.softmax_stats

    def log2_lse(s):
        m, l, _ = real_stats(s)
        return m, l, m + np.log2(l)

    monkeypatch.setattr(oattn, "softmax_stats", log2_lse)
    assert not _forward_pins_pass()


def test_planted_backward_mistakes_are_caught(monkeypatch):
    shape = (1, 1, 6, 3)
    q, k, v, do = (_rand(shape, seed=300 + i) for i in range(4))
    scale = 0.6

    def fd_ok():
        o, lse = oracle.attention_forward(q, k, v, scale, True)
        grads = oracle.attention_backward(q, k, v, o, do, lse, scale, True)
        h = 1e-6
        for x, g in zip((q, k, v), grads):
            for idx in np.ndindex(x.shape):
                old = x[idx]
                x[idx] = old + h
                lp = _loss(q, k, v, do, scale, True)
                x[idx] = old - h
                lm = _loss(q, k, v, do, scale, True)
                x[idx] = old
                if abs((lp - lm) / (2 * h) - g[idx]) > 1e-6 * max(1.0, abs(g[idx])):
                    return False
        return True

    assert fd_ok()

    # forgetting the mask in the backward: recompute P from unmasked scores
    real_scores = oattn.scores
    # (the backward asks for all rows at once; the forward passes row indices)
    monkeypatch.setattr(oattn, "scores",
                        lambda qb, kb, sc, causal, rows=None:
                        real_scores(qb, kb, sc, causal and rows is not None, rows))
    ok = fd_ok()
    monkeypatch.setattr(oattn, "scores", real_scores)
    assert not ok

    # dropping D from dS = P * (dP - D)
    real_bwd = oattn.attention_backward

    def no_delta(q_, k_, v_, o_, do_, lse_, sc, causal):
        return real_bwd(q_, k_, v_, np.zeros_like(o_), do_, lse_, sc, causal)

    monkeypatch.setattr(oattn, "attention_backward", no_delta)
    monkeypatch.setattr(oracle, "attention_backward", no_delta)
    ok = fd_ok()
    monkeypatch.setattr(oattn, "attention_backward", real_bwd)
    monkeypatch.setattr(oracle, "attention_backward", real_bwd)
    assert not ok


# ---- grouped K/V heads, query / key lengths that differ, packed batches -----------------------

def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_with_one_query_head_per_group_is_attention_forward(causal):
    q, k, v = (_rand((2, 3, 37, 8), s) for s in (1, 2, 3))
    o1, l1 = oracle.attention_forward_gqa(q, k, v, 0.3, causal)
    o2, l2 = oracle.attention_forward(q, k, v, 0.3, causal)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-13)


def _bottom_right_mask(Tq, Tk):
    i = torch.arange(Tq)[:, None]
    j = torch.arange(Tk)[None, :]
    return j <= i + (Tk - Tq)


@pytest.mark.parametrize("G,Tq,Tk,causal", [(4, 23, 23, True), (2, 9, 31, True), (8, 17, 40, False),
                                             (4, 12, 50, True), (1, 30, 7, False)])
def test_gqa_matches_torch_sdpa_float64(G, Tq, Tk, causal):
    # pinned to torch's float64 CPU attention with grouped heads and an explicit mask
    B, Hkv, D = 2, 2, 16
    q = _rand((B, Hkv * G, Tq, D), 4)
    k, v = _rand((B, Hkv, Tk, D), 5), _rand((B, Hkv, Tk, D), 6)
    o, lse = oracle.attention_forward_gqa(q, k, v, 0.25, causal)
    mask = _bottom_right_mask(Tq, Tk) if causal else None
    ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                                         attn_mask=mask, scale=0.25, enable_gqa=True).numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    # LSE against scipy on scores built with each query head's own K/V head
    kk = np.repeat(k, G, axis=1)
    s = np.einsum("bhqd,bhkd->bhqk", q, kk) * 0.25
    if causal:
        s = np.where(_bottom_right_mask(Tq, Tk).numpy(), s, -np.inf)
    np.testing.assert_allclose(lse, scipy.special.logsumexp(s, axis=-1), rtol=0, atol=1e-12)


def test_cross_causal_uniform_scores_closed_form():
    # q = 0: every visible key has score 0, so O_i = mean(V[0 : i + Tk - Tq + 1]) and
    # LSE_i = ln(i + Tk - Tq + 1); with Tk < Tq the first Tq - Tk rows see nothing.
    Tk, D = 6, 3
    v = _rand((Tk, D), 7)
    for Tq in (4, 6, 9):
        o, lse = oracle.attention_cross(np.zeros((Tq, D)), _rand((Tk, D), 8), v, 0.7, True)
        for i in range(Tq):
            n = i + Tk - Tq + 1
            if n <= 0:
                assert np.all(o[i] == 0) and lse[i] == -np.inf
            else:
                np.testing.assert_allclose(o[i], v[:n].mean(axis=0), rtol=0, atol=1e-14)
                assert abs(lse[i] - math.log(n)) < 1e-14


def test_varlen_is_attention_per_sequence():
    Hq, Hkv, D = 4, 2, 8
    lq, lk = [5, 0, 17, 1, 33], [7, 3, 17, 12, 20]
    cu_q, cu_k = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
    q = _rand((cu_q[-1], Hq, D), 9)
    k, v = _rand((cu_k[-1], Hkv, D), 10), _rand((cu_k[-1], Hkv, D), 11)
    for causal in (False, True):
        o, lse = oracle.attention_forward_varlen(q, k, v, cu_q, cu_k, 0.4, causal)
        for b in range(len(lq)):
            if lq[b] == 0:
                continue
            sl_q, sl_k = slice(cu_q[b], cu_q[b + 1]), slice(cu_k[b], cu_k[b + 1])
            qs = torch.from_numpy(np.ascontiguousarray(q[sl_q].transpose(1, 0, 2)))[None]
            ks = torch.from_numpy(np.ascontiguousarray(k[sl_k].transpose(1, 0, 2)))[None]
            vs = torch.from_numpy(np.ascontiguousarray(v[sl_k].transpose(1, 0, 2)))[None]
            mask = _bottom_right_mask(lq[b], lk[b]) if causal else None
            seen = mask.any(dim=1).numpy() if causal else np.ones(lq[b], bool)
            ref = F.scaled_dot_product_attention(qs, ks, vs, attn_mask=mask, scale=0.4,
                                                 enable_gqa=True)[0].numpy().transpose(1, 0, 2)
            np.testing.assert_allclose(o[sl_q][seen], ref[seen], rtol=0, atol=1e-12)
            assert np.all(o[sl_q][~seen] == 0) and np.all(lse[:, sl_q][:, ~seen] == -np.inf)


def test_planted_gqa_mistakes_are_caught(monkeypatch):
    # a top-left causal rule, or query head h using K/V head h % Hkv, must fail the pins
    q = _rand((1, 4, 9, 8), 12)
    k, v = _rand((1, 2, 14, 8), 13), _rand((1, 2, 14, 8), 14)
    mask = _bottom_right_mask(9, 14)
    ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                                         attn_mask=mask, scale=0.3, enable_gqa=True).numpy()

    def top_left(q_h, k_h, v_h, scale, causal):
        s = (q_h @ k_h.T) * scale
        s = np.where(np.arange(k_h.shape[0])[None] <= np.arange(q_h.shape[0])[:, None], s, -np.inf)
        _, _, lse = oattn.softmax_stats(s)
        return np.exp(s - lse[:, None]) @ v_h, lse
    monkeypatch.setattr(oattn, "attention_cross", top_left)
    o_bad, _ = oattn.attention_forward_gqa(q, k, v, 0.3, True)
    assert np.abs(o_bad - ref).max() > 1e-3
    monkeypatch.undo()
    o_ok, _ = oattn.attention_forward_gqa(q, k, v, 0.3, True)
    np.testing.assert_allclose(o_ok, ref, rtol=0, atol=1e-12)
    o_mod = np.stack([oattn.attention_cross(q[0, h], k[0, h % 2], v[0, h % 2], 0.3, True)[0]
                      for h in range(4)])[None]
    assert np.abs(o_mod - ref).max() > 1e-3


# ---------------------------------------------------------------- split-K decode
SPLIT_CASES = [(1, 50, False), (1, 50, True), (4, 37, True), (6, 4, True), (3, 20, False)]


def _split_pins(cases=SPLIT_CASES, trials=6):
    """Split-and-merge over random key ranges (empty ones included) against the definition."""
    rng = np.random.default_rng(20)
    for Tq, Tk, causal in cases:
        q, k, v = _rand((Tq, 8), 21), _rand((Tk, 8), 22), _rand((Tk, 8), 23)
        o_ref, l_ref = oracle.attention_cross(q, k, v, 0.45, causal)
        seen = np.isfinite(l_ref)
        for _ in range(trials):
            cuts = np.sort(rng.integers(0, Tk + 1, rng.integers(0, 6)))
            bounds = np.concatenate([[0], cuts, [Tk]])
            o, lse = oracle.attention_split_k(q, k, v, 0.45, causal, bounds)
            if not (np.array_equal(np.isfinite(lse), seen) and np.all(np.isfinite(o))
                    and np.max(np.abs(o - o_ref)) <= 1e-13
                    and np.max(np.abs(lse[seen] - l_ref[seen]), initial=0.0) <= 1e-13
                    and np.all(o[~seen] == 0)):
                return False
    return True


def test_split_k_reaches_the_definition():
    # [Lab06] "Check yourself" answer 2: partial (m, l, acc) per key range, merged with the
    # rescaling rule, equals exact attention; ranges a row cannot see (causal) and empty ranges
    # contribute nothing, and a row that sees no key at all ends as O = 0, LSE = -inf
    assert _split_pins()


def test_split_k_single_range_is_the_partial_normalised():
    q, k, v = _rand((3, 8), 24), _rand((11, 8), 25), _rand((11, 8), 26)
    m, l, acc = oracle.split_partial(q, k, v, 0.5, 0, 11, np.full(3, 10))
    s = (q @ k.T) * 0.5
    np.testing.assert_allclose(m, s.max(axis=1), rtol=0, atol=0)
    np.testing.assert_allclose(m + np.log(l), scipy.special.logsumexp(s, axis=1), rtol=0, atol=1e-13)
    o, lse = oracle.merge_partials([m], [l], [acc])
    np.testing.assert_allclose(o, scipy.special.softmax(s, axis=1) @ v, rtol=0, atol=1e-13)


def test_planted_merge_mistakes_are_caught(monkeypatch):
    # each plausible slip in the merge fails the split pins
    real = oattn.merge_partials

    def no_weights(ms, ls, accs):
        ms, ls, accs = np.stack(ms), np.stack(ls), np.stack(accs)
        m = np.max(ms, axis=0)
        return np.sum(accs, 0) / np.sum(ls, 0)[:, None], m + np.log(np.sum(ls, 0))

    def no_empty_guard(ms, ls, accs):
        ms, ls, accs = np.stack(ms), np.stack(ls), np.stack(accs)
        m = np.max(ms, axis=0)
        with np.errstate(invalid="ignore", divide="ignore"):
            w = np.exp(ms - m[None, :])
            l = np.sum(w * ls, 0)
            return np.sum(w[:, :, None] * accs, 0) / l[:, None], m + np.log(l)

    def unweighted_lse(ms, ls, accs):
        o, lse = real(ms, ls, accs)
        m = np.max(np.stack(ms), axis=0)
        with np.errstate(divide="ignore"):
            return o, m + np.log(np.sum(np.stack(ls), 0))

    for wrong in (no_weights, no_empty_guard, unweighted_lse):
        monkeypatch.setattr(oattn, "merge_partials", wrong)
        with np.errstate(invalid="ignore", divide="ignore", over="ignore"):
            assert not _split_pins(), wrong.__name__
    monkeypatch.setattr(oattn, "merge_partials", real)
    assert _split_pins()


@pytest.mark.parametrize("causal", [False, True])
def test_decode_matches_torch_sdpa_float64(causal):
    # pinned to torch's float64 CPU attention on each sequence's valid keys, LSE to torch's
    # logsumexp of the explicit scores
    B, Hq, Hkv, Tq, Tk, D = 4, 8, 2, 3, 40, 16
    q, k, v = _rand((B, Hq, Tq, D), 30), _rand((B, Hkv, Tk, D), 31), _rand((B, Hkv, Tk, D), 32)
    lens = [40, 17, 2, 0]
    o, lse = oracle.attention_decode(q, k, v, lens, 0.3, causal)
    G = Hq // Hkv
    for b, L in enumerate(lens):
        if L == 0:
            assert np.all(o[b] == 0) and np.all(lse[b] == -np.inf)
            continue
        mask = _bottom_right_mask(Tq, L) if causal else torch.ones(Tq, L, dtype=torch.bool)
        seen = mask.any(dim=1).numpy()
        qt = torch.from_numpy(q[b:b + 1])
        kt, vt = (torch.from_numpy(np.ascontiguousarray(x[b:b + 1, :, :L])) for x in (k, v))
        ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=0.3,
                                             enable_gqa=True)[0].numpy()
        s = torch.matmul(qt, kt.repeat_interleave(G, dim=1).transpose(-1, -2)) * 0.3
        ref_lse = torch.logsumexp(s.masked_fill(~mask, -math.inf), dim=-1)[0].numpy()
        np.testing.assert_allclose(o[b][:, seen], ref[:, seen], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[b][:, seen], ref_lse[:, seen], rtol=0, atol=1e-12)
        assert np.all(o[b][:, ~seen] == 0) and np.all(lse[b][:, ~seen] == -np.inf)


def test_decode_closed_forms():
    # Q = 0 and one query row: O is the mean of the valid V rows, LSE = ln L; counts are
    # clamped into [0, Tk]
    B, Hq, Hkv, Tk, D = 4, 4, 4, 30, 8
    v = _rand((B, Hkv, Tk, D), 33)
    lens = [30, 99, 5, -3]
    o, lse = oracle.attention_decode(np.zeros((B, Hq, 1, D)), _rand((B, Hkv, Tk, D), 34), v,
                                     lens, 0.9, True)
    for b, L in enumerate([30, 30, 5, 0]):
        if L == 0:
            assert np.all(o[b] == 0) and np.all(lse[b] == -np.inf)
            continue
        np.testing.assert_allclose(o[b, :, 0], v[b, :, :L].mean(axis=1), rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[b, :, 0], math.log(L), rtol=0, atol=1e-14)


def test_decode_without_lengths_is_gqa_forward():
    q, k, v = _rand((2, 6, 2, 8), 35), _rand((2, 3, 25, 8), 36), _rand((2, 3, 25, 8), 37)
    for causal in (False, True):
        o1, l1 = oracle.attention_decode(q, k, v, None, 0.35, causal)
        o2, l2 = oracle.attention_forward_gqa(q, k, v, 0.35, causal)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
