"""Backward parity on the GPU: fa_bwd (through the C ABI) against the CPU float64
oracle's backward. The GPU backward takes O and LSE from the GPU forward; the
oracle uses its own float64 forward.

Tolerance: max-abs <= 2e-2 on dQ, dK, dV for bf16 inputs. Outputs are stored in
bf16, so an entry of magnitude >= 8 cannot be closer than half a bf16 ulp
(0.03125) to the exact value; such entries are allowed that rounding floor
on top of 2e-2 and the test reports how many there were.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import planted
from gpu_util import as_f64, bwd_rounding_bound, device_tensor, host_f64

pytestmark = pytest.mark.gpu
TOL = 2e-2


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_tiled_attention_flash_amd as m
    return m


def _half_ulp_bf16(x):
    ax = np.abs(x)
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return 2.0 ** (e - 8)  # bf16 has 8 significant bits (7 stored)


def _check_grad(g, ref, name):
    err = np.abs(g - ref)
    assert np.all(np.isfinite(g)), name
    floor = np.where(np.abs(ref) >= 8.0, _half_ulp_bf16(ref), 0.0)
    bad = err > TOL + floor
    assert not bad.any(), (f"{name}: max-abs {err.max():.3e} at |ref| "
                           f"{np.abs(ref).ravel()[err.argmax()]:.3f}; {bad.sum()} over tolerance")
    return float(err.max()), int((np.abs(ref) >= 8.0).sum())


def _gpu_fwd_bwd(fa, d, causal, scale):
    q, k, v, do = (device_tensor(d[n], "bf16") for n in ("q", "k", "v", "do"))
    o, lse = fa.fa_fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa.fa_bwd(q, k, v, o, do, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return q, k, v, do, o, lse, dq, dk, dv


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("T", [1, 2, 7, 33, 64, 65, 127, 129, 200, 1000])
def test_bwd_sweep_vs_oracle(fa, T, causal, D):
    print(f"case bwd T={T} D={D} causal={causal}", flush=True)
    d = synth.make_inputs(1, 2, T, D, "bf16", seed=T * 3 + D, with_do=True)
    scale = 1.0 / math.sqrt(D)
    *_, dq, dk, dv = _gpu_fwd_bwd(fa, d, causal, scale)
    q64, k64, v64, do64 = (as_f64(d[n], "bf16") for n in ("q", "k", "v", "do"))
    o_ref, lse_ref = oracle.attention_forward(q64, k64, v64, scale, causal)
    ref = oracle.attention_backward(q64, k64, v64, o_ref, do64, lse_ref, scale, causal)
    for g, r, n in zip((dq, dk, dv), ref, ("dQ", "dK", "dV")):
        _check_grad(host_f64(g), r, n)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("T", [1000, 1031])
def test_bwd_spiky_keys_vs_oracle(fa, T, causal, D):
    # the long ragged workload's recipe at a size the oracle finishes quickly: 1 % of the key
    # rows scaled by 8, so some rows' softmax is dominated by one key and the gradient sums
    # cancel large terms. The bf16 roundings of O (feeding D_i) and of dS are then amplified
    # past the flat 2e-2; each entry is held to the bound derived from those roundings
    # (gpu_util.bwd_rounding_bound), which planted mistakes exceed (tests/test_bwd_bound.py).
    print(f"case bwd spiky T={T} D={D} causal={causal}", flush=True)
    d = planted.make_spiky(1, 2, T, D, seed=T + D)
    scale = 1.0 / math.sqrt(D)
    *_, dq, dk, dv = _gpu_fwd_bwd(fa, d, causal, scale)
    q64, k64, v64, do64 = (as_f64(d[n], "bf16") for n in ("q", "k", "v", "do"))
    o_ref, lse_ref = oracle.attention_forward(q64, k64, v64, scale, causal)
    ref = oracle.attention_backward(q64, k64, v64, o_ref, do64, lse_ref, scale, causal)
    rep = []
    for h in range(2):
        bounds = bwd_rounding_bound(q64[0, h], k64[0, h], v64[0, h], do64[0, h], o_ref[0, h],
                                    lse_ref[0, h], scale, causal)
        for g, r, b, n in zip((dq, dk, dv), ref, bounds, ("dQ", "dK", "dV")):
            err = np.abs(host_f64(g)[0, h] - r[0, h])
            assert np.all(np.isfinite(err)), n
            assert np.all(err <= b), (f"{n} head {h}: max-abs {err.max():.3e}, "
                                      f"{int((err > b).sum())} entries over the derived bound")
            rep.append((n, float(err.max()), float((err / b).max())))
    print("spiky backward (grad, max-abs, largest fraction of the bound):", rep)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("T", [1, 2, 7, 33, 64, 65, 129, 200, 1000])
def test_bwd_f32_sweep_vs_oracle(fa, T, causal, D):
    # the true-fp32 backward (fp32 products, P and dS kept in fp32) on the fp32 forward's O
    # and LSE, element by element against the oracle at the fp32 tolerance 1e-4
    print(f"case bwd f32 T={T} D={D} causal={causal}", flush=True)
    d = synth.make_inputs(1, 2, T, D, "f32", seed=T * 5 + D, with_do=True)
    scale = 1.0 / math.sqrt(D)
    q, k, v, do = (device_tensor(d[n], "f32") for n in ("q", "k", "v", "do"))
    o, lse = fa.fa_fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa.fa_bwd(q, k, v, o, do, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    q64, k64, v64, do64 = (as_f64(d[n], "f32") for n in ("q", "k", "v", "do"))
    o_ref, lse_ref = oracle.attention_forward(q64, k64, v64, scale, causal)
    ref = oracle.attention_backward(q64, k64, v64, o_ref, do64, lse_ref, scale, causal)
    errs = []
    for g, r, n in zip((dq, dk, dv), ref, ("dQ", "dK", "dV")):
        gh = host_f64(g)
        assert np.all(np.isfinite(gh)), n
        errs.append(float(np.max(np.abs(gh - r))))
        assert errs[-1] <= 1e-4, f"{n} max-abs {errs[-1]:.3e}"
    print("fp32 backward max-abs dQ, dK, dV:", errs)


def test_bwd_f32_batch_heads_and_spiky_keys(fa):
    # several (b, h), a ragged T, and the long workload's 1 % of keys x 8 in fp32
    for causal in (False, True):
        d = synth.make_inputs(2, 3, 150, 64, "f32", seed=31, with_do=True)
        sp = planted.make_spiky(1, 2, 300, 128, seed=32)
        for dd, dt in ((d, "f32"), ({n: as_f64(sp[n], "bf16").astype(np.float32)
                                     for n in ("q", "k", "v", "do")}, "f32")):
            D = dd["q"].shape[-1]
            scale = 1.0 / math.sqrt(D)
            q, k, v, do = (device_tensor(dd[n], dt) for n in ("q", "k", "v", "do"))
            o, lse = fa.fa_fwd(q, k, v, causal=causal, scale=scale)
            grads = fa.fa_bwd(q, k, v, o, do, lse, causal=causal, scale=scale)
            torch.cuda.synchronize()
            q64, k64, v64, do64 = (dd[n].astype(np.float64) for n in ("q", "k", "v", "do"))
            o_ref, lse_ref = oracle.attention_forward(q64, k64, v64, scale, causal)
            ref = oracle.attention_backward(q64, k64, v64, o_ref, do64, lse_ref, scale, causal)
            for g, r, n in zip(grads, ref, ("dQ", "dK", "dV")):
                err = float(np.max(np.abs(host_f64(g) - r)))
                assert err <= 1e-4, f"{n} D={D} causal={causal} max-abs {err:.3e}"


def test_bwd_batch_heads(fa):
    for causal in (False, True):
        d = synth.make_inputs(2, 3, 150, 64, "bf16", seed=21, with_do=True)
        *_, dq, dk, dv = _gpu_fwd_bwd(fa, d, causal, 0.125)
        q64, k64, v64, do64 = (as_f64(d[n], "bf16") for n in ("q", "k", "v", "do"))
        o_ref, lse_ref = oracle.attention_forward(q64, k64, v64, 0.125, causal)
        ref = oracle.attention_backward(q64, k64, v64, o_ref, do64, lse_ref, 0.125, causal)
        for g, r, n in zip((dq, dk, dv), ref, ("dQ", "dK", "dV")):
            _check_grad(host_f64(g), r, n)


@pytest.mark.parametrize("D", [64, 128])
def test_bwd_heads_in_groups_of_four_per_xcd(fa, D):
    """B * H a multiple of 32 takes the grid order that hands each XCD four heads at a time,
    in both backward kernels; every head and tile must still be computed once, in its place."""
    B, H, T = 2, 16, 300
    scale = 1.0 / math.sqrt(D)
    for causal in (False, True):
        print(f"case bwd grouped grid B={B} H={H} T={T} D={D} causal={causal}", flush=True)
        d = synth.make_inputs(B, H, T, D, "bf16", seed=410 + D, with_do=True)
        *_, dq, dk, dv = _gpu_fwd_bwd(fa, d, causal, scale)
        q64, k64, v64, do64 = (as_f64(d[n], "bf16") for n in ("q", "k", "v", "do"))
        o_ref, lse_ref = oracle.attention_forward(q64, k64, v64, scale, causal)
        ref = oracle.attention_backward(q64, k64, v64, o_ref, do64, lse_ref, scale, causal)
        for g, r, n in zip((dq, dk, dv), ref, ("dQ", "dK", "dV")):
            _check_grad(host_f64(g), r, n)


def test_workload_backward_causal_t4096(fa):
    w = synth.WORKLOADS["bwd_bf16_b2h16t4096d128_causal"]
    d = synth.make_workload_inputs(w)
    q, k, v, do, o, lse, dq, dk, dv = _gpu_fwd_bwd(fa, d, w.causal, w.scale)
    # oracle-free properties over every head: each row of P sums to 1, so the
    # key-sum of dV equals the query-sum of dO; each row of dS sums to 0, so the
    # key-sum of dK vanishes.
    sum_dv = dv.float().sum(dim=2)
    sum_do = do.float().sum(dim=2)
    assert (sum_dv - sum_do).abs().max().item() < 0.5
    assert dk.float().sum(dim=2).abs().max().item() < 0.5
    # and every head whole against the oracle
    report = []
    for idx in range(w.B * w.H):
        b, h = divmod(idx, w.H)
        sl = (slice(b, b + 1), slice(h, h + 1))
        q64, k64, v64, do64 = (as_f64(d[n][sl], "bf16") for n in ("q", "k", "v", "do"))
        o_ref, lse_ref = oracle.attention_forward(q64, k64, v64, w.scale, True)
        ref = oracle.attention_backward(q64, k64, v64, o_ref, do64, lse_ref, w.scale, True)
        for g, r, n in zip((dq, dk, dv), ref, ("dQ", "dK", "dV")):
            report.append((idx, n) + _check_grad(host_f64(g[sl]), r, f"head {idx} {n}"))
    worst = {n: max(r[2] for r in report if r[1] == n) for n in ("dQ", "dK", "dV")}
    print("B=2 H=16 T=4096 D=128 causal backward, worst max-abs over every head:", worst)


def test_bwd_million_key_sequence(fa):
    # one head of T = 2^20 + 3 (ragged), D = 128, causal: dQ of sampled rows (the first, the
    # last, the middle and random ones) and dK, dV of the last 80 keys against the oracle's
    # restricted backward, and the two gradient sums over every key
    T, D = (1 << 20) + 3, 128
    print(f"case backward one head T={T} D={D} causal", flush=True)
    d = synth.make_inputs(1, 1, T, D, "bf16", seed=41, with_do=True)
    scale = 1 / math.sqrt(D)
    q, k, v, do, o, lse, dq, dk, dv = _gpu_fwd_bwd(fa, d, True, scale)
    assert (dv.float().sum(dim=2) - do.float().sum(dim=2)).abs().max().item() < 0.5
    assert dk.float().sum(dim=2).abs().max().item() < 0.5
    q64, k64, v64, do64 = (as_f64(d[n][0, 0], "bf16") for n in ("q", "k", "v", "do"))
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, T // 2, T - 3, T - 2, T - 1],
                                     rng.integers(0, T, 8)]))
    ref = oracle.attention_backward_rows(q64, k64, v64, do64, scale, True, rows)
    e_q = _check_grad(host_f64(dq)[0, 0, rows], ref, f"dQ rows of T={T}")
    r0 = T - 80
    ref_k, ref_v = oracle.attention_backward_key_tail(q64, k64, v64, do64, scale, r0)
    e_k = _check_grad(host_f64(dk)[0, 0, r0:], ref_k, f"dK of the last keys of T={T}")
    e_v = _check_grad(host_f64(dv)[0, 0, r0:], ref_v, f"dV of the last keys of T={T}")
    # the last keys are seen by few queries of a million-key softmax: their gradients are small,
    # so the absolute tolerance says little; they must also hold to 2^-6 of their own magnitude
    # (bf16 rounding of P, dS and the output is 2^-9 each)
    for e, r, n in ((e_k, ref_k, "dK"), (e_v, ref_v, "dV")):
        assert e[0] <= 2.0 ** -6 * np.abs(r).max(), f"{n} tail: {e[0]:.3e} vs |ref| {np.abs(r).max():.3e}"
    print(f"T={T} max-abs dQ rows, dK tail, dV tail:", e_q[0], e_k[0], e_v[0],
          "| largest |dK|, |dV| in the tail:", np.abs(ref_k).max(), np.abs(ref_v).max())


def test_bwd_deterministic(fa):
    d = synth.make_inputs(1, 4, 700, 128, "bf16", seed=22, with_do=True)
    r1 = _gpu_fwd_bwd(fa, d, True, 0.09)
    q, k, v, do, o, lse = r1[:6]
    r2 = fa.fa_bwd(q, k, v, o, do, lse, causal=True, scale=0.09)
    torch.cuda.synchronize()
    for a, b in zip(r1[6:], r2):
        assert torch.equal(a, b)


def test_bwd_zero_upstream_gradient(fa):
    d = synth.make_inputs(1, 2, 300, 64, "bf16", seed=23)
    q, k, v = (device_tensor(d[n], "bf16") for n in "qkv")
    o, lse = fa.fa_fwd(q, k, v, causal=True)
    dq, dk, dv = fa.fa_bwd(q, k, v, o, torch.zeros_like(o), lse, causal=True)
    for g in (dq, dk, dv):
        assert g.abs().max().item() == 0.0


def test_bwd_argument_errors(fa):
    import ctypes
    lib = fa.load_library()
    x = torch.zeros(1, 1, 64, 64, device="cuda", dtype=torch.bfloat16)
    lse = torch.zeros(1, 1, 64, device="cuda")
    g = torch.full_like(x, 3.0)
    ws = torch.zeros(512, dtype=torch.uint8, device="cuda")
    p = x.data_ptr()

    def call(ws_bytes=512, dtype=1, D=64):
        return lib.fa_bwd(p, p, p, p, p, lse.data_ptr(), g.data_ptr(), g.data_ptr(), g.data_ptr(),
                          ws.data_ptr(), ws_bytes, 1, 1, 64, D, ctypes.c_float(0.1), 1, dtype, None)

    assert lib.fa_bwd_workspace_bytes(1, 1, 64, 64) == 512
    assert call(ws_bytes=511) == fa._lib.FA_ERR_ARG
    assert call(dtype=2) == fa._lib.FA_ERR_DTYPE
    assert call(D=96) == fa._lib.FA_ERR_HEADDIM
    torch.cuda.synchronize()
    assert bool((g == 3.0).all())
