"""Forward parity on the GPU: the HIP kernels (through the C ABI) against the CPU
float64 oracle, element by element, plus properties that need no oracle.

Tolerances (max-abs): bf16 inputs O <= 2e-2 and LSE <= 1e-3; fp32 inputs 1e-4.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import TOL, as_f64, device_tensor, host_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_tiled_attention_flash_amd as m
    return m


def _run(fa, d, dtype, causal, scale):
    q, k, v = (device_tensor(d[n], dtype) for n in "qkv")
    o, lse = fa.fa_fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return host_f64(o), lse.cpu().numpy().astype(np.float64)


def _compare(o, lse, o_ref, lse_ref, dtype, what=""):
    err_o = float(np.max(np.abs(o - o_ref))) if o.size else 0.0
    err_l = float(np.max(np.abs(lse - lse_ref))) if lse.size else 0.0
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), what
    assert err_o <= TOL[dtype]["o"], f"{what} O max-abs {err_o:.3e}"
    assert err_l <= TOL[dtype]["lse"], f"{what} LSE max-abs {err_l:.3e}"
    return err_o, err_l


SWEEP_T = [1, 2, 7, 33, 37, 63, 64, 65, 127, 128, 129, 200, 1000]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("T", SWEEP_T)
def test_fwd_sweep_vs_oracle(fa, T, causal, D, dtype):
    print(f"case fwd T={T} D={D} causal={causal} dtype={dtype}", flush=True)
    d = synth.make_inputs(1, 2, T, D, dtype, seed=T * 7 + D)
    scale = 1.0 / math.sqrt(D)
    o, lse = _run(fa, d, dtype, causal, scale)
    o_ref, lse_ref = oracle.attention_forward(*(as_f64(d[n], dtype) for n in "qkv"), scale, causal)
    _compare(o, lse, o_ref, lse_ref, dtype, f"T={T}")


@pytest.mark.parametrize("B,H", [(3, 5), (2, 1)])
def test_fwd_batch_heads(fa, B, H):
    for dtype in ("bf16", "f32"):
        for causal in (False, True):
            d = synth.make_inputs(B, H, 150, 64, dtype, seed=B * 10 + H)
            o, lse = _run(fa, d, dtype, causal, 0.125)
            o_ref, lse_ref = oracle.attention_forward(*(as_f64(d[n], dtype) for n in "qkv"),
                                                      0.125, causal)
            _compare(o, lse, o_ref, lse_ref, dtype)


@pytest.mark.parametrize("D", [64, 128])
def test_fwd_heads_in_groups_of_four_per_xcd(fa, D):
    """B * H a multiple of 32 takes the grid order that hands each XCD four heads at a time;
    every head and query tile must still be computed once, in the right place."""
    B, H, T = 2, 16, 300
    for causal in (False, True):
        print(f"case fwd grouped grid B={B} H={H} T={T} D={D} causal={causal}", flush=True)
        d = synth.make_inputs(B, H, T, D, "bf16", seed=400 + D)
        o, lse = _run(fa, d, "bf16", causal, 1.0 / math.sqrt(D))
        o_ref, lse_ref = oracle.attention_forward(*(as_f64(d[n], "bf16") for n in "qkv"),
                                                  1.0 / math.sqrt(D), causal)
        _compare(o, lse, o_ref, lse_ref, "bf16", f"causal={causal}")


def test_workload_small_f32(fa):
    w = synth.WORKLOADS["fwd_f32_b1h2t128d64"]
    d = synth.make_workload_inputs(w)
    o, lse = _run(fa, d, "f32", w.causal, w.scale)
    o_ref, lse_ref = oracle.attention_forward(*(as_f64(d[n], "f32") for n in "qkv"), w.scale, w.causal)
    e = _compare(o, lse, o_ref, lse_ref, "f32")
    print("fp32 B=1 H=2 T=128 D=64 max-abs O, LSE:", e)


@pytest.mark.parametrize("name", ["fwd_bf16_b1h8t1024d64", "fwd_bf16_b1h8t1024d64_causal"])
def test_workload_bf16_t1024(fa, name):
    w = synth.WORKLOADS[name]
    d = synth.make_workload_inputs(w)
    o, lse = _run(fa, d, "bf16", w.causal, w.scale)
    o_ref, lse_ref = oracle.attention_forward(*(as_f64(d[n], "bf16") for n in "qkv"), w.scale, w.causal)
    e = _compare(o, lse, o_ref, lse_ref, "bf16")
    print(name, "max-abs O, LSE:", e)


def _sampled_parity(fa, w, full_heads, n_rows, seed=0):
    """Full-size run; oracle on the given whole heads plus, when n_rows > 0, sampled rows of
    every head (rows 0, 1, T-1, T-2 and rows just after spike positions among them)."""
    d = synth.make_workload_inputs(w)
    o, lse = _run(fa, d, w.dtype, w.causal, w.scale)
    q, k, v = (d[n] for n in "qkv")
    rng = np.random.default_rng(seed)
    worst = (0.0, 0.0)
    BH = w.B * w.H
    for idx in full_heads:
        b, h = divmod(idx, w.H)
        qh, kh, vh = (as_f64(x[b:b + 1, h:h + 1], w.dtype) for x in (q, k, v))
        o_ref, lse_ref = oracle.attention_forward(qh, kh, vh, w.scale, w.causal)
        e = _compare(o[b:b + 1, h:h + 1], lse[b:b + 1, h:h + 1], o_ref, lse_ref, w.dtype,
                     f"head {idx}")
        worst = tuple(max(a, c) for a, c in zip(worst, e))
    extra = list(d.get("spikes", []))
    for idx in range(BH if n_rows > 0 else 0):
        b, h = divmod(idx, w.H)
        rows = np.unique(np.concatenate([
            rng.integers(0, w.T, n_rows), [0, 1, w.T - 1, w.T - 2],
            np.clip(np.array(extra[:8], dtype=np.int64) + 1, 0, w.T - 1)]))
        kh, vh = as_f64(k[b, h], w.dtype), as_f64(v[b, h], w.dtype)
        qh = as_f64(q[b, h], w.dtype)
        o_ref, lse_ref = oracle.attention_rows(qh, kh, vh, w.scale, w.causal, rows)
        e = _compare(o[b, h, rows], lse[b, h, rows], o_ref, lse_ref, w.dtype, f"rows of head {idx}")
        worst = tuple(max(a, c) for a, c in zip(worst, e))
    return worst


def test_workload_headline_causal_t4096(fa):
    # every head whole ("Triton FlashAttention-2 forward", "Correctness": the whole output
    # against the reference), at the size and in the launch configuration the benchmark times
    w = synth.WORKLOADS["fwd_bf16_b4h16t4096d128_causal"]
    worst = _sampled_parity(fa, w, full_heads=range(w.B * w.H), n_rows=0)
    print("B=4 H=16 T=4096 D=128 causal, worst max-abs O, LSE over every head:", worst)


def test_workload_long_ragged_spiky(fa):
    w = synth.WORKLOADS["fwd_bf16_b1h32t16381d128_causal_spiky"]
    worst = _sampled_parity(fa, w, full_heads=range(w.B * w.H), n_rows=0)
    print("B=1 H=32 T=16381 D=128 causal spiky, worst max-abs O, LSE over every head:", worst)


@pytest.mark.parametrize("D,causal", [(128, True), (64, False)])
def test_million_key_sequence(fa, D, causal):
    # one head of T = 2^20 + 3 (16385 key tiles, ragged): the long end of the sizes the calls
    # accept (a head stays below 2^31 bytes up to T = 2^22 at D = 128); every tile's online
    # rescale and the fp32 row sums over a million keys, on sampled rows including the last
    T = (1 << 20) + 3
    print(f"case one head T={T} D={D} causal={causal}", flush=True)
    d = synth.make_inputs(1, 1, T, D, "bf16", seed=D + 11)
    scale = 1 / math.sqrt(D)
    o, lse = _run(fa, d, "bf16", causal, scale)
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, T // 2, T - 3, T - 2, T - 1],
                                     rng.integers(0, T, 6)]))
    q, k, v = (as_f64(d[n][0, 0], "bf16") for n in "qkv")
    o_ref, lse_ref = oracle.attention_rows(q, k, v, scale, causal, rows)
    e = _compare(o[0, 0, rows], lse[0, 0, rows], o_ref, lse_ref, "bf16", f"T={T} rows")
    print(f"T={T} D={D} causal={causal} max-abs O, LSE on {len(rows)} rows:", e)


# ------------------------------------------------------------ oracle-free properties
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_v_ones_gives_ones(fa, dtype, causal):
    d = synth.make_inputs(2, 3, 333, 128, dtype, seed=11)
    q, k = device_tensor(d["q"], dtype), device_tensor(d["k"], dtype)
    v = torch.ones_like(q)
    o, _ = fa.fa_fwd(q, k, v, causal=causal)
    err = (o.float() - 1).abs().max().item()
    assert err <= (4e-3 if dtype == "bf16" else 1e-6), err


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_uniform_scores_closed_form(fa, dtype):
    # Q = 0: causal O_i = mean(V[0..i]), LSE_i = ln(i + 1); non-causal O = mean(V), LSE = ln T
    T, D = 300, 64
    d = synth.make_inputs(1, 2, T, D, dtype, seed=12)
    v64 = as_f64(d["v"], dtype)
    q = torch.zeros((1, 2, T, D), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32,
                    device="cuda")
    k, v = device_tensor(d["k"], dtype), device_tensor(d["v"], dtype)
    o, lse = fa.fa_fwd(q, k, v, causal=True)
    prefix = np.cumsum(v64, axis=2) / np.arange(1, T + 1)[None, None, :, None]
    assert np.max(np.abs(host_f64(o) - prefix)) <= TOL[dtype]["o"]
    assert np.max(np.abs(lse.cpu().numpy() - np.log(np.arange(1, T + 1)))) <= 1e-5
    o, lse = fa.fa_fwd(q, k, v, causal=False)
    assert np.max(np.abs(host_f64(o) - v64.mean(axis=2, keepdims=True))) <= TOL[dtype]["o"]
    assert np.max(np.abs(lse.cpu().numpy() - math.log(T))) <= 1e-5
    # scale = 0 has the same effect
    q2 = device_tensor(d["q"], dtype)
    o, lse = fa.fa_fwd(q2, k, v, causal=True, scale=0.0)
    assert np.max(np.abs(host_f64(o) - prefix)) <= TOL[dtype]["o"]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_causal_row_zero_is_v0(fa, dtype):
    d = synth.make_inputs(2, 2, 257, 128, dtype, seed=13)
    q, k, v = (device_tensor(d[n], dtype) for n in "qkv")
    o, lse = fa.fa_fwd(q, k, v, causal=True, scale=0.1)
    if dtype == "bf16":
        assert torch.equal(o[:, :, 0], v[:, :, 0])
    else:
        assert (o[:, :, 0] - v[:, :, 0]).abs().max().item() <= 1e-6
    s00 = 0.1 * (as_f64(d["q"], dtype)[:, :, 0] * as_f64(d["k"], dtype)[:, :, 0]).sum(-1)
    assert np.max(np.abs(lse[:, :, 0].cpu().numpy() - s00)) <= 1e-5


def test_deterministic_and_stream(fa):
    d = synth.make_inputs(2, 4, 777, 128, "bf16", seed=14)
    q, k, v = (device_tensor(d[n], "bf16") for n in "qkv")
    o1, l1 = fa.fa_fwd(q, k, v, causal=True)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o2, l2 = fa.fa_fwd(q, k, v, causal=True)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_outputs_untouched_on_error(fa):
    import ctypes
    lib = fa.load_library()
    q = torch.randn(1, 1, 64, 64, device="cuda", dtype=torch.bfloat16)
    o = torch.full_like(q, 7.0)
    lse = torch.full((1, 1, 64), 7.0, device="cuda")
    for D, scale, causal in ((96, 0.1, 0), (64, -1.0, 0), (64, 0.1, 3)):
        rc = lib.fa_fwd(q.data_ptr(), q.data_ptr(), q.data_ptr(), o.data_ptr(), lse.data_ptr(),
                        1, 1, 64, D, ctypes.c_float(scale), causal, 1, None)
        assert rc < 0
    torch.cuda.synchronize()
    assert bool((o == 7.0).all()) and bool((lse == 7.0).all())
