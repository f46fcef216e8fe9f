"""Rows past the end of every input are never read: each input sits at the start of a larger
device buffer whose remaining rows hold NaN, and the results must match the oracle (a single
NaN that reached a product or a sum would show up in the outputs). The kernels bound their
tile loads by the last valid row, so ragged lengths are the interesting cases.

Tolerances as in the other GPU parity tests (max-abs): bf16 O <= 2e-2, LSE <= 1e-3, gradients
<= 2e-2; fp32 1e-4.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.fp8 as f8
import synth
from gpu_util import TOL, as_f64, device_tensor, host_f64

pytestmark = pytest.mark.gpu

PAD = 64   # NaN rows after each input


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_tiled_attention_flash_amd as m
    return m


def _nan_padded(t: torch.Tensor, rows: int) -> torch.Tensor:
    """t (rows, ...) copied to the start of a buffer with PAD more rows of NaN; returns the
    contiguous view of the first `rows` rows."""
    buf = torch.full((rows + PAD,) + tuple(t.shape[1:]), float("nan"), dtype=t.dtype, device=t.device)
    buf[:rows].copy_(t)
    return buf[:rows]


def _nan_padded_bytes(t: torch.Tensor, rows: int, fill: int) -> torch.Tensor:
    buf = torch.full((rows + PAD,) + tuple(t.shape[1:]), fill, dtype=t.dtype, device=t.device)
    buf[:rows].copy_(t)
    return buf[:rows]


def _dense(d, name, dtype, T, D):
    """(1, 1, T, D) input whose buffer continues with NaN rows."""
    return _nan_padded(device_tensor(d[name], dtype).reshape(T, D), T).view(1, 1, T, D)


def _check(o, lse, o_ref, l_ref, dtype, what):
    assert np.all(np.isfinite(o)), f"{what}: non-finite O"
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(lse), fin), f"{what}: -inf rows differ"
    eo = float(np.max(np.abs(o - o_ref))) if o.size else 0.0
    el = float(np.max(np.abs(lse[fin] - l_ref[fin]))) if fin.any() else 0.0
    assert eo <= TOL[dtype]["o"], f"{what} O max-abs {eo:.3e}"
    assert el <= TOL[dtype]["lse"], f"{what} LSE max-abs {el:.3e}"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("T", [1, 37, 64, 65, 130])
def test_fwd_never_reads_past_T(fa, T, causal, D, dtype):
    print(f"case bounds fwd T={T} D={D} causal={causal} dtype={dtype}", flush=True)
    d = synth.make_inputs(1, 1, T, D, dtype, seed=900 + T + D)
    q, k, v = (_dense(d, n, dtype, T, D) for n in "qkv")
    scale = 1 / math.sqrt(D)
    o, lse = fa.fa_fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_forward(*(as_f64(d[n], dtype) for n in "qkv"), scale, causal)
    _check(host_f64(o), lse.cpu().numpy().astype(np.float64), o_ref, l_ref, dtype, f"T={T}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("T", [1, 65, 130])
def test_bwd_never_reads_past_T(fa, T, causal, D, dtype):
    print(f"case bounds bwd T={T} D={D} causal={causal} dtype={dtype}", flush=True)
    d = synth.make_inputs(1, 1, T, D, dtype, seed=950 + T + D, with_do=True)
    q, k, v, do = (_dense(d, n, dtype, T, D) for n in ("q", "k", "v", "do"))
    scale = 1 / math.sqrt(D)
    o, lse = fa.fa_fwd(q, k, v, causal=causal, scale=scale)
    o = _nan_padded(o.reshape(T, D), T).view(1, 1, T, D)
    lse = _nan_padded(lse.reshape(T), T).view(1, 1, T)
    dq, dk, dv = fa.fa_bwd(q, k, v, o, do, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    q64, k64, v64, do64 = (as_f64(d[n], dtype) for n in ("q", "k", "v", "do"))
    o_ref, lse_ref = oracle.attention_forward(q64, k64, v64, scale, causal)
    ref = oracle.attention_backward(q64, k64, v64, o_ref, do64, lse_ref, scale, causal)
    for g, r, name in zip((dq, dk, dv), ref, ("dQ", "dK", "dV")):
        gh = host_f64(g)
        assert np.all(np.isfinite(gh)), name
        err = float(np.max(np.abs(gh - r)))
        assert err <= TOL[dtype]["grad"], f"{name} max-abs {err:.3e}"


def test_varlen_never_reads_past_the_last_sequence(fa):
    lens = [5, 70, 1, 129]
    H, D = 2, 128
    rng = np.random.default_rng(977)
    total = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    arrays = {n: synth.f32_to_bf16_bits(rng.standard_normal((total, H, D)).astype(np.float32))
              for n in "qkv"}
    q, k, v = (_nan_padded(device_tensor(arrays[n], "bf16"), total) for n in "qkv")
    cu_t = torch.from_numpy(cu).cuda()
    scale = 1 / math.sqrt(D)
    for causal in (False, True):
        o, lse = fa.fa_fwd_varlen(q, k, v, cu_t, cu_t, max(lens), causal=causal, scale=scale)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.attention_forward_varlen(*(as_f64(arrays[n], "bf16") for n in "qkv"),
                                                       cu, cu, scale, causal)
        # LSE is (H, total); its transpose lines up with O's (total, H) rows
        _check(host_f64(o), lse.cpu().numpy().astype(np.float64).T, o_ref, l_ref.T, "bf16",
               f"varlen causal={causal}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("T", [33, 100])
def test_fp8qk_never_reads_past_T(fa, T, D):
    print(f"case bounds fp8 T={T} D={D}", flush=True)
    d = synth.make_inputs(1, 1, T, D, "bf16", seed=990 + T + D)
    q8, qs = fa.fa_quantize_mxfp8(device_tensor(d["q"], "bf16"))
    k8, ks = fa.fa_quantize_mxfp8(device_tensor(d["k"], "bf16"))
    # E4M3 code 0x7F and scale byte 0xFF are NaN
    k8 = _nan_padded_bytes(k8.reshape(T, D), T, 0x7F).view(1, 1, T, D)
    ks = _nan_padded_bytes(ks.reshape(T, D // 32), T, 0xFF).view(1, 1, T, D // 32)
    v = _dense(d, "v", "bf16", T, D)
    scale = 1 / math.sqrt(D)
    for causal in (False, True):
        o, lse = fa.fa_fwd_fp8qk(q8, qs, k8, ks, v, causal=causal, scale=scale)
        torch.cuda.synchronize()
        o_ref, l_ref = f8.attention_forward_fp8qk(*(as_f64(d[n], "bf16") for n in "qkv"), scale, causal)
        _check(host_f64(o), lse.cpu().numpy().astype(np.float64), o_ref, l_ref, "bf16",
               f"fp8 T={T} causal={causal}")


def test_decode_never_reads_past_the_valid_keys(fa):
    # keys at or past a sequence's valid length hold NaN inside the cache itself
    B, Hq, Hkv, Tk, D = 3, 8, 2, 300, 128
    lens = [1, 129, 300]
    rng = np.random.default_rng(991)
    qb = synth.f32_to_bf16_bits(rng.standard_normal((B, Hq, 1, D)).astype(np.float32))
    kb = synth.f32_to_bf16_bits(rng.standard_normal((B, Hkv, Tk, D)).astype(np.float32))
    vb = synth.f32_to_bf16_bits(rng.standard_normal((B, Hkv, Tk, D)).astype(np.float32))
    k, v = device_tensor(kb, "bf16"), device_tensor(vb, "bf16")
    for b, n in enumerate(lens):
        k[b, :, n:] = float("nan")
        v[b, :, n:] = float("nan")
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    scale = 1 / math.sqrt(D)
    for splits in (0, 1, 7):
        o, lse = fa.fa_fwd_decode(device_tensor(qb, "bf16"), k, v, cache_seqlens=sl,
                                  num_splits=splits, scale=scale)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.attention_decode(as_f64(qb, "bf16"), as_f64(kb, "bf16"),
                                               as_f64(vb, "bf16"), lens, scale, False)
        _check(host_f64(o), lse.cpu().numpy().astype(np.float64), o_ref, l_ref, "bf16",
               f"decode splits={splits}")
