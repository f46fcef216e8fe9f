"""Split-K decode on the GPU (fa_fwd_decode through the C ABI) against the CPU float64 oracle.

Tolerances as for the forward: bf16 O max-abs <= 2e-2, LSE <= 1e-3. Rows that see no key
(causal with Tq above the valid length, or a sequence with no valid keys) must come back as
O = 0 and LSE = -inf exactly.
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


def _bf16(shape, seed):
    a = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)
    return synth.f32_to_bf16_bits(a)


def _check(o, lse, o_ref, lse_ref, what):
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse), fin), f"{what}: -inf rows differ"
    assert np.all(lse[~fin] == -np.inf) and np.all(o[~fin] == 0), f"{what}: unseen rows"
    err_o = float(np.max(np.abs(o - o_ref))) if o.size else 0.0
    err_l = float(np.max(np.abs(lse[fin] - lse_ref[fin]))) if fin.any() else 0.0
    assert err_o <= TOL["bf16"]["o"], f"{what} O max-abs {err_o:.3e}"
    assert err_l <= TOL["bf16"]["lse"], f"{what} LSE max-abs {err_l:.3e}"
    return err_o, err_l


def _run(fa, B, Hq, Hkv, Tq, Tk, D, causal, lens=None, splits=0, seed=0):
    qb = _bf16((B, Hq, Tq, D), seed + 1)
    kb, vb = _bf16((B, Hkv, Tk, D), seed + 2), _bf16((B, Hkv, Tk, D), seed + 3)
    scale = 1 / math.sqrt(D)
    sl = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda")
    o, lse = fa.fa_fwd_decode(device_tensor(qb, "bf16"), device_tensor(kb, "bf16"),
                              device_tensor(vb, "bf16"), cache_seqlens=sl, num_splits=splits,
                              causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_decode(as_f64(qb, "bf16"), as_f64(kb, "bf16"),
                                           as_f64(vb, "bf16"), lens, scale, causal)
    return host_f64(o), lse.cpu().numpy().astype(np.float64), o_ref, l_ref


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("G,Tq,Tk", [(1, 1, 1), (4, 1, 31), (4, 1, 32), (8, 1, 33), (4, 1, 1000),
                                     (2, 3, 100), (8, 4, 257), (1, 2, 4097), (4, 8, 5),
                                     (16, 2, 700), (32, 1, 65)])
def test_decode_vs_oracle(fa, G, Tq, Tk, causal, D):
    print(f"case decode G={G} Tq={Tq} Tk={Tk} D={D} causal={causal}", flush=True)
    o, lse, o_ref, l_ref = _run(fa, 2, 2 * G, 2, Tq, Tk, D, causal)
    _check(o, lse, o_ref, l_ref, f"G={G} Tq={Tq} Tk={Tk}")


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 64, 1000])
def test_decode_split_counts(fa, splits):
    # every split count (including more splits than key tiles) gives the same attention
    print(f"case decode splits={splits}", flush=True)
    o, lse, o_ref, l_ref = _run(fa, 2, 8, 2, 1, 1500, 128, True, splits=splits, seed=4)
    _check(o, lse, o_ref, l_ref, f"splits={splits}")


@pytest.mark.parametrize("causal", [False, True])
def test_decode_cache_lengths(fa, causal):
    # per-sequence valid lengths, clamped into [0, Tk]: empty, shorter than Tq, ragged, beyond Tk
    print(f"case decode lengths causal={causal}", flush=True)
    lens = [0, 2, 37, 600, 5000, 1025]
    o, lse, o_ref, l_ref = _run(fa, len(lens), 8, 2, 4, 1100, 128, causal, lens=lens, seed=5)
    _check(o, lse, o_ref, l_ref, "lengths")
    assert np.all(o[0] == 0) and np.all(lse[0] == -np.inf)


@pytest.mark.parametrize("n_seq,splits", [(64, 0), (64, 1), (64, 3), (65, 0), (7, 1000)])
def test_decode_many_lengths(fa, n_seq, splits):
    # up to 64 sequences: split slots shared out by length; 65: one split count for all. Lengths
    # from empty to the whole cache, with automatic, single, few and very many split slots
    print(f"case decode {n_seq} lengths splits={splits}", flush=True)
    rng = np.random.default_rng(n_seq + splits)
    lens = [int(x) for x in rng.integers(0, 700, n_seq)]
    lens[0], lens[1], lens[-1] = 0, 700, 1
    o, lse, o_ref, l_ref = _run(fa, n_seq, 8, 2, 1, 700, 64, True, lens=lens, splits=splits,
                                seed=13)
    _check(o, lse, o_ref, l_ref, f"{n_seq} lengths splits={splits}")


def test_decode_negative_length_is_empty(fa):
    o, lse, o_ref, l_ref = _run(fa, 2, 4, 4, 1, 64, 64, False, lens=[-5, 64], seed=6)
    _check(o, lse, o_ref, l_ref, "negative length")
    assert np.all(lse[0] == -np.inf)


def test_decode_matches_forward_kernel(fa):
    # the decode and the grouped forward compute the same rows (within rounding)
    B, Hq, Hkv, Tq, Tk, D = 2, 16, 4, 2, 3000, 128
    q = device_tensor(_bf16((B, Hq, Tq, D), 7), "bf16")
    k = device_tensor(_bf16((B, Hkv, Tk, D), 8), "bf16")
    v = device_tensor(_bf16((B, Hkv, Tk, D), 9), "bf16")
    o1, l1 = fa.fa_fwd_decode(q, k, v, causal=True)
    o2, l2 = fa.fa_fwd_gqa(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert (o1.float() - o2.float()).abs().max().item() <= 2 * 2 ** -8
    assert (l1 - l2).abs().max().item() <= 1e-4


def test_decode_deterministic(fa):
    B, Hq, Hkv, Tk, D = 3, 32, 8, 2049, 128
    q = device_tensor(_bf16((B, Hq, 1, D), 10), "bf16")
    k = device_tensor(_bf16((B, Hkv, Tk, D), 11), "bf16")
    v = device_tensor(_bf16((B, Hkv, Tk, D), 12), "bf16")
    o1, l1 = fa.fa_fwd_decode(q, k, v)
    o2, l2 = fa.fa_fwd_decode(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_v_ones_gives_ones(fa):
    # V = 1: O = 1 for every row, whatever the splits (the normaliser is the rounded-P sum)
    B, Hq, Hkv, Tk, D = 2, 8, 2, 3333, 64
    q = device_tensor(_bf16((B, Hq, 1, D), 13), "bf16")
    k = device_tensor(_bf16((B, Hkv, Tk, D), 14), "bf16")
    v = torch.ones((B, Hkv, Tk, D), dtype=torch.bfloat16, device="cuda")
    for splits in (0, 5):
        o, _ = fa.fa_fwd_decode(q, k, v, num_splits=splits)
        torch.cuda.synchronize()
        assert (o.float() - 1).abs().max().item() <= 4e-3


# ------------------------------------------------ full-size workloads, as the benchmark runs them
@pytest.mark.parametrize("name", sorted(synth.DECODE_WORKLOADS))
def test_decode_workload_full_size(fa, name):
    w = synth.DECODE_WORKLOADS[name]
    print(f"case {name}", flush=True)
    d = synth.make_gqa_inputs(w)
    lens = synth.decode_lengths(w)
    sl = torch.from_numpy(lens).cuda() if w.B > 1 else None
    o, lse = fa.fa_fwd_decode(*(device_tensor(d[n], "bf16") for n in "qkv"), cache_seqlens=sl,
                              causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_decode(*(as_f64(d[n], "bf16") for n in "qkv"),
                                           lens if w.B > 1 else None, w.scale, w.causal)
    e = _check(host_f64(o), lse.cpu().numpy().astype(np.float64), o_ref, l_ref, name)
    print(name, "max-abs O, LSE:", e)
