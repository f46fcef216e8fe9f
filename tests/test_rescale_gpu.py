"""The exp(m - m') rescale of the online softmax, on the GPU, in every forward instantiation.

"Lab 06 - Attention kernels", section 2 and "What to implement" item 1 (a row maximum that
jumps from -40 to 1000 across tiles), and "Common bugs" (the first tile already holds the
maximum). The bf16 forward moves a row's reference maximum only when a tile beats it by more
than 2^8 in the exp2 domain, in a wave-uniform branch; with N(0,1) inputs that branch is
practically never taken after the first tile. The inputs here (synth/planted.py) plant key
scores that make it happen: a late jump to 1000, a rising staircase past the margin, one just
below it, a maximum held by the first tile, and rows of one wave of which only half see the
planted scores. Every case is compared element by element with the float64 oracle at the
usual tolerances (bf16: O <= 2e-2, LSE <= 1e-3; fp32: 1e-4) through the C ABI: dense (D 64 and
128, causal and not, bf16 and fp32), grouped K/V heads with Tq == Tk and Tq != Tk, packed
variable-length batches, block-scaled E4M3 Q K^T, and the split-K decode.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.fp8 as f8
from gpu_util import TOL, as_f64, device_tensor, e4m3_tolerances, host_f64
from synth import planted

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_tiled_attention_flash_amd as m
    return m


def _check(o, lse, o_ref, l_ref, what, dtype="bf16"):
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(lse), fin), f"{what}: -inf rows differ"
    assert np.all(o[~fin] == 0), f"{what}: rows that see no key"
    assert np.all(np.isfinite(o)), f"{what}: non-finite O"
    eo = float(np.max(np.abs(o - o_ref))) if o.size else 0.0
    el = float(np.max(np.abs(lse[fin] - l_ref[fin]))) if fin.any() else 0.0
    assert eo <= TOL[dtype]["o"], f"{what} O max-abs {eo:.3e}"
    assert el <= TOL[dtype]["lse"], f"{what} LSE max-abs {el:.3e}"
    return eo, el


CASES = [("jump", False, None), ("jump", True, None), ("jump", False, 70), ("jump", False, 995),
         ("first_tile_max", False, None), ("staircase", False, None), ("staircase", True, None),
         ("below_margin", False, None)]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("scenario,mixed,p", CASES)
def test_dense_bf16(fa, scenario, mixed, p, causal, D):
    print(f"case rescale dense bf16 {scenario} mixed={mixed} p={p} D={D} causal={causal}",
          flush=True)
    T = 1000
    d = planted.make_planted(1, 2, 2, T, T, D, scenario, seed=D + 3, mixed=mixed, p=p)
    q, k, v = (device_tensor(d[n], "bf16") for n in "qkv")
    o, lse = fa.fa_fwd(q, k, v, causal=causal, scale=d["scale"])
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_forward(*(as_f64(d[n], "bf16") for n in "qkv"), d["scale"],
                                            causal)
    e = _check(host_f64(o), lse.cpu().numpy().astype(np.float64), o_ref, l_ref, scenario)
    print("max-abs O, LSE:", e)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("scenario", ["staircase", "first_tile_max", "below_margin"])
def test_dense_f32(fa, scenario, causal, D):
    # the fp32 kernel keeps an exact running maximum; its rescale runs on every raised max
    print(f"case rescale dense f32 {scenario} D={D} causal={causal}", flush=True)
    T = 700
    d = planted.make_planted(1, 2, 2, T, T, D, scenario, seed=D + 5)
    q, k, v = (device_tensor(as_f64(d[n], "bf16").astype(np.float32), "f32") for n in "qkv")
    o, lse = fa.fa_fwd(q, k, v, causal=causal, scale=d["scale"])
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_forward(*(as_f64(d[n], "bf16") for n in "qkv"), d["scale"],
                                            causal)
    _check(host_f64(o), lse.cpu().numpy().astype(np.float64), o_ref, l_ref, scenario, "f32")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("G,Tq,Tk", [(4, 700, 700), (2, 300, 900), (8, 129, 1000)])
@pytest.mark.parametrize("scenario,mixed", [("jump", True), ("staircase", False)])
def test_gqa(fa, scenario, mixed, G, Tq, Tk, causal, D):
    print(f"case rescale gqa {scenario} G={G} Tq={Tq} Tk={Tk} D={D} causal={causal}", flush=True)
    Hkv = 2
    d = planted.make_planted(1, Hkv * G, Hkv, Tq, Tk, D, scenario, seed=G * 10 + D, mixed=mixed)
    o, lse = fa.fa_fwd_gqa(*(device_tensor(d[n], "bf16") for n in "qkv"), causal=causal,
                           scale=d["scale"])
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_forward_gqa(*(as_f64(d[n], "bf16") for n in "qkv"),
                                                d["scale"], causal)
    _check(host_f64(o), lse.cpu().numpy().astype(np.float64), o_ref, l_ref,
           f"gqa {scenario} G={G}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("scenario,mixed", [("jump", False), ("jump", True), ("staircase", False)])
def test_varlen(fa, scenario, mixed, causal, D):
    print(f"case rescale varlen {scenario} mixed={mixed} D={D} causal={causal}", flush=True)
    G, Hkv = 2, 2
    d = planted.make_planted_varlen([700, 1, 300, 0, 129, 1000], Hkv * G, Hkv, D, scenario,
                                    seed=D + 7, mixed=mixed)
    cu = torch.from_numpy(d["cu"]).cuda()
    o, lse = fa.fa_fwd_varlen(*(device_tensor(d[n], "bf16") for n in "qkv"), cu, cu,
                              int(d["lens"].max()), causal=causal, scale=d["scale"])
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_forward_varlen(*(as_f64(d[n], "bf16") for n in "qkv"),
                                                   d["cu"], d["cu"], d["scale"], causal)
    _check(host_f64(o), lse.cpu().numpy().astype(np.float64).T, o_ref, l_ref.T,
           f"varlen {scenario}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("G", [1, 2])
@pytest.mark.parametrize("scenario,mixed", [("jump", False), ("jump", True), ("staircase", False),
                                            ("first_tile_max", False)])
def test_fp8qk(fa, scenario, mixed, G, causal, D):
    # Parity against the oracle on the dequantized Q and K, with the tolerance widened by
    # what the E4M3 product's own summation can move a score (gpu_util.e4m3_tolerances):
    # planted scores of about -40 are a -448 x 1 product cancelling small ones, and the
    # matrix core sums a block of products to about 12 bits of its largest product.
    print(f"case rescale fp8qk {scenario} mixed={mixed} G={G} D={D} causal={causal}", flush=True)
    Hkv, T = 2, 1000
    d = planted.make_planted(1, Hkv * G, Hkv, T, T, D, scenario, seed=G + D, mixed=mixed)
    q8, qs = fa.fa_quantize_mxfp8(device_tensor(d["q"], "bf16"))
    k8, ks = fa.fa_quantize_mxfp8(device_tensor(d["k"], "bf16"))
    o, lse = fa.fa_fwd_fp8qk(q8, qs, k8, ks, device_tensor(d["v"], "bf16"), causal=causal,
                             scale=d["scale"])
    torch.cuda.synchronize()
    q, k, v = (as_f64(d[n], "bf16") for n in "qkv")
    o_ref, l_ref = f8.attention_forward_fp8qk(q, k, v, d["scale"], causal)
    o, lse = host_f64(o), lse.cpu().numpy().astype(np.float64)
    qd = f8.dequantize_mxfp8(*f8.quantize_mxfp8(q))
    kd = f8.dequantize_mxfp8(*f8.quantize_mxfp8(k))
    worst = 0.0
    for h in range(Hkv * G):
        tol_o, tol_l = e4m3_tolerances(qd[0, h], kd[0, h // G], v[0, h // G], d["scale"], causal)
        eo = np.abs(o[0, h] - o_ref[0, h]).max(axis=1)
        el = np.abs(lse[0, h] - l_ref[0, h])
        assert np.all(np.isfinite(o[0, h])) and np.all(np.isfinite(lse[0, h])), f"head {h}"
        assert np.all(eo <= tol_o), f"head {h}: O row {int(np.argmax(eo - tol_o))} {eo.max():.3e}"
        assert np.all(el <= tol_l), f"head {h}: LSE row {int(np.argmax(el - tol_l))} {el.max():.3e}"
        worst = max(worst, float(np.max(el / tol_l)), float(np.max(eo / tol_o)))
    print(f"fp8qk {scenario}: largest fraction of a row's tolerance used {worst:.2f}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G,Tq", [(8, 1), (4, 4)])
@pytest.mark.parametrize("scenario,mixed", [("jump", False), ("jump", True), ("staircase", False)])
def test_decode(fa, scenario, mixed, G, Tq, D):
    print(f"case rescale decode {scenario} mixed={mixed} G={G} Tq={Tq} D={D}", flush=True)
    Hkv, Tk = 2, 5000
    d = planted.make_planted(2, Hkv * G, Hkv, Tq, Tk, D, scenario, seed=G + Tq + D, mixed=mixed)
    lens = [Tk, 3001]
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    for splits in (0, 7):
        o, lse = fa.fa_fwd_decode(*(device_tensor(d[n], "bf16") for n in "qkv"), cache_seqlens=sl,
                                  num_splits=splits, causal=True, scale=d["scale"])
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.attention_decode(*(as_f64(d[n], "bf16") for n in "qkv"), lens,
                                               d["scale"], True)
        _check(host_f64(o), lse.cpu().numpy().astype(np.float64), o_ref, l_ref,
               f"decode {scenario} splits={splits}")


def test_long_jump_d128_causal(fa):
    # several query tiles and a jump inside the unmasked main loop of later tiles
    print("case rescale dense bf16 jump T=4099 D=128 causal", flush=True)
    T, D = 4099, 128
    d = planted.make_planted(1, 1, 1, T, T, D, "jump", seed=99, p=2100)
    o, lse = fa.fa_fwd(*(device_tensor(d[n], "bf16") for n in "qkv"), causal=True,
                       scale=d["scale"])
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_forward(*(as_f64(d[n], "bf16") for n in "qkv"), d["scale"],
                                            True)
    _check(host_f64(o), lse.cpu().numpy().astype(np.float64), o_ref, l_ref, "jump T=4099")
    assert math.isclose(float(l_ref[0, 0, -1]), 1000.0, abs_tol=2.0)
