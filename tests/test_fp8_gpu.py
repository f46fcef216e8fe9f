"""FP8 (block-scaled E4M3) Q K^T on the GPU, through the C ABI, against the CPU oracle.

The quantizer must reproduce the oracle's codes and scale bytes exactly (integer outputs).
The attention on those codes is compared with the oracle's float64 attention on the same
dequantized Q and K, to the bf16 forward's tolerances (O <= 2e-2, LSE <= 1e-3). The error
against exact attention on the unquantized inputs is the price of FP8: it is reported and held,
row by row, to the bound that row's score error implies.
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


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_tiled_attention_flash_amd as m
    return m


def _bf16(shape, seed, spread=0):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(shape, dtype=np.float32)
    if spread:
        a *= np.exp2(rng.integers(-spread, spread + 1, shape[:-1] + (1,))).astype(np.float32)
    return synth.f32_to_bf16_bits(a)


def _quant(fa, bits):
    c, s = fa.fa_quantize_mxfp8(device_tensor(bits, "bf16"))
    torch.cuda.synchronize()
    return c.cpu().numpy(), s.cpu().numpy()


@pytest.mark.parametrize("D", [32, 64, 128, 96, 256])
def test_quantizer_bit_exact(fa, D):
    bits = _bf16((3, 5, 77, D), D, spread=20)
    codes, scales = _quant(fa, bits)
    rc, rs = f8.quantize_mxfp8(as_f64(bits, "bf16"))
    np.testing.assert_array_equal(scales, rs)
    np.testing.assert_array_equal(codes, rc)


def test_quantizer_edge_values(fa):
    x = np.zeros((6, 64), dtype=np.float32)
    x[1] = -0.0                                              # signed zeros
    x[2, :32] = 2.0 ** -133                                  # bf16 subnormals, one per block
    x[2, 32:] = np.linspace(-1e-30, 1e-30, 32)
    x[3] = np.linspace(-448, 448, 64)                        # exact fit
    x[4, :32] = 3e38                                         # near the bf16 maximum
    x[4, 32:] = 1.0
    x[4, 40] = 2.0 ** -100                                   # tiny beside a large block max
    x[5] = (np.arange(64) % 7 - 3) * 2.0 ** -9              # subnormal E4M3 grid after scaling
    bits = synth.f32_to_bf16_bits(x)
    codes, scales = _quant(fa, bits)
    rc, rs = f8.quantize_mxfp8(as_f64(bits, "bf16"))
    np.testing.assert_array_equal(scales, rs)
    np.testing.assert_array_equal(codes, rc)
    assert np.all(scales[0] == 127) and np.all(codes[0] == 0) and np.all(codes[1] == 0x80)


def _fp8_run(fa, B, Hq, Hkv, Tq, Tk, D, causal, seed=0):
    qb, kb = _bf16((B, Hq, Tq, D), seed + 1), _bf16((B, Hkv, Tk, D), seed + 2)
    vb = _bf16((B, Hkv, Tk, D), seed + 3)
    scale = 1 / math.sqrt(D)
    q8, qs = fa.fa_quantize_mxfp8(device_tensor(qb, "bf16"))
    k8, ks = fa.fa_quantize_mxfp8(device_tensor(kb, "bf16"))
    o, lse = fa.fa_fwd_fp8qk(q8, qs, k8, ks, device_tensor(vb, "bf16"), causal=causal, scale=scale)
    torch.cuda.synchronize()
    q, k, v = (as_f64(x, "bf16") for x in (qb, kb, vb))
    return host_f64(o), lse.cpu().numpy().astype(np.float64), (q, k, v, scale)


def _check(o, lse, o_ref, l_ref, what):
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(lse), fin), f"{what}: -inf rows differ"
    assert np.all(o[~fin] == 0), f"{what}: unseen rows"
    eo = float(np.max(np.abs(o - o_ref)))
    el = float(np.max(np.abs(lse[fin] - l_ref[fin]))) if fin.any() else 0.0
    assert eo <= TOL["bf16"]["o"], f"{what} O max-abs {eo:.3e}"
    assert el <= TOL["bf16"]["lse"], f"{what} LSE max-abs {el:.3e}"
    return eo, el


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("G,Tq,Tk", [(1, 1, 1), (1, 33, 33), (1, 64, 64), (1, 65, 65), (1, 200, 200),
                                     (4, 129, 129), (2, 37, 300), (4, 300, 45), (1, 1000, 1000)])
def test_fp8qk_vs_oracle(fa, G, Tq, Tk, causal, D):
    print(f"case fp8qk G={G} Tq={Tq} Tk={Tk} D={D} causal={causal}", flush=True)
    o, lse, (q, k, v, scale) = _fp8_run(fa, 2, 2 * G, 2, Tq, Tk, D, causal)
    o_ref, l_ref = f8.attention_forward_fp8qk(q, k, v, scale, causal)
    _check(o, lse, o_ref, l_ref, f"G={G} Tq={Tq} Tk={Tk}")


def test_fp8qk_headline_full_size(fa):
    # the benchmark's workload: parity on sampled heads and rows, and the FP8 error against
    # exact attention on the unquantized inputs
    w = synth.WORKLOADS["fwd_bf16_b4h16t4096d128_causal"]
    print("case fp8qk headline", flush=True)
    d = synth.make_workload_inputs(w)
    q8, qs = fa.fa_quantize_mxfp8(device_tensor(d["q"], "bf16"))
    k8, ks = fa.fa_quantize_mxfp8(device_tensor(d["k"], "bf16"))
    o, lse = fa.fa_fwd_fp8qk(q8, qs, k8, ks, device_tensor(d["v"], "bf16"), causal=True, scale=w.scale)
    torch.cuda.synchronize()
    o, lse = host_f64(o), lse.cpu().numpy().astype(np.float64)
    qd = f8.dequantize_mxfp8(q8.cpu().numpy(), qs.cpu().numpy())
    kd = f8.dequantize_mxfp8(k8.cpu().numpy(), ks.cpu().numpy())
    v = as_f64(d["v"], "bf16")
    for idx in (0, 37, 63):
        b, h = divmod(idx, w.H)
        sl = (slice(b, b + 1), slice(h, h + 1))
        o_ref, l_ref = oracle.attention_forward(qd[sl], kd[sl], v[sl], w.scale, True)
        _check(o[sl], lse[sl], o_ref, l_ref, f"head {idx}")
        # the price of FP8 against exact attention on the unquantized inputs, row by row:
        # with delta_i = max_j |S8_ij - S_ij| every softmax weight of row i moves by a factor
        # within [e^-2delta_i, e^2delta_i], so sum_j |p8_ij - p_ij| <= e^(2 delta_i) - 1 and
        # |dO_i| <= (e^(2 delta_i) - 1) max_j |V_j| (plus the kernel's own parity error), and
        # |dLSE_i| <= delta_i
        q, k = as_f64(d["q"][b, h], "bf16"), as_f64(d["k"][b, h], "bf16")
        rows = np.arange(0, w.T, 7)
        s_ex = oracle.scores(q, k, w.scale, True, rows)
        s_8 = oracle.scores(qd[b, h], kd[b, h], w.scale, True, rows)
        fin = np.isfinite(s_ex)
        dif = np.zeros_like(s_ex)
        dif[fin] = np.abs(s_8[fin] - s_ex[fin])
        delta = dif.max(axis=1)
        p_ex = np.exp(s_ex - np.max(s_ex, axis=1, keepdims=True))
        p_ex /= p_ex.sum(axis=1, keepdims=True)
        p_8 = np.exp(s_8 - np.max(s_8, axis=1, keepdims=True))
        p_8 /= p_8.sum(axis=1, keepdims=True)
        assert np.all(np.abs(p_8 - p_ex).sum(axis=1) <= np.expm1(2 * delta) + 1e-12)
        vmax = np.maximum.accumulate(np.abs(v[b, h]).max(axis=1))[rows]   # max over keys <= i
        oe, le = oracle.attention_rows(q, k, v[b, h], w.scale, True, rows)
        err_o = np.abs(o[b, h, rows] - oe).max(axis=1)
        err_l = np.abs(lse[b, h, rows] - le)
        bound_o = np.expm1(2 * delta) * vmax + TOL["bf16"]["o"]
        print(f"head {idx}: FP8 against exact attention max-abs O {err_o.max():.4f}, "
              f"LSE {err_l.max():.4f}; max score error {delta.max():.4f}; "
              f"tightest row uses {float(np.max(err_o / bound_o)):.2f} of its bound")
        assert np.all(err_o <= bound_o), int(np.argmax(err_o - bound_o))
        assert np.all(err_l <= delta + TOL["bf16"]["lse"])


def test_e4m3_product_summation_precision(fa):
    # The tolerance model of the E4M3 path (gpu_util.E4M3_SUM_REL): a score from one query
    # row and one key row (T = 1, so LSE = S exactly) differs from the exact dot product of
    # the dequantized rows by at most 2^-10 of the largest product of each 64-element block.
    # Rows carry one large coordinate (up to 3000) beside N(0,1) ones, the shape of the
    # planted -40 scores in the rescale tests.
    from gpu_util import e4m3_score_error_bound
    D, H = 128, 2048
    rng = np.random.default_rng(5)
    worst = 0.0
    for big in (0.0, 16.0, 452.0, 3000.0):
        q = rng.standard_normal((1, H, 1, D), dtype=np.float32)
        k = rng.standard_normal((1, H, 1, D), dtype=np.float32)
        q[..., 0] = 1.0
        if big:
            k[..., 0] = -big
        qb, kb = synth.f32_to_bf16_bits(q), synth.f32_to_bf16_bits(k)
        vb = synth.f32_to_bf16_bits(np.ones((1, H, 1, D), np.float32))
        q8, qs = fa.fa_quantize_mxfp8(device_tensor(qb, "bf16"))
        k8, ks = fa.fa_quantize_mxfp8(device_tensor(kb, "bf16"))
        _, lse = fa.fa_fwd_fp8qk(q8, qs, k8, ks, device_tensor(vb, "bf16"), scale=1.0)
        torch.cuda.synchronize()
        qd = f8.dequantize_mxfp8(*f8.quantize_mxfp8(as_f64(qb, "bf16")))[0, :, 0]
        kd = f8.dequantize_mxfp8(*f8.quantize_mxfp8(as_f64(kb, "bf16")))[0, :, 0]
        exact = np.sum(qd * kd, axis=-1)
        bound = np.array([e4m3_score_error_bound(qd[i:i + 1], kd[i:i + 1], 1.0)[0, 0]
                          for i in range(H)])
        err = np.abs(lse.cpu().numpy()[0, :, 0].astype(np.float64) - exact)
        assert np.all(err <= bound + 1e-6 * np.abs(exact)), f"big={big}: {np.max(err / bound):.2f}"
        worst = max(worst, float(np.max(err / bound)))
    print(f"E4M3 summation: largest error {worst:.2f} of the 2^-10 bound")
