"""Race check of the LDS tile pipelines: the race-check build (libfa_synccheck.so, compiled with
FA_SYNC_CHECK=1) waits for every outstanding load and LDS access and takes a workgroup barrier
before each stage that reads a tile from LDS, so none of its reads can overtake a direct
HBM-to-LDS load or another wave's accesses. Its outputs must equal the release build's bit for
bit on every entry point; a read that the release build's hand-placed waits let through too
early would show up as a difference. The pages' software pipelining ("Lab 06 - Attention
kernels", "Stretch": num_stages) is what these waits protect.
"""
import ctypes
import math

import numpy as np
import pytest
import torch

import synth
from gpu_util import device_tensor

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def libs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_tiled_attention_flash_amd as fa
    from exact_tiled_attention_flash_amd import _lib
    return fa.load_library(), _lib.load_variant(_lib.SYNC_CHECK_LIB_PATH)


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _f(x):
    return ctypes.c_float(x)


def _fwd(lib, q, k, v, causal, dtype):
    B, H, T, D = q.shape
    o, lse = torch.empty_like(q), torch.empty((B, H, T), dtype=torch.float32, device="cuda")
    assert lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                      B, H, T, D, _f(1 / math.sqrt(D)), int(causal), dtype, _stream()) == 0
    return o, lse


def _bwd(lib, q, k, v, o, do, lse, causal, dtype):
    B, H, T, D = q.shape
    ws = torch.empty(lib.fa_bwd_workspace_bytes(B, H, T, D), dtype=torch.uint8, device="cuda")
    g = [torch.empty_like(q) for _ in range(3)]
    assert lib.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                      lse.data_ptr(), *(t.data_ptr() for t in g), ws.data_ptr(), ws.numel(),
                      B, H, T, D, _f(1 / math.sqrt(D)), int(causal), dtype, _stream()) == 0
    return g


def _same(a, b, what):
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y), what


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("T", [1, 37, 64, 65, 129, 200, 1000])
def test_fwd_bwd_bitwise_equal(libs, T, causal, D, dtype):
    print(f"case race check fwd/bwd T={T} D={D} causal={causal} dtype={dtype}", flush=True)
    rel, chk = libs
    code = 1 if dtype == "bf16" else 0
    d = synth.make_inputs(2, 3, T, D, dtype, seed=T + D, with_do=True)
    q, k, v, do = (device_tensor(d[n], dtype) for n in ("q", "k", "v", "do"))
    o1, l1 = _fwd(rel, q, k, v, causal, code)
    o2, l2 = _fwd(chk, q, k, v, causal, code)
    _same((o1, l1), (o2, l2), "forward")
    _same(_bwd(rel, q, k, v, o1, do, l1, causal, code), _bwd(chk, q, k, v, o1, do, l1, causal, code),
          "backward")


def test_headline_and_backward_workloads_bitwise_equal(libs):
    rel, chk = libs
    w = synth.WORKLOADS["fwd_bf16_b4h16t4096d128_causal"]
    print("case race check headline workload", flush=True)
    d = synth.make_workload_inputs(w)
    q, k, v = (device_tensor(d[n], "bf16") for n in "qkv")
    _same(_fwd(rel, q, k, v, True, 1), _fwd(chk, q, k, v, True, 1), "headline forward")
    wb = synth.WORKLOADS["bwd_bf16_b2h16t4096d128_causal"]
    print("case race check backward workload", flush=True)
    d = synth.make_workload_inputs(wb)
    q, k, v, do = (device_tensor(d[n], "bf16") for n in ("q", "k", "v", "do"))
    o, lse = _fwd(rel, q, k, v, True, 1)
    _same(_bwd(rel, q, k, v, o, do, lse, True, 1), _bwd(chk, q, k, v, o, do, lse, True, 1),
          "backward workload")


@pytest.mark.parametrize("causal", [False, True])
def test_grouped_packed_fp8_decode_bitwise_equal(libs, causal):
    print(f"case race check grouped/packed/fp8/decode causal={causal}", flush=True)
    rel, chk = libs
    rng = np.random.default_rng(7)

    def bf(shape):
        return device_tensor(synth.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32)),
                             "bf16")

    B, Hq, Hkv, Tq, Tk, D = 2, 8, 2, 300, 700, 128
    q, k, v = bf((B, Hq, Tq, D)), bf((B, Hkv, Tk, D)), bf((B, Hkv, Tk, D))
    outs = []
    for lib in (rel, chk):
        o, lse = torch.empty_like(q), torch.empty((B, Hq, Tq), device="cuda")
        assert lib.fa_fwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                              lse.data_ptr(), B, Hq, Hkv, Tq, Tk, D, _f(0.09), int(causal), 1,
                              _stream()) == 0
        outs.append((o, lse))
    _same(*outs, "grouped")

    lens = [700, 1, 0, 129, 300]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda")
    tot = int(sum(lens))
    qp, kp, vp = bf((tot, Hq, D)), bf((tot, Hkv, D)), bf((tot, Hkv, D))
    outs = []
    for lib in (rel, chk):
        o, lse = torch.zeros_like(qp), torch.zeros((Hq, tot), device="cuda")
        assert lib.fa_fwd_varlen(qp.data_ptr(), kp.data_ptr(), vp.data_ptr(), o.data_ptr(),
                                 lse.data_ptr(), cu.data_ptr(), cu.data_ptr(), len(lens), Hq, Hkv,
                                 tot, tot, max(lens), D, _f(0.09), int(causal), 1, _stream()) == 0
        outs.append((o, lse))
    _same(*outs, "packed")

    # a skewed batch with 8 head groups: the longest-first grid order
    lens = [2100, 1, 0, 129, 300]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda")
    tot = int(sum(lens))
    qp, kp, vp = bf((tot, 8, D)), bf((tot, 8, D)), bf((tot, 8, D))
    outs = []
    for lib in (rel, chk):
        o, lse = torch.zeros_like(qp), torch.zeros((8, tot), device="cuda")
        assert lib.fa_fwd_varlen(qp.data_ptr(), kp.data_ptr(), vp.data_ptr(), o.data_ptr(),
                                 lse.data_ptr(), cu.data_ptr(), cu.data_ptr(), len(lens), 8, 8,
                                 tot, tot, max(lens), D, _f(0.09), int(causal), 1, _stream()) == 0
        outs.append((o, lse))
    _same(*outs, "packed, skewed")

    q8 = torch.empty((B, Hq, Tq, D), dtype=torch.uint8, device="cuda")
    qs = torch.empty((B, Hq, Tq, D // 32), dtype=torch.uint8, device="cuda")
    k8 = torch.empty((B, Hkv, Tk, D), dtype=torch.uint8, device="cuda")
    ks = torch.empty((B, Hkv, Tk, D // 32), dtype=torch.uint8, device="cuda")
    assert rel.fa_quantize_mxfp8(q.data_ptr(), q8.data_ptr(), qs.data_ptr(), B * Hq * Tq, D, 1,
                                 _stream()) == 0
    assert rel.fa_quantize_mxfp8(k.data_ptr(), k8.data_ptr(), ks.data_ptr(), B * Hkv * Tk, D, 1,
                                 _stream()) == 0
    outs = []
    for lib in (rel, chk):
        o, lse = torch.empty_like(q), torch.empty((B, Hq, Tq), device="cuda")
        assert lib.fa_fwd_fp8qk(q8.data_ptr(), qs.data_ptr(), k8.data_ptr(), ks.data_ptr(),
                                v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, Hq, Hkv, Tq, Tk, D,
                                _f(0.09), int(causal), _stream()) == 0
        outs.append((o, lse))
    _same(*outs, "fp8")

    qd = bf((B, Hq, 2, D))
    sl = torch.tensor([700, 333], dtype=torch.int32, device="cuda")
    outs = []
    for lib in (rel, chk):
        nbytes = lib.fa_decode_workspace_bytes(B, Hq, Hkv, 2, Tk, D, 0)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        o, lse = torch.empty_like(qd), torch.empty((B, Hq, 2), device="cuda")
        assert lib.fa_fwd_decode(qd.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                 lse.data_ptr(), sl.data_ptr(), ws.data_ptr(), nbytes, B, Hq, Hkv,
                                 2, Tk, D, 0, _f(0.09), int(causal), 1, _stream()) == 0
        outs.append((o, lse))
    _same(*outs, "decode")
