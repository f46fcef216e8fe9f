"""fa_bwd_noalloc (the backward whose row statistics live in the library's fixed scratch
array, for callers that cannot allocate) against fa_bwd with a caller workspace, through the
C ABI: bit-identical gradients on two calls in a row, the second smaller than the first, for
bf16 and fp32, causal and not; sizes past the array are refused without touching anything."""
import ctypes

import pytest
import torch

import synth
from gpu_util import device_tensor

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_tiled_attention_flash_amd as m
    return m


def _case(fa, B, H, T, D, dtype, causal, seed):
    d = synth.make_inputs(B, H, T, D, dtype, seed=seed, with_do=True)
    q, k, v, do = (device_tensor(d[n], dtype) for n in ("q", "k", "v", "do"))
    o, lse = fa.fa_fwd(q, k, v, causal=causal)
    ref = fa.fa_bwd(q, k, v, o, do, lse, causal=causal)
    got = fa.fa_bwd_noalloc(q, k, v, o, do, lse, causal=causal)
    torch.cuda.synchronize()
    for r, g, n in zip(ref, got, ("dQ", "dK", "dV")):
        assert torch.equal(r, g), f"{n} B={B} H={H} T={T} D={D} {dtype} causal={causal}"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_noalloc_matches_fa_bwd_twice(fa, dtype, causal):
    print(f"case noalloc {dtype} causal={causal}", flush=True)
    _case(fa, 2, 4, 700, 128, dtype, causal, seed=1)   # larger first
    _case(fa, 1, 3, 129, 64, dtype, causal, seed=2)    # then smaller: stale rows must not leak


def test_noalloc_full_backward_workload(fa):
    w = synth.WORKLOADS["bwd_bf16_b2h16t4096d128_causal"]
    print("case noalloc backward workload", flush=True)
    _case(fa, w.B, w.H, w.T, w.D, "bf16", True, seed=3)


def test_noalloc_refuses_sizes_past_the_array(fa):
    lib = fa.load_library()
    cap = fa.fa_bwd_noalloc_max_bytes()
    assert cap == 16 << 20
    x = torch.full((1, 1, 64, 64), 3.0, device="cuda", dtype=torch.bfloat16)
    lse = torch.zeros(1, 1, 64, device="cuda")
    p = x.data_ptr()
    T = cap // 8 + 1                  # one row more than the array holds
    rc = lib.fa_bwd_noalloc(p, p, p, p, p, lse.data_ptr(), p, p, p, 1, 1, T, 64,
                            ctypes.c_float(0.1), 1, 1, None)
    assert rc == fa._lib.FA_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((x == 3.0).all())
