"""The Python binding refuses caller-supplied buffers that the library cannot use.

A host tensor's pointer would pass the C ABI's null and alignment checks and reach a
kernel; the binding must raise before calling the library when an output, an LSE buffer or
a workspace is not a contiguous device tensor on the inputs' device. None of these calls
launches a kernel.
"""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_tiled_attention_flash_amd as m
    return m


def _qkv(B=1, H=2, T=64, D=64, dtype=torch.bfloat16):
    return [torch.randn(B, H, T, D, device="cuda", dtype=dtype) for _ in range(3)]


def test_fwd_rejects_host_lse_and_out(fa):
    q, k, v = _qkv()
    with pytest.raises(ValueError):
        fa.fa_fwd(q, k, v, lse=torch.empty(1, 2, 64))
    with pytest.raises(ValueError):
        fa.fa_fwd(q, k, v, out=torch.empty(1, 2, 64, 64, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        fa.fa_fwd(q, k, v, lse=torch.empty(1, 2, 128, device="cuda")[:, :, ::2])
    with pytest.raises(ValueError):
        fa.fa_fwd(q, k, v, lse=torch.empty(1, 2, 64, device="cuda", dtype=torch.float64))


def test_bwd_rejects_host_lse_and_workspace(fa):
    q, k, v = _qkv()
    o, lse = fa.fa_fwd(q, k, v)
    do = torch.randn_like(q)
    with pytest.raises(ValueError):
        fa.fa_bwd(q, k, v, o, do, lse.cpu())
    need = fa.fa_bwd_workspace_bytes(1, 2, 64, 64)
    with pytest.raises(ValueError):
        fa.fa_bwd(q, k, v, o, do, lse, workspace=torch.empty(need, dtype=torch.uint8))
    with pytest.raises(ValueError):
        fa.fa_bwd(q, k, v, o, do, lse,
                  workspace=torch.empty(2 * need, dtype=torch.uint8, device="cuda")[::2])
    with pytest.raises(ValueError):
        fa.fa_bwd(q, k, v, o, do, lse,
                  workspace=torch.empty(need - 16, dtype=torch.uint8, device="cuda"))


def test_grouped_and_packed_reject_host_outputs(fa):
    q, k, v = _qkv()
    with pytest.raises(ValueError):
        fa.fa_fwd_gqa(q, k, v, lse=torch.empty(1, 2, 64))
    with pytest.raises(ValueError):
        fa.fa_fwd_gqa(q, k, v, out=torch.empty(1, 2, 64, 64, dtype=torch.bfloat16))
    qp, kp, vp = (t[0].transpose(0, 1).contiguous() for t in (q, k, v))
    cu = torch.tensor([0, 64], dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        fa.fa_fwd_varlen(qp, kp, vp, cu, cu, 64, lse=torch.empty(2, 64))
    with pytest.raises(ValueError):
        fa.fa_fwd_varlen(qp, kp, vp, cu.cpu(), cu, 64)


def test_decode_rejects_host_workspace(fa):
    q = torch.randn(1, 4, 1, 64, device="cuda", dtype=torch.bfloat16)
    k = torch.randn(1, 2, 300, 64, device="cuda", dtype=torch.bfloat16)
    need = fa.fa_decode_workspace_bytes(1, 4, 2, 1, 300, 64)
    with pytest.raises(ValueError):
        fa.fa_fwd_decode(q, k, k, workspace=torch.empty(need, dtype=torch.uint8))
    with pytest.raises(ValueError):
        fa.fa_fwd_decode(q, k, k, lse=torch.empty(1, 4, 1))
    with pytest.raises(ValueError):
        fa.fa_fwd_decode(q, k, k, cache_seqlens=torch.tensor([5], dtype=torch.int32))


def test_fp8_rejects_host_scales(fa):
    x = torch.randn(1, 2, 64, 64, device="cuda", dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fa_quantize_mxfp8(x, scales=torch.empty(1, 2, 64, 2, dtype=torch.uint8))
    q8, qs = fa.fa_quantize_mxfp8(x)
    with pytest.raises(ValueError):
        fa.fa_fwd_fp8qk(q8, qs.cpu(), q8, qs, x)
