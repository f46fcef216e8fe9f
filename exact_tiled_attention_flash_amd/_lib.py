"""ctypes binding to libfa.so: argument marshalling only.

Every step of the attention computation runs in the HIP kernels behind the C
ABI (include/fa.h). torch supplies device memory and the current stream. If
the library is missing the import fails loudly: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa.so")
SYNC_CHECK_LIB_PATH = os.path.join(_PKG, "libfa_synccheck.so")

FA_F32 = 0
FA_BF16 = 1
FA_OK = 0
FA_ERR_NULL = -1
FA_ERR_SHAPE = -2
FA_ERR_HEADDIM = -3
FA_ERR_DTYPE = -4
FA_ERR_ALIGN = -5
FA_ERR_SCALE = -6
FA_ERR_ARG = -7
FA_ERR_HIP = -8
FA_ERR_SCRATCH = -9

_lib = None


def _declare(lib: ctypes.CDLL) -> ctypes.CDLL:
    """Declare the C signatures of include/fa.h on a loaded library."""
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_abi_version.restype = i
    lib.fa_abi_version.argtypes = []
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_status_string.argtypes = [i]
    lib.fa_fwd.restype = i
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
    lib.fa_fwd_gqa.restype = i
    lib.fa_fwd_gqa.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp]
    lib.fa_fwd_varlen.restype = i
    lib.fa_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, i, vp]
    lib.fa_quantize_mxfp8.restype = i
    lib.fa_quantize_mxfp8.argtypes = [vp, vp, vp, i, i, i, vp]
    lib.fa_fwd_fp8qk.restype = i
    lib.fa_fwd_fp8qk.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
    lib.fa_decode_workspace_bytes.restype = sz
    lib.fa_decode_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.fa_fwd_decode.restype = i
    lib.fa_fwd_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, i, f, i, i, vp]
    lib.fa_bwd.restype = i
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, f, i, i, vp]
    lib.fa_bwd_workspace_bytes.restype = sz
    lib.fa_bwd_workspace_bytes.argtypes = [i, i, i, i]
    if hasattr(lib, "fa_bwd_noalloc"):
        lib.fa_bwd_noalloc.restype = i
        lib.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
        lib.fa_bwd_noalloc_max_bytes.restype = sz
        lib.fa_bwd_noalloc_max_bytes.argtypes = []
    return lib


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfa.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python exact_tiled_attention_flash_amd/build.py`")
    _lib = _declare(ctypes.CDLL(path))
    return _lib


def load_variant(path: str) -> ctypes.CDLL:
    """Another build of the same library (the race-check build, libfa_synccheck.so), loaded
    beside libfa.so with the same declarations; the Python wrappers keep using libfa.so."""
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python exact_tiled_attention_flash_amd/build.py`")
    return _declare(ctypes.CDLL(path))


class FaError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(f"libfa status {status}: {fa_status_string(status)}")


def fa_status_string(status: int) -> str:
    return load_library().fa_status_string(int(status)).decode()


def fa_abi_version() -> int:
    return load_library().fa_abi_version()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float32:
        return FA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _check(name: str, t: torch.Tensor, like: torch.Tensor | None = None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (B, H, T, D)")
    if like is not None and (t.shape != like.shape or t.dtype != like.dtype
                             or t.device != like.device):
        raise ValueError(f"{name} must match q in shape, dtype and device")


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def fa_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
           scale: float | None = None, out: torch.Tensor | None = None,
           lse: torch.Tensor | None = None):
    """o, lse = softmax(scale q k^T [causal]) v, per-row log-sum-exp. Enqueued on the
    current stream. q, k, v: contiguous (B, H, T, D) bf16 or fp32 device tensors."""
    lib = load_library()
    _check("q", q)
    _check("k", k, q)
    _check("v", v, q)
    if q.dim() != 4:
        raise ValueError("q must be (B, H, T, D)")
    B, H, T, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = torch.empty_like(q) if out is None else out
    l = torch.empty((B, H, T), dtype=torch.float32, device=q.device) if lse is None else lse
    _check("out", o, q)
    _check_plain("lse", l, torch.float32, 3, q.device)
    if tuple(l.shape) != (B, H, T):
        raise ValueError("lse must be a contiguous float32 (B, H, T) tensor")
    rc = lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), l.data_ptr(),
                    B, H, T, D, float(scale), int(bool(causal)), _dtype_code(q), _stream(q))
    if rc != FA_OK:
        raise FaError(rc)
    return o, l


def _check_plain(name: str, t: torch.Tensor, dtype: torch.dtype, dims: int,
                 device: torch.device | None = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda or not t.is_contiguous() or t.dtype != dtype or t.dim() != dims:
        raise ValueError(f"{name} must be a contiguous {dims}-d {dtype} device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, like the inputs")


def _check_workspace(ws: torch.Tensor, need: int, device: torch.device):
    """A caller's workspace: a contiguous device tensor on the inputs' device, of any dtype,
    holding at least `need` bytes (the library checks the size again)."""
    if not isinstance(ws, torch.Tensor):
        raise TypeError("workspace must be a torch.Tensor")
    if not ws.is_cuda or not ws.is_contiguous() or ws.device != device:
        raise ValueError(f"workspace must be a contiguous device tensor on {device}")
    if ws.numel() * ws.element_size() < need:
        raise ValueError(f"workspace holds {ws.numel() * ws.element_size()} bytes, "
                         f"{need} are needed")


def fa_fwd_gqa(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
               scale: float | None = None, out: torch.Tensor | None = None,
               lse: torch.Tensor | None = None):
    """Grouped K/V heads and separate lengths: q (B, Hq, Tq, D), k and v (B, Hkv, Tk, D),
    bf16; query head h uses K/V head h // (Hq // Hkv). Causal is aligned at the bottom right.
    Returns o (B, Hq, Tq, D) and lse (B, Hq, Tq) float32. Enqueued on the current stream."""
    lib = load_library()
    _check_plain("q", q, torch.bfloat16, 4)
    for name, t in (("k", k), ("v", v)):
        _check_plain(name, t, torch.bfloat16, 4, q.device)
    if k.shape != v.shape or k.shape[0] != q.shape[0] or k.shape[3] != q.shape[3]:
        raise ValueError("k and v must be (B, Hkv, Tk, D) with q's B and D")
    B, Hq, Tq, D = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = torch.empty_like(q) if out is None else out
    l = torch.empty((B, Hq, Tq), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_plain("out", o, torch.bfloat16, 4, q.device)
    _check_plain("lse", l, torch.float32, 3, q.device)
    if o.shape != q.shape or tuple(l.shape) != (B, Hq, Tq):
        raise ValueError("out must match q and lse must be (B, Hq, Tq)")
    rc = lib.fa_fwd_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), l.data_ptr(),
                        B, Hq, Hkv, Tq, Tk, D, float(scale), int(bool(causal)), FA_BF16, _stream(q))
    if rc != FA_OK:
        raise FaError(rc)
    return o, l


def fa_fwd_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
                  cu_seqlens_k: torch.Tensor, max_seqlen_q: int, causal: bool = False,
                  scale: float | None = None, out: torch.Tensor | None = None,
                  lse: torch.Tensor | None = None):
    """Packed batch: q (total_q, Hq, D), k and v (total_k, Hkv, D), bf16; cu_seqlens_q / _k
    int32 device tensors of B + 1 offsets. Returns o (total_q, Hq, D) and lse (Hq, total_q)
    float32. Enqueued on the current stream."""
    lib = load_library()
    _check_plain("q", q, torch.bfloat16, 3)
    for name, t in (("k", k), ("v", v)):
        _check_plain(name, t, torch.bfloat16, 3, q.device)
    _check_plain("cu_seqlens_q", cu_seqlens_q, torch.int32, 1, q.device)
    _check_plain("cu_seqlens_k", cu_seqlens_k, torch.int32, 1, q.device)
    if cu_seqlens_q.numel() != cu_seqlens_k.numel() or cu_seqlens_q.numel() < 2:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold B + 1 offsets")
    if k.shape != v.shape or k.shape[2] != q.shape[2]:
        raise ValueError("k and v must be (total_k, Hkv, D) with q's D")
    total_q, Hq, D = q.shape
    total_k, Hkv = k.shape[0], k.shape[1]
    B = cu_seqlens_q.numel() - 1
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = torch.empty_like(q) if out is None else out
    l = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_plain("out", o, torch.bfloat16, 3, q.device)
    _check_plain("lse", l, torch.float32, 2, q.device)
    if o.shape != q.shape or tuple(l.shape) != (Hq, total_q):
        raise ValueError("out must match q and lse must be (Hq, total_q)")
    rc = lib.fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), l.data_ptr(),
                           cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), B, Hq, Hkv, total_q,
                           total_k, int(max_seqlen_q), D, float(scale), int(bool(causal)), FA_BF16,
                           _stream(q))
    if rc != FA_OK:
        raise FaError(rc)
    return o, l


def fa_quantize_mxfp8(x: torch.Tensor, codes: torch.Tensor | None = None,
                      scales: torch.Tensor | None = None):
    """Block-scaled E4M3 of a contiguous bf16 device tensor (..., D), D a multiple of 32: codes
    uint8 (..., D) and scale bytes uint8 (..., D / 32). Enqueued on the current stream."""
    lib = load_library()
    if not x.is_cuda or not x.is_contiguous() or x.dtype != torch.bfloat16 or x.dim() < 1:
        raise ValueError("x must be a contiguous bf16 device tensor")
    D = x.shape[-1]
    rows = x.numel() // D if D else 0
    c = torch.empty(x.shape, dtype=torch.uint8, device=x.device) if codes is None else codes
    s = (torch.empty(tuple(x.shape[:-1]) + (D // 32,), dtype=torch.uint8, device=x.device)
         if scales is None else scales)
    _check_plain("codes", c, torch.uint8, x.dim(), x.device)
    _check_plain("scales", s, torch.uint8, x.dim(), x.device)
    if c.shape != x.shape or tuple(s.shape) != tuple(x.shape[:-1]) + (D // 32,):
        raise ValueError("codes must match x and scales must be (..., D / 32)")
    rc = lib.fa_quantize_mxfp8(x.data_ptr(), c.data_ptr(), s.data_ptr(), rows, D, FA_BF16, _stream(x))
    if rc != FA_OK:
        raise FaError(rc)
    return c, s


def fa_fwd_fp8qk(q8: torch.Tensor, q_scale: torch.Tensor, k8: torch.Tensor, k_scale: torch.Tensor,
                 v: torch.Tensor, causal: bool = False, scale: float | None = None,
                 out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    """Forward with E4M3 Q and K (codes and scales from fa_quantize_mxfp8): q8 (B, Hq, Tq, D),
    k8 (B, Hkv, Tk, D) uint8, v (B, Hkv, Tk, D) bf16. Returns o (B, Hq, Tq, D) bf16 and lse
    (B, Hq, Tq) float32. Enqueued on the current stream."""
    lib = load_library()
    _check_plain("q8", q8, torch.uint8, 4)
    _check_plain("k8", k8, torch.uint8, 4, q8.device)
    _check_plain("v", v, torch.bfloat16, 4, q8.device)
    B, Hq, Tq, D = q8.shape
    Hkv, Tk = k8.shape[1], k8.shape[2]
    if v.shape != k8.shape or k8.shape[0] != B or k8.shape[3] != D:
        raise ValueError("k8 and v must be (B, Hkv, Tk, D) with q8's B and D")
    _check_plain("q_scale", q_scale, torch.uint8, 4, q8.device)
    _check_plain("k_scale", k_scale, torch.uint8, 4, q8.device)
    if tuple(q_scale.shape) != (B, Hq, Tq, D // 32) or tuple(k_scale.shape) != (B, Hkv, Tk, D // 32):
        raise ValueError("scales must be (..., D / 32) of the codes' leading shape")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = torch.empty((B, Hq, Tq, D), dtype=torch.bfloat16, device=q8.device) if out is None else out
    l = torch.empty((B, Hq, Tq), dtype=torch.float32, device=q8.device) if lse is None else lse
    _check_plain("out", o, torch.bfloat16, 4, q8.device)
    _check_plain("lse", l, torch.float32, 3, q8.device)
    if tuple(o.shape) != (B, Hq, Tq, D) or tuple(l.shape) != (B, Hq, Tq):
        raise ValueError("out must be (B, Hq, Tq, D) and lse (B, Hq, Tq)")
    rc = lib.fa_fwd_fp8qk(q8.data_ptr(), q_scale.data_ptr(), k8.data_ptr(), k_scale.data_ptr(),
                          v.data_ptr(), o.data_ptr(), l.data_ptr(), B, Hq, Hkv, Tq, Tk, D,
                          float(scale), int(bool(causal)), _stream(q8))
    if rc != FA_OK:
        raise FaError(rc)
    return o, l


def fa_decode_workspace_bytes(B: int, Hq: int, Hkv: int, Tq: int, Tk: int, D: int,
                              num_splits: int = 0) -> int:
    return load_library().fa_decode_workspace_bytes(B, Hq, Hkv, Tq, Tk, D, num_splits)


def fa_fwd_decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                  cache_seqlens: torch.Tensor | None = None, num_splits: int = 0,
                  causal: bool = False, scale: float | None = None,
                  out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None):
    """Split-K decode against a K/V cache: q (B, Hq, Tq, D) with (Hq / Hkv) * Tq <= 32, k and v
    (B, Hkv, Tk, D), bf16; cache_seqlens an int32 (B,) device tensor of valid keys per
    sequence (None: all Tk). num_splits 0 picks the split count. Returns o (B, Hq, Tq, D) and
    lse (B, Hq, Tq) float32. Enqueued on the current stream."""
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_plain(name, t, torch.bfloat16, 4)
    if k.shape != v.shape or k.shape[0] != q.shape[0] or k.shape[3] != q.shape[3]:
        raise ValueError("k and v must be (B, Hkv, Tk, D) with q's B and D")
    B, Hq, Tq, D = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    if cache_seqlens is not None:
        _check_plain("cache_seqlens", cache_seqlens, torch.int32, 1, q.device)
        if cache_seqlens.numel() != B:
            raise ValueError("cache_seqlens must hold B counts")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = torch.empty_like(q) if out is None else out
    l = torch.empty((B, Hq, Tq), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_plain("out", o, torch.bfloat16, 4, q.device)
    _check_plain("lse", l, torch.float32, 3, q.device)
    if o.shape != q.shape or tuple(l.shape) != (B, Hq, Tq):
        raise ValueError("out must match q and lse must be (B, Hq, Tq)")
    need = lib.fa_decode_workspace_bytes(B, Hq, Hkv, Tq, Tk, D, int(num_splits))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, need, q.device)
    rc = lib.fa_fwd_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), l.data_ptr(),
                           None if cache_seqlens is None else cache_seqlens.data_ptr(),
                           workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                           B, Hq, Hkv, Tq, Tk, D, int(num_splits), float(scale),
                           int(bool(causal)), FA_BF16, _stream(q))
    if rc != FA_OK:
        raise FaError(rc)
    return o, l


def fa_bwd_workspace_bytes(B: int, H: int, T: int, D: int) -> int:
    return load_library().fa_bwd_workspace_bytes(B, H, T, D)


def fa_bwd(q, k, v, o, dout, lse, causal: bool = False, scale: float | None = None,
           workspace: torch.Tensor | None = None):
    """dq, dk, dv of L with dL/do = dout, from the forward's o and lse. Enqueued on the
    current stream."""
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _check(name, t, None if name == "q" else q)
    B, H, T, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    _check_plain("lse", lse, torch.float32, 3, q.device)
    if tuple(lse.shape) != (B, H, T):
        raise ValueError("lse must be a contiguous float32 (B, H, T) tensor")
    need = fa_bwd_workspace_bytes(B, H, T, D)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, need, q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    rc = lib.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                    lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                    workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                    B, H, T, D, float(scale), int(bool(causal)), _dtype_code(q), _stream(q))
    if rc != FA_OK:
        raise FaError(rc)
    return dq, dk, dv


def fa_bwd_noalloc_max_bytes() -> int:
    return load_library().fa_bwd_noalloc_max_bytes()


def fa_bwd_noalloc(q, k, v, o, dout, lse, causal: bool = False, scale: float | None = None,
                   dq: torch.Tensor | None = None, dk: torch.Tensor | None = None,
                   dv: torch.Tensor | None = None):
    """fa_bwd without a workspace: the library's fixed scratch array holds the per-row
    statistics. With dq, dk and dv supplied the call allocates nothing (usable under graph
    capture). Calls that overlap on one GPU race on that array. Enqueued on the current
    stream."""
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _check(name, t, None if name == "q" else q)
    B, H, T, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    _check_plain("lse", lse, torch.float32, 3, q.device)
    if tuple(lse.shape) != (B, H, T):
        raise ValueError("lse must be a contiguous float32 (B, H, T) tensor")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check(name, t, q)
    rc = lib.fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                            dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                            dv.data_ptr(), B, H, T, D, float(scale), int(bool(causal)),
                            _dtype_code(q), _stream(q))
    if rc != FA_OK:
        raise FaError(rc)
    return dq, dk, dv
