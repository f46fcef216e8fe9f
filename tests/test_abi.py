"""The C ABI on the host: libfa.so loads, exports every function include/fa.h
declares, and rejects bad arguments before touching the GPU (no compute calls)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(fa_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    import exact_tiled_attention_flash_amd as fa
    return fa.load_library()


def test_header_declares_entry_points():
    names = declared_functions()
    assert {"fa_fwd", "fa_status_string", "fa_abi_version"} <= set(names)


def test_library_exports_every_declared_symbol(lib):
    from exact_tiled_attention_flash_amd import LIB_PATH
    out = subprocess.run(["nm", "-D", "--defined-only", LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_abi_version(lib):
    assert lib.fa_abi_version() == 5


def test_status_strings(lib):
    for code in range(-9, 1):
        assert lib.fa_status_string(code)
    assert lib.fa_status_string(0) == b"ok"
    assert lib.fa_status_string(-99) == b"unknown status"


# Fake, 16-byte aligned, never dereferenced: every call below fails validation
# before anything is enqueued.
P = 4096


def fwd(lib, q=P, k=P, v=P, o=P, lse=P, B=1, H=1, T=16, D=64, scale=0.125, causal=0, dtype=1):
    return lib.fa_fwd(q, k, v, o, lse, B, H, T, D, ctypes.c_float(scale), causal, dtype, None)


@pytest.mark.parametrize("which", ["q", "k", "v", "o", "lse"])
def test_null_pointers(lib, which):
    assert fwd(lib, **{which: None}) == -1


@pytest.mark.parametrize("B,H,T", [(0, 1, 16), (1, 0, 16), (1, 1, 0), (-1, 1, 16),
                                   (1 << 20, 1 << 11, 1 << 20)])
def test_bad_shapes(lib, B, H, T):
    assert fwd(lib, B=B, H=H, T=T) == -2


def test_head_size_bound(lib):
    # one head of one tensor must stay below 2^31 bytes (in-head offsets are 32-bit)
    assert fwd(lib, B=1, H=1, T=1 << 23, D=128) == -2
    assert fwd(lib, B=1, H=1, T=1 << 24, D=64) == -2
    assert lib.fa_bwd_workspace_bytes(1, 1, 1 << 23, 128) == 0
    assert lib.fa_bwd_workspace_bytes(1, 1, (1 << 23) - 1, 128) == 8 * ((1 << 23) - 1)


@pytest.mark.parametrize("D", [0, 32, 96, 256, 127])
def test_bad_head_dim(lib, D):
    assert fwd(lib, D=D) == -3


@pytest.mark.parametrize("dtype", [-1, 2, 7])
def test_bad_dtype(lib, dtype):
    assert fwd(lib, dtype=dtype) == -4


@pytest.mark.parametrize("which", ["q", "k", "v", "o", "lse"])
def test_misaligned(lib, which):
    assert fwd(lib, **{which: P + 8}) == -5


@pytest.mark.parametrize("scale", [-0.5, float("nan"), float("inf")])
def test_bad_scale(lib, scale):
    assert fwd(lib, scale=scale) == -6


def test_bad_causal(lib):
    assert fwd(lib, causal=2) == -7


def test_bwd_workspace_bytes(lib):
    assert lib.fa_bwd_workspace_bytes(2, 16, 4096, 128) == 8 * 2 * 16 * 4096
    assert lib.fa_bwd_workspace_bytes(0, 16, 4096, 128) == 0
    assert lib.fa_bwd_workspace_bytes(1, 1, 16, 96) == 0


def bwd(lib, ws_bytes=1 << 20, dtype=1, D=64, T=16, causal=1, scale=0.1, nulls=()):
    ptrs = [None if i in nulls else P for i in range(10)]
    return lib.fa_bwd(*ptrs, ws_bytes, 1, 1, T, D, ctypes.c_float(scale), causal, dtype, None)


def test_bwd_validation(lib):
    for i in range(10):
        assert bwd(lib, nulls=(i,)) == -1
    assert bwd(lib, T=0) == -2
    assert bwd(lib, D=32) == -3
    assert bwd(lib, dtype=2) == -4      # FA_F32 (0) and FA_BF16 (1) only
    assert bwd(lib, dtype=-1) == -4
    assert bwd(lib, scale=-1.0) == -6
    assert bwd(lib, causal=5) == -7
    assert bwd(lib, ws_bytes=127) == -7  # needs 8*B*H*T = 128 bytes


def gqa(lib, Hq=4, Hkv=2, Tq=16, Tk=16, D=64, dtype=1, causal=0, scale=0.125, nulls=()):
    ptrs = [None if i in nulls else P for i in range(5)]
    return lib.fa_fwd_gqa(*ptrs, 1, Hq, Hkv, Tq, Tk, D, ctypes.c_float(scale), causal, dtype, None)


def test_gqa_validation(lib):
    for i in range(5):
        assert gqa(lib, nulls=(i,)) == -1
    assert gqa(lib, Hq=3, Hkv=2) == -2          # Hq not a multiple of Hkv
    assert gqa(lib, Tq=0) == -2 and gqa(lib, Tk=0) == -2
    assert gqa(lib, Tk=1 << 23, D=128) == -2    # one K head reaches 2^31 bytes
    assert gqa(lib, D=96) == -3
    assert gqa(lib, dtype=0) == -4              # bf16 only
    assert gqa(lib, causal=3) == -7
    assert gqa(lib, scale=float("nan")) == -6


def varlen(lib, B=2, Hq=4, Hkv=2, tq=32, tk=32, maxq=16, D=64, dtype=1, cu=P, nulls=()):
    ptrs = [None if i in nulls else P for i in range(5)]
    cq = None if 5 in nulls else cu
    ck = None if 6 in nulls else cu
    return lib.fa_fwd_varlen(*ptrs, cq, ck, B, Hq, Hkv, tq, tk, maxq, D, ctypes.c_float(0.1), 1,
                             dtype, None)


def test_varlen_validation(lib):
    for i in range(7):
        assert varlen(lib, nulls=(i,)) == -1
    assert varlen(lib, maxq=0) == -2 and varlen(lib, maxq=33) == -2   # 1 <= max <= total
    assert varlen(lib, B=0) == -2
    assert varlen(lib, tq=1 << 22, Hq=4, D=128, maxq=16) == -2          # (rows, heads, D) >= 2^31 B
    assert varlen(lib, D=32) == -3
    assert varlen(lib, dtype=0) == -4
    assert varlen(lib, cu=P + 2) == -5                                  # offsets 4-byte aligned


def test_decode_workspace_bytes(lib):
    # 4 * B * Hq * Tq * splits * (D + 4); automatic splits: ceil(1024 / (B * Hkv)) within
    # [1, min(ceil(Tk / 32), 1024)]
    assert lib.fa_decode_workspace_bytes(1, 32, 8, 1, 32768, 128, 0) == 4 * 32 * 128 * 132
    assert lib.fa_decode_workspace_bytes(1, 32, 8, 1, 32768, 128, 7) == 4 * 32 * 7 * 132
    assert lib.fa_decode_workspace_bytes(1, 32, 8, 1, 100, 64, 0) == 4 * 32 * 4 * 68     # 4 tiles
    assert lib.fa_decode_workspace_bytes(1, 1, 1, 1, 1 << 20, 64, 5000) == 4 * 1024 * 68  # cap
    assert lib.fa_decode_workspace_bytes(64, 8, 8, 1, 4096, 128, 0) == 4 * 64 * 8 * 2 * 132
    assert lib.fa_decode_workspace_bytes(1, 64, 1, 1, 128, 128, 0) == 0   # 64 rows per group
    assert lib.fa_decode_workspace_bytes(1, 8, 2, 9, 128, 128, 0) == 0    # 4 * 9 > 32
    assert lib.fa_decode_workspace_bytes(1, 8, 2, 8, 128, 128, 0) > 0     # 4 * 8 = 32
    assert lib.fa_decode_workspace_bytes(1, 8, 2, 1, 128, 128, -1) == 0


def decode(lib, Hq=8, Hkv=2, Tq=1, Tk=64, D=128, ws=1 << 20, splits=0, dtype=1, causal=0,
           scale=0.1, lens=P, nulls=()):
    ptrs = [None if i in nulls else P for i in range(5)]
    return lib.fa_fwd_decode(*ptrs, lens, None if 5 in nulls else P, ws, 2, Hq, Hkv, Tq, Tk, D,
                             splits, ctypes.c_float(scale), causal, dtype, None)


def test_decode_validation(lib):
    for i in range(6):
        assert decode(lib, nulls=(i,)) == -1
    assert decode(lib, Hq=9) == -2                # Hq not a multiple of Hkv
    assert decode(lib, Tq=9) == -2                # 4 * 9 query rows per group > 32
    assert decode(lib, Tk=0) == -2
    assert decode(lib, D=96) == -3
    assert decode(lib, dtype=0) == -4
    assert decode(lib, lens=P + 2) == -5          # lengths 4-byte aligned
    assert decode(lib, scale=-1.0) == -6
    assert decode(lib, causal=2) == -7
    assert decode(lib, splits=-1) == -7
    need = lib.fa_decode_workspace_bytes(2, 8, 2, 1, 64, 128, 0)
    assert decode(lib, ws=need - 1) == -7


def test_quantize_validation(lib):
    q = lambda x=P, c=P, s=P, rows=4, D=64, dtype=1: lib.fa_quantize_mxfp8(x, c, s, rows, D, dtype, None)
    assert q(x=None) == -1 and q(c=None) == -1 and q(s=None) == -1
    assert q(rows=0) == -2 and q(D=48) == -2 and q(D=0) == -2
    assert q(rows=1 << 30, D=4096) == -2          # 2^42 elements
    assert q(dtype=0) == -4
    assert q(x=P + 8) == -5 and q(c=P + 4) == -5 and q(s=P + 2) == -5


def test_fp8qk_validation(lib):
    def f(nulls=(), Hq=4, Hkv=2, D=128, causal=1, scale=0.1, mis=None):
        ptrs = [None if i in nulls else P for i in range(7)]
        if mis is not None:
            ptrs[mis[0]] = P + mis[1]
        return lib.fa_fwd_fp8qk(*ptrs, 1, Hq, Hkv, 16, 16, D, ctypes.c_float(scale), causal, None)
    for i in range(7):
        assert f(nulls=(i,)) == -1
    assert f(Hq=3) == -2 and f(D=96) == -3 and f(causal=2) == -7 and f(scale=float("inf")) == -6
    assert f(mis=(0, 8)) == -5 and f(mis=(1, 2)) == -5 and f(mis=(2, 8)) == -5 and f(mis=(3, 2)) == -5


def test_bwd_noalloc_validation(lib):
    # every refusal happens on the host, before the runtime is touched
    def call(T=16, D=64, dtype=1, causal=1, scale=0.1, nulls=()):
        ptrs = [None if i in nulls else P for i in range(9)]
        return lib.fa_bwd_noalloc(*ptrs, 1, 1, T, D, ctypes.c_float(scale), causal, dtype, None)
    for i in range(9):
        assert call(nulls=(i,)) == -1
    assert call(T=0) == -2 and call(D=96) == -3 and call(dtype=2) == -4
    assert call(causal=3) == -7 and call(scale=-1.0) == -6
    cap = lib.fa_bwd_noalloc_max_bytes()
    assert cap == 16 << 20
    assert call(T=cap // 8 + 1) == -9            # one row more than the scratch array holds
    assert lib.fa_status_string(-9).startswith(b"sizes exceed")
