"""Build libfa.so (the HIP kernels for gfx950 plus the C ABI) in-tree with hipcc.

Usage: python exact_tiled_attention_flash_amd/build.py [--asm DIR]
(run by path: importing the package itself needs the built library)

Each source compiles in its own hipcc process (in parallel), then one link
step writes exact_tiled_attention_flash_amd/libfa.so. Packed fp32 vector
instructions are disabled for all device code.

The same sources are also built with -DFA_SYNC_CHECK=1 into libfa_synccheck.so:
the race-check variant, with a full wait and a workgroup barrier before every
stage that reads a tile from LDS. Only the tests load it (their outputs must
equal the release library's bit for bit).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfa.so")
SYNC_LIB = os.path.join(PKG, "libfa_synccheck.so")

ARCH = "gfx950"
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-fno-honor-nans", "-mno-amdgpu-ieee"]
# per-source extra device flags
EXTRA = {}
COMMON = ["-O3", "-std=c++17", "-fPIC", f"-I{os.path.join(ROOT, 'include')}", "-Wall",
          "-Wno-unused-function"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain is required to build libfa.so)")


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".hip") or f.endswith(".cpp"))


def _compile(src: str, asm_dir: str | None, variant: str = "") -> str:
    bdir = os.path.join(BUILD, variant) if variant else BUILD
    obj = os.path.join(bdir, os.path.basename(src) + ".o")
    defs = ["-DFA_SYNC_CHECK=1"] if variant == "synccheck" else []
    cmd = [_hipcc(), f"--offload-arch={ARCH}", *COMMON, *defs, "-c", src, "-o", obj]
    if src.endswith(".hip"):
        cmd += DEVICE_FLAGS + EXTRA.get(os.path.basename(src), [])
        if asm_dir and not variant:
            asm = os.path.join(asm_dir, os.path.basename(src) + ".s")
            subprocess.run([_hipcc(), f"--offload-arch={ARCH}", *COMMON, *DEVICE_FLAGS,
                            *EXTRA.get(os.path.basename(src), []),
                            "--cuda-device-only", "-S", src, "-o", asm],
                           capture_output=True, text=True, check=True)
    res = subprocess.run(cmd, cwd=bdir, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "is not a recognized feature for this target" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if out.strip():
        print(out, file=sys.stderr)
    return obj


def _link(objs: list[str], lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, lib)


def build(asm_dir: str | None = None, jobs: int = 8, sync_check: bool = True) -> str:
    """Build libfa.so (and, unless sync_check is False, libfa_synccheck.so); returns the path
    of libfa.so."""
    variants = ["", "synccheck"] if sync_check else [""]
    for v in variants:
        os.makedirs(os.path.join(BUILD, v) if v else BUILD, exist_ok=True)
    if asm_dir:
        os.makedirs(asm_dir, exist_ok=True)
    srcs = sources()
    todo = [(s, v) for v in variants for s in srcs]
    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(todo))) as ex:
        objs = list(ex.map(lambda sv: _compile(sv[0], asm_dir, sv[1]), todo))
    for v in variants:
        _link([o for o, (_, vv) in zip(objs, todo) if vv == v], SYNC_LIB if v else LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", default=None, help="also write device assembly (.s) of each HIP source to this dir")
    ap.add_argument("--no-sync-check", action="store_true",
                    help="skip the race-check library (libfa_synccheck.so)")
    args = ap.parse_args()
    print(build(args.asm, sync_check=not args.no_sync_check))
