"""Benchmark: attention forward TFLOP/s on one MI355X, and % of the bf16 MFMA peak.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step is one forward pass (fa_fwd: one kernel launch) over the headline
workload: causal bf16, B=4, H=16, T=4096, D=128, scale 1/sqrt(128), seeded
N(0,1) inputs already resident in HBM. FLOPs per step = 4*B*H*T^2*D / 2.
The backward (fa_bwd, three kernels) is measured the same way on its own
workload (causal bf16, B=2, H=16, T=4096, D=128) and reported under
"backward". The further rows of the forward are timed on their own workloads
and reported under "next_rows": grouped K/V heads (B=4, 32 query heads over 8
K/V heads, T=4096, causal) and a packed batch of 32 causal sequences of 64 to
8192 tokens (16 heads); the split-K decode of one query row against a 32768-key
cache (batch 1, 32 query heads over 8 K/V heads; also a batch of 8 with valid
lengths of 1k to 32k keys) in GB/s against the HBM peak, beside the forward
kernel's time on the same cache; and the forward with block-scaled E4M3 Q and K for Q K^T on
the headline workload (TFLOP/s, with and without the quantization of Q and K, and its
difference from the bf16 kernel's O and LSE). "library_gemm" times the vendor library's bf16 GEMM
(8192^3) in the same process, as the dense bf16 rate reachable on this GPU at its sustained
clock. The CPU baseline times the float64 oracle on a bounded sample of the forward workload
(whole (b, h) heads) on the host cores.
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FWD_WORKLOAD = "fwd_bf16_b4h16t4096d128_causal"
BWD_WORKLOAD = "bwd_bf16_b2h16t4096d128_causal"


def _dev(a, torch):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to("cuda")


def _time_launches(torch, fn, steps, warmup):
    """Warm up, then time `steps` calls of fn() with one event pair per call on the
    current stream (where fn enqueues its kernels). Returns (total_ms, per_call_ms)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    per = [a.elapsed_time(b) for a, b in ev]
    total = ev[0][0].elapsed_time(ev[-1][1])
    return total, per, wall_ms


def library_gemm(torch, peak):
    """Context for the roofline: the vendor library's dense bf16 GEMM (8192^3 through
    torch.matmul, i.e. hipBLASLt) on the same GPU in the same process. Under sustained matrix
    work the chip clocks below the 2.4 GHz the published peak assumes; this is the dense bf16
    rate a library reaches here."""
    n = 8192
    a = torch.randn(n, n, dtype=torch.bfloat16, device="cuda")
    b = torch.randn(n, n, dtype=torch.bfloat16, device="cuda")
    ms = _time_loop(torch, lambda: torch.matmul(a, b), 20, 5)
    tflops = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    return {"op": "bf16 GEMM 8192x8192x8192 (torch.matmul -> hipBLASLt)", "ms": round(ms, 4),
            "tflops": round(tflops, 1), "pct_of_bf16_peak": round(100.0 * tflops / peak, 2)}


def _time_loop(torch, fn, steps, warmup):
    """Warm up, then time `steps` back-to-back calls of fn() with one event pair around the
    loop (for calls of tens of microseconds, where an event pair per call would leave gaps
    of host time between the launches). Returns milliseconds per call."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


COPY_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd_bf16_b4h16t4096d128_causal_traffic.json")
# the sources the headline forward kernel is compiled from
FWD_SOURCES = [os.path.join(ROOT, "exact_tiled_attention_flash_amd", "csrc", f)
               for f in ("fa_fwd_bf16.hip", "fa_fwd_parts.h", "fa_swz.h", "fa_common.h")]


def fwd_source_digest():
    import hashlib
    h = hashlib.sha256()
    for f in FWD_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def committed_traffic(flops):
    """HBM bytes per launch of the forward kernel from the committed rocprofv3 FETCH_SIZE and
    WRITE_SIZE runs (scaled by the same counters on a copy of known size), provided the kernel
    source is unchanged since they were taken; else None."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != fwd_source_digest():
        return None
    return {"bytes_per_launch": rec["hbm_bytes_per_launch"], "source": os.path.relpath(TRAFFIC_FILE, ROOT)}


def cpu_baseline(w, d, budget_s: float):
    """Time the float64 oracle on whole (b, h) heads of the same inputs, in order,
    until budget_s has passed."""
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = len(os.sched_getaffinity(0))
    heads = 0
    t0 = time.perf_counter()
    while True:
        b, h = divmod(heads, w.H)
        q, k, v = (synth.bf16_bits_to_f64(d[n][b:b + 1, h:h + 1]) for n in "qkv")
        oracle.attention_forward(q, k, v, w.scale, w.causal)
        heads += 1
        el = time.perf_counter() - t0
        if el >= budget_s or heads >= w.B * w.H:
            break
    flops = 4.0 * heads * w.T * w.T * w.D / (2.0 if w.causal else 1.0)
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{heads} of {w.B * w.H} (b,h) heads of B={w.B} H={w.H} T={w.T} D={w.D} "
                      f"{'causal' if w.causal else 'non-causal'}; float64, full S materialised; "
                      f"{el:.1f} s", "seconds": el}


def next_rows(torch, fa, metrics, steps, warmup):
    """Time the grouped-head and packed variable-length forwards; one launch per step."""
    import synth
    peak = metrics.PEAK_TFLOPS["bf16"]
    rows = {}

    w = synth.GQA_WORKLOADS["gqa_bf16_b4hq32hkv8t4096d128_causal"]
    d = synth.make_gqa_inputs(w, seed=0)
    q, k, v = (_dev(d[n], torch) for n in "qkv")
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Tq), dtype=torch.float32, device="cuda")
    total, per, _ = _time_launches(
        torch, lambda: fa.fa_fwd_gqa(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse),
        steps, warmup)
    flops = metrics.gqa_flops(w.B, w.Hq, w.Tq, w.Tk, w.D, w.causal)
    ms = total / steps
    rows["gqa"] = {"workload": w.name, "ms_per_step": round(ms, 5),
                   "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
                   "pct_of_bf16_peak": round(100.0 * flops / (ms * 1e-3) / 1e12 / peak, 2),
                   "flops_per_step": flops,
                   "algorithmic_bytes_per_step": metrics.gqa_bytes(w.B, w.Hq, w.Hkv, w.Tq, w.Tk,
                                                                   w.D, 2)}
    del q, k, v, o, lse

    w = synth.VARLEN_WORKLOADS["varlen_bf16_n32l64to8192h16d128_causal"]
    d = synth.make_varlen_inputs(w, seed=0)
    q, k, v = (_dev(d[n], torch) for n in "qkv")
    cu = torch.from_numpy(d["cu"]).to("cuda")
    maxlen = int(d["lens"].max())
    o = torch.empty_like(q)
    lse = torch.empty((w.Hq, q.shape[0]), dtype=torch.float32, device="cuda")
    total, per, _ = _time_launches(
        torch, lambda: fa.fa_fwd_varlen(q, k, v, cu, cu, maxlen, causal=w.causal, scale=w.scale,
                                        out=o, lse=lse), steps, warmup)
    flops = metrics.varlen_flops(d["lens"], d["lens"], w.Hq, w.D, w.causal)
    ms = total / steps
    rows["varlen"] = {"workload": w.name, "total_tokens": int(d["cu"][-1]), "max_len": maxlen,
                      "ms_per_step": round(ms, 5),
                      "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
                      "pct_of_bf16_peak": round(100.0 * flops / (ms * 1e-3) / 1e12 / peak, 2),
                      "flops_per_step": flops,
                      "algorithmic_bytes_per_step": metrics.varlen_bytes(
                          q.shape[0], k.shape[0], w.Hq, w.Hkv, w.D, 2)}
    # FP8 (block-scaled E4M3) Q K^T on the headline workload: quantize Q and K, then the
    # forward on the codes; accuracy as the difference from the bf16 kernel's result
    w = synth.WORKLOADS["fwd_bf16_b4h16t4096d128_causal"]
    d = synth.make_workload_inputs(w, seed=0)
    q, k, v = (_dev(d[n], torch) for n in "qkv")
    q8, qs = fa.fa_quantize_mxfp8(q)
    k8, ks = fa.fa_quantize_mxfp8(k)
    o8 = torch.empty_like(q)
    l8 = torch.empty((w.B, w.H, w.T), dtype=torch.float32, device="cuda")
    total, _, _ = _time_launches(
        torch, lambda: fa.fa_fwd_fp8qk(q8, qs, k8, ks, v, causal=True, scale=w.scale, out=o8, lse=l8),
        steps, warmup)
    ms = total / steps
    qms = _time_loop(torch, lambda: (fa.fa_quantize_mxfp8(q, q8, qs), fa.fa_quantize_mxfp8(k, k8, ks)),
                     steps, warmup)
    flops = metrics.fwd_flops(w.B, w.H, w.T, w.D, True)
    ob, lb = fa.fa_fwd(q, k, v, causal=True, scale=w.scale)
    fa.fa_fwd_fp8qk(q8, qs, k8, ks, v, causal=True, scale=w.scale, out=o8, lse=l8)
    torch.cuda.synchronize()
    # S is half the flops at the fp8 rate (5.0 PFLOP/s), P V half at the bf16 rate
    mixed_peak = 1.0 / (0.5 / 5000.0 + 0.5 / peak)
    rows["fp8qk"] = {"workload": w.name, "ms_per_step": round(ms, 5),
                     "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
                     "pct_of_bf16_peak": round(100.0 * flops / (ms * 1e-3) / 1e12 / peak, 2),
                     "pct_of_mixed_peak": round(100.0 * flops / (ms * 1e-3) / 1e12 / mixed_peak, 2),
                     "mixed_peak_tflops": round(mixed_peak, 1),
                     "quantize_q_and_k_ms": round(qms, 5),
                     "tflops_with_quantize": round(flops / ((ms + qms) * 1e-3) / 1e12, 2),
                     "max_abs_o_vs_bf16_kernel": round((o8.float() - ob.float()).abs().max().item(), 5),
                     "max_abs_lse_vs_bf16_kernel": round((l8 - lb).abs().max().item(), 5),
                     "flops_per_step": flops}
    del q, k, v, q8, k8, qs, ks, o8, l8, ob, lb

    for name in ("decode_bf16_b1hq32hkv8tk32768d128", "decode_bf16_b8hq32hkv8tk32768d128_lens"):
        w = synth.DECODE_WORKLOADS[name]
        d = synth.make_gqa_inputs(w, seed=0)
        q, k, v = (_dev(d[n], torch) for n in "qkv")
        lens = synth.decode_lengths(w)
        sl = torch.from_numpy(lens).to("cuda") if w.B > 1 else None
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.Hq, w.Tq), dtype=torch.float32, device="cuda")
        ws = torch.empty(fa.fa_decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.Tq, w.Tk, w.D),
                         dtype=torch.uint8, device="cuda")
        ms = _time_loop(
            torch, lambda: fa.fa_fwd_decode(q, k, v, cache_seqlens=sl, causal=w.causal,
                                            scale=w.scale, out=o, lse=lse, workspace=ws),
            4 * steps, warmup)
        nbytes = metrics.decode_bytes(w.B, w.Hq, w.Hkv, w.Tq, w.D, int(lens.sum()), 2)
        row = {"workload": w.name, "ms_per_step": round(ms, 5),
               "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
               "pct_of_hbm_peak": round(100.0 * nbytes / (ms * 1e-3) / 1e9 / metrics.PEAK_HBM_GBS, 2),
               "algorithmic_bytes_per_step": nbytes,
               "kernels": "split kernel + merge kernel, one step each"}
        if w.B == 1:
            # the forward kernel on the same cache with one query row, as the pages ask
            fo = torch.empty_like(q)
            fl = torch.empty_like(lse)
            ftot, _, _ = _time_launches(
                torch, lambda: fa.fa_fwd_gqa(q, k, v, causal=w.causal, scale=w.scale, out=fo,
                                             lse=fl), max(3, steps // 4), 2)
            row["forward_kernel_ms_per_step"] = round(ftot / max(3, steps // 4), 5)
        rows["decode" if w.B == 1 else "decode_lens"] = row
        del q, k, v, o, lse, ws
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-next-rows", action="store_true")
    ap.add_argument("--no-library-gemm", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 256 MiB device-to-device copy (counter calibration under rocprofv3)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import exact_tiled_attention_flash_amd as fa
    import synth
    from exact_tiled_attention_flash_amd import metrics

    w = synth.WORKLOADS[FWD_WORKLOAD]
    d = synth.make_workload_inputs(w, seed=0)
    q, k, v = (_dev(d[n], torch) for n in "qkv")
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.T), dtype=torch.float32, device="cuda")

    def step():
        fa.fa_fwd(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse)

    total_ms, per, wall_ms = _time_launches(torch, step, args.steps, args.warmup)
    flops = metrics.fwd_flops(w.B, w.H, w.T, w.D, w.causal)
    ms_per_step = total_ms / args.steps
    avg_launch_ms = float(np.mean(per))
    achieved = flops / (avg_launch_ms * 1e-3) / 1e12
    peak = metrics.PEAK_TFLOPS["bf16"]
    value = flops / (ms_per_step * 1e-3) / 1e12

    out = {
        "metric": "attention fwd TFLOP/s (4*B*H*T^2*D, causal halved) and % of bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), numpy PCG64 seed 0, RNE to bf16)",
        "config": {"workload": FWD_WORKLOAD, "B": w.B, "H": w.H, "T": w.T, "D": w.D,
                   "causal": w.causal, "scale": w.scale},
        "pct_of_bf16_peak": round(100.0 * value / peak, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": None,
                     "kernel": "fwd_q32_kernel<128, causal>",
                     "avg_launch_ms": round(avg_launch_ms, 5),
                     "min_launch_ms": round(float(np.min(per)), 5),
                     "median_launch_ms": round(float(np.median(per)), 5),
                     "algorithmic_flops_per_launch": flops,
                     "algorithmic_bytes_per_launch": metrics.fwd_bytes(w.B, w.H, w.T, w.D, 2)},
        "wall_ms_timed_region": round(wall_ms, 3),
    }

    traffic = committed_traffic(flops)
    if traffic is not None:
        out["roofline"]["traffic"] = traffic["bytes_per_launch"]
        out["roofline"]["traffic_source"] = traffic["source"]

    if args.calibrate_copy:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = COPY_BYTES

    lib = fa.load_library()
    if not args.no_backward and hasattr(lib, "fa_bwd"):
        wb = synth.WORKLOADS[BWD_WORKLOAD]
        db = synth.make_workload_inputs(wb, seed=0)
        bq, bk, bv, bdo = (_dev(db[n], torch) for n in ("q", "k", "v", "do"))
        bo, blse = fa.fa_fwd(bq, bk, bv, causal=wb.causal, scale=wb.scale)
        ws = torch.empty(fa.fa_bwd_workspace_bytes(wb.B, wb.H, wb.T, wb.D), dtype=torch.uint8,
                         device="cuda")

        def bstep():
            fa.fa_bwd(bq, bk, bv, bo, bdo, blse, causal=wb.causal, scale=wb.scale, workspace=ws)

        btotal, bper, _ = _time_launches(torch, bstep, max(5, args.steps // 2), args.warmup)
        bflops = metrics.bwd_flops(wb.B, wb.H, wb.T, wb.D, wb.causal)
        bms = btotal / max(5, args.steps // 2)
        out["backward"] = {"workload": BWD_WORKLOAD, "ms_per_step": round(bms, 5),
                           "tflops": round(bflops / (bms * 1e-3) / 1e12, 2),
                           "flops_per_step": bflops,
                           "flop_count": "10*B*H*T^2*D/2 (S recompute, dP, dV, dQ, dK)",
                           "pct_of_bf16_peak": round(100.0 * bflops / (bms * 1e-3) / 1e12 / peak, 2)}

    if not args.no_next_rows:
        out["next_rows"] = next_rows(torch, fa, metrics, max(5, args.steps // 2), args.warmup)

    if not args.no_library_gemm:
        out["library_gemm"] = library_gemm(torch, peak)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, d, args.cpu_budget)
        out["cpu_baseline"]["value"] = round(out["cpu_baseline"]["value"], 5)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
