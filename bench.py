"""Benchmark: attention forward TFLOP/s on one MI355X, and % of the bf16 MFMA peak.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--seed S] [--configs 1,2,4,5]
                [--no-cpu-baseline] [--no-next-rows] [--no-library-gemm]

One step is one forward pass (fa_fwd: one kernel launch) over the headline workload
(configuration 3): causal bf16, B=4, H=16, T=4096, D=128, scale 1/sqrt(128), seeded N(0,1)
inputs already resident in HBM. FLOPs per step = 4*B*H*T^2*D / 2. The float64 oracle runs on
every (b, h) head of the same inputs on the host: it is timed (cpu_baseline) and its O and LSE
are compared with the timed kernel's output over the whole tensor ("parity").

The other four configurations are reported under "configs", each with its GPU time, its
parity against the oracle and the oracle's own time:
  1  fp32 non-causal B=1 H=2 T=128 D=64 (latency-bound; parity at 1e-4)
  2  bf16 B=1 H=8 T=1024 D=64, non-causal and causal (latency-bound)
  4  bf16 causal B=1 H=32 T=16381 D=128 with 1 % of the key rows x8 (roofline fields; oracle on
     two whole heads plus sampled rows of every head)
  5  bf16 causal backward B=2 H=16 T=4096 D=128, O and LSE from the forward (oracle on two
     heads)
"next_rows" times the grouped-head, packed-batch, split-K decode and E4M3 Q K^T calls on their
own workloads; "library_gemm" times the vendor library's bf16 GEMM (8192^3) in the same process
as the dense bf16 rate reachable on this GPU at its sustained clock, and "library_copy" a 1 GiB
device copy as the streaming rate reachable for the HBM-bound rows; "device_peak" recomputes
the bf16 peak from the compute-unit count and peak clock the device reports. Prints one JSON
line.
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


def _device_warmup(torch, fn, seconds):
    """Run fn() untimed until `seconds` of wall time have passed (at least once): the GPU
    leaves its idle clock over tens of milliseconds of sustained work, and a handful of warm-up
    steps ends before that. Returns the number of calls."""
    n = 0
    t0 = time.perf_counter()
    while True:
        for _ in range(8):
            fn()
        n += 8
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return n


def _time_launches(torch, fn, steps, warmup, warm_s=0.2):
    """Warm up, then time `steps` back-to-back calls of fn() (enqueued on the current stream)
    between one pair of events, bracketed by device synchronisations: the whole-job rate.
    Then time `steps` more calls with one event pair around each call: the duration of one
    launch on its own (each event record makes the stream wait for the kernel before it, so
    this pass has no overlap between consecutive launches and is kept out of the first).
    Returns (total_ms of the back-to-back pass, per-launch ms list, host wall ms of the
    back-to-back pass). Before all of it, warm_s seconds of untimed calls (_device_warmup):
    each workload's inputs are drawn on the host while the GPU idles."""
    if warm_s > 0:
        _device_warmup(torch, fn, warm_s)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record(stream)
    for _ in range(steps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    total = a.elapsed_time(b)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for x, y in ev:
        x.record(stream)
        fn()
        y.record(stream)
    torch.cuda.synchronize()
    per = [x.elapsed_time(y) for x, y in ev]
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


def library_copy(torch):
    """Context for the HBM-bound rows (decode): a device-to-device copy of 1 GiB through torch
    (the runtime's copy kernel), bytes read plus bytes written per second. The published 8 TB/s
    is the interface's peak; this is what a plain streaming kernel reaches on this GPU."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    ms = _time_loop(torch, lambda: b.copy_(a), 20, 5)
    gbs = 2.0 * n / (ms * 1e-3) / 1e9
    return {"op": "device-to-device copy of 1 GiB (torch copy_)", "ms": round(ms, 4),
            "gbs_read_plus_write": round(gbs, 1), "pct_of_hbm_peak": round(100.0 * gbs / 8000.0, 2)}


def _time_loop(torch, fn, steps, warmup, warm_s=0.2):
    """Warm up (warm_s seconds of untimed calls, then `warmup` calls), then time `steps`
    back-to-back calls of fn() with one event pair around the loop (for calls of tens of
    microseconds, where an event pair per call would leave gaps of host time between the
    launches). Returns milliseconds per call."""
    if warm_s > 0:
        _device_warmup(torch, fn, warm_s)
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


def _threads():
    """BLAS threads the oracle's numpy uses (the cores the CPU baseline runs on)."""
    try:
        from threadpoolctl import threadpool_info
        return int(max([p.get("num_threads", 1) for p in threadpool_info()] or [1]))
    except Exception:  # noqa: BLE001
        return len(os.sched_getaffinity(0))


def _host_f64(t):
    """A device tensor (bf16 or fp32) as float64 numpy."""
    import torch
    import synth
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return synth.bf16_bits_to_f64(t.view(torch.int16).numpy().view(np.uint16))
    return t.numpy().astype(np.float64)


def _err(a, b):
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def headline_oracle(w, d, o_dev, lse_dev):
    """The float64 oracle on every (b, h) head of the headline inputs, timed (the CPU
    baseline), and its O and LSE compared with the kernel's output over the whole tensor."""
    import oracle
    import synth
    o, lse = _host_f64(o_dev), lse_dev.cpu().numpy().astype(np.float64)
    err_o = err_l = 0.0
    el = 0.0
    for idx in range(w.B * w.H):
        b, h = divmod(idx, w.H)
        q, k, v = (synth.bf16_bits_to_f64(d[n][b:b + 1, h:h + 1]) for n in "qkv")
        t0 = time.perf_counter()
        o_ref, l_ref = oracle.attention_forward(q, k, v, w.scale, w.causal)
        el += time.perf_counter() - t0
        err_o = max(err_o, _err(o[b, h], o_ref[0, 0]))
        err_l = max(err_l, _err(lse[b, h], l_ref[0, 0]))
    heads = w.B * w.H
    flops = 4.0 * heads * w.T * w.T * w.D / (2.0 if w.causal else 1.0)
    base = {"value": round(flops / el / 1e12, 5), "unit": "TFLOP/s", "cores": _threads(),
            "kind": "oracle",
            "sample": f"all {heads} (b,h) heads of B={w.B} H={w.H} T={w.T} D={w.D} "
                      f"{'causal' if w.causal else 'non-causal'} (the whole workload); float64, "
                      f"full S materialised in row chunks; {el:.1f} s",
            "seconds": round(el, 3)}
    parity = {"compared": f"whole tensors: O {tuple(o.shape)}, LSE {tuple(lse.shape)}",
              "max_abs_o": err_o, "max_abs_lse": err_l, "tol_o": 2e-2, "tol_lse": 1e-3,
              "pass": bool(err_o <= 2e-2 and err_l <= 1e-3)}
    return base, parity


def device_peak(torch):
    """The bf16 dense matrix-core peak recomputed from what the device reports: compute
    units x peak engine clock x 4096 flops per clock per compute unit (one 32x32x16 bf16
    product, 32768 flops, every 32 clocks on each of a compute unit's 4 SIMDs)."""
    import ctypes
    try:
        hip = ctypes.CDLL("libamdhip64.so")
    except OSError as e:
        return {"error": str(e)}
    dev = torch.cuda.current_device()
    val = ctypes.c_int(0)
    attrs = {"clock_khz": 5, "compute_units": 63}   # hipDeviceAttributeClockRate, ...MultiprocessorCount
    got = {}
    for name, code in attrs.items():
        if hip.hipDeviceGetAttribute(ctypes.byref(val), code, dev) != 0:
            return {"error": f"hipDeviceGetAttribute({name}) failed"}
        got[name] = val.value
    if got["compute_units"] != torch.cuda.get_device_properties(dev).multi_processor_count:
        return {"error": "compute-unit count disagrees with torch's"}
    tf = got["compute_units"] * got["clock_khz"] * 1e3 * 4096 / 1e12
    return {"compute_units": got["compute_units"], "peak_clock_mhz": got["clock_khz"] / 1e3,
            "bf16_tflops": round(tf, 1),
            "published_bf16_tflops": 2516.6}


# Figures the pages give with their own hardware: context only, none measured here.
PAGE_CONTEXT = [
    {"figure": "max-abs error of a Triton FA2 forward against the PyTorch math path: goal below 1e-3",
     "workload": "B=1 H=8 T=1024 D=64 causal, fp16 inputs, seed 0",
     "hardware": "NVIDIA Ampere or newer",
     "source": "Triton FlashAttention-2 forward, 'Correctness'"},
    {"figure": "speed of the Triton FA2 forward against naive attention: goal at least 3x, "
               "3 warm-ups and 20 timed iterations",
     "workload": "B=1 H=8 T=2048 D=64 causal, fp16", "hardware": "NVIDIA Ampere or newer",
     "source": "Triton FlashAttention-2 forward, 'Performance'"},
    {"figure": "a first Triton kernel about 2x behind the vendor attention kernel is normal",
     "workload": "B=8 H=16 T=2048 D=64 causal, bf16, 64/64 blocks", "hardware": "RTX 5060",
     "source": "Lab 06 - Attention kernels, 'On your RTX 5060'"},
    {"figure": "tolerance 2e-3 when the dots run in tf32", "workload": "T=16 and 37, D=32",
     "hardware": "RTX 5060", "source": "Lab 06 - Attention kernels, test table 'Tip'"},
]


def _fwd_parity(fa, torch, w, d, dtype):
    """Run fa_fwd once on a whole workload and compare O and LSE with the oracle."""
    import oracle
    import synth
    conv = (lambda a: synth.bf16_bits_to_f64(a)) if dtype == "bf16" else (lambda a: a.astype(np.float64))
    if dtype == "bf16":
        q, k, v = (_dev(d[n], torch) for n in "qkv")
    else:
        q, k, v = (torch.from_numpy(np.ascontiguousarray(d[n], dtype=np.float32)).cuda() for n in "qkv")
    o, lse = fa.fa_fwd(q, k, v, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    o_ref, l_ref = oracle.attention_forward(*(conv(d[n]) for n in "qkv"), w.scale, w.causal)
    el = time.perf_counter() - t0
    return (q, k, v), {"max_abs_o": _err(_host_f64(o), o_ref),
                       "max_abs_lse": _err(lse.cpu().numpy().astype(np.float64), l_ref)}, el


def config_rows(torch, fa, metrics, which, steps, warmup, seed, peak):
    """Configurations 1, 2, 4 and 5: GPU time, parity against the oracle, the oracle's time."""
    import oracle
    import synth
    rows = {}
    small = [("1", "fwd_f32_b1h2t128d64", 1e-4, 1e-4)]
    small += [("2", "fwd_bf16_b1h8t1024d64", 2e-2, 1e-3), ("2", "fwd_bf16_b1h8t1024d64_causal", 2e-2, 1e-3)]
    for cfg, name, to, tl in small:
        if cfg not in which:
            continue
        w = synth.WORKLOADS[name]
        d = synth.make_workload_inputs(w, seed=seed)
        (q, k, v), par, el = _fwd_parity(fa, torch, w, d, w.dtype)
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.T), dtype=torch.float32, device="cuda")
        ms = _time_loop(torch, lambda: fa.fa_fwd(q, k, v, causal=w.causal, scale=w.scale, out=o,
                                                 lse=lse), 10 * steps, warmup)
        flops = metrics.fwd_flops(w.B, w.H, w.T, w.D, w.causal)
        par.update({"tol_o": to, "tol_lse": tl, "compared": "whole tensors",
                    "pass": bool(par["max_abs_o"] <= to and par["max_abs_lse"] <= tl)})
        # one workgroup per 128 query rows of a (b, h)
        wgs = w.B * w.H * -(-w.T // 128)
        rows.setdefault(cfg, {})[name] = {
            "ms_per_step": round(ms, 5), "tflops": round(flops / (ms * 1e-3) / 1e12, 3),
            "flops_per_step": flops,
            "bound": f"latency: {wgs} workgroups for 256 compute units, each walking every key "
                     "tile of its rows in turn (parity configuration)",
            "parity": par,
            "oracle": {"seconds": round(el, 4), "tflops": round(flops / el / 1e12, 6),
                       "cores": _threads(), "sample": "whole workload"}}

    if "4" in which:
        w = synth.WORKLOADS["fwd_bf16_b1h32t16381d128_causal_spiky"]
        d = synth.make_workload_inputs(w, seed=seed)
        q, k, v = (_dev(d[n], torch) for n in "qkv")
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.T), dtype=torch.float32, device="cuda")
        n4 = max(3, steps // 4)
        total, per, _ = _time_launches(
            torch, lambda: fa.fa_fwd(q, k, v, causal=True, scale=w.scale, out=o, lse=lse), n4, 2)
        flops = metrics.fwd_flops(w.B, w.H, w.T, w.D, True)
        avg = float(np.mean(per))
        ms = total / n4
        oh, lh = _host_f64(o), lse.cpu().numpy().astype(np.float64)
        err_o = err_l = 0.0
        el = 0.0
        for hh in (5, 31):   # two whole heads
            qh, kh, vh = (synth.bf16_bits_to_f64(d[n][:, hh:hh + 1]) for n in "qkv")
            t0 = time.perf_counter()
            o_ref, l_ref = oracle.attention_forward(qh, kh, vh, w.scale, True)
            el += time.perf_counter() - t0
            err_o = max(err_o, _err(oh[0, hh], o_ref[0, 0]))
            err_l = max(err_l, _err(lh[0, hh], l_ref[0, 0]))
        rng = np.random.default_rng(seed)
        spikes = np.asarray(d["spikes"])
        for hh in range(w.H):   # sampled rows of every head: rows after spikes, the ragged tail
            sel = np.unique(np.concatenate([rng.integers(0, w.T, 8), [0, w.T - 1, w.T - 2],
                                            np.clip(spikes[:4] + 1, 0, w.T - 1)]))
            qh, kh, vh = (synth.bf16_bits_to_f64(d[n][0, hh]) for n in "qkv")
            o_ref, l_ref = oracle.attention_rows(qh, kh, vh, w.scale, True, sel)
            err_o = max(err_o, _err(oh[0, hh, sel], o_ref))
            err_l = max(err_l, _err(lh[0, hh, sel], l_ref))
        ach = flops / (avg * 1e-3) / 1e12
        rows4 = {"workload": w.name, "ms_per_step": round(ms, 5),
                 "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
                 "pct_of_bf16_peak": round(100.0 * flops / (ms * 1e-3) / 1e12 / peak, 2),
                 "roofline": {"bound": "mfma", "achieved": round(ach, 2), "peak": peak,
                              "unit": "TFLOP/s", "frac": round(ach / peak, 4),
                              "kernel": "fwd_q32_kernel<128, causal>",
                              "avg_launch_ms": round(avg, 5),
                              "algorithmic_flops_per_launch": flops,
                              "algorithmic_bytes_per_launch": metrics.fwd_bytes(w.B, w.H, w.T, w.D, 2)},
                 "parity": {"compared": "heads 5 and 31 whole, 8 random rows + rows 0, T-1, T-2 "
                                        "and 4 rows after spike positions of every head",
                            "max_abs_o": err_o, "max_abs_lse": err_l, "tol_o": 2e-2,
                            "tol_lse": 1e-3, "pass": bool(err_o <= 2e-2 and err_l <= 1e-3)},
                 "oracle": {"seconds": round(el, 3),
                            "tflops": round(2 * 4.0 * w.T * w.T * w.D / 2 / el / 1e12, 5),
                            "cores": _threads(), "sample": "2 of 32 (b,h) heads, whole"}}
        rows["4"] = rows4
        del q, k, v, o, lse

    if "5" in which:
        wb = synth.WORKLOADS[BWD_WORKLOAD]
        db = synth.make_workload_inputs(wb, seed=seed)
        bq, bk, bv, bdo = (_dev(db[n], torch) for n in ("q", "k", "v", "do"))
        bo, blse = fa.fa_fwd(bq, bk, bv, causal=wb.causal, scale=wb.scale)
        ws = torch.empty(fa.fa_bwd_workspace_bytes(wb.B, wb.H, wb.T, wb.D), dtype=torch.uint8,
                         device="cuda")
        res = {}

        def bstep():
            res["g"] = fa.fa_bwd(bq, bk, bv, bo, bdo, blse, causal=wb.causal, scale=wb.scale,
                                 workspace=ws)

        nb = max(5, steps // 2)
        btotal, bper, _ = _time_launches(torch, bstep, nb, warmup)
        bflops = metrics.bwd_flops(wb.B, wb.H, wb.T, wb.D, wb.causal)
        bms = btotal / nb
        dq, dk, dv = (_host_f64(g) for g in res["g"])
        errs = [0.0, 0.0, 0.0]
        el = 0.0
        for idx in (0, 31):
            b, h = divmod(idx, wb.H)
            sl = (slice(b, b + 1), slice(h, h + 1))
            q64, k64, v64, do64 = (synth.bf16_bits_to_f64(db[n][sl]) for n in ("q", "k", "v", "do"))
            t0 = time.perf_counter()
            o_ref, l_ref = oracle.attention_forward(q64, k64, v64, wb.scale, True)
            ref = oracle.attention_backward(q64, k64, v64, o_ref, do64, l_ref, wb.scale, True)
            el += time.perf_counter() - t0
            for i, (g, r) in enumerate(zip((dq, dk, dv), ref)):
                errs[i] = max(errs[i], _err(g[sl], r))
        rows["5"] = {"workload": BWD_WORKLOAD, "ms_per_step": round(bms, 5),
                     "tflops": round(bflops / (bms * 1e-3) / 1e12, 2),
                     "flops_per_step": bflops,
                     "flop_count": "10*B*H*T^2*D/2 (S recompute, dP, dV, dQ, dK)",
                     "pct_of_bf16_peak": round(100.0 * bflops / (bms * 1e-3) / 1e12 / peak, 2),
                     "kernels": "bwd_dq (with D_i) + bwd_dkdv, one step each",
                     "parity": {"compared": "(b,h) heads 0 and 31, whole dQ, dK, dV",
                                "max_abs_dq": errs[0], "max_abs_dk": errs[1], "max_abs_dv": errs[2],
                                "tol": 2e-2, "pass": bool(max(errs) <= 2e-2 + 0.03125)},
                     "oracle": {"seconds": round(el, 3),
                                "tflops": round(2 * bflops / (wb.B * wb.H) / el / 1e12, 5),
                                "cores": _threads(),
                                "sample": "2 of 32 (b,h) heads: float64 forward and dense backward"}}
        del bq, bk, bv, bdo, bo, blse, ws, res
    return rows


def next_rows(torch, fa, metrics, steps, warmup, seed=0):
    """Time the grouped-head and packed variable-length forwards; one launch per step."""
    import synth
    peak = metrics.PEAK_TFLOPS["bf16"]
    rows = {}

    w = synth.GQA_WORKLOADS["gqa_bf16_b4hq32hkv8t4096d128_causal"]
    d = synth.make_gqa_inputs(w, seed=seed)
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
    d = synth.make_varlen_inputs(w, seed=seed)
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
    d = synth.make_workload_inputs(w, seed=seed)
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
        d = synth.make_gqa_inputs(w, seed=seed)
        q, k, v = (_dev(d[n], torch) for n in "qkv")
        lens = synth.decode_lengths(w, seed=seed)
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
    ap.add_argument("--seed", type=int, default=0, help="seed of every synthetic input")
    ap.add_argument("--device-warmup", type=float, default=1.0,
                    help="seconds of untimed headline steps before the W warm-up steps")
    ap.add_argument("--configs", default="1,2,4,5",
                    help="comma-separated configurations reported besides the headline (3)")
    ap.add_argument("--backward-only", action="store_true",
                    help="time only configuration 5 (the backward), for the backward's profiles")
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

    if args.backward_only:
        if args.calibrate_copy:
            src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
            dst = torch.empty_like(src)
            for _ in range(3):
                dst.copy_(src)
            torch.cuda.synchronize()
        rows = config_rows(torch, fa, metrics, {"5"}, args.steps, args.warmup, args.seed,
                           metrics.PEAK_TFLOPS["bf16"])
        print(json.dumps({"backward_only": rows["5"]}))
        return

    w = synth.WORKLOADS[FWD_WORKLOAD]
    d = synth.make_workload_inputs(w, seed=args.seed)
    q, k, v = (_dev(d[n], torch) for n in "qkv")
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.T), dtype=torch.float32, device="cuda")

    def step():
        fa.fa_fwd(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse)

    dev_warm = _device_warmup(torch, step, args.device_warmup)
    total_ms, per, wall_ms = _time_launches(torch, step, args.steps, args.warmup, warm_s=0)
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
        "data": f"synthetic (seeded N(0,1), numpy PCG64 seed {args.seed}, RNE to bf16)",
        "config": {"workload": FWD_WORKLOAD, "B": w.B, "H": w.H, "T": w.T, "D": w.D,
                   "causal": w.causal, "scale": w.scale, "seed": args.seed},
        "pct_of_bf16_peak": round(100.0 * value / peak, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": None,
                     "kernel": "fwd_q32_kernel<128, causal>",
                     "avg_launch_ms": round(avg_launch_ms, 5),
                     "launch_timing": "one event pair around each of K further launches "
                                      "(no overlap between launches)",
                     "min_launch_ms": round(float(np.min(per)), 5),
                     "median_launch_ms": round(float(np.median(per)), 5),
                     "algorithmic_flops_per_launch": flops,
                     "algorithmic_bytes_per_launch": metrics.fwd_bytes(w.B, w.H, w.T, w.D, 2)},
        "wall_ms_timed_region": round(wall_ms, 3),
        "timing": "value and ms_per_step: K back-to-back steps between one event pair, "
                  "device synchronised before and after",
        "device_warmup": {"seconds": args.device_warmup, "steps": dev_warm,
                          "why": "untimed steps before the W warm-up steps, so that the GPU has "
                                 "left its idle clock when the timed region starts"},
        "device_peak": device_peak(torch),
        "context_from_pages": PAGE_CONTEXT,
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

    which = {c.strip() for c in args.configs.split(",") if c.strip() and c.strip() != "none"}
    if args.no_backward:
        which.discard("5")
    if which:
        out["configs"] = config_rows(torch, fa, metrics, which, args.steps, args.warmup,
                                     args.seed, peak)
        if "5" in out["configs"]:
            out["backward"] = out["configs"]["5"]

    if not args.no_next_rows:
        out["next_rows"] = next_rows(torch, fa, metrics, max(5, args.steps // 2), args.warmup,
                                     args.seed)

    if not args.no_library_gemm:
        out["library_gemm"] = library_gemm(torch, peak)
        out["library_copy"] = library_copy(torch)

    if not args.no_cpu_baseline:
        out["cpu_baseline"], out["parity"] = headline_oracle(w, d, o, lse)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
