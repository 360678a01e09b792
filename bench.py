#!/usr/bin/env python3
"""Benchmark of the integer attention forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config bert]

A step is one intattn_forward call over the whole workload (every head of
every batch entry: Q.K^T, IndexSoftmax, P.V, requantisation), with inputs
already resident in HBM. Prints one JSON line. The default workload is
BERT-base encoder attention (B=8, H=12, S=512, d=64, non-causal); --config
selects one of the other four workloads (tiny, vit, llama_prefill, decode).

Work counted (algorithmic only): 4*d integer ops per allowed score (2*d for
Q.K^T, 2*d for P.V; causal counts the lower triangle with the diagonal), and
Q + K + V + O bytes of int8 read or written once.

Timing: 0.3 s of untimed calls (the GPU leaves its idle clocks), W untimed
calls, then exactly K calls bracketed by synchronisation and HIP events
recorded on the stream the library launches on (the caller's current
stream). The same events give the kernel's average duration per launch used
for the roofline fraction. Five more blocks of K calls give the median, and
one block cycling through copies of the inputs (more than 512 MB in all, so
they do not stay in the caches) gives the cold-input rate. Key "graph": the
same calls captured in a HIP graph (50 calls a graph) and replayed, five
blocks of replays (median), with the first replay's output checked against
the eager output;
`value` stays the rate of plain calls, one launch each.

The default run (BERT) also times every other workload in the same process
(key "workloads": tiny, BERT, ViT, causal prefill and batched decode, the
last one giving the metric's decode GB/s), each with both roofline fractions,
its outputs on a sample of heads compared with the oracle, and the oracle's
own rate on a short sample.

    python bench.py --calibrate peaks   # measured copy GB/s, int8 MFMA TOPS, VALU ops/s
    python bench.py --calibrate copy    # three 256 MiB device copies (counter scaling run)
    python bench.py --breakdown         # per-stage times of the unfused pipelines
    python bench.py --variants          # finer tables, grouped K/V heads, cache update
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0        # MI355X dense int8 MFMA, 5.0 POP/s
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
# 32-bit VALU: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz = 39.3e12 lane-ops/s
# (a wave64 VALU instruction occupies its SIMD for 4 cycles)
PEAK_VALU_TLANEOPS = 39.3
VALU_CYCLES_PER_INSTR = 4
N_SIMD = 1024
CLOCK_GHZ = 2.4

DEFAULT_STEPS = {"tiny": 2000, "bert": 500, "vit": 500, "llama_prefill": 50, "decode": 100}
# untimed calls before the timed region: about 0.4 s of work, so the GPU has
# left its idle clocks (shorter warm-ups measure the clock ramp-up)
DEFAULT_WARMUP = {"tiny": 50000, "bert": 30000, "vit": 25000, "llama_prefill": 2000, "decode": 2000}
# binding roofline per workload (ViT: 197 keys a row, arithmetic intensity 197 ops/byte, HBM)
BOUND = {"tiny": "mfma", "bert": "mfma", "vit": "hbm", "llama_prefill": "mfma", "decode": "hbm"}
# kernel the library dispatches for each workload, and its source file
# (the sources a summary's kernel_source_sha256 covers: the kernel's own files and ia_device.h)
_SHORT = ("ia_short.hip", "ia_short_impl.h")
KERNEL = {"tiny": ("ia_short_kernel", _SHORT), "bert": ("ia_short_kernel", _SHORT),
          "vit": ("ia_short_kernel", _SHORT), "llama_prefill": ("ia_long_kernel", ("ia_long.hip",)),
          "decode": ("ia_decode_kernel", ("ia_decode.hip",))}


def kernel_source_sha(srcs) -> str:
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "integer_only_quantized_amd", "csrc")
    for f in (*srcs, "ia_device.h"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(config: str):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary, or None when there is none or the kernel source changed since."""
    kname, src = KERNEL[config]
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{kname}_{config}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line:
                k, _, val = line.partition(":")
                fields[k.strip()] = val.strip()
    if fields.get("kernel_source_sha256") != kernel_source_sha(src):
        return None
    try:
        return int(fields["fetch_bytes_per_launch"]) + int(fields["write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def measured_valu(config):
    """SQ_INSTS_VALU per launch from the committed rocprofv3 counter summary, or
    None when there is none or the kernel source changed since."""
    kname, src = KERNEL[config]
    path = os.path.join(ROOT, "profiles", f"valu_{kname}_{config}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line:
                k, _, val = line.partition(":")
                fields[k.strip()] = val.strip()
    if fields.get("kernel_source_sha256") != kernel_source_sha(src):
        return None
    try:
        return float(fields["valu_wave_instrs_per_launch"])
    except (KeyError, ValueError):
        return None


def algorithmic_work(w):
    """(ops, bytes, allowed scores) of one forward call."""
    B, H, Sq, Skv, D = w.shape
    if w.causal:
        shift = Skv - Sq
        # row i attends keys 0 .. i + shift
        scores_per_head = sum(min(Skv, i + shift + 1) for i in range(Sq))
    else:
        scores_per_head = Sq * Skv
    scores = B * H * scores_per_head
    ops = 4 * D * scores
    nbytes = B * H * D * (2 * Sq + 2 * Skv)
    return ops, nbytes, scores


def cpu_baseline(w, budget_s=10.0):
    """Time the CPU oracle on a bounded sample of the workload's heads.

    Heads are processed one oracle call each, cycling over the workload's
    (b, h) pairs until about budget_s seconds of CPU work have run (a large
    workload stops part-way through its heads; a small one is repeated).
    Returns (summary dict, {(b, h): oracle output of the first pass}).
    """
    from oracle import intattn_oracle as O
    from integer_only_quantized_amd import workloads as W

    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    cores = len(os.sched_getaffinity(0))
    sub = W.slice_heads(w, heads[:1])               # warm-up (BLAS thread start-up)
    O.forward(sub.q, sub.k, sub.v, sub.scales, sub.clip, sub.causal)
    n_calls, t_total, results = 0, 0.0, {}
    while t_total < budget_s:
        bh = heads[n_calls % len(heads)]
        sub = W.slice_heads(w, [bh])
        t0 = time.perf_counter()
        o = O.forward(sub.q, sub.k, sub.v, sub.scales, sub.clip, sub.causal)
        t_total += time.perf_counter() - t0
        if bh not in results:
            results[bh] = o[0, 0]
        n_calls += 1
    ops_all, _, _ = algorithmic_work(w)
    frac = n_calls / len(heads)                       # workload calls' worth of heads
    tops = ops_all * frac / t_total / 1e12
    info = {
        "value": tops, "unit": "TOPS", "cores": cores, "kind": "oracle",
        "sample": f"{n_calls} single-head oracle calls cycling over the {len(heads)} (b,h) heads "
                  f"of the same workload ({frac:.3g} workload calls), {t_total:.2f} s wall; "
                  f"numpy float64 BLAS contractions (exact) + int64 elementwise; "
                  f"CPU {platform.processor() or platform.machine()}",
        "seconds": t_total,
        "calls_per_s": frac / t_total,
    }
    return info, results


def calibrate(mode):
    """Peaks measured on this GPU (mode 'peaks'), or the plain-copy run that
    scales FETCH_SIZE / WRITE_SIZE (mode 'copy': three 256 MiB copies)."""
    import ctypes
    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if mode == "copy":
        n = 256 << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev).random_(0, 255)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes_per_copy": n, "copies": 3}), flush=True)
        return 0
    out = {"calibration": "peaks"}
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev).random_(0, 255)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(20):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    out["copy_GBs"] = 2 * n * 20 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    lib = ctypes.CDLL(os.path.join(ROOT, "integer_only_quantized_amd", "libintattn_probe.so"))
    for fn in (lib.intattn_probe_mfma_i8, lib.intattn_probe_valu):
        fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        fn.restype = ctypes.c_int
    blocks = 2048
    sink = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    for name, fn, iters, work in (
            ("mfma_i8_TOPS", lib.intattn_probe_mfma_i8, 20000, lambda it: blocks * 4 * 4 * it * 65536 / 1e12),
            ("valu_Tlaneops", lib.intattn_probe_valu, 100000, lambda it: blocks * 256 * 8 * it / 1e12)):
        if fn(blocks, 100, ctypes.c_void_p(sink.data_ptr()), stream) != 0:
            raise RuntimeError(f"{name}: probe launch failed")
        torch.cuda.synchronize()
        e0.record()
        if fn(blocks, iters, ctypes.c_void_p(sink.data_ptr()), stream) != 0:
            raise RuntimeError(f"{name}: probe launch failed")
        e1.record()
        torch.cuda.synchronize()
        out[name] = work(iters) / (e0.elapsed_time(e1) * 1e-3)
    out["spec"] = {"hbm_GBs": PEAK_HBM_GBS, "mfma_i8_TOPS": PEAK_INT8_TOPS, "valu_Tlaneops": PEAK_VALU_TLANEOPS}
    print(json.dumps(out), flush=True)
    return 0


def breakdown(config, steps=None):
    """Per-stage times of the pipeline run as separate kernels (scores and P in
    HBM), with the integer softmax and with the float32 comparator, beside the
    fused call: the softmax share of each pipeline and the speedups."""
    import torch

    from integer_only_quantized_amd import _binding as ia
    from integer_only_quantized_amd import workloads as W

    w = W.make_config(config)
    if w.Skv > 4096:
        raise SystemExit(f"--breakdown needs Skv <= 4096 (the softmax stages hold a row in registers); "
                         f"{config} has Skv = {w.Skv}")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = (torch.from_numpy(x).to(dev) for x in (w.q, w.k, w.v))
    B, H, Sq, Skv, D = w.shape
    S = torch.empty((B, H, Sq, Skv), dtype=torch.int32, device=dev)
    P = torch.empty((B, H, Sq, Skv), dtype=torch.uint8, device=dev)
    C = torch.empty_like(P)
    out = torch.empty_like(q)
    outc = torch.empty_like(q)
    calls = {
        "fused": lambda: ia.forward(q, k, v, w.scales, w.clip, w.causal, out=out),
        "qk_scores": lambda: ia.qk_scores(q, k, out=S),
        "index_softmax": lambda: ia.index_softmax(S, D, w.scales, w.clip, w.causal, probs=P),
        "fp_softmax": lambda: ia.fp_softmax(S, D, w.scales, w.causal, probs=C),
        "pv": lambda: ia.pv(P, v, w.scales, w.clip, w.causal, out=outc),
    }
    for name in ("qk_scores", "index_softmax", "fp_softmax", "pv", "fused"):
        calls[name]()
    torch.cuda.synchronize(dev)
    if not torch.equal(outc, out):
        raise RuntimeError("the integer stages chained differ from the fused call")
    stream = torch.cuda.current_stream(dev)
    times = {}
    for name, fn in calls.items():
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.3:      # warm-up (clock ramp)
            fn()
        torch.cuda.synchronize(dev)
        n = steps or 200
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize(dev)
        times[name] = e0.elapsed_time(e1) / n * 1e3      # us per call
    _, _, scores = algorithmic_work(w)
    n_sc = B * H * Sq * Skv
    hbm = {   # bytes each stage moves at least once
        "qk_scores": B * H * (Sq + Skv) * D + 4 * n_sc,
        "index_softmax": 5 * n_sc,
        "fp_softmax": 5 * n_sc,
        "pv": n_sc + B * H * (Skv + Sq) * D,
    }
    t_int = times["qk_scores"] + times["index_softmax"] + times["pv"]
    t_fp = times["qk_scores"] + times["fp_softmax"] + times["pv"]
    line = {
        "breakdown": config,
        "shape": {"B": B, "H": H, "Sq": Sq, "Skv": Skv, "D": D, "causal": w.causal},
        "us_per_call": times,
        "stage_GBs": {k2: hbm[k2] / (times[k2] * 1e-6) / 1e9 for k2 in hbm},
        "stage_hbm_frac": {k2: hbm[k2] / (times[k2] * 1e-6) / 1e9 / PEAK_HBM_GBS for k2 in hbm},
        "integer_pipeline_us": t_int,
        "fp_pipeline_us": t_fp,
        "softmax_share_integer_pipeline": times["index_softmax"] / t_int,
        "softmax_share_fp_pipeline": times["fp_softmax"] / t_fp,
        "speedup_integer_vs_fp_pipeline": t_fp / t_int,
        "speedup_fused_vs_fp_pipeline": t_fp / times["fused"],
        "softmax_stage_speedup": times["fp_softmax"] / times["index_softmax"],
        "scores_allowed": scores,
    }
    print(json.dumps(line), flush=True)
    return 0


def _time_calls(fn, stream, n, warm_s=0.3):
    """Median-free event timing: warm-up for warm_s seconds, then n calls; us per call."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < warm_s:
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n * 1e3


def _time_calls_held(fn, stream, n, warm_s=0.3):
    """(GPU us per call, host us per call) for calls whose host submission
    may be as long as their GPU time (several launches a call): the host
    time is taken over n calls first, then the GPU is held by a spin kernel
    long enough for the host to queue n more, and the events time those."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < warm_s:
        fn()
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    for _ in range(n):
        fn()
    host_us = (time.perf_counter() - h0) / n * 1e6
    torch.cuda.synchronize()
    hold_gpu(stream)                          # calibrates the spin rate on first use
    torch.cuda._sleep(int((1.5 * n * host_us + 200.0) * _SLEEP_CYCLES_PER_US))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n * 1e3, host_us


def variants(steps=None):
    """The variants beside the 32-entry MHA path: finer exp tables (64, 128
    entries), uint8 table entries and uint16 probabilities on the BERT and
    causal-prefill workloads (int8 TOPS and MFMA fraction; uint8 entries and
    uint16 also on the decode shape), grouped
    K/V heads on the batched decode shape (HBM GB/s of
    Q + K + V + O with K/V read once per K/V head), and the decode-step cache
    update (HBM GB/s of 4 bytes read and 1 written per value), and decode
    with keys split over workgroups (batch 1, and caches longer than 16384
    keys) against the same calls without a workspace. One JSON line."""
    import torch

    from integer_only_quantized_amd import _binding as ia
    from integer_only_quantized_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    res = {"variants": True, "fine_tables": {}, "grouped_decode": {}, "kv_append": {}, "decode_step": {}}

    for cfg in ("bert", "llama_prefill"):
        w = W.make_config(cfg)
        q, k, v = (torch.from_numpy(x).to(dev) for x in (w.q, w.k, w.v))
        out = torch.empty_like(q)
        ops, _, _ = algorithmic_work(w)
        row = {}
        for n in (32, 64, 128):
            try:
                ia.derive_params_ex(w.D, w.scales, w.clip, n)
            except ia.IntAttnError:
                row[str(n)] = {"refused": "index multiplier outside [2^-24, 2^14) for this table"}
                continue
            fn = lambda n=n: ia.forward_ex(q, k, v, w.scales, w.clip, w.causal, n, out=out)
            us = _time_calls(fn, stream, steps or (200 if cfg == "bert" else 30))
            tops = ops / (us * 1e-6) / 1e12
            row[str(n)] = {"us_per_call": us, "int8_TOPS": tops, "mfma_frac": tops / PEAK_INT8_TOPS}
        res["fine_tables"][cfg] = row
        # uint16 probabilities (32-entry table): the short-row kernel's uint16 instances on BERT, the
        # long-row kernel on causal prefill
        fn = lambda: ia.forward_ex(q, k, v, w.scales, w.clip, w.causal, 32, out=out, prob_bits=16)
        us = _time_calls(fn, stream, steps or (200 if cfg == "bert" else 30))
        tops = ops / (us * 1e-6) / 1e12
        res.setdefault("uint16_probabilities", {})[cfg] = {"us_per_call": us, "int8_TOPS": tops,
                                                          "mfma_frac": tops / PEAK_INT8_TOPS}
        # uint8 table entries (32 entries): the same kernels, the table in Q15 units
        fn = lambda: ia.forward_ex(q, k, v, w.scales, w.clip, w.causal, 32, out=out, lut_bits=8)
        us = _time_calls(fn, stream, steps or (200 if cfg == "bert" else 30))
        tops = ops / (us * 1e-6) / 1e12
        res.setdefault("uint8_table", {})[cfg] = {"us_per_call": us, "int8_TOPS": tops,
                                                  "mfma_frac": tops / PEAK_INT8_TOPS}
        print(f"# variants: tables and widths on {cfg} done", file=sys.stderr, flush=True)

    # grouped K/V heads on the decode shape: B=16, H=32, Skv=8192, d=128
    B, H, Skv, D = 16, 32, 8192, 128
    g = torch.Generator(device=dev)
    g.manual_seed(4)
    def codes(shape):
        x = torch.randn(shape, generator=g, device=dev) * (127.0 / 4.5)
        return x.round().clamp_(-127, 127).to(torch.int8)
    q = codes((B, H, 1, D))
    scales = (4.5 / 127, 4.5 / 127, 4.5 / 127, 0.6 / 127)
    for hkv in (32, 8, 1):
        k = codes((B, hkv, Skv, D))
        v = codes((B, hkv, Skv, D))
        out = torch.empty_like(q)
        fn = lambda: ia.forward_ex(q, k, v, scales, W.DEFAULT_CLIP, False, 32, out=out)
        us = _time_calls(fn, stream, steps or 100)
        nbytes = 2 * B * H * D + 2 * B * hkv * Skv * D
        gbs = nbytes / (us * 1e-6) / 1e9
        res["grouped_decode"][f"Hkv={hkv}"] = {"us_per_call": us, "bytes": nbytes, "GBs": gbs,
                                               "hbm_frac": gbs / PEAK_HBM_GBS}
        if hkv == 32:
            fn16 = lambda: ia.forward_ex(q, k, v, scales, W.DEFAULT_CLIP, False, 32, out=out, prob_bits=16)
            us16 = _time_calls(fn16, stream, steps or 100)
            gbs16 = nbytes / (us16 * 1e-6) / 1e9
            res.setdefault("uint16_probabilities", {})["decode"] = {"us_per_call": us16, "GBs": gbs16,
                                                                    "hbm_frac": gbs16 / PEAK_HBM_GBS}
            fn8 = lambda: ia.forward_ex(q, k, v, scales, W.DEFAULT_CLIP, False, 32, out=out, lut_bits=8)
            us8 = _time_calls(fn8, stream, steps or 100)
            gbs8 = nbytes / (us8 * 1e-6) / 1e9
            res.setdefault("uint8_table", {})["decode"] = {"us_per_call": us8, "GBs": gbs8,
                                                           "hbm_frac": gbs8 / PEAK_HBM_GBS}
        del k, v
        print(f"# variants: grouped decode Hkv={hkv} done", file=sys.stderr, flush=True)
    torch.cuda.empty_cache()

    # cache update: one decode token and a 4096-token prefill chunk
    for name, (Bc, hkv, T, cap) in {"decode_token": (16, 8, 1, 8192), "prefill_chunk": (1, 32, 4096, 4096)}.items():
        kc = torch.zeros((Bc, hkv, cap, D), dtype=torch.int8, device=dev)
        vc = torch.zeros_like(kc)
        kn = torch.randn((Bc, hkv, T, D), generator=g, device=dev)
        vn = torch.randn((Bc, hkv, T, D), generator=g, device=dev)
        pos = cap - T
        fn = lambda: ia.kv_append(kn, vn, kc, vc, pos, 0.035, 0.035)
        us = _time_calls(fn, stream, steps or 200)
        nbytes = 2 * 5 * Bc * hkv * T * D
        gbs = nbytes / (us * 1e-6) / 1e9
        res["kv_append"][name] = {"shape": [Bc, hkv, T, D], "us_per_call": us, "bytes": nbytes, "GBs": gbs,
                                  "hbm_frac": gbs / PEAK_HBM_GBS}
        del kc, vc, kn, vn

    # one grouped-query decode step: append the token, attend over the cache
    Bc, hkv, cap, filled = 16, 8, 8192, 8191
    kc = codes((Bc, hkv, cap, D))
    vc = codes((Bc, hkv, cap, D))
    kn = torch.randn((Bc, hkv, 1, D), generator=g, device=dev)
    vn = torch.randn((Bc, hkv, 1, D), generator=g, device=dev)
    out = torch.empty_like(q)
    def step():
        ia.kv_append(kn, vn, kc, vc, filled, 4.5 / 127, 4.5 / 127)
        ia.forward_ex(q, kc, vc, scales, W.DEFAULT_CLIP, False, 32, out=out, skv=filled + 1)
    us = _time_calls(step, stream, steps or 100)
    res["decode_step"] = {"shape": {"B": Bc, "H": H, "Hkv": hkv, "Skv": filled + 1, "D": D},
                          "us_per_step": us, "steps_per_s": 1e6 / us}
    del kc, vc, kn, vn
    torch.cuda.empty_cache()

    # decode with keys split over several workgroups per head (workspace):
    # batch 1 (32 heads: one workgroup each on the decode kernel) and caches
    # past the decode kernel's 16384 keys (without a workspace: one workgroup
    # per head streaming K three times); HBM GB/s of K + V read once. A split
    # call is four launches, whose host submission through the binding can
    # outlast the GPU work at batch 1, so the GPU time is taken with the
    # calls queued ahead, and the host time per call is reported beside it
    res["split_decode"] = {}
    for (Bc, Hc, Skv) in ((1, 32, 8192), (8, 32, 32768), (2, 32, 65535)):
        ql = codes((Bc, Hc, 1, D))
        kl = codes((Bc, Hc, Skv, D))
        vl = codes((Bc, Hc, Skv, D))
        ol = torch.empty_like(ql)
        ws = torch.empty(ia.workspace_bytes(Bc, Hc, 1, Skv, D), dtype=torch.uint8, device=dev)
        nbytes = 2 * Bc * Hc * Skv * D
        row = {"workspace_bytes": ws.numel(), "bytes": nbytes}
        for name, w in (("split", ws), ("without_workspace", False)):
            fn = lambda w=w: ia.forward_ex(ql, kl, vl, scales, W.DEFAULT_CLIP, False, 32, out=ol, workspace=w)
            us, host_us = _time_calls_held(fn, stream, steps or 30)
            gbs = nbytes / (us * 1e-6) / 1e9
            row[name] = {"us_per_call": us, "host_us_per_call": host_us, "GBs": gbs, "hbm_frac": gbs / PEAK_HBM_GBS}
        res["split_decode"][f"B={Bc} H={Hc} Skv={Skv}"] = row
        print(f"# variants: split decode B={Bc} H={Hc} Skv={Skv} done", file=sys.stderr, flush=True)
        del ql, kl, vl, ol, ws
        torch.cuda.empty_cache()
    print(json.dumps(res), flush=True)
    return 0


CLOCK_SETTLE_S = 0.3
# parity sample per workload: (b, h) heads compared with the oracle
PARITY_HEADS = {"tiny": [(0, 0)], "bert": [(0, 0), (3, 7), (5, 2), (7, 11)],
                "vit": [(0, 0), (13, 5), (31, 11)], "llama_prefill": [(0, 0), (0, 31)],
                "decode": [(0, 0), (7, 19), (15, 31)]}


def np_equal(a, b):
    import numpy as np
    return bool(np.array_equal(a, b))


def roofline(config, tops, gbs):
    """Roofline of a workload: its binding unit (int8 MFMA or HBM) and both
    fractions, from the algorithmic ops and bytes per call."""
    bound = BOUND[config]
    if bound == "mfma":
        roof = {"bound": "mfma", "achieved": tops, "peak": PEAK_INT8_TOPS, "unit": "TOPS",
                "frac": tops / PEAK_INT8_TOPS}
    else:
        roof = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": gbs / PEAK_HBM_GBS}
    roof["mfma_frac"] = tops / PEAK_INT8_TOPS
    roof["hbm_frac"] = gbs / PEAK_HBM_GBS
    return roof


_SLEEP_CYCLES_PER_US = None


def hold_gpu(stream):
    """Queue a 150 us spin kernel ahead of a timed region, so that the host
    has enqueued the first dozen or so calls (about 8 us each through the
    Python binding) when the first event is reached: the region then starts
    with the GPU's first call, not with the host's submission of it. Later
    calls are submitted while earlier ones run, so a workload whose calls
    are shorter than their submission still measures the host-bound rate. A
    longer hold would idle the GPU (one spinning wave) long enough for its
    clock to drop."""
    import torch

    global _SLEEP_CYCLES_PER_US
    if _SLEEP_CYCLES_PER_US is None:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000)
        e0.record(stream)
        torch.cuda._sleep(1_000_000)
        e1.record(stream)
        torch.cuda.synchronize()
        _SLEEP_CYCLES_PER_US = 1_000_000 / max(1.0, e0.elapsed_time(e1) * 1e3)
    torch.cuda._sleep(int(150.0 * _SLEEP_CYCLES_PER_US))


GRAPH_CALLS = 50          # forward calls captured in one HIP graph (graph timing)


def graph_timing(call, out, stream, steps):
    """The same calls captured in one HIP graph (GRAPH_CALLS forward calls,
    torch.cuda.CUDAGraph over the library's launches on the capture stream)
    and replayed: the GPU's rate once the host submits one graph per
    GRAPH_CALLS calls instead of one launch per call. The first replay's
    output must equal the eager output left in `out`."""
    import torch

    dev = out.device
    ref = out.clone()
    side = torch.cuda.Stream(dev)
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        call()                                   # warm on the capture stream
    stream.wait_stream(side)
    torch.cuda.synchronize(dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(GRAPH_CALLS):
            call()
    torch.cuda.synchronize(dev)
    out.zero_()
    g.replay()
    torch.cuda.synchronize(dev)
    equal = bool(torch.equal(out, ref))
    # one replay submits GRAPH_CALLS calls in less host time than the GPU
    # takes to run them, so the host stays ahead without a spin kernel
    reps = max(2, steps // GRAPH_CALLS)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.3:
        g.replay()
    torch.cuda.synchronize(dev)
    blocks = []
    for _ in range(5):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize(dev)
        blocks.append(e0.elapsed_time(e1) / (reps * GRAPH_CALLS))
    ms = sorted(blocks)[2]
    del g
    return {"ms_per_step": ms, "calls_per_s": 1e3 / ms, "calls_per_graph": GRAPH_CALLS,
            "replays_per_block": reps, "blocks_ms_per_step": blocks, "first_replay_equals_eager": equal}


def measure(w, steps, warmup, extra_timing=False, settle_s=CLOCK_SETTLE_S, graph=False):
    """Times intattn_forward over workload w with inputs resident in HBM.

    First settle_s seconds of untimed calls (the GPU leaves its idle clocks),
    then `warmup` untimed calls, then exactly `steps` calls bracketed by
    synchronisation and HIP events recorded on the stream the library
    launches on (the caller's current stream); a spin kernel queued before
    the first event keeps the GPU busy while the host enqueues the calls. Returns ms_per_step, the wall
    time of the timed region, the output (numpy) and, with extra_timing,
    five more blocks (median) and one block over input copies totalling more
    than 512 MB (cold caches), and with graph the rate of the same calls
    replayed from a captured HIP graph (graph_timing).
    """
    import torch

    from integer_only_quantized_amd import _binding as ia

    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(x).to(dev) for x in (w.q, w.k, w.v))
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream(dev)
    call = lambda: ia.forward(q, k, v, w.scales, w.clip, w.causal, out=out)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < settle_s:
        call()
    # the warm-up calls run between the same two events as the timed region,
    # so the events' first-use cost falls outside it
    ev0.record(stream)
    for _ in range(warmup):
        call()
    ev1.record(stream)
    torch.cuda.synchronize(dev)
    t_wall0 = time.perf_counter()
    hold_gpu(stream)
    ev0.record(stream)
    for _ in range(steps):
        call()
    ev1.record(stream)
    torch.cuda.synchronize(dev)
    res = {"wall_s": time.perf_counter() - t_wall0, "ms_per_step": ev0.elapsed_time(ev1) / steps}
    if extra_timing:
        def timed_block(sets):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize(dev)
            hold_gpu(stream)
            e0.record(stream)
            for i in range(steps):
                qs, ks, vs, os_ = sets[i % len(sets)]
                ia.forward(qs, ks, vs, w.scales, w.clip, w.causal, out=os_)
            e1.record(stream)
            torch.cuda.synchronize(dev)
            return e0.elapsed_time(e1) / steps
        warm = [(q, k, v, out)]
        reps = [timed_block(warm) for _ in range(5)]
        per_set = 2 * q.numel() + 2 * k.numel()
        # input copies totalling > 512 MB (twice the 256 MB last-level cache),
        # at most 4096 of them (tiny inputs are launch-bound either way)
        n_sets = 1 if per_set > (512 << 20) else min(4096, (512 << 20) // per_set + 2)
        cold_sets = warm + [(q.clone(), k.clone(), v.clone(), torch.empty_like(out)) for _ in range(n_sets - 1)]
        cold = timed_block(cold_sets)
        del cold_sets
        res["timing"] = {"repeats_ms_per_step": reps, "median_ms_per_step": sorted(reps)[2],
                         "cold_ms_per_step": cold, "cold_input_sets": n_sets,
                         "cold_input_bytes": n_sets * per_set}
    if graph:
        res["graph"] = graph_timing(call, out, stream, steps)
    res["out"] = out.cpu().numpy()
    del q, k, v, out
    torch.cuda.empty_cache()
    return res


def all_workloads(bert_w, args):
    """Every workload of the metric timed in this run (exactly
    DEFAULT_STEPS[name] calls each after the same clock settle and
    DEFAULT_WARMUP-capped warm-up), with the rates, both roofline fractions
    and the output of a sample of heads compared with the oracle, plus the
    oracle's own rate on a short sample of the same workload."""
    from oracle import intattn_oracle as O
    from integer_only_quantized_amd import workloads as W

    res = {}
    for name in ("tiny", "bert", "vit", "llama_prefill", "decode"):
        w = bert_w if name == "bert" else W.make_config(name)
        steps = DEFAULT_STEPS[name]
        warmup = min(DEFAULT_WARMUP[name], 200)
        m = measure(w, steps, warmup, graph=True)
        ops, nbytes, scores = algorithmic_work(w)
        sec = m["ms_per_step"] / 1e3
        tops, gbs = ops / sec / 1e12, nbytes / sec / 1e9
        prm = O.derive_params(w.D, *w.scales, w.clip)
        heads = PARITY_HEADS[name]
        parity = all(np_equal(m["out"][b, h], O.head_forward(w.q[b, h], w.k[b, h], w.v[b, h], prm, w.causal)[0])
                     for b, h in heads)
        entry = {
            "shape": {"B": w.B, "H": w.H, "Sq": w.Sq, "Skv": w.Skv, "D": w.D, "causal": w.causal},
            "kernel": KERNEL[name][0], "steps": steps, "warmup": warmup,
            "ms_per_step": m["ms_per_step"], "calls_per_s": 1.0 / sec,
            "int8_tops": tops, "gb_per_s": gbs, "roofline": roofline(name, tops, gbs),
            "parity_on_sample": parity, "parity_heads": [list(bh) for bh in heads],
            "graph": m["graph"],
        }
        if not args.no_cpu_baseline:
            cpu, _ = cpu_baseline(w, min(args.cpu_budget, 2.0))
            entry["cpu_oracle"] = {"TOPS": cpu["value"], "calls_per_s": cpu["calls_per_s"],
                                   "GB_per_s": nbytes * cpu["calls_per_s"] / 1e9, "cores": cpu["cores"],
                                   "seconds": cpu["seconds"]}
        res[name] = entry
        print(f"# workload {name}: {m['ms_per_step'] * 1e3:.2f} us/call, parity {parity}",
              file=sys.stderr, flush=True)
        del m
        if name != "bert":
            del w
    return res


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--config", default="bert",
                    choices=["tiny", "bert", "vit", "llama_prefill", "decode"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--calibrate", choices=["peaks", "copy"], default=None)
    ap.add_argument("--breakdown", action="store_true",
                    help="per-stage times of the unfused pipelines (integer and float32 softmax)")
    ap.add_argument("--variants", action="store_true",
                    help="finer exp tables, grouped K/V heads and the cache update (one JSON line)")
    ap.add_argument("--no-extra-timing", action="store_true",
                    help="skip the median-of-5, cold-input and HIP-graph blocks")
    ap.add_argument("--no-workloads", action="store_true",
                    help="time the headline workload only (default: also every other workload)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: attention heads are independent, so a "
              "multi-GPU run is the same kernel on each GPU's share of the heads, and this "
              "library runs on one GPU. Run with --gpus 1.", file=sys.stderr)
        return 2

    if args.calibrate:
        return calibrate(args.calibrate)
    if args.breakdown:
        return breakdown(args.config, args.steps)
    if args.variants:
        return variants(args.steps)

    import torch

    from integer_only_quantized_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    steps = args.steps or DEFAULT_STEPS[args.config]
    warmup = DEFAULT_WARMUP[args.config] if args.warmup is None else args.warmup
    w = W.make_config(args.config)
    m = measure(w, steps, warmup, extra_timing=not args.no_extra_timing, graph=not args.no_extra_timing)
    ms_per_step = m["ms_per_step"]
    ops, nbytes, scores = algorithmic_work(w)
    sec = ms_per_step / 1e3
    tops = ops / sec / 1e12
    gbs = nbytes / sec / 1e9

    roof = roofline(args.config, tops, gbs)
    roof["kernel"] = KERNEL[args.config][0]
    roof["per_launch"] = {"ops": ops, "bytes": nbytes, "scores": scores,
                          "avg_launch_us": ms_per_step * 1e3}
    roof["traffic"] = measured_traffic(args.config)
    valu_instrs = measured_valu(args.config)
    valu = None
    if valu_instrs is not None:
        lane_ops = valu_instrs * 64
        achieved = lane_ops / sec / 1e12
        valu = {"bound": "alu", "achieved": achieved, "peak": PEAK_VALU_TLANEOPS, "unit": "T lane-ops/s",
                "frac": achieved / PEAK_VALU_TLANEOPS, "lane_ops_per_score": lane_ops / scores,
                "source": f"profiles/valu_{KERNEL[args.config][0]}_{args.config}.txt"}

    cpu = None
    if not args.no_cpu_baseline:
        cpu, ref = cpu_baseline(w, args.cpu_budget)
        cpu["parity_on_sample"] = all(
            np_equal(m["out"][b, h], r) for (b, h), r in ref.items())

    if args.config == "decode":
        metric_value, unit = gbs, "GB/s"
    else:
        metric_value, unit = tops, "TOPS"
    line = {
        "metric": "int8 attention TOPS + calls/s (BERT-base S=512) and decode GB/s; % of roofline"
        if args.config == "bert" else f"int8 attention throughput ({args.config})",
        "value": metric_value,
        "unit": unit,
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": args.config, "description": w.meta.get("description"),
                   "B": w.B, "H": w.H, "Sq": w.Sq, "Skv": w.Skv, "D": w.D, "causal": w.causal},
        "calls_per_s": 1.0 / sec,
        "int8_tops": tops,
        "gb_per_s": gbs,
        "clock_settle_s": CLOCK_SETTLE_S,
        "wall_s_timed_region": m["wall_s"],
        "roofline": roof,
        "valu_roofline": valu,
        "timing": m.get("timing"),
        "graph": m.get("graph"),
        "cpu_baseline": cpu,
    }
    del m
    if args.config == "bert" and not args.no_workloads:
        # the rest of the metric (decode GB/s) and every other workload, timed
        # in the same run
        line["workloads"] = all_workloads(w, args)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
