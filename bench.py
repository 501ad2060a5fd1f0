#!/usr/bin/env python3
"""Benchmark of the GPTQ weight-only quantized linear layer on one MI355X.

One step = one gptq_gemm call (the whole per-call path: dispatch, activation staging, packed
weight stream, in-register dequant, fp32 MFMA accumulation, epilogue) on the Llama-3-8B-shaped
MLP up projection (K=4096, N=14336, 4-bit, group 128, fp16, M=1).  The load-time repack is not
part of a step ("Kernel Backends Reference", pitfalls: do not time repacking as steady state).

Inputs are synthetic and seeded (gptq_inputs).  Every call streams its weights from HBM: calls
rotate over enough distinct repacked copies (>= 512 MiB) that the 256 MiB Infinity Cache cannot
serve them.

Timing.  Every timed region starts with a short device-side wait kernel queued ahead of it, so the
calls are already queued when the start event is reached and the region holds device time only
(not the host's launch latency before the first call).  The headline `value`: W warm-up calls, then
exactly K calls between two HIP events on the launch stream, with torch.cuda.synchronize() on both
sides, measured after the decode-sized records and before the compute-bound ones.  A region still
holds one dispatch latency that no earlier call overlaps (the start event waits for the wait
kernel), so a short region reads a little above the batches' steady state.  Every record (the
headline's too, in `headline_batches`) also reports the median and the 10th / 90th percentiles of
the per-call time over 7 batches of at least 50 calls (20 for M >= 1024) after at least 10 warm-up
calls, with its own counts.

Prints ONE JSON line.  `value` is microseconds per call (lower is better); `roofline` reports the
dominant kernel's algorithmic bytes per launch / its average launch time against 8 TB/s; `extra`
holds the other workloads measured with the same protocol (not bench lines of their own), the
device read floor at the decode layers' byte counts, and a dense bf16 matmul of the prefill shape
as context; `cpu_baseline` is the float64 CPU oracle timed on this host.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16/fp16 MFMA, published
ROTATE_BYTES = 512 << 20        # > 256 MiB Infinity Cache
PROFILES = os.path.join(ROOT, "profiles")
BATCHES = 7


def algorithmic_bytes(K, N, M, bits, gs, desc_act, scale_bytes=2, act_bytes=2):
    """Bytes the method must move per call: qweight + qzeros + scales + x + y (+ 4 K for the
    act-order permutation)."""
    G = 1 if gs == -1 else -(-K // gs)
    b = K * bits // 32 * N * 4 + G * (N * bits // 32) * 4 + G * N * scale_bytes + M * K * act_bytes + M * N * act_bytes
    if desc_act:
        b += 4 * K
    return b


# Sources that make up each measured kernel family (its own files plus the shared headers).
SHARED_SOURCES = ["bufmem.h", "dequant.h", "internal.h", "layout.h"]
FAMILY_SOURCES = {"skinny": ["skinny_impl.h", "plans.h", "skinny.hip", "skinny_b4.hip"],
                  "tiled": ["tiled.hip", "plans.h"]}


def csrc_digest(family):
    """Digest of the sources of one kernel family; stored counter readings are used only while it
    is unchanged."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "weight_only_quantized_amd", "csrc")
    for f in sorted(FAMILY_SOURCES[family] + SHARED_SOURCES):
        h.update(f.encode())
        h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:16]


def stored_traffic(kernel_key):
    """HBM bytes per launch from the committed rocprofv3 counter runs (profiles/traffic.json), only
    if the sources of the kernel's family are unchanged since they were taken; else None."""
    p = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        t = json.load(open(p))
    except Exception:
        return None
    e = t.get(kernel_key)
    if not e or e.get("csrc_sha") != csrc_digest(kernel_key.split("_")[0]):
        return None
    return {"bytes_per_launch": e.get("bytes_per_launch"), "kernel": e.get("kernel"), "from": "profiles/traffic.json"}


def profile_of(label):
    """Committed rocprofv3 kernel-trace summary of this workload, if any (names the kernel)."""
    hits = sorted(glob.glob(os.path.join(PROFILES, f"*_{label}_kernel_trace.md")))
    return os.path.relpath(hits[0], ROOT) if hits else None


class Workload:
    def __init__(self, name, K, N, M, bits, gs, desc_act, sdt, xdt, seed, bias=False, fmt="gptq"):
        self.name, self.K, self.N, self.M, self.bits, self.gs = name, K, N, M, bits, gs
        self.desc_act, self.sdt, self.xdt, self.seed, self.bias = desc_act, sdt, xdt, seed, bias
        self.fmt = fmt   # checkpoint the layer is repacked from: "gptq", "gptq_p" or "awq_gemm"

    def label(self):
        g = "g-1" if self.gs == -1 else f"g{self.gs}"
        return f"{self.name}_M{self.M}_b{self.bits}_{g}" + ("_actorder" if self.desc_act else "")


class DeviceTimer:
    """HIP-event timing on one stream, with a device-side wait queued ahead of each region so that
    the timed calls are queued before the start event is reached."""

    def __init__(self, stream):
        import torch
        self.torch = torch
        self.stream = stream
        with torch.cuda.stream(stream):
            torch.cuda._sleep(1000)
        torch.cuda.synchronize()
        # cycles of torch.cuda._sleep per microsecond on this device
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n = 2_000_000
        with torch.cuda.stream(stream):
            e0.record(stream)
            torch.cuda._sleep(n)
            e1.record(stream)
        torch.cuda.synchronize()
        self.cycles_per_us = n / max(e0.elapsed_time(e1) * 1e3, 1.0)

    def region(self, call, n, offset=0, lead_us=None):
        """Average microseconds per call of call(offset) .. call(offset + n - 1)."""
        torch = self.torch
        lead = lead_us if lead_us is not None else min(4000.0, 10.0 * n + 50.0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(self.stream):
            torch.cuda._sleep(int(lead * self.cycles_per_us))
            e0.record(self.stream)
            for i in range(n):
                call(offset + i)
            e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    def batches(self, call, per_batch, offset=0):
        ts = sorted(self.region(call, per_batch, offset + b * per_batch) for b in range(BATCHES))
        pct = lambda q: ts[min(len(ts) - 1, max(0, int(round(q * (len(ts) - 1)))))]
        return {"median_us": round(pct(0.5), 3), "p10_us": round(pct(0.1), 3), "p90_us": round(pct(0.9), 3),
                "mean_us": round(sum(ts) / len(ts), 3), "batches": BATCHES, "calls_per_batch": per_batch}


def build_handles(w: Workload, copies: int):
    import numpy as np
    import torch
    import gptq_inputs as gi
    import weight_only_quantized_amd as wq
    dev = torch.device("cuda:0")
    if w.fmt == "awq_gemm":
        L = gi.make_awq_layer(w.K, w.N, w.gs, scales_dtype=w.sdt, seed=w.seed)
        g = None
    else:
        L = gi.make_layer(w.K, w.N, w.bits, w.gs, desc_act=w.desc_act, scales_dtype=w.sdt, seed=w.seed)
        g = torch.from_numpy(L.g_idx).to(dev)
    qw = torch.from_numpy(L.qweight).to(dev)
    qz = torch.from_numpy(L.qzeros).to(dev)
    sc = torch.from_numpy(L.scales.view(np.int16).copy()).to(dev).view(
        torch.float16 if w.sdt == "f16" else torch.bfloat16)
    hs = [wq.repack(qw, qz, sc, g, bits=w.bits, group_size=w.gs, desc_act=w.desc_act, checkpoint_format=w.fmt)
          for _ in range(copies)]
    del qw, qz, sc, g
    return L, hs


def time_layer(w: Workload, timer: DeviceTimer, warmup: int, per_batch: int, steps: int = 0):
    """Warm-up, then (steps > 0) exactly `steps` timed calls, then the batches.  Returns a dict."""
    import numpy as np
    import torch
    import gptq_inputs as gi
    import weight_only_quantized_amd as wq
    wbytes = algorithmic_bytes(w.K, w.N, 0, w.bits, w.gs, w.desc_act)
    R = max(1, math.ceil(ROTATE_BYTES / wbytes))
    L, hs = build_handles(w, R)
    lib = wq.load_library()
    dev = torch.device("cuda:0")
    tdt = torch.float16 if w.xdt == "f16" else torch.bfloat16
    xb = gi.make_x(w.M, w.K, w.xdt, seed=w.seed + 1)
    nx = min(R, 4)
    xs = [torch.from_numpy(xb.view(np.int16).copy()).to(dev).view(tdt) for _ in range(nx)]
    ys = [torch.empty((w.M, w.N), dtype=tdt, device=dev) for _ in range(nx)]
    need = hs[0].workspace_size(w.M, tdt)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    sp = timer.stream.cuda_stream
    xcode = 0 if w.xdt == "f16" else 1
    args = [(hs[i % R].ptr, xs[i % nx].data_ptr(), ys[i % nx].data_ptr()) for i in range(R * nx)]
    bias = None
    if w.bias:   # the layer's [N] bias in the scales' dtype, through gptq_gemm_bias
        bb = gi.make_bias(w.N, w.sdt, seed=w.seed + 2)
        bias = torch.from_numpy(bb.view(np.int16).copy()).to(dev)

    def call(i):
        h, x, y = args[i % len(args)]
        if bias is None:
            st = lib.gptq_gemm(h, x, w.M, xcode, y, ws.data_ptr(), ws.numel(), 0, sp)
        else:
            st = lib.gptq_gemm_bias(h, x, w.M, xcode, bias.data_ptr(), y, ws.data_ptr(), ws.numel(), 0, sp)
        if st:
            raise wq.GPTQError(st, "gptq_gemm", lib)

    with torch.cuda.stream(timer.stream):
        for i in range(warmup):
            call(i)
    torch.cuda.synchronize()
    out = {"copies": R, "warmup": warmup}
    if steps:
        out["timed_us"] = timer.region(call, steps, warmup)
        out["steps"] = steps
    out.update(timer.batches(call, per_batch, warmup + steps))
    for h in hs:
        h.close()
    torch.cuda.synchronize()
    return out


def time_read_floor(nbytes, timer: DeviceTimer, warmup: int, per_batch: int):
    """The device read floor (gptq_read_floor) at a layer's byte count, over rotated buffers."""
    import torch
    import weight_only_quantized_amd as wq
    lib = wq.load_library()
    nb = (nbytes + 15) // 16 * 16
    R = max(2, math.ceil(ROTATE_BYTES / nb))
    bufs = [torch.full((nb,), i + 1, dtype=torch.uint8, device="cuda") for i in range(R)]
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    sp = timer.stream.cuda_stream

    def call(i):
        st = lib.gptq_read_floor(bufs[i % R].data_ptr(), nb, sink.data_ptr(), sp)
        if st:
            raise wq.GPTQError(st, "gptq_read_floor", lib)

    with torch.cuda.stream(timer.stream):
        for i in range(warmup):
            call(i)
    out = {"copies": R, "warmup": warmup}
    out.update(timer.batches(call, per_batch, warmup))
    del bufs
    torch.cuda.synchronize()
    return out


def time_dense_mm(M, K, N, timer: DeviceTimer, warmup: int, per_batch: int):
    """A dense bf16 matmul of the same shape through torch (hipBLASLt): context for the MFMA path."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(20261202)
    a = torch.randn((M, K), dtype=torch.bfloat16, device="cuda", generator=g)
    b = torch.randn((K, N), dtype=torch.bfloat16, device="cuda", generator=g).contiguous()
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def call(i):
        torch.mm(a, b, out=c)

    with torch.cuda.stream(timer.stream):
        for i in range(warmup):
            call(i)
    out = {"warmup": warmup}
    out.update(timer.batches(call, per_batch, warmup))
    del a, b, c
    torch.cuda.synchronize()
    return out


def cpu_oracle_baseline(w: Workload, budget_s=20.0):
    """The float64 oracle as it stands, timed on this host: whole calls of the headline layer, plus
    its two phases timed apart on one call (unpack + dequant; the float64 matmul)."""
    import numpy as np
    import gptq_inputs as gi
    import oracle as o
    L = gi.make_layer(w.K, w.N, w.bits, w.gs, desc_act=w.desc_act, scales_dtype=w.sdt, seed=w.seed)
    x = gi.make_x(w.M, w.K, w.xdt, seed=w.seed + 1)
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        threads = None
    t0 = time.perf_counter()
    W = o.dequant(L.qweight, L.qzeros, L.scales, w.sdt, L.g_idx, w.bits)
    t1 = time.perf_counter()
    _ = o.decode_float_bits(x, w.xdt) @ W.T
    t2 = time.perf_counter()
    del W
    runs, t_total = 0, 0.0
    while runs < 1 or (t_total < budget_s and runs < 10):
        t0w = time.perf_counter()
        o.gemm(x, w.xdt, L.qweight, L.qzeros, L.scales, w.sdt, L.g_idx, w.bits)
        t_total += time.perf_counter() - t0w
        runs += 1
        if t_total / runs * (runs + 1) > budget_s * 1.5:
            break
    return {"value": round(t_total / runs * 1e6, 1), "unit": "us/call", "cores": threads or os.cpu_count(),
            "kind": "oracle",
            "unpack_dequant_us": round((t1 - t0) * 1e6, 1), "matmul_us": round((t2 - t1) * 1e6, 1),
            "sample": f"{runs} whole call(s) of {w.label()} (unpack + float64 dequant + float64 matmul, chunked "
                      f"over the outputs); phases of one call timed apart: unpack + dequant on one thread, the "
                      f"matmul on the BLAS pool ({threads} threads); host has {os.cpu_count()} logical CPUs"}


HEADLINE = Workload("llama3_8b_up_proj", 4096, 14336, 1, 4, 128, False, "f16", "f16", 20262202)


def extra_workloads():
    import gptq_inputs as gi
    out = []
    for M in (4, 16, 64, 128, 256):
        out.append(Workload("llama3_8b_up_proj", 4096, 14336, M, 4, 128, False, "f16", "f16", gi.seed_for(1)))
    for M in (1, 8, 16, 32, 64, 128, 256):
        out.append(Workload("llama3_70b_gate_proj", 8192, 28672, M, 4, 128, False, "f16", "bf16", gi.seed_for(2)))
    # the down projection of the same 8B MLP: 14336 inputs at decode sizes
    for M in (1, 4):
        out.append(Workload("llama3_8b_down_proj", 14336, 4096, M, 4, 128, False, "f16", "f16", gi.seed_for(7)))
    for bits in (2, 3, 4, 8):
        for gs in (128, -1):
            for M in (1, 32):
                out.append(Workload("act_order_8192x8192", 8192, 8192, M, bits, gs, True, "f16", "f16",
                                    gi.seed_for(3, bits)))
    out.append(Workload("prefill_4096x8192x28672", 8192, 28672, 4096, 4, 128, False, "bf16", "bf16",
                        gi.seed_for(4)))
    # the same layers with their bias (gptq_gemm_bias)
    out.append(Workload("bias_llama3_8b_up_proj", 4096, 14336, 1, 4, 128, False, "f16", "f16", gi.seed_for(1),
                        bias=True))
    out.append(Workload("bias_prefill_4096x8192x28672", 8192, 28672, 4096, 4, 128, False, "bf16", "bf16",
                        gi.seed_for(4), bias=True))
    # GPTQ_P planar checkpoints, each in the runtime layout of its own width
    for bits in (3, 5, 6, 7):
        out.append(Workload(f"gptq_p_llama3_8b_up_proj", 4096, 14336, 1, bits, 128, False, "f16", "f16",
                            gi.seed_for(6, bits), fmt="gptq_p"))
    # the same shapes repacked from AutoAWQ GEMM tensors (same runtime layout and kernels)
    out.append(Workload("awq_llama3_8b_up_proj", 4096, 14336, 1, 4, 128, False, "f16", "f16", gi.seed_for(5),
                        fmt="awq_gemm"))
    out.append(Workload("awq_prefill_4096x8192x28672", 8192, 28672, 4096, 4, 128, False, "bf16", "bf16",
                        gi.seed_for(5), fmt="awq_gemm"))
    return out


def time_quantize(K, N, S, bits, gs, act, reps=3):
    """Wall time of the GPU quantizer on one layer: Hessian of S calibration rows, then GPTQ."""
    import numpy as np
    import torch
    import gptq_inputs as gi
    import weight_only_quantized_amd as wq
    x = torch.from_numpy(gi.make_calib(S, K, "bf16", seed=K + S).view(np.int16).copy()).cuda().view(torch.bfloat16)
    W = torch.from_numpy(gi.make_weight(N, K, seed=N + K)).cuda()
    wq.quantize(W, wq.hessian(x), bits=bits, group_size=gs, act_order=act)       # loads the solver libraries
    th, tq = [], []
    for _ in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        H = wq.hessian(x)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        wq.quantize(W, H, bits=bits, group_size=gs, act_order=act)
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        th.append(t1 - t0)
        tq.append(t2 - t1)
    g = "g-1" if gs == -1 else f"g{gs}"
    return {"workload": f"quantize_{K}x{N}_S{S}_b{bits}_{g}" + ("_actorder" if act else ""),
            "hessian_ms": round(min(th) * 1e3, 3), "quantize_ms": round(min(tq) * 1e3, 3),
            "ms_per_layer": round((min(th) + min(tq)) * 1e3, 3)}


def layer_record(e: Workload, t: dict) -> dict:
    """A layer record: timing counts and percentiles, bytes, and the roofline of its bound (HBM for
    the streaming calls, dense 16-bit MFMA for M >= 1024), on the median per-call time."""
    us = t["median_us"]
    rec = {"workload": e.label(), "us_per_call": us}
    rec.update({k: v for k, v in t.items() if k != "median_us"})
    b = algorithmic_bytes(e.K, e.N, e.M, e.bits, e.gs, e.desc_act, scale_bytes=2) + (2 * e.N if e.bias else 0)
    rec["algorithmic_bytes"] = b
    rec["TB_per_s"] = round(b / (us * 1e-6) / 1e12, 3)
    fam = "tiled" if e.M > 32 else "skinny"
    traffic = stored_traffic(f"{fam}_{e.label()}")
    prof = profile_of(e.label())
    if e.M >= 1024:
        fl = 2.0 * e.M * e.N * e.K
        tf = fl / (us * 1e-6) / 1e12
        rec["roofline"] = {"bound": "mfma", "achieved": round(tf, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                           "traffic": traffic["bytes_per_launch"] if traffic else None,
                           "algorithmic_flops_per_launch": fl, "timed": "whole call (x prep + GEMM)"}
    else:
        gbs = b / (us * 1e-6) / 1e9
        rec["roofline"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(gbs / HBM_PEAK_GBS, 4),
                           "traffic": traffic["bytes_per_launch"] if traffic else None,
                           "algorithmic_bytes_per_launch": b}
    if prof:
        rec["roofline"]["profile"] = prof
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-extra", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only", default=None, help="time the workloads whose label starts with this prefix and exit")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before timing, run 3 plain device copies of this many MiB (a known-size kernel for "
                         "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE readings); outside the timed region")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the kernels run one GPU's share "
              f"of a layer; no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import torch
    import weight_only_quantized_amd as wq
    assert torch.cuda.is_available(), "needs a GPU"
    wq.load_library()
    torch.cuda.set_device(0)
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    timer = DeviceTimer(torch.cuda.Stream())     # default priority
    xw = max(10, min(args.warmup, 100))          # warm-up of the extra records

    if args.only:
        for w in [HEADLINE] + extra_workloads():
            if w.label().startswith(args.only):
                t = time_layer(w, timer, xw, 50 if w.M < 1024 else 20)
                print(json.dumps(layer_record(w, t)), flush=True)
        return

    w = HEADLINE
    extra = []
    light = [e for e in extra_workloads() if e.M < 1024]
    heavy = [e for e in extra_workloads() if e.M >= 1024]

    def record(rec):
        extra.append(rec)
        print(json.dumps({"progress": rec}), file=sys.stderr, flush=True)

    if not args.no_extra:
        for e in light:
            record(layer_record(e, time_layer(e, timer, xw, 50)))
        # the device's own read rate at the decode layers' byte counts (rotated buffers)
        for name, fw in (("llama3_8b_up_proj_M1", HEADLINE),
                         ("llama3_70b_gate_proj_M1", Workload("g", 8192, 28672, 1, 4, 128, False, "f16", "bf16", 0))):
            nb = algorithmic_bytes(fw.K, fw.N, fw.M, fw.bits, fw.gs, fw.desc_act)
            t = time_read_floor(nb, timer, xw, 50)
            rec = {"workload": f"read_floor_{name}_bytes", "bytes": nb, "us_per_call": t.pop("median_us"), **t}
            rec["TB_per_s"] = round(nb / (rec["us_per_call"] * 1e-6) / 1e12, 3)
            rec["frac_hbm"] = round(rec["TB_per_s"] * 1e3 / HBM_PEAK_GBS, 4)
            rec["note"] = "gptq_read_floor: a plain read of the same byte count, nothing else (context)"
            record(rec)
    # the headline: W warm-up calls, then exactly K timed calls, on a device the decode records above
    # have brought to its working clocks and before the compute-bound records below (timed after
    # them, the same call measured 8.2 us, batch median 8.8, against 7.6 - 7.75 us for the same
    # kernel earlier in that run)
    head = time_layer(w, timer, args.warmup, max(50, min(args.steps, 500)), steps=args.steps)
    if not args.no_extra:
        for e in heavy:
            record(layer_record(e, time_layer(e, timer, xw, 20)))
        # dense bf16 matmul of the prefill shape (hipBLASLt through torch): context for the MFMA path
        t = time_dense_mm(4096, 8192, 28672, timer, 10, 20)
        fl = 2.0 * 4096 * 8192 * 28672
        rec = {"workload": "dense_bf16_mm_4096x8192x28672", "us_per_call": t.pop("median_us"), **t}
        rec["TFLOP_per_s"] = round(fl / (rec["us_per_call"] * 1e-6) / 1e12, 1)
        rec["frac_mfma_bf16"] = round(rec["TFLOP_per_s"] / BF16_PEAK_TFLOPS, 4)
        rec["note"] = "torch.mm on dense bf16 operands of the prefill shape (context, not this method)"
        record(rec)
        # the step before the path: GPTQ on the GPU for the same 4096 x 14336 layer
        record(time_quantize(4096, 14336, 512, 4, 128, True))
    us = head["timed_us"]
    abytes = algorithmic_bytes(w.K, w.N, w.M, w.bits, w.gs, w.desc_act)
    achieved = abytes / (us * 1e-6) / 1e9
    print(json.dumps({"progress": {"headline_us": round(us, 3), **head}}), file=sys.stderr, flush=True)
    cpu = None if args.no_cpu else cpu_oracle_baseline(w)
    traffic = stored_traffic("skinny_" + w.label())
    line = {
        "metric": "GPTQ-W4A16 linear: us/call + achieved TB/s (M=1) and TFLOP/s (M=4096) vs roofline",
        "value": round(us, 3), "unit": "us/call", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 6), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic",
        "config": {"workload": w.label(), "K": w.K, "N": w.N, "M": w.M, "bits": w.bits, "group_size": w.gs,
                   "desc_act": w.desc_act, "handles_rotated": head["copies"]},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic["bytes_per_launch"] if traffic else None,
                     "algorithmic_bytes_per_launch": abytes, "profile": profile_of(w.label())},
        "headline_batches": {k: v for k, v in head.items() if k not in ("timed_us",)},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
