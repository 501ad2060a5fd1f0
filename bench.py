#!/usr/bin/env python3
"""Benchmark of the GPTQ weight-only quantized linear layer on one MI355X.

One step = one gptq_gemm call (the whole per-call path: dispatch, activation staging, packed
weight stream, in-register dequant, fp32 MFMA accumulation, epilogue) on the Llama-3-8B-shaped
MLP up projection (K=4096, N=14336, 4-bit, group 128, fp16, M=1).  The load-time repack is not
part of a step ("Kernel Backends Reference", pitfalls: do not time repacking as steady state).

Inputs are synthetic and seeded (gptq_inputs).  Every call streams its weights from HBM: calls
rotate over enough distinct repacked copies (>= 512 MiB) that the 256 MiB Infinity Cache cannot
serve them.  Timing: W warm-up calls, then exactly K calls between two HIP events on the stream
the kernels run on, with torch.cuda.synchronize() on both sides.

Prints ONE JSON line.  `value` is microseconds per call (lower is better); `roofline` reports the
dominant kernel's algorithmic bytes per launch / its average launch time against 8 TB/s; `extra`
holds the other workloads measured with the same protocol (not bench lines of their own);
`cpu_baseline` is the float64 CPU oracle timed on this host.
"""
from __future__ import annotations

import argparse
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
FAMILY_SOURCES = {"skinny": ["skinny_impl.h", "skinny.hip", "skinny_b4.hip"],
                  "tiled": ["tiled.hip"]}


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
    if the sources of the kernel's family are unchanged since they were taken."""
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
    return e.get("bytes_per_launch")


class Workload:
    def __init__(self, name, K, N, M, bits, gs, desc_act, sdt, xdt, seed, bias=False, fmt="gptq"):
        self.name, self.K, self.N, self.M, self.bits, self.gs = name, K, N, M, bits, gs
        self.desc_act, self.sdt, self.xdt, self.seed, self.bias = desc_act, sdt, xdt, seed, bias
        self.fmt = fmt   # checkpoint the layer is repacked from: "gptq" or "awq_gemm"

    def label(self):
        g = "g-1" if self.gs == -1 else f"g{self.gs}"
        return f"{self.name}_M{self.M}_b{self.bits}_{g}" + ("_actorder" if self.desc_act else "")


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


def time_calls(w: Workload, steps: int, warmup: int, copies=None, graph=False):
    """Average microseconds per gptq_gemm call, HIP events on the launch stream."""
    import numpy as np
    import torch
    import gptq_inputs as gi
    import weight_only_quantized_amd as wq
    wbytes = algorithmic_bytes(w.K, w.N, 0, w.bits, w.gs, w.desc_act)
    R = copies or max(1, math.ceil(ROTATE_BYTES / wbytes))
    L, hs = build_handles(w, R)
    lib = wq.load_library()
    dev = torch.device("cuda:0")
    tdt = torch.float16 if w.xdt == "f16" else torch.bfloat16
    xb = gi.make_x(w.M, w.K, w.xdt, seed=w.seed + 1)
    xs = [torch.from_numpy(xb.view(np.int16).copy()).to(dev).view(tdt) for _ in range(min(R, 4))]
    ys = [torch.empty((w.M, w.N), dtype=tdt, device=dev) for _ in range(min(R, 4))]
    need = hs[0].workspace_size(w.M, tdt)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    # graph capture needs a side stream (default priority); eager calls use the current stream
    stream = torch.cuda.Stream() if graph else torch.cuda.current_stream()
    sp = stream.cuda_stream
    xcode = 0 if w.xdt == "f16" else 1
    args = [(hs[i % R].ptr, xs[i % len(xs)].data_ptr(), ys[i % len(ys)].data_ptr()) for i in range(R * len(xs))]
    bias = None
    if w.bias:   # the layer's [N] bias in the scales' dtype, through gptq_gemm_bias
        bb = gi.make_bias(w.N, w.sdt, seed=w.seed + 2)
        bias = (torch.from_numpy(np.ascontiguousarray(bb, dtype=np.float32)) if w.sdt == "f32" else
                torch.from_numpy(bb.view(np.int16).copy())).to(dev)

    def call(i):
        h, x, y = args[i % len(args)]
        if bias is None:
            st = lib.gptq_gemm(h, x, w.M, xcode, y, ws.data_ptr(), ws.numel(), 0, sp)
        else:
            st = lib.gptq_gemm_bias(h, x, w.M, xcode, bias.data_ptr(), y, ws.data_ptr(), ws.numel(), 0, sp)
        if st:
            raise wq.GPTQError(st, "gptq_gemm", lib)

    with torch.cuda.stream(stream):
        for i in range(warmup):
            call(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(steps):
                call(i)
        with torch.cuda.stream(stream):
            g.replay()
            torch.cuda.synchronize()
            e0.record(stream)
            g.replay()
            e1.record(stream)
    else:
        e0.record(stream)
        for i in range(steps):
            call(i)
        e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    for h in hs:
        h.close()
    torch.cuda.synchronize()
    return us, R


def cpu_oracle_baseline(w: Workload, budget_s=20.0):
    """The float64 oracle as it stands, timed on this host on whole calls of the headline layer."""
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
    runs, t_total = 0, 0.0
    while runs < 1 or (t_total < budget_s and runs < 10):
        t0 = time.perf_counter()
        o.gemm(x, w.xdt, L.qweight, L.qzeros, L.scales, w.sdt, L.g_idx, w.bits)
        t_total += time.perf_counter() - t0
        runs += 1
        if t_total / runs * (runs + 1) > budget_s * 1.5:
            break
    return {"value": round(t_total / runs * 1e6, 1), "unit": "us/call", "cores": threads or os.cpu_count(),
            "kind": "oracle",
            "sample": f"{runs} whole call(s) of {w.label()} (unpack + float64 dequant + float64 matmul); "
                      f"host has {os.cpu_count()} logical CPUs, unpack/dequant run on one thread, the matmul "
                      f"on the BLAS pool"}


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
    # GPTQ_P planar checkpoints: 3-bit (its own runtime width) and 5-bit (run as 8-bit codes)
    for bits in (3, 5):
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--graph", action="store_true", help="replay the timed calls from one HIP graph")
    ap.add_argument("--no-extra", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only", default=None, help="time one extra workload (by label prefix) and exit")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before timing, run 3 plain device copies of this many MiB (a known-size kernel for "
                         "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE readings); outside the timed region")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the kernels run one GPU's share of a layer; no multi-GPU path)",
              file=sys.stderr)
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

    if args.only:
        for w in [HEADLINE] + extra_workloads():
            if w.label().startswith(args.only):
                steps = args.steps if w.M < 1024 else max(3, args.steps // 100)
                us, R = time_calls(w, steps, min(args.warmup, steps), graph=args.graph)
                print(json.dumps({"workload": w.label(), "us_per_call": round(us, 3), "copies": R}), flush=True)
        return

    w = HEADLINE
    us, R = time_calls(w, args.steps, args.warmup, graph=args.graph)
    abytes = algorithmic_bytes(w.K, w.N, w.M, w.bits, w.gs, w.desc_act)
    achieved = abytes / (us * 1e-6) / 1e9
    extra = []
    if not args.no_extra:
        for e in extra_workloads():
            steps = args.steps if e.M < 1024 else max(3, args.steps // 200)
            eus, eR = time_calls(e, steps, min(args.warmup, steps), graph=args.graph)
            rec = {"workload": e.label(), "us_per_call": round(eus, 3), "copies": eR}
            b = algorithmic_bytes(e.K, e.N, e.M, e.bits, e.gs, e.desc_act, scale_bytes=2) + (2 * e.N if e.bias else 0)
            rec["algorithmic_bytes"] = b
            rec["TB_per_s"] = round(b / (eus * 1e-6) / 1e12, 3)
            rec["frac_hbm"] = round(b / (eus * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
            if e.M >= 1024:
                fl = 2.0 * e.M * e.N * e.K
                tf = fl / (eus * 1e-6) / 1e12
                rec["TFLOP_per_s"] = round(tf, 1)
                rec["frac_mfma_bf16"] = round(tf / BF16_PEAK_TFLOPS, 4)
                # whole call (the fp16 copy of x plus the GEMM), against the dense 16-bit MFMA peak
                rec["roofline"] = {"bound": "mfma", "achieved": round(tf, 1), "peak": BF16_PEAK_TFLOPS,
                                   "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                                   "traffic": stored_traffic("tiled_" + e.label()),
                                   "kernel": "gq::tiled_kernel<4,1,16,2,4,8,1>", "algorithmic_flops_per_launch": fl}
            extra.append(rec)
            print(json.dumps({"progress": rec}), file=sys.stderr, flush=True)
        # the step before the path: GPTQ on the GPU for the same 4096 x 14336 layer
        rec = time_quantize(4096, 14336, 512, 4, 128, True)
        extra.append(rec)
        print(json.dumps({"progress": rec}), file=sys.stderr, flush=True)
    cpu = None if args.no_cpu else cpu_oracle_baseline(w)
    line = {
        "metric": "GPTQ-W4A16 linear: us/call + achieved TB/s (M=1) and TFLOP/s (M=4096) vs roofline",
        "value": round(us, 3), "unit": "us/call", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 6), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic",
        "config": {"workload": w.label(), "K": w.K, "N": w.N, "M": w.M, "bits": w.bits, "group_size": w.gs,
                   "desc_act": w.desc_act, "handles_rotated": R, "graph": bool(args.graph)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": stored_traffic("skinny_" + w.label()),
                     "kernel": "gq::skinny_kernel<4,0,1,1,2,4,1,4,16,0,0>", "algorithmic_bytes_per_launch": abytes},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
