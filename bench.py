#!/usr/bin/env python3
"""Throughput of the fused conv2d path on one MI355X.

One step is one forward pass of the ResNet-18-D-style backbone (N=4, 640x640x3,
NHWC bf16: 22 fused convs, 1 max pool, 3 average pools; 134.09 GFLOP), which
runs every part of the path: the low-Cin stem kernel, the matrix-core implicit
GEMM for 3x3 (stride 1 and 2) and 1x1 convs with bias, ReLU and the residual
fused in the epilogue, and both pools. All inputs, weights and output buffers
are resident in device memory before timing starts. The metric is conv TFLOP/s
= sum over convs of 2*N*OH*OW*Cout*Cin*kh*kw, divided by the step time.

Prints one JSON line. Besides the headline number it carries the roofline of
the dominant kernel (per-kernel durations from HIP events on the launch stream)
and the CPU oracle's throughput on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16/f16 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--mode", choices=["graph", "eager"], default="graph",
                   help="replay one captured HIP graph per step, or launch eagerly")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--layer-reps", type=int, default=10)
    p.add_argument("--layers-out", default=None, help="write per-layer timings (JSON) here")
    return p.parse_args()


class Net:
    """The backbone's layers with preallocated device buffers and prebuilt C-ABI arguments."""

    def __init__(self, work, dev):
        import torch

        import conv2d_bias_activation_amd as c2d

        self.c2d = c2d
        self.lib = c2d._load()
        self.work = work
        self.t = {"x": work.x.to(dev)}
        self.layers = []
        dt = c2d.DTYPE_BF16
        for spec in work.layers:
            src = self.t[spec.src]
            n, h, w, c = src.shape
            if hasattr(spec, "cin"):
                oh = c2d.out_dim(h, spec.k, spec.stride, spec.pad)
                ow = c2d.out_dim(w, spec.k, spec.stride, spec.pad)
                out = torch.empty((n, oh, ow, spec.cout), dtype=src.dtype, device=dev)
                wdev = spec.w.to(dev)
                bdev = spec.bias.to(dev)
                res = self.t[spec.res] if spec.res else None
                act = {"none": 0, "relu": 1, "silu": 2, "prelu": 3}[spec.act]
                act |= c2d.RES_BEFORE_ACT if spec.res_before_act else 0
                keep = (wdev, bdev)
                args = [ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(wdev.data_ptr()),
                        ctypes.c_void_p(bdev.data_ptr()), None,
                        ctypes.c_void_p(res.data_ptr()) if res is not None else None,
                        ctypes.c_void_p(out.data_ptr()), n, h, w, c, spec.cout, spec.k, spec.k,
                        spec.stride, spec.pad, act, c2d.LAYOUT_NHWC, dt]
                flops = 2 * n * oh * ow * spec.cout * c * spec.k * spec.k
                nbytes = 2 * (src.numel() + spec.w.numel() + out.numel() +
                              (res.numel() if res is not None else 0)) + 4 * spec.cout
                plan = c2d.plan(n, h, w, c, spec.cout, spec.k, spec.k, spec.stride, spec.pad, act,
                                c2d.LAYOUT_NHWC, dt)
                self.layers.append(dict(name=spec.name, fn=self.lib.conv2d_fused, args=args,
                                        flops=flops, bytes=nbytes, plan=plan, keep=keep))
            else:
                if spec.kind == "max":
                    oh, ow, fn = (h - 1) // 2 + 1, (w - 1) // 2 + 1, self.lib.maxpool3x3s2
                    plan = "maxpool3x3s2"
                else:
                    oh, ow, fn = h // 2, w // 2, self.lib.avgpool2x2
                    plan = "avgpool2x2"
                out = torch.empty((n, oh, ow, c), dtype=src.dtype, device=dev)
                args = [ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(out.data_ptr()), n, h, w,
                        c, c2d.LAYOUT_NHWC, dt]
                self.layers.append(dict(name=spec.name, fn=fn, args=args, flops=0,
                                        bytes=2 * (src.numel() + out.numel()), plan=plan, keep=()))
            self.t[spec.out] = out
        self.flops = sum(L["flops"] for L in self.layers)
        self.out_name = work.layers[-1].out

    def run_layer(self, L, stream_handle):
        rc = L["fn"](*L["args"], stream_handle)
        if rc != 0:
            raise RuntimeError(f"{L['name']}: {self.c2d.last_error()}")

    def step(self, stream):
        h = ctypes.c_void_p(stream.cuda_stream)
        for L in self.layers:
            self.run_layer(L, h)


def prefill(torch, ms=20.0):
    """Keep the GPU busy while the host queues work, so the timed region is GPU time."""
    torch.cuda._sleep(int(ms * 1e-3 * 2.4e9))


def time_steps(torch, net, steps, warmup, mode):
    stream = torch.cuda.current_stream()
    graph = None
    if mode == "graph":
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for _ in range(2):
                net.step(side)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            net.step(torch.cuda.current_stream())
        torch.cuda.synchronize()
    run = (lambda: graph.replay()) if graph is not None else (lambda: net.step(stream))
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    prefill(torch, ms=min(200.0, 2.0 * steps))
    e0.record(stream)
    for _ in range(steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, graph


def time_layers(torch, net, reps):
    """Per-layer average durations (ms) from events between back-to-back launches."""
    stream = torch.cuda.current_stream()
    h = ctypes.c_void_p(stream.cuda_stream)
    n = len(net.layers)
    tot = [0.0] * n
    for _ in range(reps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        prefill(torch, ms=10.0)
        ev[0].record(stream)
        for i, L in enumerate(net.layers):
            net.run_layer(L, h)
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        for i in range(n):
            tot[i] += ev[i].elapsed_time(ev[i + 1])
    return [t / reps for t in tot]


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "conv2d_bias_activation_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp")):
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(plan, launches_bytes):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it was taken on
    the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash():
        return None
    k = rec.get("kernels", {}).get(plan)
    if not k:
        return None
    return k.get("bytes_per_launch")


def cpu_baseline(work):
    """The oracle (fp64 direct loops, all host threads) on one image of the same backbone."""
    import numpy as np

    import oracle
    import workloads as wl

    one = wl.conv5_resnet18d(n=1)
    t = {"x": one.x.to(__import__("torch").float64).numpy()}
    flops = 0
    t0 = time.perf_counter()
    for spec in one.layers:
        src = t[spec.src]
        if isinstance(spec, wl.ConvSpec):
            r = t[spec.res] if spec.res else None
            y = oracle.conv2d(src, spec.w.double().numpy(), spec.bias.double().numpy(), None, r,
                              stride=spec.stride, pad=spec.pad, act=spec.act,
                              res_before_act=spec.res_before_act)
            n, h, w, c = src.shape
            flops += 2 * n * y.shape[1] * y.shape[2] * spec.cout * c * spec.k * spec.k
            t[spec.out] = oracle.quantize(y, "bf16")
        elif spec.kind == "max":
            t[spec.out] = oracle.maxpool3x3s2(src)
        else:
            t[spec.out] = oracle.quantize(oracle.avgpool2x2(src).astype(np.float64), "bf16")
    dt = time.perf_counter() - t0
    return dict(value=round(flops / dt / 1e12, 6), unit="TFLOP/s", cores=oracle.threads(),
                kind="oracle",
                sample=f"one of the 4 images: full 22-conv forward in fp64 ({flops / 1e9:.2f} GFLOP, "
                       f"{dt:.1f} s)")


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; multi-GPU runs are not "
                                   "part of this build", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    work = wl.conv5_resnet18d()
    net = Net(work, dev)
    ms, graph = time_steps(torch, net, args.steps, args.warmup, args.mode)
    value = net.flops / (ms * 1e-3) / 1e12

    layer_ms = time_layers(torch, net, args.layer_reps)
    groups = {}
    for L, t in zip(net.layers, layer_ms):
        g = groups.setdefault(L["plan"], dict(ms=0.0, flops=0, bytes=0, launches=0))
        g["ms"] += t
        g["flops"] += L["flops"]
        g["bytes"] += L["bytes"]
        g["launches"] += 1
    dom_plan = max(groups, key=lambda k: groups[k]["ms"])
    g = groups[dom_plan]
    avg_ms = g["ms"] / g["launches"]
    if g["flops"] > 0:
        achieved = g["flops"] / g["launches"] / (avg_ms * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 2), peak=PEAK_BF16_TFLOPS,
                    unit="TFLOP/s", frac=round(achieved / PEAK_BF16_TFLOPS, 4))
    else:
        achieved = g["bytes"] / g["launches"] / (avg_ms * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=round(achieved / PEAK_HBM_GBS, 4))
    roof["traffic"] = measured_traffic(dom_plan, None)
    roof["kernel"] = dom_plan
    roof["avg_launch_us"] = round(avg_ms * 1e3, 2)
    roof["launches_per_step"] = g["launches"]

    if args.layers_out:
        rows = []
        for L, t in zip(net.layers, layer_ms):
            rows.append(dict(name=L["name"], plan=L["plan"], us=round(t * 1e3, 2),
                             tflops=round(L["flops"] / (t * 1e-3) / 1e12, 1) if L["flops"] else None,
                             gbs=round(L["bytes"] / (t * 1e-3) / 1e9, 1),
                             mfma_frac=round(L["flops"] / (t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
                             if L["flops"] else None,
                             hbm_frac=round(L["bytes"] / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)))
        os.makedirs(os.path.dirname(os.path.abspath(args.layers_out)), exist_ok=True)
        with open(args.layers_out, "w") as f:
            json.dump(dict(step_ms=ms, sum_layer_ms=sum(layer_ms), layers=rows), f, indent=1)

    cpu = None if args.no_cpu_baseline else cpu_baseline(work)
    line = {
        "metric": "conv TFLOP/s (2*N*OH*OW*Cout*Cin*kh*kw) and % of MFMA/HBM roofline, 1 GPU",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded PCG64: x~U[0,1] image, He-normal weights, bias~U[-0.1,0.1])",
        "config": {"workload": "resnet18d_backbone_4x640x640_nhwc_bf16", "global_batch": 4,
                   "image": "640x640x3", "convs": 22, "pools": 4, "gflop_per_step": round(net.flops / 1e9, 3),
                   "launch": args.mode},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
