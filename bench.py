"""Benchmark of the W4A16 + gated-EC linear layer on one MI355X.

Default workload (C2, decode): K = N = 4096 (7B-class attention projection),
int4 asymmetric per-channel weights with bf16 scales, EC rank 32 with a soft
gate.  One step is one pass of the layer for each decode batch M in {1, 4, 8}
(three calls of spear_w4_linear, each one fused launch).  The weights and EC
factors rotate over 64 device copies (538 MB, more than twice the 256 MB
Infinity Cache) so every call streams them from HBM.  The timed steps are
captured once in a HIP graph and replayed, so host launch overhead stays out of
the timed region; the time is taken with HIP events on the launch stream.

`value` is algorithmic bytes moved per second (packed weights, scales, zero
points, EC factors and gate weights, activations in, fp32 outputs out), in GB/s.
The line also carries the plain-W4 time of the same steps (EC overhead), the
roofline of the decode kernel and the CPU oracle timed on a bounded sample.

--workload c1 times the small layer (M = 16, K = N = 1024, rank 16; launch
latency bound, reported in microseconds a call and GB/s); --workload c4 times
the prefill configuration instead (M = N = K = 4096,
TFLOP/s); --workload c3 the MLP up-projection at M = 64 (K = 4096, N = 14336,
rank 64, hard gate); --workload c5 a 28-layer stack of a 1.5B-class decoder's
seven linears (ECs on 4 layers) at --c5-m tokens, reporting the stack time
and the EC share.  None of these is the default line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A16+gated-EC linear: decode GB/s, prefill TFLOP/s, EC overhead vs plain W4"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="c2", choices=["c1", "c2", "c3", "c4", "c5"])
    p.add_argument("--c5-m", type=int, default=1, choices=[1, 16, 128, 2048],
                   help="tokens per call of the C5 stack")
    p.add_argument("--copies", type=int, default=64)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="approximate CPU time budget of the oracle sample")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain device copy of known size (for counter scaling)")
    return p.parse_args()


def profiled_traffic():
    """HBM bytes per fused decode launch from the committed rocprofv3 counter
    record (FETCH_SIZE + WRITE_SIZE, calibrated on a device copy), or None when
    the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "decode_fused_c2_hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    h = hashlib.sha256()
    for name in ("decode.hip", "api.hip", "spear_internal.hpp"):
        with open(os.path.join(ROOT, "quantized_gemm_w4a16_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return rec.get("traffic_bytes_per_launch") if h.hexdigest() == rec.get("source_sha256") else None


def dev(a, torch):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def layer_bytes(M, N, K, r, asym, out_bytes=4):
    w = N * K / 2 + 4 * N + (N if asym else 0)
    ec = 2 * K * r + 2 * r * N + 2 * K if r else 0
    io = 2 * M * K + out_bytes * M * N
    return w, ec, io


def build_copies(d, copies, torch, sp):
    codes = dev(d["codes"], torch)
    e = d["ec"]
    ws, ecs = [], []
    for _ in range(copies):
        packed = sp.spear_pack_w4(codes, d["kind"])
        ws.append(sp.W4(packed, dev(d["scales"], torch),
                        dev(d["zeros"], torch) if d["zeros"] is not None else None,
                        d["N"], d["K"]))
        ecs.append(sp.EC(dev(e["A"], torch), dev(e["B"], torch), dev(e["w_g"], torch),
                         e["b"], e["tau"], e["hard"]))
    del codes
    return ws, ecs


def time_graph(torch, record_steps, steps):
    """Capture `steps` steps in one graph, replay once untimed, then time one replay."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            record_steps(steps)
    torch.cuda.current_stream().wait_stream(s)
    g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    g.replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1), g


def cpu_baseline_c2(Ms, budget_s):
    """The oracle (never tuned for speed) on C2 layers, whole layers, until the
    budget is used; rate in the same unit as the GPU value."""
    import oracle
    from quantized_gemm_w4a16_amd import inputs as gen
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    done_bytes, t_used, calls = 0.0, 0.0, 0
    cached = {}
    while t_used < budget_s and calls < 5000:
        M = Ms[calls % len(Ms)]
        if M not in cached:
            d = gen.make(2, M=M)
            packed, _ = oracle.pack_w4(d["codes"], d["kind"])
            cached[M] = (d, packed)
        d, packed = cached[M]
        t = time.perf_counter()
        oracle.w4_linear(d["x"], packed, d["scales"], d["zeros"], d["ec"])
        t_used += time.perf_counter() - t
        w, ec, io = layer_bytes(M, d["N"], d["K"], d["ec"]["r"], True)
        done_bytes += w + ec + io
        calls += 1
    return {"value": round(done_bytes / t_used / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{calls} whole C2 layer calls cycling M in {Ms} "
                      f"({t_used:.1f} s of oracle time, fp64 sums, {threads} OpenMP threads)"}


def copy_calibration(torch):
    n = 256 << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    return n


def run_c2(args, torch, sp, gen):
    Ms = (1, 4, 8)
    d0 = gen.make(2, M=1)
    N, K, r = d0["N"], d0["K"], d0["ec"]["r"]
    R = args.copies
    ws, ecs = build_copies(d0, R, torch, sp)
    xs = {M: dev(gen.make(2, M=M)["x"], torch) if M > 1 else dev(d0["x"], torch) for M in Ms}
    ys = {M: torch.empty((M, N), dtype=torch.float32, device="cuda") for M in Ms}
    wsp = sp.new_workspace(max(Ms), N, K, r)
    for M in Ms:
        assert wsp.numel() >= sp.spear_w4_linear_workspace_size(M, N, K, r)

    def steps_fn(use_ec):
        def record(n):
            for i in range(n):
                c = i % R
                for M in Ms:
                    sp.spear_w4_linear(xs[M], ws[c], ecs[c] if use_ec else None, y=ys[M],
                                       workspace=wsp, path=sp.PATH_AUTO)
        return record

    for i in range(args.warmup):
        steps_fn(True)(1)
    torch.cuda.synchronize()
    t_ec, _ = time_graph(torch, steps_fn(True), args.steps)
    t_plain, _ = time_graph(torch, steps_fn(False), args.steps)
    assert sp.spear_workspace_timeouts(wsp) == 0

    per_step_bytes = 0.0
    per_step_plain = 0.0
    for M in Ms:
        w, ec, io = layer_bytes(M, N, K, r, True)
        per_step_bytes += w + ec + io
        per_step_plain += w + io
    ms_step = t_ec / args.steps
    launches = len(Ms)
    achieved = (per_step_bytes / launches) / (ms_step / launches * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(per_step_bytes / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "C2 decode GEMV: M in {1,4,8} per step, K=N=4096, int4 "
                               "asymmetric per-channel (bf16 scales, zero points 6..9), "
                               "bf16 activations N(0,1), EC rank 32 soft gate, fp32 output",
                   "rotating_weight_copies": R, "launches_per_step": launches,
                   "timing": "HIP graph replay, HIP events on the launch stream"},
        "ec_overhead": round(t_ec / t_plain - 1.0, 4),
        "plain_ms_per_step": round(t_plain / args.steps, 6),
        "plain_GBps": round(per_step_plain / (t_plain / args.steps * 1e-3) / 1e9, 2),
        "us_per_launch": round(ms_step / launches * 1e3, 3),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": profiled_traffic(),
                     "traffic_unit": "bytes per launch (profiles/decode_fused_c2_hbm_traffic.md)",
                     "kernel": "decode_kernel<1,1,*,*> (fused EC, fp32 out)",
                     "bytes_per_launch": round(per_step_bytes / launches)},
    }
    return out


def run_c4(args, torch, sp, gen):
    d = gen.make(4)
    M, N, K, r = d["M"], d["N"], d["K"], d["ec"]["r"]
    R = max(2, min(args.copies, 4))
    ws, ecs = build_copies(d, R, torch, sp)
    x = dev(d["x"], torch)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    wsp = sp.new_workspace(M, N, K, r)

    def steps_fn(use_ec):
        def record(n):
            for i in range(n):
                sp.spear_w4_linear(x, ws[i % R], ecs[i % R] if use_ec else None, y=y,
                                   workspace=wsp)
        return record

    for _ in range(args.warmup):
        steps_fn(True)(1)
    torch.cuda.synchronize()
    t_ec, _ = time_graph(torch, steps_fn(True), args.steps)
    t_plain, _ = time_graph(torch, steps_fn(False), args.steps)
    flops = 2.0 * M * N * K
    ec_flops = 2.0 * M * K * r + 2.0 * M * r * N
    ms = t_ec / args.steps
    tf = (flops + ec_flops) / (ms * 1e-3) / 1e12
    tf_plain = flops / (t_plain / args.steps * 1e-3) / 1e12
    return {
        "metric": METRIC, "value": round(tf, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "C4 prefill: M=N=K=4096, int4 symmetric per-channel, "
                               "Student-t(4) activations, EC rank 32 soft gate, fp32 output"},
        "ec_overhead": round(t_ec / t_plain - 1.0, 4),
        "plain_TFLOPs": round(tf_plain, 2),
        "roofline": {"bound": "mfma", "achieved": round(tf_plain, 2), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf_plain / BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "kernel": "gemm2_kernel<2,4,0,0,1,1,4,4,1> (plain, whole K)"},
    }


def run_c1(args, torch, sp, gen):
    """C1: M = 16, K = N = 1024, symmetric codes with fp32 scales, EC rank 16
    with the soft gate.  One call moves about 0.6 MB, so it is bound by launch
    latency; the weights rotate over 512 copies (more than the Infinity Cache)."""
    d = gen.make(1)
    M, N, K, r = d["M"], d["N"], d["K"], d["ec"]["r"]
    R = max(2, min(args.copies * 8, 512))
    ws, ecs = build_copies(d, R, torch, sp)
    x = dev(d["x"], torch)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    wsp = sp.new_workspace(M, N, K, r)

    def steps_fn(use_ec):
        def record(n):
            for i in range(n):
                sp.spear_w4_linear(x, ws[i % R], ecs[i % R] if use_ec else None, y=y,
                                   workspace=wsp)
        return record

    for _ in range(args.warmup):
        steps_fn(True)(1)
    torch.cuda.synchronize()
    t_ec, _ = time_graph(torch, steps_fn(True), args.steps)
    t_plain, _ = time_graph(torch, steps_fn(False), args.steps)
    assert sp.spear_workspace_timeouts(wsp) == 0
    w, ecb, io = layer_bytes(M, N, K, r, False)
    ms = t_ec / args.steps
    gbs = (w + ecb + io) / (ms * 1e-3) / 1e9
    return {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "C1 small layer: M=16, K=N=1024, int4 symmetric per-channel "
                               "(fp32 scales), bf16 activations N(0,1), EC rank 16 soft gate, "
                               "fp32 output",
                   "rotating_weight_copies": R},
        "us_per_call": round(ms * 1e3, 3),
        "plain_us_per_call": round(t_plain / args.steps * 1e3, 3),
        "ec_overhead": round(t_ec / t_plain - 1.0, 4),
        "plain_GBps": round((w + io) / (t_plain / args.steps * 1e-3) / 1e9, 2),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "decode_kernel<1,1,2,0> (fused EC, 16 tokens)"},
    }


def run_c3(args, torch, sp, gen):
    """C3: M = 64, K = 4096, N = 14336, EC rank 64 with the hard gate (about 40 %
    of tokens skip).  Near the ridge: GB/s and TFLOP/s both reported."""
    d = gen.make(3)
    M, N, K, r = d["M"], d["N"], d["K"], d["ec"]["r"]
    R = max(2, min(args.copies, 16))                     # 16 x 29 MB > 2 x the Infinity Cache
    ws, ecs = build_copies(d, R, torch, sp)
    x = dev(d["x"], torch)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    wsp = sp.new_workspace(M, N, K, r)

    def steps_fn(use_ec):
        def record(n):
            for i in range(n):
                sp.spear_w4_linear(x, ws[i % R], ecs[i % R] if use_ec else None, y=y,
                                   workspace=wsp)
        return record

    for _ in range(args.warmup):
        steps_fn(True)(1)
    torch.cuda.synchronize()
    t_ec, _ = time_graph(torch, steps_fn(True), args.steps)
    t_plain, _ = time_graph(torch, steps_fn(False), args.steps)
    w, ecb, io = layer_bytes(M, N, K, r, True)
    ms = t_ec / args.steps
    gbs = (w + ecb + io) / (ms * 1e-3) / 1e9
    flops = 2.0 * M * N * K + 2.0 * M * K * r + 2.0 * M * r * N
    return {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "C3 MLP up-projection: M=64, K=4096, N=14336, int4 asymmetric "
                               "per-channel, x N(0,1) with 1% of channels x20, EC rank 64, "
                               "hard gate (~40% of tokens skip), fp32 output",
                   "rotating_weight_copies": R},
        "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 2),
        "ec_overhead": round(t_ec / t_plain - 1.0, 4),
        "plain_GBps": round((w + io) / (t_plain / args.steps * 1e-3) / 1e9, 2),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "gemm2_kernel<2,2,0,2,1,2,2,2,1> (64 x 64 tiles over all of K, EC pre-pass as its first blocks)"},
    }


def run_c5(args, torch, sp, gen):
    """C5: the stack of 28 layers x 7 linears (q, k, v, o 2048 -> 2048; gate, up
    2048 -> 8192; down 8192 -> 2048) with ECs on 4 seeded layers, one call per
    linear at M tokens, each layer with its own weights (896 MB packed, so the
    stack streams from HBM).  One step = the whole stack; EC share = the stack
    time the ECs add, over the compensated stack time."""
    M = args.c5_m
    layers = []
    ec_layers = set(gen.c5_ec_layers())
    for layer in range(gen.C5_LAYERS):
        for lin in gen.C5_LINEARS:
            d = gen.make_c5(layer, lin, M)
            codes = dev(d["codes"], torch)
            w = sp.W4(sp.spear_pack_w4(codes, d["kind"]), dev(d["scales"], torch),
                      dev(d["zeros"], torch), d["N"], d["K"])
            del codes
            e = d["ec"]
            ec = (sp.EC(dev(e["A"], torch), dev(e["B"], torch), dev(e["w_g"], torch), e["b"],
                        e["tau"], e["hard"]) if e is not None else None)
            layers.append((d["N"], d["K"], w, ec, e["r"] if e is not None else 0))
    xs = {K: dev(gen.make_c5(0, "down" if K == gen.C5_FF else "q", M)["x"], torch)
          for K in (gen.C5_D, gen.C5_FF)}
    ys = {N: torch.empty((M, N), dtype=torch.float32, device="cuda") for N in (gen.C5_D, gen.C5_FF)}
    # one workspace for every layer: the largest any of their shapes needs
    need = max(sp.spear_w4_linear_workspace_size(M, N, K, r) for (N, K, _, _, r) in layers)
    wsp = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda")

    def steps_fn(use_ec):
        def record(n):
            for _ in range(n):
                for (N, K, w, ec, r) in layers:
                    sp.spear_w4_linear(xs[K], w, ec if use_ec else None, y=ys[N], workspace=wsp)
        return record

    for _ in range(args.warmup):
        steps_fn(True)(1)
    torch.cuda.synchronize()
    t_ec, _ = time_graph(torch, steps_fn(True), args.steps)
    t_plain, _ = time_graph(torch, steps_fn(False), args.steps)
    assert sp.spear_workspace_timeouts(wsp) == 0
    byts = sum(sum(layer_bytes(M, N, K, r, True)) for (N, K, w, ec, r) in layers)
    flops = sum(2.0 * M * N * K + (2.0 * M * K * r + 2.0 * M * r * N if r else 0.0)
                for (N, K, w, ec, r) in layers)
    ms = t_ec / args.steps
    big = M >= 128
    val = flops / (ms * 1e-3) / 1e12 if big else byts / (ms * 1e-3) / 1e9
    unit = "TFLOP/s" if big else "GB/s"
    peak = BF16_PEAK_TFLOPS if big else HBM_PEAK_GBS
    return {
        "metric": METRIC, "value": round(val, 2), "unit": unit, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"C5 decoder stack: 28 layers x (q,k,v,o 2048->2048, gate,up "
                               f"2048->8192, down 8192->2048), M={M}, int4 asymmetric "
                               f"per-channel, ECs rank 32 hard gate on layers "
                               f"{sorted(ec_layers)}, fp32 output",
                   "linears_per_step": len(layers)},
        "stack_ms": round(ms, 4),
        "plain_stack_ms": round(t_plain / args.steps, 4),
        "ec_share": round((t_ec - t_plain) / t_ec, 4),
        "ec_overhead": round(t_ec / t_plain - 1.0, 4),
        "roofline": {"bound": "mfma" if big else "hbm", "achieved": round(val, 2), "peak": peak,
                     "unit": unit, "frac": round(val / peak, 4), "traffic": None,
                     "kernel": "whole stack (all kernels)"},
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the layer is "
              "benchmarked at one GPU's shard shape.", file=sys.stderr)
        sys.exit(2)
    import torch
    from quantized_gemm_w4a16_amd import inputs as gen
    from quantized_gemm_w4a16_amd import spear as sp
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    sp.load()
    run = {"c1": run_c1, "c2": run_c2, "c3": run_c3, "c4": run_c4, "c5": run_c5}[args.workload]
    out = run(args, torch, sp, gen)
    if args.copy_calibration:
        out["copy_calibration_bytes"] = copy_calibration(torch)
    if args.workload == "c2" and not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_c2((1, 4, 8), args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
