"""Benchmark of the W4A16 + gated-EC linear layer on one MI355X.

Default run (the JSON line's `value`): workload C2, decode.  K = N = 4096
(7B-class attention projection), int4 asymmetric per-channel weights with bf16
scales, EC rank 32 with a soft gate.  One step is one pass of the layer for each
decode batch M in {1, 4, 8} (three calls of spear_w4_linear, each one fused
launch).  The weights and EC factors rotate over 64 device copies (538 MB, more
than twice the 256 MB Infinity Cache) so every call streams them from HBM.  The
K timed steps are captured once in a HIP graph; the graph is replayed
`--replays` times (each replay exactly K steps, bracketed by synchronisation and
timed with HIP events on the launch stream) and the median replay gives
`ms_per_step`, with p10 / p90 beside it.  `value` is algorithmic bytes moved per
second (packed weights, scales, zero points, EC factors and gate weights,
activations in, fp32 outputs out), in GB/s.

The same line also carries:
  * the plain-W4 time of the same steps (EC overhead), and per M the average
    launch time of the fused and the plain decode kernel (one graph per M);
  * `roofline` of the fused decode kernel against 8 TB/s, plus the rate of a
    plain streaming read of the same 64 rotating weight buffers (the same-size
    read floor, `stream_floor_GBps`) and of one 1 GiB buffer
    (`stream_floor_1GiB_GBps`), and the rate on the packed weights plus the EC
    factors alone (`achieved_weights_ec_GBps`, the spec's headline count);
  * `prefill`: workload C4 (M = N = K = 4096, Student-t activations, EC rank 32
    soft gate): TFLOP/s with and without the EC, the EC overhead, the plain
    GEMM's fraction of the 2.5 PFLOP/s bf16 peak, and the CPU oracle on a
    sample of C4 outputs;
  * `cpu_baseline`: the CPU oracle on whole C2 layer calls.

--workload c1|c3|c4|c5 times one other workload alone, same JSON contract
(C1: M = 16, K = N = 1024, launch-latency bound; C3: M = 64, K = 4096,
N = 14336, rank 64, hard gate; C4: prefill; C5: a 28-layer stack of a
1.5B-class decoder's seven linears with ECs on 4 layers at --c5-m tokens).
--workload slo measures the kernel-latency table of the C5 stack's linear
kinds (2048 -> 2048, 2048 -> 8192, 8192 -> 2048, each with and without its EC)
at token counts 1 .. 4096, then runs a seeded synthetic request trace through
continuous batching with the native chunk picker against fixed chunk sizes.
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
    p.add_argument("--replays", type=int, default=7,
                   help="timed replays of the K-step graph (median, p10, p90 reported)")
    p.add_argument("--no-prefill", action="store_true",
                   help="leave the C4 prefill object out of the default C2 line")
    p.add_argument("--prefill-steps", type=int, default=20,
                   help="layer calls per replay of the C4 prefill graph in the default line")
    p.add_argument("--workload", default="c2", choices=["c1", "c2", "c3", "c4", "c5", "slo"])
    p.add_argument("--lut-out", default="",
                   help="slo workload: also write the measured latency table to this JSON file")
    p.add_argument("--c5-m", type=int, default=1, choices=[1, 16, 128, 2048],
                   help="tokens per call of the C5 stack")
    p.add_argument("--copies", type=int, default=64)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="approximate CPU time budget of each oracle sample")
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


def time_graph(torch, record_steps, steps, replays):
    """Capture `steps` steps in one graph, replay it once untimed, then time
    `replays` replays (each exactly `steps` steps, synchronised on both sides,
    HIP events on the replay stream).  -> dict of ms per step: median, p10, p90,
    and every replay."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            record_steps(steps)
    torch.cuda.current_stream().wait_stream(s)
    g.replay()
    torch.cuda.synchronize()
    per = []
    for _ in range(max(1, replays)):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        g.replay()
        t1.record()
        torch.cuda.synchronize()
        per.append(t0.elapsed_time(t1) / steps)
    a = np.array(per)
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90)), "all": [round(v, 6) for v in per]}


def stats_ms(t, nd=6):
    return {"replays": len(t["all"]), "median_ms_per_step": round(t["median"], nd),
            "p10_ms_per_step": round(t["p10"], nd), "p90_ms_per_step": round(t["p90"], nd)}


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


def cpu_baseline_c4(budget_s):
    """The oracle on sampled outputs of the C4 prefill layer (whole rows of the
    fp64 dot products, the gate and the EC of each sampled token), until the
    budget is used.  Rate: algorithmic flops of the sampled outputs (2 K for the
    main term and 2 r for the EC up-projection per output, plus 2 K for the gate
    and 2 K r for the EC down-projection per distinct token) per second."""
    import oracle
    from quantized_gemm_w4a16_amd import inputs as gen
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    d = gen.make(4)
    packed, _ = oracle.pack_w4(d["codes"], d["kind"])
    M, N, K, r = d["M"], d["N"], d["K"], d["ec"]["r"]
    rng = np.random.default_rng(404)
    flops, t_used, outs = 0.0, 0.0, 0
    S = 4096
    while t_used < budget_s and outs < 50_000_000:
        m = rng.integers(0, M, 64)
        ms = np.repeat(m, S // 64)
        ns = rng.integers(0, N, S)
        t = time.perf_counter()
        oracle.w4_linear_sampled(d["x"], packed, d["scales"], d["zeros"], d["ec"], ms, ns)
        t_used += time.perf_counter() - t
        flops += S * (2.0 * K + 2.0 * r) + len(np.unique(m)) * (2.0 * K + 2.0 * K * r)
        outs += S
    return {"value": round(flops / t_used / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{outs} sampled C4 outputs (64 tokens x {S // 64} channels per batch; "
                      f"{t_used:.1f} s of oracle time, fp64 sums, {threads} OpenMP threads)"}


def stream_floor(torch, sp, bufs, steps, replays):
    """Plain streaming read of the rotating buffers, one launch per buffer as
    the layer does: GB/s and the average microseconds per buffer."""
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    nbytes = bufs[0].numel() * bufs[0].element_size()

    def record(n):
        for i in range(n):
            sp.spear_stream_read(bufs[i % len(bufs)], sink)
    t = time_graph(torch, record, steps, replays)
    return nbytes / (t["median"] * 1e-3) / 1e9, t["median"] * 1e3, nbytes


def stream_floor_large(torch, sp, nbytes=1 << 30, replays=5):
    """The same read over one 1 GiB buffer: the rate a long stream reaches."""
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")

    def record(n):
        for _ in range(n):
            sp.spear_stream_read(buf, sink)
    t = time_graph(torch, record, 1, replays)
    del buf
    return nbytes / (t["median"] * 1e-3) / 1e9


def launch_floor(torch, sp, replays, launches=200):
    """Fixed cost of one dependent launch in a captured graph: back-to-back
    launches of the library's read kernel over 16 KiB (one workgroup), in
    microseconds a launch."""
    buf = torch.ones(16384, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")

    def record(n):
        for _ in range(n):
            sp.spear_stream_read(buf, sink)
    t = time_graph(torch, record, launches, replays)
    return t["median"] * 1e3


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

    def steps_fn(use_ec, only=None):
        def record(n):
            for i in range(n):
                c = i % R
                for M in (Ms if only is None else (only,)):
                    sp.spear_w4_linear(xs[M], ws[c], ecs[c] if use_ec else None, y=ys[M],
                                       workspace=wsp, path=sp.PATH_AUTO)
        return record

    for i in range(args.warmup):
        steps_fn(True)(1)
    torch.cuda.synchronize()
    t_ec = time_graph(torch, steps_fn(True), args.steps, args.replays)
    t_plain = time_graph(torch, steps_fn(False), args.steps, args.replays)
    per_m = {}
    for M in Ms:
        te = time_graph(torch, steps_fn(True, M), args.steps, args.replays)
        tp = time_graph(torch, steps_fn(False, M), args.steps, args.replays)
        per_m[str(M)] = {"fused_us": round(te["median"] * 1e3, 3),
                         "plain_us": round(tp["median"] * 1e3, 3),
                         "ec_overhead": round(te["median"] / tp["median"] - 1.0, 4)}
    assert sp.spear_workspace_timeouts(wsp) == 0
    floor_gbs, floor_us, floor_bytes = stream_floor(torch, sp, [w.packed for w in ws],
                                                    args.steps, args.replays)
    floor_large = stream_floor_large(torch, sp)

    per_step_bytes = 0.0
    per_step_plain = 0.0
    for M in Ms:
        w, ec, io = layer_bytes(M, N, K, r, True)
        per_step_bytes += w + ec + io
        per_step_plain += w + io
    ms_step = t_ec["median"]
    launches = len(Ms)
    achieved = (per_step_bytes / launches) / (ms_step / launches * 1e-3) / 1e9
    w_b, ec_b, _ = layer_bytes(1, N, K, r, True)            # packed weights plus EC factors
    achieved_w_ec = (w_b + ec_b) / (ms_step / launches * 1e-3) / 1e9
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
                   "timing": f"median of {len(t_ec['all'])} replays of a {args.steps}-step "
                             "HIP graph, HIP events on the launch stream"},
        "timing": stats_ms(t_ec),
        "ec_overhead": round(t_ec["median"] / t_plain["median"] - 1.0, 4),
        "plain_ms_per_step": round(t_plain["median"], 6),
        "plain_timing": stats_ms(t_plain),
        "plain_GBps": round(per_step_plain / (t_plain["median"] * 1e-3) / 1e9, 2),
        "us_per_launch": round(ms_step / launches * 1e3, 3),
        "per_M_launch": per_m,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": profiled_traffic(),
                     "traffic_unit": "bytes per launch (profiles/decode_fused_c2_hbm_traffic.md)",
                     "kernel": "decode_kernel<1,1,*,*> (fused EC, fp32 out)",
                     "bytes_per_launch": round(per_step_bytes / launches),
                     "stream_floor_GBps": round(floor_gbs, 2),
                     "stream_floor_us_per_buffer": round(floor_us, 3),
                     "stream_floor_buffer_bytes": floor_bytes,
                     "frac_of_stream_floor": round(achieved / floor_gbs, 4),
                     "stream_floor_1GiB_GBps": round(floor_large, 2),
                     "achieved_weights_ec_GBps": round(achieved_w_ec, 2),
                     "weights_ec_bytes_per_launch": round(w_b + ec_b),
                     "plain_frac_of_stream_floor": round(
                         (per_step_plain / launches) / (t_plain["median"] / launches * 1e-3)
                         / 1e9 / floor_gbs, 4)},
    }
    return out


def measure_c4(args, torch, sp, gen, steps):
    """C4 prefill: the layer with the EC and without, `steps` calls per graph
    replay; -> dict of the measured quantities."""
    d = gen.make(4)
    M, N, K, r = d["M"], d["N"], d["K"], d["ec"]["r"]
    R = max(2, min(args.copies, 4))
    ws, ecs = build_copies(d, R, torch, sp)
    x = dev(d["x"], torch)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    wsp = sp.new_workspace(M, N, K, r)

    sf = sp.SemiFused()

    def steps_fn(use_ec, semi=False):
        def record(n):
            for i in range(n):
                if semi:
                    sp.spear_w4_linear_semifused(x, ws[i % R], ecs[i % R], sf, y=y, workspace=wsp)
                else:
                    sp.spear_w4_linear(x, ws[i % R], ecs[i % R] if use_ec else None, y=y,
                                       workspace=wsp)
        return record

    for _ in range(args.warmup):
        steps_fn(True)(1)
        steps_fn(True, True)(1)
    torch.cuda.synchronize()
    t_ec = time_graph(torch, steps_fn(True), steps, args.replays)
    t_plain = time_graph(torch, steps_fn(False), steps, args.replays)
    t_semi = time_graph(torch, steps_fn(True, True), steps, args.replays)
    assert sp.spear_workspace_timeouts(wsp) == 0
    flops = 2.0 * M * N * K
    ec_flops = 2.0 * M * K * r + 2.0 * M * r * N
    return {"M": M, "N": N, "K": K, "r": r, "flops": flops, "ec_flops": ec_flops,
            "t_ec": t_ec, "t_plain": t_plain, "t_semi": t_semi}


def prefill_object(args, torch, sp, gen):
    m = measure_c4(args, torch, sp, gen, args.prefill_steps)
    ms, ms0 = m["t_ec"]["median"], m["t_plain"]["median"]
    tf = (m["flops"] + m["ec_flops"]) / (ms * 1e-3) / 1e12
    tf0 = m["flops"] / (ms0 * 1e-3) / 1e12
    out = {"workload": "C4 prefill: M=N=K=4096, int4 symmetric per-channel, Student-t(4) "
                       "activations, EC rank 32 soft gate, fp32 output",
           "unit": "TFLOP/s", "TFLOPs": round(tf, 2), "plain_TFLOPs": round(tf0, 2),
           "ms_per_call": round(ms, 5), "plain_ms_per_call": round(ms0, 5),
           "ec_overhead": round(ms / ms0 - 1.0, 4),
           "timing": stats_ms(m["t_ec"], 5), "plain_timing": stats_ms(m["t_plain"], 5),
           "semifused": {"what": "EC as a separate kernel on a second stream beside the plain "
                                 "GEMM, joined by events (the pages' prefill form)",
                         "ms_per_call": round(m["t_semi"]["median"], 5),
                         "ec_overhead": round(m["t_semi"]["median"] / ms0 - 1.0, 4),
                         "timing": stats_ms(m["t_semi"], 5)},
           "roofline": {"bound": "mfma", "achieved": round(tf0, 2), "peak": BF16_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(tf0 / BF16_PEAK_TFLOPS, 4),
                        "traffic": None,
                        "kernel": "gemm2_kernel<2,4,0,0,1,1,4,4,1> (plain, 256 x 128 tiles, "
                                  "whole K; one launch a call)",
                        "flops_per_launch": m["flops"]}}
    return out


def run_c4(args, torch, sp, gen):
    m = measure_c4(args, torch, sp, gen, args.steps)
    ms, ms0 = m["t_ec"]["median"], m["t_plain"]["median"]
    tf = (m["flops"] + m["ec_flops"]) / (ms * 1e-3) / 1e12
    tf0 = m["flops"] / (ms0 * 1e-3) / 1e12
    return {
        "metric": METRIC, "value": round(tf, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "C4 prefill: M=N=K=4096, int4 symmetric per-channel, "
                               "Student-t(4) activations, EC rank 32 soft gate, fp32 output"},
        "timing": stats_ms(m["t_ec"]),
        "ec_overhead": round(ms / ms0 - 1.0, 4),
        "semifused_ms_per_call": round(m["t_semi"]["median"], 6),
        "semifused_ec_overhead": round(m["t_semi"]["median"] / ms0 - 1.0, 4),
        "plain_TFLOPs": round(tf0, 2),
        "plain_timing": stats_ms(m["t_plain"]),
        "roofline": {"bound": "mfma", "achieved": round(tf0, 2), "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf0 / BF16_PEAK_TFLOPS, 4),
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
    t_ec = time_graph(torch, steps_fn(True), args.steps, args.replays)["median"] * args.steps
    t_plain = time_graph(torch, steps_fn(False), args.steps, args.replays)["median"] * args.steps
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
    sf = sp.SemiFused()

    def steps_fn(use_ec, semi=False):
        def record(n):
            for i in range(n):
                if semi:
                    sp.spear_w4_linear_semifused(x, ws[i % R], ecs[i % R], sf, y=y, workspace=wsp)
                else:
                    sp.spear_w4_linear(x, ws[i % R], ecs[i % R] if use_ec else None, y=y,
                                       workspace=wsp)
        return record

    for _ in range(args.warmup):
        steps_fn(True)(1)
        steps_fn(True, True)(1)
    torch.cuda.synchronize()
    t_ec = time_graph(torch, steps_fn(True), args.steps, args.replays)["median"] * args.steps
    t_plain = time_graph(torch, steps_fn(False), args.steps, args.replays)["median"] * args.steps
    t_semi = time_graph(torch, steps_fn(True, True), args.steps, args.replays)["median"] * args.steps
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
        "semifused_ec_overhead": round(t_semi / t_plain - 1.0, 4),
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
    t_ec = time_graph(torch, steps_fn(True), args.steps, args.replays)["median"] * args.steps
    t_plain = time_graph(torch, steps_fn(False), args.steps, args.replays)["median"] * args.steps
    assert sp.spear_workspace_timeouts(wsp) == 0
    floor_us = launch_floor(torch, sp, args.replays)
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
        "launch_floor": {"us_per_launch": round(floor_us, 3), "launches_per_step": len(layers),
                         "ms_per_step": round(floor_us * len(layers) / 1e3, 4),
                         "share_of_stack": round(floor_us * len(layers) / 1e3 / ms, 4),
                         "what": "graph-captured back-to-back launches of the library's read kernel "
                                 "over 16 KiB (one workgroup): the fixed cost each of the stack's "
                                 "dependent launches pays"},
        "roofline": {"bound": "mfma" if big else "hbm", "achieved": round(val, 2), "peak": peak,
                     "unit": unit, "frac": round(val / peak, 4), "traffic": None,
                     "kernel": "whole stack (all kernels)"},
    }


def c5_stack(torch, sp, gen, M_max):
    """The C5 stack's 196 linears on the device (each its own weights), and
    input / output buffers for up to M_max tokens."""
    layers = []
    ec_layers = set(gen.c5_ec_layers())
    for layer in range(gen.C5_LAYERS):
        for lin in gen.C5_LINEARS:
            d = gen.make_c5(layer, lin, 1)
            codes = dev(d["codes"], torch)
            w = sp.W4(sp.spear_pack_w4(codes, d["kind"]), dev(d["scales"], torch),
                      dev(d["zeros"], torch), d["N"], d["K"])
            del codes
            e = d["ec"]
            ec = (sp.EC(dev(e["A"], torch), dev(e["B"], torch), dev(e["w_g"], torch), e["b"],
                        e["tau"], e["hard"]) if e is not None else None)
            layers.append((lin, d["N"], d["K"], w, ec, e["r"] if e is not None else 0))
    xs = {K: dev(gen.make_c5(0, "down" if K == gen.C5_FF else "q", M_max)["x"], torch)
          for K in (gen.C5_D, gen.C5_FF)}
    ys = {N: torch.empty((M_max, N), dtype=torch.float32, device="cuda")
          for N in (gen.C5_D, gen.C5_FF)}
    need = max(sp.spear_w4_linear_workspace_size(M_max, N, K, max(r, 32))
               for (_, N, K, _, _, r) in layers)
    wsp = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda")
    return layers, ec_layers, xs, ys, wsp


SLO_KINDS = (("attn", ("q", "k", "v", "o")), ("up", ("gate", "up")), ("down", ("down",)))
SLO_GRID = (1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096)


def run_slo(args, torch, sp, gen):
    """Latency table of the C5 stack's linear kinds, then the chunking trace."""
    from quantized_gemm_w4a16_amd import chunking
    layers, ec_layers, xs, ys, wsp = c5_stack(torch, sp, gen, max(SLO_GRID))
    kinds, counts, table = [], [], []
    for name, lins in SLO_KINDS:
        for use_ec in (0, 1):
            calls = [(N, K, w, ec) for (lin, N, K, w, ec, r) in layers
                     if lin in lins and (ec is not None) == bool(use_ec)]
            row = []
            for M in SLO_GRID:
                def record(n, calls=calls, M=M):
                    for _ in range(n):
                        for (N, K, w, ec) in calls:
                            sp.spear_w4_linear(xs[K][:M], w, ec, y=ys[N][:M], workspace=wsp)
                record(1)
                torch.cuda.synchronize()
                t = time_graph(torch, record, 2, 3)
                row.append(t["median"] * 1e3 / len(calls))          # us per call
            kinds.append(f"{name}{'_ec' if use_ec else ''}")
            counts.append(len(calls))
            table.append(row)
    assert sp.spear_workspace_timeouts(wsp) == 0
    lut = sp.SloLut(SLO_GRID, table, counts, 0.0)
    trace = chunking.make_trace(gen.SEED_BASE + 7, 300, mean_gap_us=12000.0)
    n_ref = 16
    out_slo = []
    for extra in (256, 1024):
        slo = lut.predict(n_ref + extra)
        res = [chunking.simulate(trace, lut, pol, slo, align=16).summary(slo)
               for pol in ("dynamic", "static:256", "static:1024", "static:4096")]
        out_slo.append({"slo_ms": round(slo / 1e3, 4),
                        "slo_reading": f"predicted step of {n_ref} decode + {extra} prefill tokens",
                        "policies": res})
    # EC-aware: the chunk the picker allows at the tight objective as EC density grows
    by_density = {}
    slo = out_slo[0]["slo_ms"] * 1e3
    for n_ec in (0, 4, 8, 16, 28):
        cnt = []
        for k in kinds:
            per_layer = {"attn": 4, "up": 2, "down": 1}[k.split("_")[0]]
            cnt.append(per_layer * (n_ec if k.endswith("_ec") else gen.C5_LAYERS - n_ec))
        L = sp.SloLut(SLO_GRID, table, cnt, 0.0)
        by_density[str(n_ec)] = L.pick_chunk(n_ref, 4096, slo, 16)[0]
    lut_json = {"tokens": list(SLO_GRID), "kinds": kinds, "us_per_call": table,
                "calls_per_step": counts,
                "source": "measured by bench.py --workload slo: median of 3 replays of a "
                          "graph over every call of the kind in the C5 stack"}
    if args.lut_out:
        with open(args.lut_out, "w") as f:
            json.dump(lut_json, f, indent=1)
    dyn = out_slo[0]["policies"][0]
    return {
        "metric": METRIC, "value": dyn["decode_tokens_per_s"], "unit": "decode tokens/s",
        "n_gpus": 1, "steps": 2, "warmup": 1, "ms_per_step": None, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "EC-aware prefill chunking on the C5 stack (28 layers, ECs "
                               f"on layers {sorted(ec_layers)}): latency table measured here, "
                               "300 seeded requests (Poisson arrivals, mean gap 12 ms, "
                               "log-normal prompts 64..4096, outputs 32..256)"},
        "lut": lut_json, "slo": out_slo, "chunk_at_tight_slo_by_ec_layers": by_density,
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
    run = {"c1": run_c1, "c2": run_c2, "c3": run_c3, "c4": run_c4, "c5": run_c5,
           "slo": run_slo}[args.workload]
    out = run(args, torch, sp, gen)
    if args.copy_calibration:
        out["copy_calibration_bytes"] = copy_calibration(torch)
    if args.workload == "c2" and not args.no_prefill:
        out["prefill"] = prefill_object(args, torch, sp, gen)
    if args.workload == "c2" and not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_c2((1, 4, 8), args.cpu_seconds)
        if "prefill" in out:
            out["prefill"]["cpu_baseline"] = cpu_baseline_c4(args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
