"""Prefill chunking under an inter-token-latency objective, on a synthetic
request trace (host only).

The chunk is chosen by the library's native picker (spear_slo_pick_chunk):
the largest prefill chunk whose predicted step time, from a table of measured
kernel latencies, meets the objective -- the scheduler of "SPEAR: A System for
Post-Quantization Error-Adaptive Recovery Enabling Efficient Low-Bit LLM
Serving" (gist.science summary, section 2.2 C), compared here with fixed chunk
sizes as in its section 3.2.  This module holds only the trace and the
continuous-batching bookkeeping; it makes no GPU call.

Model of a serving step: every running request decodes one token and at most
one waiting request (first come, first served) prefills a chunk of its prompt;
the step processes n_decode + chunk tokens through the model's linears, and
takes the time the table predicts for that many tokens.  A request's first
token comes with the step that finishes its prompt; its later tokens come one
per step, so each step's time is the inter-token latency of every running
request.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass
class Request:
    arrival_us: float
    prompt: int
    output: int


def make_trace(seed: int, n: int, mean_gap_us: float, prompt_median: int = 768,
               prompt_range=(64, 4096), output_range=(32, 256)) -> list:
    """Seeded synthetic requests: Poisson arrivals (exponential gaps), log-normal
    prompt lengths clipped to prompt_range, uniform output lengths."""
    rng = np.random.Generator(np.random.PCG64(seed))
    t = np.cumsum(rng.exponential(mean_gap_us, n))
    p = np.clip(np.round(rng.lognormal(np.log(prompt_median), 0.8, n)), *prompt_range)
    o = rng.integers(output_range[0], output_range[1] + 1, n)
    return [Request(float(a), int(b), int(c)) for a, b, c in zip(t, p, o)]


@dataclass
class Result:
    policy: str
    steps: int = 0
    itl_us: list = field(default_factory=list)      # step times with running requests
    ttft_us: list = field(default_factory=list)
    decode_tokens: int = 0
    end_us: float = 0.0

    def summary(self, slo_us: float) -> dict:
        itl = np.array(self.itl_us) if self.itl_us else np.zeros(1)
        ttft = np.array(self.ttft_us) if self.ttft_us else np.zeros(1)
        return {"policy": self.policy, "steps": self.steps,
                "slo_met": round(float(np.mean(itl <= slo_us)), 4),
                "itl_p50_ms": round(float(np.percentile(itl, 50)) / 1e3, 4),
                "itl_p99_ms": round(float(np.percentile(itl, 99)) / 1e3, 4),
                "itl_max_ms": round(float(itl.max()) / 1e3, 4),
                "ttft_mean_ms": round(float(ttft.mean()) / 1e3, 3),
                "ttft_p90_ms": round(float(np.percentile(ttft, 90)) / 1e3, 3),
                "decode_tokens_per_s": round(self.decode_tokens / (self.end_us * 1e-6), 1)}


def simulate(trace: list, lut, policy: str, slo_us: float, align: int = 16) -> Result:
    """Run the trace.  policy: "dynamic" (the native picker under slo_us) or
    "static:S" (chunks of at most S tokens).  With nothing running, a step that
    the objective cannot fit still prefills `align` tokens (no inter-token
    latency is at stake then)."""
    res = Result(policy)
    static = int(policy.split(":")[1]) if policy.startswith("static:") else 0
    clock, i = 0.0, 0
    waiting = []          # [request, prompt tokens left]
    running = []          # [request, output tokens left]
    n = len(trace)
    while i < n or waiting or running:
        while i < n and trace[i].arrival_us <= clock:
            waiting.append([trace[i], trace[i].prompt])
            i += 1
        if not waiting and not running:
            clock = trace[i].arrival_us
            continue
        n_dec = len(running)
        chunk = 0
        if waiting:
            pending = waiting[0][1]
            if static:
                chunk = min(pending, static)
            else:
                chunk, _ = lut.pick_chunk(n_dec, pending, slo_us, align)
                if chunk == 0 and n_dec == 0:
                    chunk = min(pending, align)
        step = lut.predict(n_dec + chunk)
        clock += step
        res.steps += 1
        if n_dec:
            res.itl_us.append(step)
            res.decode_tokens += n_dec
        for r in running:
            r[1] -= 1
        running = [r for r in running if r[1] > 0]
        if chunk:
            waiting[0][1] -= chunk
            if waiting[0][1] == 0:
                req = waiting.pop(0)[0]
                res.ttft_us.append(clock - req.arrival_us)
                if req.output > 1:
                    running.append([req, req.output - 1])
    res.end_us = clock
    return res
