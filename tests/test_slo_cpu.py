"""The EC-aware chunk picker and its latency prediction (host only, summary
section 2.2 C), and the trace simulation around it."""
import math

import numpy as np
import pytest

from quantized_gemm_w4a16_amd import chunking
from quantized_gemm_w4a16_amd import spear as sp


def lut1(tokens, us, count=1, overhead=0.0):
    return sp.SloLut(tokens, [us], [count], overhead)


def test_predict_closed_forms():
    # one kind, two points: exact linear interpolation, flat below, slope above
    L = lut1([16, 48], [10.0, 30.0])
    assert L.predict(0) == 0.0
    assert L.predict(1) == 10.0 and L.predict(16) == 10.0
    assert L.predict(32) == 20.0 and L.predict(48) == 30.0
    assert L.predict(80) == 50.0
    # counts multiply, overhead adds once, kinds add
    L = sp.SloLut([16, 48], [[10.0, 30.0], [1.0, 2.0]], [3, 5], 7.5)
    assert L.predict(32) == 7.5 + 3 * 20.0 + 5 * 1.5
    # a kind with count 0 is ignored
    L = sp.SloLut([16, 48], [[10.0, 30.0], [1e6, 1e6]], [1, 0], 0.0)
    assert L.predict(32) == 20.0


def test_predict_monotone_envelope():
    """A measured dip (noise) is replaced by the running maximum, so the
    prediction never decreases as the batch grows."""
    L = lut1([1, 2, 4, 8], [5.0, 9.0, 7.0, 11.0])
    assert L.predict(2) == 9.0 and L.predict(4) == 9.0 and L.predict(3) == 9.0
    assert L.predict(6) == 10.0 and L.predict(8) == 11.0
    v = [L.predict(m) for m in range(0, 40)]
    assert all(b >= a for a, b in zip(v, v[1:]))


def brute_pick(L, n_dec, pending, align, slo):
    cands = [c for c in range(0, pending + 1) if c == pending or c % align == 0]
    ok = [c for c in cands if L.predict(n_dec + c) <= slo]
    return max(ok) if ok else 0


@pytest.mark.parametrize("seed", range(6))
def test_pick_is_largest_fitting_chunk(seed):
    rng = np.random.default_rng(seed)
    pts = np.unique(np.sort(rng.integers(1, 3000, 7)))
    us = np.maximum.accumulate(rng.uniform(1, 100, (3, len(pts))), axis=1)
    L = sp.SloLut(pts, us, rng.integers(0, 4, 3), float(rng.uniform(0, 20)))
    for _ in range(60):
        n_dec = int(rng.integers(0, 64))
        pending = int(rng.integers(0, 3000))
        align = int(rng.choice([1, 8, 16, 64]))
        slo = float(rng.uniform(0, 2) * L.predict(n_dec + pending // 2 + 1) + 1)
        c, pred = L.pick_chunk(n_dec, pending, slo, align)
        assert c == brute_pick(L, n_dec, pending, align, slo), (n_dec, pending, align, slo)
        assert pred == pytest.approx(L.predict(n_dec + c), rel=1e-6)
        if c:
            assert L.predict(n_dec + c) <= slo


def test_pick_edges():
    L = lut1([1, 1024], [100.0, 1100.0])          # 100 us + ~0.977 us a token
    assert L.pick_chunk(4, 0, 1e9)[0] == 0          # nothing pending
    assert L.pick_chunk(4, 500, 1e9)[0] == 500      # everything fits: the whole prompt
    assert L.pick_chunk(4, 500, 50.0)[0] == 0       # not even decode alone fits
    c, _ = L.pick_chunk(4, 5000, L.predict(4 + 256), 16)
    assert c == 256
    c, _ = L.pick_chunk(4, 5000, L.predict(4 + 256) - 1e-3, 16)
    assert c == 240


def test_lut_validation():
    lib = sp.load()
    bad = [sp.SloLut([4, 2], [[1.0, 2.0]], [1]),           # not ascending
           sp.SloLut([0, 2], [[1.0, 2.0]], [1]),           # tokens < 1
           sp.SloLut([1, 2], [[1.0, float("nan")]], [1]),  # a NaN time
           sp.SloLut([1, 2], [[1.0, 2.0]], [-1]),          # negative count
           sp.SloLut([1, 2], [[1.0, 2.0]], [1], -1.0)]     # negative overhead
    for L in bad:
        with pytest.raises(sp.SpearError):
            L.predict(3)
    L = lut1([1, 2], [1.0, 2.0])
    with pytest.raises(sp.SpearError):
        L.pick_chunk(-1, 10, 5.0)
    with pytest.raises(sp.SpearError):
        L.pick_chunk(1, 10, 5.0, align=0)


def test_trace_dynamic_meets_objective_static_does_not():
    """On a trace where long prompts arrive while requests decode, the picker
    keeps every step with running requests within the objective, while one
    whole-prompt chunk per step breaks it; the picker's chunks let prompts
    through at a comparable time to first token."""
    L = lut1([1, 64, 512, 4096], [40.0, 60.0, 300.0, 2200.0], count=10, overhead=100.0)
    trace = chunking.make_trace(7, 200, mean_gap_us=4000.0)
    slo = L.predict(16 + 256)
    dyn = chunking.simulate(trace, L, "dynamic", slo, align=16).summary(slo)
    big = chunking.simulate(trace, L, "static:4096", slo).summary(slo)
    small = chunking.simulate(trace, L, "static:64", slo).summary(slo)
    print(dyn, big, small)
    assert dyn["slo_met"] == 1.0
    assert big["slo_met"] < 0.9
    assert dyn["ttft_mean_ms"] < small["ttft_mean_ms"]


def test_measured_table_trace():
    """The latency table measured on MI355X for the C5 stack's linear kinds
    (data/slo_lut_c5_mi355x.json, written by bench.py --workload slo): under
    the picker every step with running requests meets the objective; with
    more EC layers the picker allows a smaller chunk (EC-aware)."""
    import json
    import os
    here = os.path.dirname(os.path.abspath(chunking.__file__))
    t = json.load(open(os.path.join(here, "data", "slo_lut_c5_mi355x.json")))
    L = sp.SloLut(t["tokens"], t["us_per_call"], t["calls_per_step"])
    slo = L.predict(16 + 256)
    trace = chunking.make_trace(11, 120, mean_gap_us=12000.0)
    dyn = chunking.simulate(trace, L, "dynamic", slo, align=16).summary(slo)
    assert dyn["slo_met"] == 1.0
    big = chunking.simulate(trace, L, "static:4096", slo).summary(slo)
    assert big["slo_met"] < 1.0
    per_layer = {"attn": 4, "up": 2, "down": 1}
    chunks = []
    for n_ec in (0, 4, 28):
        cnt = [per_layer[k.split("_")[0]] * (n_ec if k.endswith("_ec") else 28 - n_ec)
               for k in t["kinds"]]
        chunks.append(sp.SloLut(t["tokens"], t["us_per_call"], cnt).pick_chunk(16, 4096, slo, 16)[0])
    assert chunks[0] >= chunks[1] >= chunks[2] and chunks[0] > chunks[2]
