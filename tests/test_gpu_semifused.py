"""The semi-fused prefill (the summary's section 2.2 A: at prefill the EC is a
separate kernel beside the low-bit GEMM, joined through the graph) against the
oracle; the hard gate's compacted token list drives the EC kernel."""
import math

import numpy as np
import pytest
import torch

import oracle
from quantized_gemm_w4a16_amd import inputs as gen
from quantized_gemm_w4a16_amd import spear as sp
from gpu_util import assert_close, dev, gpu_ec, gpu_weights, host, run_oracle
from test_gpu_parity import random_case
from test_gpu_vector_gate import with_vgate

pytestmark = pytest.mark.gpu


def run_sf(d, sf, w=None, ws=None):
    w = gpu_weights(d) if w is None else w
    e = gpu_ec(d["ec"], d["M"]) if d["ec"] is not None else None
    y = sp.spear_w4_linear_semifused(dev(d["x"]), w, e, sf, workspace=ws)
    torch.cuda.synchronize()
    return host(y), e


@pytest.fixture(scope="module")
def sf():
    return sp.SemiFused()


@pytest.mark.parametrize("M,N,K,r", [(17, 96, 256, 8), (40, 1000, 160, 40), (100, 200, 544, 64),
                                     (130, 129, 1024, 32), (257, 300, 2080, 24),
                                     (600, 520, 1024, 256), (2100, 96, 1056, 24)])
@pytest.mark.parametrize("hard", [0, 1])
def test_semifused_parity(sf, M, N, K, r, hard):
    d = random_case(M, N, K, r, oracle.CODES_U4, hard, seed=3000 + M + N + K + r + hard)
    ref = run_oracle(d)
    gref = oracle.gate(d["x"], d["ec"]["w_g"], d["ec"]["b"], d["ec"]["tau"], hard)
    y, e = run_sf(d, sf)
    assert_close(y, ref, f"semifused {M}x{N}x{K} r={r} hard={hard}")
    n = int(e.n_active_out.item())
    assert n == gref["n_active"]
    assert np.array_equal(host(e.idx_out)[:n], gref["idx"])
    np.testing.assert_allclose(host(e.g_out), gref["g"], rtol=2e-7)


@pytest.mark.parametrize("M", [24, 300])
def test_semifused_vector_gate(sf, M):
    d = with_vgate(random_case(M, 256, 1024, 32, oracle.CODES_S4, 1, seed=77 + M), 8, seed=M)
    assert_close(run_sf(d, sf)[0], run_oracle(d), f"semifused vector gate M={M}")


def test_semifused_c4_sampled(sf):
    d = gen.make(4)
    rng = np.random.default_rng(45)
    S = 2000
    ms, ns = rng.integers(0, d["M"], S), rng.integers(0, d["N"], S)
    ms[:32] = d["M"] - 1
    ns[32:64] = d["N"] - 1
    packed, _ = oracle.pack_w4(d["codes"], d["kind"])
    ref = oracle.w4_linear_sampled(d["x"], packed, d["scales"], d["zeros"], d["ec"], ms, ns)
    y, e = run_sf(d, sf)
    assert np.all(np.isfinite(y))
    assert_close(y[ms, ns], ref, "semifused C4 sampled")
    assert int(e.n_active_out.item()) == d["M"]


def test_semifused_no_active_token_and_plain(sf):
    """tau = 1 leaves the token list empty: the EC kernel adds nothing, and the
    result is the plain GEMM's bit for bit; ec = NULL is the plain layer."""
    d = random_case(150, 300, 1024, 32, oracle.CODES_U4, 1, seed=11)
    w = gpu_weights(d)
    plain = host(sp.spear_w4_linear(dev(d["x"]), w, None))
    y, e = run_sf(dict(d, ec=dict(d["ec"], tau=1.0)), sf, w=w)
    assert int(e.n_active_out.item()) == 0
    assert np.array_equal(y, plain)
    y0, _ = run_sf(dict(d, ec=None), sf, w=w)
    assert np.array_equal(y0, plain)
    assert_close(y0, run_oracle(d, ec=None), "semifused plain")


def test_semifused_graph_replays(sf):
    """Captured in a HIP graph (the fork and join become graph edges) and
    replayed three times, with eager work between the replays: every replay
    equals the eager call bit for bit."""
    d = random_case(96, 512, 2048, 32, oracle.CODES_U4, 1, seed=21)
    w = gpu_weights(d)
    x = dev(d["x"])
    e = gpu_ec(d["ec"], d["M"])
    ws = sp.new_workspace(96, 512, 2048, 32)
    y = torch.empty((96, 512), dtype=torch.float32, device="cuda")
    sp.spear_w4_linear_semifused(x, w, e, sf, y=y, workspace=ws)
    torch.cuda.synchronize()
    want = host(y).copy()
    assert_close(want, run_oracle(d), "semifused eager")
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            sp.spear_w4_linear_semifused(x, w, e, sf, y=y, workspace=ws, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for i in range(3):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(y), want), i
        junk = sp.spear_w4_linear(x, w, None)            # eager work between replays
        torch.cuda.synchronize()
        del junk
