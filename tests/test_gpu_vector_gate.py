"""GPU parity of the vector gate (the summary's diag(gamma(Ax)) with gamma a
bottleneck MLP on the rank-r projection, section 2.1 A) against the oracle,
on every path; gamma = 1 reduces to the scalar form bit for bit."""
import math

import numpy as np
import pytest

import oracle
from quantized_gemm_w4a16_amd import spear as sp
from gpu_util import assert_close, gpu_weights, host, run_gpu, run_oracle
from test_gpu_parity import random_case

pytestmark = pytest.mark.gpu

PATHS = [sp.PATH_DECODE, sp.PATH_DECODE_2PASS, sp.PATH_PREFILL, sp.PATH_PREFILL_LARGE]


def with_vgate(d, h, seed, alpha=0.8, c2=None):
    rng = np.random.default_rng(seed)
    r = d["ec"]["r"]
    ec = dict(d["ec"], gate_h=h, alpha=alpha,
              gate_w1=rng.normal(0, 2.0 / math.sqrt(r), (h, r)).astype(np.float32),
              gate_c1=rng.normal(0, 0.1, h).astype(np.float32),
              gate_w2=rng.normal(0, 2.0 / math.sqrt(h), (r, h)).astype(np.float32),
              gate_c2=(rng.normal(0, 0.5, r) if c2 is None else c2).astype(np.float32))
    return dict(d, ec=ec)


@pytest.mark.parametrize("M,N,K,r,h", [(1, 256, 1024, 32, 8), (4, 300, 2080, 64, 16),
                                       (16, 512, 4096, 32, 4), (40, 200, 1056, 96, 64),
                                       (150, 520, 1024, 32, 8), (600, 256, 2048, 256, 32)])
@pytest.mark.parametrize("hard", [0, 1])
def test_vector_gate_parity(M, N, K, r, h, hard):
    d = with_vgate(random_case(M, N, K, r, oracle.CODES_U4, hard, seed=M + N + K + r + hard),
                   h, seed=h + M)
    ref = run_oracle(d)
    gref = oracle.gate(d["x"], d["ec"]["w_g"], d["ec"]["b"], d["ec"]["tau"], hard)
    if gref["n_active"]:
        # the EC term with the vector gate is not that of the scalar form
        assert not np.allclose(ref, run_oracle(dict(d, ec=dict(d["ec"], gate_h=0))), atol=1e-4)
    w = gpu_weights(d)
    for path in (PATHS if M <= 16 else PATHS[2:]):
        y, e = run_gpu(d, path=path, w=w)
        assert_close(y, ref, f"vector gate M={M} N={N} K={K} r={r} h={h} hard={hard} path={path}")
        n = int(e.n_active_out.item())
        assert n == gref["n_active"]
        assert np.array_equal(host(e.idx_out)[:n], gref["idx"])
        np.testing.assert_allclose(host(e.g_out), gref["g"], rtol=2e-7)


@pytest.mark.parametrize("M", [3, 70])
def test_vector_gate_one_is_scalar_form_bitwise(M):
    """c2 = +inf: gamma = 1 exactly, alpha = 1: the same bits as the scalar form."""
    d = random_case(M, 272, 1024, 32, oracle.CODES_S4, 1, seed=800 + M)
    dv = with_vgate(d, 8, seed=5, alpha=1.0, c2=np.full(32, np.inf))
    w = gpu_weights(d)
    for path in (PATHS if M <= 16 else PATHS[2:]):
        y0, _ = run_gpu(d, path=path, w=w)
        y1, _ = run_gpu(dv, path=path, w=w)
        assert np.array_equal(y0, y1), path
