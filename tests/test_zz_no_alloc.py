"""The allocation-free entry point against the workspace entry point: same
kernels, so the outputs must agree bit for bit (and both meet the oracle's
tolerance), on two calls in a row, the second with a smaller input."""
import math

import numpy as np
import pytest
import torch

import oracle
from quantized_gemm_w4a16_amd import inputs as gen
from quantized_gemm_w4a16_amd import spear as sp
from gpu_util import assert_close, dev, gpu_ec, gpu_weights, host, run_oracle

pytestmark = pytest.mark.gpu


def case(M, N, K, r, hard, seed):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    ec = {"A": gen.bf16_bits(rng.normal(0, 0.05, size=(r, K)).astype(np.float32)),
          "B": gen.bf16_bits(rng.normal(0, 0.05, size=(N, r)).astype(np.float32)),
          "w_g": gen.bf16_bits(rng.normal(0, 1 / math.sqrt(K), size=K).astype(np.float32)),
          "b": 0.1, "tau": 0.5, "hard": hard, "r": r}
    return {"M": M, "N": N, "K": K, "kind": oracle.CODES_U4, "codes": codes,
            "scales": rng.uniform(0.005, 0.02, N).astype(np.float32),
            "zeros": rng.integers(0, 16, size=N, dtype=np.uint8),
            "x": gen.bf16_bits(rng.normal(0, 1, size=(M, K)).astype(np.float32)), "ec": ec}


def test_noalloc_matches_workspace_entry():
    # first a prefill-sized call (the pre-pass in the GEMM's launch, tagged
    # exchange), then a smaller decode call (fused EC, tagged exchange)
    for (M, N, K, r, hard) in [(96, 1024, 4096, 64, 1), (4, 512, 2048, 32, 0)]:
        d = case(M, N, K, r, hard, seed=M + N + K)
        print(f"[noalloc] M={M} N={N} K={K} r={r} hard={hard}", flush=True)
        w = gpu_weights(d)
        x = dev(d["x"])
        e_ws, e_na = gpu_ec(d["ec"], M), gpu_ec(d["ec"], M)
        y_ws = sp.spear_w4_linear(x, w, e_ws)
        y_na = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        sp.spear_w4_linear_noalloc(x, w, e_na, y=y_na)
        torch.cuda.synchronize()
        a, b = host(y_ws), host(y_na)
        assert np.array_equal(a, b)
        assert_close(b, run_oracle(d), f"noalloc M={M}")
        n = int(e_na.n_active_out.item())
        assert n == int(e_ws.n_active_out.item())
        assert np.array_equal(host(e_na.idx_out)[:n], host(e_ws.idx_out)[:n])
        assert np.array_equal(host(e_na.g_out), host(e_ws.g_out))


def test_noalloc_rejects_oversize_before_any_hip_call():
    lib = sp.load()
    A16 = 0x10000
    w = sp._W4(A16, A16, None, 8192, 65536)        # needs far more than the scratch
    assert sp.spear_w4_linear_workspace_size(4096, 8192, 65536, 0) > sp.NOALLOC_MAX_WORKSPACE
    st = lib.spear_w4_linear_noalloc(A16, 4096, __import__("ctypes").byref(w), None, A16, 1, 0,
                                     None)
    assert st == -5
