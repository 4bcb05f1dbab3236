"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded bf16 inputs.  Packing, token selection and the one-hot unpack
probe are bit-exact; fp32 outputs are within rel-L2 1e-3 and max-abs 2e-2."""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from quantized_gemm_w4a16_amd import inputs as gen
from quantized_gemm_w4a16_amd import spear as sp
from gpu_util import (assert_close, assert_reordered, dev, errors, gpu_ec, gpu_weights, host,
                      run_gpu, run_oracle)

pytestmark = pytest.mark.gpu

ALL_PATHS_SMALL = [sp.PATH_DECODE, sp.PATH_DECODE_2PASS, sp.PATH_PREFILL, sp.PATH_PREFILL_LARGE]


def test_library_is_in_tree():
    lib = sp.load()
    assert os.path.samefile(lib._name, sp.LIB_PATH)
    assert torch.cuda.is_available()
    print("[device]", torch.cuda.get_device_properties(0).gcnArchName, flush=True)


# ------------------------------------------------------------------ packing

@pytest.mark.parametrize("cfg", [1, 2])
def test_pack_bit_exact(cfg):
    d = gen.make(cfg)
    want, _ = oracle.pack_w4(d["codes"], d["kind"])
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = sp.spear_pack_w4(dev(d["codes"]), d["kind"], bad_codes=bad)
    torch.cuda.synchronize()
    assert np.array_equal(host(got), want)
    assert int(bad.item()) == 0


@pytest.mark.parametrize("kind", [oracle.CODES_S4, oracle.CODES_U4])
def test_pack_ragged_and_bad_codes(kind):
    rng = np.random.default_rng(31 + kind)
    N, K = 37, 96
    if kind == oracle.CODES_S4:
        codes = rng.integers(-128, 128, size=(N, K), dtype=np.int16).astype(np.int8)
    else:
        codes = rng.integers(0, 256, size=(N, K), dtype=np.int16).astype(np.uint8)
    want, nbad = oracle.pack_w4(codes, kind)
    bad = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = sp.spear_pack_w4(dev(codes), kind, bad_codes=bad)
    torch.cuda.synchronize()
    assert np.array_equal(host(got), want)
    assert int(bad.item()) == nbad > 0


# ---------------------------------------------------------------------- gate

@pytest.mark.parametrize("M,K", [(0, 64), (1, 32), (5, 4096), (64, 4096), (1500, 1024)])
@pytest.mark.parametrize("hard,tau", [(0, 0.5), (1, 0.5), (1, 0.35), (1, 1.0), (1, 0.0)])
def test_gate_parity(M, K, hard, tau):
    rng = np.random.default_rng(M * 7 + K + int(tau * 100) + hard)
    x = gen.bf16_bits(rng.normal(0, 1, size=(M, K)).astype(np.float32))
    wg = gen.bf16_bits(rng.normal(0, 1 / math.sqrt(K), size=K).astype(np.float32))
    b = 0.125
    ref = oracle.gate(x, wg, b, tau, hard)
    if M and hard and 0 < tau < 1:
        assert np.min(np.abs(ref["z"] - oracle.logit_threshold(tau))) > 1e-9
    g, idx, n = sp.spear_gate(dev(x) if M else torch.empty((0, K), dtype=torch.int16,
                                                          device="cuda"),
                              dev(wg), b, tau, hard)
    torch.cuda.synchronize()
    n = int(n.item())
    assert n == ref["n_active"]
    assert np.array_equal(host(idx)[:n], ref["idx"])
    if M:
        np.testing.assert_allclose(host(g), ref["g"], rtol=2e-7, atol=0)


# ----------------------------------------------------------- one-hot probe

@pytest.mark.parametrize("path,M", [(sp.PATH_DECODE, 16), (sp.PATH_DECODE, 3),
                                    (sp.PATH_DECODE, 1),
                                    (sp.PATH_DECODE_2PASS, 16), (sp.PATH_PREFILL, 16),
                                    (sp.PATH_PREFILL, 40), (sp.PATH_PREFILL, 200),
                                    (sp.PATH_PREFILL_LARGE, 16), (sp.PATH_PREFILL_LARGE, 200)])
@pytest.mark.parametrize("K", [256, 4096])
def test_one_hot_unpack_probe(path, M, K):
    """x[m] = e_{k_m}, s = 1: y[m][n] = u[n][k_m] - z_n exactly (fp32 output).  Pins
    the in-kernel nibble order, the pair permutation and the offset removal."""
    rng = np.random.default_rng(K + M + path)
    N = 48
    u = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    z = rng.integers(0, 16, size=N, dtype=np.uint8)
    ks = rng.choice(K, size=M, replace=M > K)
    x = np.zeros((M, K), np.uint16)
    x[np.arange(M), ks] = 0x3F80
    d = {"M": M, "N": N, "K": K, "kind": oracle.CODES_U4, "codes": u,
         "scales": np.ones(N, np.float32), "zeros": z, "x": x, "ec": None}
    y, _ = run_gpu(d, path=path, ec=False)
    want = u[:, ks].T.astype(np.float32) - z[None, :].astype(np.float32)
    assert np.array_equal(y, want)


# ----------------------------------------------------------- full workloads

@pytest.mark.parametrize("path", ALL_PATHS_SMALL)
@pytest.mark.parametrize("out", [sp.OUT_F32, sp.OUT_BF16])
def test_c1(path, out):
    d = gen.make(1)
    ref = run_oracle(d)
    y, e = run_gpu(d, path=path, out=out)
    if out == sp.OUT_F32:
        assert_close(y, ref, f"C1 path={path}")
    else:
        # bf16 output: within one bf16 ulp (of |ref|) of the oracle
        a = np.maximum(np.abs(ref), 2.0 ** -120)
        ulp = 2.0 ** (np.floor(np.log2(a)) - 7)
        assert np.all(np.abs(y.astype(np.float64) - ref) <= ulp)
        want = gen.bf16_bits(ref.astype(np.float32))
        same = np.mean(gen.bf16_bits(y) == want)
        print(f"[parity] C1 bf16 path={path} bit-equal to RNE(oracle): {same:.5f}")
        assert same >= 0.999
    gref = oracle.gate(d["x"], d["ec"]["w_g"], d["ec"]["b"], d["ec"]["tau"], d["ec"]["hard"])
    np.testing.assert_allclose(host(e.g_out), gref["g"], rtol=2e-7)
    assert int(e.n_active_out.item()) == 16


@pytest.mark.parametrize("M", [1, 4, 8])
@pytest.mark.parametrize("path", ALL_PATHS_SMALL)
def test_c2_decode(M, path):
    d = gen.make(2, M=M)
    ref = run_oracle(d)
    y, e = run_gpu(d, path=path)
    assert_close(y, ref, f"C2 M={M} path={path}")
    assert int(e.n_active_out.item()) == M
    plain, _ = run_gpu(d, path=path, ec=False)
    assert_close(plain, run_oracle(d, ec=None), f"C2 plain M={M} path={path}")


def test_c3_hard_gate_selection():
    d = gen.make(3)
    ec = d["ec"]
    gref = oracle.gate(d["x"], ec["w_g"], ec["b"], ec["tau"], ec["hard"])
    t = oracle.logit_threshold(ec["tau"])
    print(f"[C3] active {gref['n_active']}/64, margin {np.min(np.abs(gref['z'] - t)):.3e}")
    ref = run_oracle(d)
    y, e = run_gpu(d)
    n = int(e.n_active_out.item())
    assert n == gref["n_active"]
    assert np.array_equal(host(e.idx_out)[:n], gref["idx"])
    np.testing.assert_allclose(host(e.g_out), gref["g"], rtol=2e-7)
    assert_close(y, ref, "C3")


def test_c4_full_size_sampled():
    d = gen.make(4)
    rng = np.random.default_rng(44)
    S = 3000
    ms = rng.integers(0, d["M"], S)
    ns = rng.integers(0, d["N"], S)
    ms[:64] = d["M"] - 1          # the last tile row and column
    ns[64:128] = d["N"] - 1
    packed, _ = oracle.pack_w4(d["codes"], d["kind"])
    ref = oracle.w4_linear_sampled(d["x"], packed, d["scales"], d["zeros"], d["ec"], ms, ns)
    y, e = run_gpu(d)
    assert np.all(np.isfinite(y))
    assert_close(y[ms, ns], ref, "C4 sampled")
    assert int(e.n_active_out.item()) == d["M"]
    plain, _ = run_gpu(d, ec=False)
    ref0 = oracle.w4_linear_sampled(d["x"], packed, d["scales"], d["zeros"], None, ms, ns)
    assert_close(plain[ms, ns], ref0, "C4 plain sampled")


def random_case(M, N, K, r, kind, hard, seed):
    rng = np.random.default_rng(seed)
    if kind == oracle.CODES_S4:
        codes, zeros = rng.integers(-8, 8, size=(N, K), dtype=np.int8), None
    else:
        codes = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
        zeros = rng.integers(0, 16, size=N, dtype=np.uint8)
    x = gen.bf16_bits(rng.normal(0, 1, size=(M, K)).astype(np.float32))
    ec = {"A": gen.bf16_bits(rng.normal(0, 0.05, size=(r, K)).astype(np.float32)),
          "B": gen.bf16_bits(rng.normal(0, 0.05, size=(N, r)).astype(np.float32)),
          "w_g": gen.bf16_bits(rng.normal(0, 1 / math.sqrt(K), size=K).astype(np.float32)),
          "b": 0.1, "tau": 0.5, "hard": hard, "r": r}
    return {"M": M, "N": N, "K": K, "kind": kind, "codes": codes,
            "scales": rng.uniform(0.005, 0.02, N).astype(np.float32), "zeros": zeros,
            "x": x, "ec": ec}


RAGGED = [(1, 16, 32, 8), (3, 40, 96, 16), (16, 1000, 160, 40), (5, 17, 1056, 256),
          (17, 1000, 160, 40), (33, 24, 4096, 8), (100, 200, 544, 64), (130, 129, 1024, 32),
          (257, 300, 2080, 24), (200, 300, 352, 32), (129, 513, 192, 16),
          # K split over workgroups with a K tail and EC rank chunks spread over
          # the slices; 64 x 64 tiles up to 128 tokens, 128 x 256 above
          (64, 260, 1184, 96), (65, 700, 1280, 48), (128, 2050, 1024, 32), (129, 300, 1024, 16),
          # 128 x 256 tiles over two K slices with the pre-pass in the GEMM's
          # launch: each slice's epilogue takes two rank chunks in one poll
          (160, 300, 1024, 128),
          # rank 32 with at least 128 token groups: 64-token pre-pass blocks over
          # K slices, a partial last block and a ragged last slice
          (2100, 96, 1056, 24),
          # 64-token pre-pass blocks whose last block holds one partial group of
          # 16 (the other three lie past M), K split into 4 slices of 520
          (4100, 64, 2080, 32),
          # decode with K split over workgroups (16 tokens do not fit one
          # workgroup's LDS at this depth): three ranges, a ragged last one
          (12, 1000, 5024, 40)]


@pytest.mark.parametrize("M,N,K,r", RAGGED)
@pytest.mark.parametrize("kind", [oracle.CODES_S4, oracle.CODES_U4])
@pytest.mark.parametrize("hard", [0, 1])
def test_ragged_shapes(M, N, K, r, kind, hard):
    d = random_case(M, N, K, r, kind, hard, seed=M * 1000 + N + K + r + kind * 7 + hard)
    ref = run_oracle(d)
    gref = oracle.gate(d["x"], d["ec"]["w_g"], d["ec"]["b"], d["ec"]["tau"], hard)
    paths = ALL_PATHS_SMALL if M <= 16 else [sp.PATH_PREFILL, sp.PATH_PREFILL_LARGE]
    for path in paths:
        y, e = run_gpu(d, path=path)
        assert_close(y, ref, f"ragged {M}x{N}x{K} r={r} kind={kind} hard={hard} path={path}")
        n = int(e.n_active_out.item())
        assert n == gref["n_active"]
        assert np.array_equal(host(e.idx_out)[:n], gref["idx"])


@pytest.mark.parametrize("path,M", [(sp.PATH_DECODE, 1), (sp.PATH_DECODE, 16),
                                    (sp.PATH_DECODE_2PASS, 8), (sp.PATH_PREFILL, 16),
                                    (sp.PATH_PREFILL, 150)])
def test_invariants_bitwise(path, M):
    """tau = 1, A = 0 and b = -inf each make the EC term an exact zero: the three
    outputs are bitwise identical, and bitwise equal to plain W4 where the plain
    layer runs the same stream form (the two-pass decode and the prefill); the
    fused decode always streams with 4 waves, the plain decode with 8 on long K
    ranges, so there they agree to the rounding of the reordered sum.  Repeated
    calls are bitwise identical (no floating-point atomics)."""
    d = random_case(M, 272, 1024, 32, oracle.CODES_U4, 0, seed=500 + M + path)
    w = gpu_weights(d)
    plain, _ = run_gpu(d, path=path, w=w, ec=False)
    off = []
    for mod in [dict(hard=1, tau=1.0), dict(A=np.zeros_like(d["ec"]["A"])),
                dict(b=-math.inf)]:
        y, _ = run_gpu(d, path=path, w=w, ec=dict(d["ec"], **mod))
        if path == sp.PATH_DECODE:
            assert_reordered(y, plain, f"EC off {mod}")
        else:
            assert np.array_equal(y, plain), mod
        off.append(y)
    assert np.array_equal(off[0], off[1]) and np.array_equal(off[0], off[2])
    y1, _ = run_gpu(d, path=path, w=w)
    y2, _ = run_gpu(d, path=path, w=w)
    assert np.array_equal(y1, y2)
    assert not np.array_equal(y1, plain)


def test_rows_independent_of_batch():
    d = random_case(12, 96, 512, 16, oracle.CODES_S4, 1, seed=77)
    w = gpu_weights(d)
    y, _ = run_gpu(d, path=sp.PATH_DECODE, w=w)
    for m in [0, 5, 11]:
        dm = dict(d, M=1, x=d["x"][m:m + 1])
        ym, _ = run_gpu(dm, path=sp.PATH_DECODE, w=w)
        np.testing.assert_allclose(ym[0], y[m], rtol=0, atol=1e-5)


def test_workspace_reuse_across_calls():
    """One workspace serves a sequence of calls of different shapes that each
    make one launch with a launch epoch (the fused decode kernel, or the K-split
    GEMM with the pre-pass in its first blocks): each call advances every one of
    the 64 launch counters after the 256-byte header (64-bit, 128 bytes apart)
    by exactly 2^32, whatever its grid, and leaves the header words zero."""
    ws = sp.new_workspace(64, 1024, 4096, 64)
    shapes = [(1, 1024, 4096, 64, sp.PATH_DECODE), (64, 1024, 4096, 64, sp.PATH_PREFILL),
              (16, 512, 2048, 32, sp.PATH_DECODE), (40, 1024, 4096, 64, sp.PATH_PREFILL),
              (4, 1024, 4096, 64, sp.PATH_DECODE), (1, 1024, 4096, 64, sp.PATH_DECODE)]
    for (M, N, K, r, path) in shapes:
        d = random_case(M, N, K, r, oracle.CODES_U4, 1, seed=M + N + K)
        assert ws.numel() >= sp.spear_w4_linear_workspace_size(M, N, K, r)
        y, _ = run_gpu(d, path=path, ws=ws)
        assert_close(y, run_oracle(d), f"ws reuse {M}x{N}x{K} path={path}")
    head = host(ws[:256 + 64 * 128])
    assert np.all(head[:256] == 0)
    ctr = head[256:].view(np.uint64)[::16]
    assert ctr.shape == (64,)
    assert np.all(ctr == np.uint64(len(shapes) << 32)), ctr


def nan_or_exact(y, full, n, blocks, what):
    """After a forced short wait: every output is NaN or equal to the full
    result, NaN comes in whole blocks (each NaN element lies in some fully NaN
    block of one of the listed (rows, cols) shapes), and some wait expired
    (n > 0) exactly when some output is NaN."""
    nan = np.isnan(y)
    ok = nan | np.isclose(y, full, rtol=0, atol=1e-5)
    assert np.all(ok), what
    M, N = y.shape
    for (m, c) in zip(*np.nonzero(nan)):
        covered = False
        for (br, bc) in blocks:
            r0, c0 = (m // br) * br, (c // bc) * bc
            if np.all(nan[r0:min(r0 + br, M), c0:min(c0 + bc, N)]):
                covered = True
                break
        assert covered, (what, m, c)
    print(f"[timeout] {what}: expired waits {n}, NaN outputs {int(nan.sum())}", flush=True)
    assert (n > 0) == bool(nan.any()), (what, n, int(nan.sum()))


def test_forced_wait_timeout_is_reported():
    """A wait limit of one poll makes the fused decode epilogues give up early:
    the call still completes, each 16-channel group's outputs are either exact
    or NaN for every token (never a finite wrong value), the expired waits are
    counted, n_active is -1 when the first group gave up, and the next call with
    the default limit is exact again."""
    d = random_case(4, 4096, 4096, 32, oracle.CODES_U4, 0, seed=9)
    w = gpu_weights(d)
    ws = sp.new_workspace(4, 4096, 4096, 32)
    full, e = run_gpu(d, path=sp.PATH_DECODE, w=w, ws=ws)
    assert sp.spear_workspace_timeouts(ws) == 0
    assert_close(full, run_oracle(d), "fused decode before the forced timeouts")
    try:
        sp.spear_set_wait_limit(1)
        y, e = run_gpu(d, path=sp.PATH_DECODE, w=w, ws=ws)
        n = sp.spear_workspace_timeouts(ws)
    finally:
        sp.spear_set_wait_limit(0)
    nan_or_exact(y, full, n, [(4, 16)], "fused decode")
    nact = int(e.n_active_out.item())
    assert nact in (-1, 4)
    if nact == -1:
        assert np.all(np.isnan(y[:, :16]))
        assert np.all(np.isnan(host(e.g_out)))
    y, _ = run_gpu(d, path=sp.PATH_DECODE, w=w, ws=ws)
    assert np.array_equal(y, full)


def test_decode_ksplit_wait_timeout_is_reported():
    """Decode with K split over workgroups: the channel group's last range waits,
    bounded, for the other ranges' tagged sums.  With a wait limit of one poll it
    may give up: those channels are then NaN for every token and the expiry is
    counted; with the default limit the next call is exact."""
    d = random_case(16, 512, 8192, 32, oracle.CODES_U4, 0, seed=23)
    w = gpu_weights(d)
    ws = sp.new_workspace(16, 512, 8192, 32)
    full, _ = run_gpu(d, path=sp.PATH_DECODE, w=w, ws=ws, ec=False)
    assert_close(full, run_oracle(d, ec=None), "decode K split")
    assert sp.spear_workspace_timeouts(ws) == 0
    try:
        sp.spear_set_wait_limit(1)
        y, _ = run_gpu(d, path=sp.PATH_DECODE, w=w, ws=ws, ec=False)
        n = sp.spear_workspace_timeouts(ws)
    finally:
        sp.spear_set_wait_limit(0)
    nan_or_exact(y, full, n, [(16, 16)], "decode K split")
    y, _ = run_gpu(d, path=sp.PATH_DECODE, w=w, ws=ws, ec=False)
    assert np.array_equal(y, full)


@pytest.mark.parametrize("r", [32, 64])
def test_prepass_wait_timeout_gives_nan(r):
    """The split pre-pass's finisher waits, bounded, for the other slices' tagged
    words, and here (the pre-pass in the GEMM's launch) the GEMM epilogues wait
    the same way for the pre-pass blocks' tagged v.  With a wait limit of one
    poll either may give up: a 16-token group's rows (pre-pass) or a 64 x 64
    tile (epilogue) are then NaN, n_active is -1 if the gate is incomplete, the
    expiry is counted, and the next call with the default limit is exact."""
    d = random_case(32, 512, 4096, r, oracle.CODES_U4, 0, seed=19 + r)
    w = gpu_weights(d)
    ws = sp.new_workspace(32, 512, 4096, r)
    full, _ = run_gpu(d, path=sp.PATH_PREFILL, w=w, ws=ws)
    assert_close(full, run_oracle(d), f"split pre-pass r={r}")
    assert sp.spear_workspace_timeouts(ws) == 0
    try:
        sp.spear_set_wait_limit(1)
        y, e = run_gpu(d, path=sp.PATH_PREFILL, w=w, ws=ws)
        n = sp.spear_workspace_timeouts(ws)
    finally:
        sp.spear_set_wait_limit(0)
    nan_or_exact(y, full, n, [(16, 512), (64, 64)], f"prefill r={r}")
    nact = int(e.n_active_out.item())
    assert nact in (-1, 32)
    gnan = np.isnan(host(e.g_out))
    assert (nact == -1) == bool(gnan.any())
    for g0 in range(0, 32, 16):
        if gnan[g0:g0 + 16].any():
            assert np.all(gnan[g0:g0 + 16]) and np.all(np.isnan(y[g0:g0 + 16]))
    y, _ = run_gpu(d, path=sp.PATH_PREFILL, w=w, ws=ws)
    assert np.array_equal(y, full)


@pytest.mark.parametrize("M", [1, 16, 128, 2048])
def test_c5_stack_layers_sampled(M):
    ec_layer = gen.c5_ec_layers()[0]
    for (layer, lin) in [(ec_layer, "down"), (ec_layer, "q"), (ec_layer, "up"),
                         (0 if ec_layer else 1, "up")]:
        d = gen.make_c5(layer, lin, M)
        rng = np.random.default_rng(M + layer)
        S = 1500
        ms, ns = rng.integers(0, M, S), rng.integers(0, d["N"], S)
        packed, _ = oracle.pack_w4(d["codes"], d["kind"])
        ref = oracle.w4_linear_sampled(d["x"], packed, d["scales"], d["zeros"], d["ec"], ms, ns)
        y, e = run_gpu(d)
        assert_close(y[ms, ns], ref, f"C5 {d['name']} M={M}")
        if d["ec"] is not None:
            gref = oracle.gate(d["x"], d["ec"]["w_g"], 0.0, 0.5, 1)
            n = int(e.n_active_out.item())
            assert n == gref["n_active"]
            assert np.array_equal(host(e.idx_out)[:n], gref["idx"])


@pytest.mark.parametrize("M,N,K", [(1, 4096, 4096), (4, 4112, 4096), (1, 2048, 8192), (8, 2048, 8192),
                                   (12, 2048, 8192), (16, 1000, 4096)])
def test_decode_stream_waves_parity(M, N, K):
    """Plain and two-pass decode stream with 8 waves a workgroup where the
    workgroup's K range is at least 32 super-steps and the grid at most 256
    workgroups, else 4 (4112 channels: 257 groups; 12 and 16 tokens: K split):
    both sides of that choice match the oracle, plain and with the EC."""
    d = random_case(M, N, K, 32, oracle.CODES_U4, 0, seed=40 + M + N + K)
    w = gpu_weights(d)
    plain, _ = run_gpu(d, path=sp.PATH_DECODE, w=w, ec=False)
    assert_close(plain, run_oracle(d, ec=None), f"plain decode {M}x{N}x{K}")
    ref = run_oracle(d)
    for path in (sp.PATH_DECODE, sp.PATH_DECODE_2PASS):
        y, _ = run_gpu(d, path=path, w=w)
        assert_close(y, ref, f"decode {M}x{N}x{K} path={path}")


@pytest.mark.parametrize("K", [1056, 4096, 8192])
@pytest.mark.parametrize("bias", [-4.0, 0.0, 4.0])
def test_decode_one_token_hard_gate(K, bias):
    """One token, hard gate: the stream workgroups form the gate logit
    themselves (all of K in one workgroup) and a skipped token takes no EC
    exchange; with K split over workgroups the producers' logit decides.  The
    bias moves the token to either side of the threshold; the output, the gate
    value and the selection match the oracle."""
    d = random_case(1, 1000, K, 32, oracle.CODES_U4, 1, seed=900 + K)
    d["ec"] = dict(d["ec"], b=bias)
    gref = oracle.gate(d["x"], d["ec"]["w_g"], bias, d["ec"]["tau"], 1)
    w = gpu_weights(d)
    for path in (sp.PATH_DECODE, sp.PATH_DECODE_2PASS):
        y, e = run_gpu(d, path=path, w=w)
        assert_close(y, run_oracle(d), f"one token hard gate K={K} b={bias} path={path}")
        n = int(e.n_active_out.item())
        assert n == gref["n_active"]
        assert np.array_equal(host(e.idx_out)[:n], gref["idx"])
        np.testing.assert_allclose(host(e.g_out)[:1], gref["g"], rtol=2e-7)
    if gref["n_active"] == 0:
        # the skipped token's output is the fused kernel's own W4 sum: bitwise
        # that of a selected token whose EC term is an exact zero (A = 0), and
        # the plain layer's up to the reordered sum
        plain, _ = run_gpu(d, path=sp.PATH_DECODE, w=w, ec=False)
        y, _ = run_gpu(d, path=sp.PATH_DECODE, w=w)
        zero_a = dict(d["ec"], A=np.zeros_like(d["ec"]["A"]), b=bias + 100.0)
        y0, e0 = run_gpu(d, path=sp.PATH_DECODE, w=w, ec=zero_a)
        assert int(e0.n_active_out.item()) == 1
        assert np.array_equal(y, y0)
        assert_reordered(y, plain, f"one token skipped K={K}")


@pytest.mark.parametrize("M", [2, 16])
def test_decode_mixed_activity(M):
    """Several tokens under the hard gate, some selected and some not (the
    bias puts the threshold inside the tokens' logits): per-token EC terms,
    the selection list and the count match the oracle on every decode path."""
    d = random_case(M, 640, 2048, 32, oracle.CODES_S4, 1, seed=70 + M)
    gref = oracle.gate(d["x"], d["ec"]["w_g"], d["ec"]["b"], d["ec"]["tau"], 1)
    z = np.sort(gref["z"])
    b = float(d["ec"]["b"] - (z[M // 2 - 1] + z[M // 2]) / 2)   # about half selected
    d["ec"] = dict(d["ec"], b=b)
    gref = oracle.gate(d["x"], d["ec"]["w_g"], b, d["ec"]["tau"], 1)
    assert 0 < gref["n_active"] < M
    ref = run_oracle(d)
    w = gpu_weights(d)
    for path in (sp.PATH_DECODE, sp.PATH_DECODE_2PASS, sp.PATH_PREFILL):
        y, e = run_gpu(d, path=path, w=w)
        assert_close(y, ref, f"mixed activity M={M} path={path}")
        n = int(e.n_active_out.item())
        assert n == gref["n_active"]
        assert np.array_equal(host(e.idx_out)[:n], gref["idx"])
