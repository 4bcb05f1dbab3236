"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The oracle (plain C) and the chunk picker (plain C++ host code of the library)
are rebuilt with -fsanitize=address,undefined into a temporary directory and
exercised in a child Python process that preloads the sanitizer runtimes:
pack / unpack, the gate, the full and the sampled layer with the scalar and
the vector gate, and the chunk picker's prediction and choice.  Any report
aborts the child, so the test fails on the first memory error or undefined
operation.
"""
import os
import shutil
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = textwrap.dedent(r"""
    import ctypes, sys
    import numpy as np
    sys.path.insert(0, ROOT)
    import oracle
    from quantized_gemm_w4a16_amd import inputs as gen
    from quantized_gemm_w4a16_amd import spear as sp
    oracle._LIB = ORACLE_LIB

    d = gen.make(1)                                   # M = 16, K = N = 1024, rank 16
    packed, bad = oracle.pack_w4(d["codes"], d["kind"])
    assert bad == 0
    u = d["codes"].astype(np.int16) + (8 if d["kind"] == oracle.CODES_S4 else 0)
    assert np.array_equal(oracle.unpack_w4(packed, d["K"]), u)     # stored nibbles
    e = d["ec"]
    g = oracle.gate(d["x"], e["w_g"], e["b"], e["tau"], 1)
    y = oracle.w4_linear(d["x"], packed, d["scales"], d["zeros"], e)
    rng = np.random.default_rng(7)
    r, h = e["r"], 8
    ev = dict(e, gate_h=h, alpha=0.8,
              gate_w1=rng.normal(0, 0.5, (h, r)).astype(np.float32),
              gate_c1=rng.normal(0, 0.1, h).astype(np.float32),
              gate_w2=rng.normal(0, 0.5, (r, h)).astype(np.float32),
              gate_c2=rng.normal(0, 0.5, r).astype(np.float32))
    yv = oracle.w4_linear(d["x"], packed, d["scales"], d["zeros"], ev)
    ms, ns = rng.integers(0, d["M"], 64), rng.integers(0, d["N"], 64)
    ys = oracle.w4_linear_sampled(d["x"], packed, d["scales"], d["zeros"], ev, ms, ns)
    assert np.allclose(ys, yv[ms, ns], rtol=0, atol=0)
    assert np.isfinite(y).all() and np.isfinite(yv).all()

    lib = ctypes.CDLL(SLO_LIB)
    lut_t = sp._LUT
    tok = np.array([1, 16, 128, 1024, 4096], np.int32)
    us = np.array([[5, 6, 9, 40, 150], [7, 8, 12, 50, 170]], np.float32)
    cnt = np.array([24, 4], np.int32)
    lut = lut_t(len(tok), tok.ctypes.data, 2, us.ctypes.data, cnt.ctypes.data, 30.0)
    f = ctypes.c_float()
    for t in (0, 1, 50, 4096, 10000):
        assert lib.spear_slo_predict(ctypes.byref(lut), t, ctypes.byref(f)) == 0
    c = ctypes.c_int32()
    for (nd, pend, align, slo) in [(16, 5000, 64, 3000.0), (0, 0, 1, 100.0), (300, 4096, 256, 1.0)]:
        assert lib.spear_slo_pick_chunk(ctypes.byref(lut), nd, pend, align, ctypes.c_float(slo),
                                        ctypes.byref(c), ctypes.byref(f)) == 0
    print("sanitized host code: ok")
""")


def _tool(name):
    p = shutil.which(name)
    if p is None:
        pytest.skip(f"{name} not found")
    return p


def test_host_code_under_asan_ubsan(tmp_path):
    gcc, gxx = _tool("gcc"), _tool("g++")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", "-g", "-O1"]
    olib = str(tmp_path / "liboracle_asan.so")
    subprocess.run([gcc, "-std=c99", "-fopenmp", "-fPIC", "-shared", *san, "-o", olib,
                    os.path.join(ROOT, "oracle", "spear_oracle.c"), "-lm"], check=True)
    slib = str(tmp_path / "libslo_asan.so")
    subprocess.run([gxx, "-std=c++17", "-fPIC", "-shared", *san, "-o", slib,
                    os.path.join(ROOT, "quantized_gemm_w4a16_amd", "csrc", "slo.cpp")], check=True)
    runtimes = [subprocess.run([gcc, f"-print-file-name={n}"], capture_output=True, text=True,
                               check=True).stdout.strip() for n in ("libasan.so", "libubsan.so")]
    # the sanitizer runtimes must come first; whatever the environment already
    # preloads stays, after them
    pre = ":".join(runtimes + ([os.environ["LD_PRELOAD"]] if os.environ.get("LD_PRELOAD") else []))
    env = dict(os.environ,
               LD_PRELOAD=pre,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               OMP_NUM_THREADS="2")
    code = f"ROOT = {ROOT!r}\nORACLE_LIB = {olib!r}\nSLO_LIB = {slib!r}\n" + CHILD
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "sanitized host code: ok" in r.stdout
