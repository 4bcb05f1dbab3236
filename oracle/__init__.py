"""CPU oracle for the W4A16 + gated Error-Compensator linear layer.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke``
and by the CPU-baseline leg of ``bench.py``; never by the product package.
It wraps ``spear_oracle.c`` (plain C, fp64 sums) through ctypes.  See that
file's header for the sources and the readings it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "spear_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CODES_S4 = 0
CODES_U4 = 1

_lib = None


def build(verbose: bool = False) -> str:
    """Compile liboracle.so with gcc (always recompiles)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-Wall",
           "-o", _LIB + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i64 = ctypes.c_int64
    lib.oracle_pack_w4.argtypes = [P, ctypes.c_int, i64, i64, P]
    lib.oracle_pack_w4.restype = i64
    lib.oracle_unpack_w4.argtypes = [P, i64, i64, P]
    lib.oracle_unpack_w4.restype = None
    lib.oracle_dequant_w4.argtypes = [P, P, P, i64, i64, P]
    lib.oracle_dequant_w4.restype = None
    lib.oracle_logit_threshold.argtypes = [ctypes.c_float]
    lib.oracle_logit_threshold.restype = ctypes.c_double
    lib.oracle_gate.argtypes = [P, i64, i64, P, ctypes.c_float, ctypes.c_float, ctypes.c_int,
                                P, P, P, P]
    lib.oracle_gate.restype = None
    lin = [P, i64, i64, i64, P, P, P, ctypes.c_int, P, P, i64, P,
           ctypes.c_float, ctypes.c_float, ctypes.c_int, i64, P, P, P, P, ctypes.c_float]
    lib.oracle_w4_linear.argtypes = lin + [P]
    lib.oracle_w4_linear.restype = ctypes.c_int
    lib.oracle_w4_linear_sampled.argtypes = lin + [i64, P, P, P]
    lib.oracle_w4_linear_sampled.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def pack_w4(codes: np.ndarray, kind: int):
    """codes [N][K] (int8 for S4, uint8 for U4) -> (packed [N][K/2] uint8, bad count)."""
    dt = np.int8 if kind == CODES_S4 else np.uint8
    codes = _c(codes, dt)
    N, K = codes.shape
    assert K % 8 == 0, "the packed layout works in words of 8 codes"
    out = np.empty((N, K // 2), dtype=np.uint8)
    bad = _load().oracle_pack_w4(_ptr(codes), kind, N, K, _ptr(out))
    return out, int(bad)


def unpack_w4(packed: np.ndarray, K: int) -> np.ndarray:
    assert K % 8 == 0, "the packed layout works in words of 8 codes"
    packed = _c(packed, np.uint8)
    N = packed.shape[0]
    out = np.empty((N, K), dtype=np.uint8)
    _load().oracle_unpack_w4(_ptr(packed), N, K, _ptr(out))
    return out


def dequant_w4(packed, scales, zeros, K: int) -> np.ndarray:
    packed = _c(packed, np.uint8)
    N = packed.shape[0]
    out = np.empty((N, K), dtype=np.float32)
    _load().oracle_dequant_w4(_ptr(packed), _ptr(_c(scales, np.float32)),
                              _ptr(_c(zeros, np.uint8)), N, K, _ptr(out))
    return out


def logit_threshold(tau: float) -> float:
    return float(_load().oracle_logit_threshold(float(tau)))


def gate(x_bits, w_g_bits, b: float, tau: float, hard: int):
    """-> dict(z fp64 [M], g fp32 [M], idx int32 [n_active], n_active int)."""
    x = _c(x_bits, np.uint16)
    M, K = x.shape
    z = np.empty(M, dtype=np.float64)
    g = np.empty(M, dtype=np.float32)
    idx = np.empty(max(M, 1), dtype=np.int32)
    n = np.zeros(1, dtype=np.int32)
    _load().oracle_gate(_ptr(x), M, K, _ptr(_c(w_g_bits, np.uint16)), float(b), float(tau),
                        int(hard), _ptr(z), _ptr(g), _ptr(idx), _ptr(n))
    return {"z": z, "g": g, "idx": idx[: int(n[0])].copy(), "n_active": int(n[0])}


def _lin_args(x, packed, scales, zeros, ec):
    x = _c(x, np.uint16)
    M, K = x.shape
    packed = _c(packed, np.uint8)
    N = packed.shape[0]
    assert packed.shape[1] * 2 == K
    keep = [x, packed, _c(scales, np.float32), _c(zeros, np.uint8)]
    if ec is None:
        ecargs = [0, None, None, 0, None, 0.0, 0.0, 0, 0, None, None, None, None, 1.0]
    else:
        A = _c(ec["A"], np.uint16)
        B = _c(ec["B"], np.uint16)
        wg = _c(ec["w_g"], np.uint16)
        r = A.shape[0]
        assert A.shape == (r, K) and B.shape == (N, r) and wg.shape == (K,)
        keep += [A, B, wg]
        ecargs = [1, _ptr(A), _ptr(B), r, _ptr(wg), float(ec["b"]), float(ec["tau"]),
                  int(ec["hard"])]
        h = int(ec.get("gate_h", 0) or 0)
        if h:
            W1 = _c(ec["gate_w1"], np.float32)
            c1 = _c(ec["gate_c1"], np.float32)
            W2 = _c(ec["gate_w2"], np.float32)
            c2 = _c(ec["gate_c2"], np.float32)
            assert W1.shape == (h, r) and c1.shape == (h,) and W2.shape == (r, h)
            assert c2.shape == (r,)
            keep += [W1, c1, W2, c2]
            ecargs += [h, _ptr(W1), _ptr(c1), _ptr(W2), _ptr(c2), float(ec.get("alpha", 1.0))]
        else:
            ecargs += [0, None, None, None, None, 1.0]
    args = [_ptr(keep[0]), M, K, N, _ptr(keep[1]), _ptr(keep[2]), _ptr(keep[3])] + ecargs
    return args, keep, M, N


def w4_linear(x_bits, packed, scales, zeros=None, ec=None) -> np.ndarray:
    """Full layer output y [M][N] in fp64.  ec: dict(A [r][K] bf16 bits, B [N][r] bf16 bits,
    w_g [K] bf16 bits, b, tau, hard) or None for the plain W4 linear.  Optional vector
    gate in ec: gate_h (hidden width, 0 = none), gate_w1 [h][r], gate_c1 [h],
    gate_w2 [r][h], gate_c2 [r] (fp32) and alpha."""
    args, keep, M, N = _lin_args(x_bits, packed, scales, zeros, ec)
    y = np.empty((M, N), dtype=np.float64)
    rc = _load().oracle_w4_linear(*args, _ptr(y))
    assert rc == 0, rc
    return y


def w4_linear_sampled(x_bits, packed, scales, zeros, ec, ms, ns) -> np.ndarray:
    """y[ms[i]][ns[i]] in fp64 for the listed output positions."""
    args, keep, M, N = _lin_args(x_bits, packed, scales, zeros, ec)
    ms = _c(ms, np.int64)
    ns = _c(ns, np.int64)
    assert ms.shape == ns.shape
    out = np.empty(ms.shape[0], dtype=np.float64)
    rc = _load().oracle_w4_linear_sampled(*args, ms.shape[0], _ptr(ms), _ptr(ns), _ptr(out))
    assert rc == 0, rc
    return out
