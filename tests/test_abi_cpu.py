"""The C ABI on the CPU: the library loads, exports every function that
include/spear.h declares, sizes workspaces, and rejects bad arguments with the
documented status before making any HIP call (no GPU is touched here)."""
import ctypes
import os
import re

import pytest

from quantized_gemm_w4a16_amd import spear as sp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spear.h")

E_NULL, E_SHAPE, E_ALIGN, E_ARG, E_WS = -1, -2, -3, -4, -5


@pytest.fixture(scope="module")
def lib():
    return sp.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spear_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(sp.EXPORTS)
    assert lib.spear_abi_version() == sp.ABI_VERSION == 2


def test_status_strings(lib):
    for st in range(-7, 1):
        assert sp.spear_status_string(st)
    assert sp.spear_status_string(-99) == "unknown status"


def test_workspace_size_layout(lib):
    f = sp.spear_w4_linear_workspace_size
    for (M, N, K, r) in [(1, 4096, 4096, 32), (16, 1024, 1024, 16), (64, 14336, 4096, 64),
                         (4096, 4096, 4096, 32), (3, 17, 96, 8), (1, 16, 32, 0)]:
        n = f(M, N, K, r)
        assert n > 0 and n % 256 == 0
        assert f(M, N, K, 0) <= n
    assert f(-1, 16, 32, 0) == 0 and f(1, 0, 32, 0) == 0 and f(1, 16, 16, 0) == 0


def test_workspace_size_monotone_in_tokens(lib):
    """A workspace sized for M tokens serves every smaller M (decode and prefill
    share one allocation): the size never decreases as M grows."""
    f = sp.spear_w4_linear_workspace_size
    for (N, K, r) in [(4096, 4096, 32), (1024, 11008, 64), (512, 2048, 256), (17, 96, 8),
                      (4096, 32768, 32), (64, 4096, 0), (2048, 2048, 32), (8192, 2048, 32),
                      (2048, 8192, 32), (14336, 4096, 64)]:
        # across the tile switches (64-token tiles up to 128 tokens) and K splits
        Ms = list(range(1, 40)) + [63, 64, 65, 96, 127, 128, 129, 150, 255, 256, 257, 300,
                                   512, 1000, 2047, 2048, 2049, 4096]
        sizes = [f(M, N, K, r) for M in Ms]
        assert all(b >= a for a, b in zip(sizes, sizes[1:])), (N, K, r, sizes)


A16 = 0x10000          # fake, suitably aligned device addresses: never dereferenced


def linear(lib, x=A16, M=4, N=64, K=128, ec=None, y=A16, out=1, ws=A16, wsb=1 << 20,
           path=0, packed=A16, scales=A16, zeros=None):
    w = sp._W4(packed, scales, zeros, N, K)
    return lib.spear_w4_linear_path(x, M, ctypes.byref(w), ctypes.byref(ec) if ec else None,
                                    y, out, ws, wsb, path, None)


def ec_struct(r=16, tau=0.5, hard=0, A=A16, B=A16, wg=A16, b=0.0, gate_h=0, alpha=1.0,
              w1=A16, c1=A16, w2=A16, c2=A16):
    return sp._EC(A, B, wg, b, tau, hard, r, None, None, None, gate_h, alpha, w1, c1, w2, c2)


def test_linear_validation(lib):
    assert linear(lib, x=None) == E_NULL
    assert linear(lib, y=None) == E_NULL
    assert linear(lib, ws=None) == E_NULL
    assert linear(lib, packed=None) == E_NULL
    assert linear(lib, ec=ec_struct(A=None)) == E_NULL
    assert linear(lib, K=48) == E_SHAPE
    assert linear(lib, K=0) == E_SHAPE
    assert linear(lib, N=0) == E_SHAPE
    assert linear(lib, M=-1) == E_SHAPE
    assert linear(lib, ec=ec_struct(r=12)) == E_SHAPE
    assert linear(lib, ec=ec_struct(r=264)) == E_SHAPE
    assert linear(lib, M=17, path=sp.PATH_DECODE) == E_SHAPE
    assert linear(lib, M=17, path=sp.PATH_DECODE_2PASS) == E_SHAPE
    assert linear(lib, path=7) == E_ARG
    assert linear(lib, out=2) == E_ARG
    assert linear(lib, ec=ec_struct(tau=float("nan"))) == E_ARG
    assert linear(lib, ec=ec_struct(hard=2)) == E_ARG
    assert linear(lib, x=A16 + 8) == E_ALIGN
    assert linear(lib, y=A16 + 4) == E_ALIGN
    assert linear(lib, ws=A16 + 16) == E_ALIGN
    assert linear(lib, ec=ec_struct(B=A16 + 2)) == E_ALIGN
    need = sp.spear_w4_linear_workspace_size(4, 64, 128, 16)
    assert linear(lib, ec=ec_struct(), wsb=need - 1) == E_WS
    # the vector gate's MLP
    assert linear(lib, ec=ec_struct(gate_h=65)) == E_SHAPE
    assert linear(lib, ec=ec_struct(gate_h=-1)) == E_SHAPE
    assert linear(lib, ec=ec_struct(gate_h=4, w1=None)) == E_NULL
    assert linear(lib, ec=ec_struct(gate_h=4, c2=None)) == E_NULL
    assert linear(lib, ec=ec_struct(gate_h=4, alpha=float("nan"))) == E_ARG
    assert linear(lib, ec=ec_struct(gate_h=4, w2=A16 + 2)) == E_ALIGN
    # gate_h = 0: the MLP pointers are not read
    assert linear(lib, ec=ec_struct(gate_h=0, w1=None, c1=None, w2=None, c2=None),
                  wsb=need - 1) == E_WS


def test_pack_and_gate_validation(lib):
    assert lib.spear_pack_w4(None, 0, 4, 64, A16, None, None) == E_NULL
    assert lib.spear_pack_w4(A16, 0, 4, 48, A16, None, None) == E_SHAPE
    assert lib.spear_pack_w4(A16, 0, 0, 64, A16, None, None) == E_SHAPE
    assert lib.spear_pack_w4(A16, 3, 4, 64, A16, None, None) == E_ARG
    assert lib.spear_pack_w4(A16 + 1, 0, 4, 64, A16, None, None) == E_ALIGN
    assert lib.spear_gate(A16, 4, 64, None, 0.0, 0.5, 0, A16, A16, A16, None) == E_NULL
    assert lib.spear_gate(A16, 4, 40, A16, 0.0, 0.5, 0, A16, A16, A16, None) == E_SHAPE
    assert lib.spear_gate(A16, 4, 64, A16, 0.0, float("nan"), 0, A16, A16, A16, None) == E_ARG
    assert lib.spear_gate(A16, 4, 64, A16, 0.0, 0.5, 5, A16, A16, A16, None) == E_ARG
    assert lib.spear_gate(A16 + 2, 4, 64, A16, 0.0, 0.5, 0, A16, A16, A16, None) == E_ALIGN
    assert lib.spear_workspace_init(None, 1024, None) == E_NULL
    assert lib.spear_workspace_init(A16, 16, None) == E_WS
    assert lib.spear_workspace_init(A16 + 64, 1024, None) == E_ALIGN
