"""Thin ctypes binding of libspear (the C ABI declared in include/spear.h).

Argument marshalling only: tensors are passed as device pointers together with
torch's current HIP stream; every step of the layer runs in the library's
kernels.  The library is opened on first use; if it has not been built the
call raises (there is no fallback path).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspear.so")

SPEAR_OK = 0
CODES_S4 = 0
CODES_U4 = 1
OUT_BF16 = 0
OUT_F32 = 1
PATH_AUTO = 0
PATH_DECODE = 1
PATH_PREFILL = 2
PATH_DECODE_2PASS = 3
PATH_PREFILL_LARGE = 4
MAX_RANK = 256
MAX_GATE_HIDDEN = 64
ABI_VERSION = 2

EXPORTS = ("spear_pack_w4", "spear_gate", "spear_w4_linear_workspace_size",
           "spear_workspace_init", "spear_w4_linear", "spear_w4_linear_path",
           "spear_w4_linear_noalloc", "spear_w4_linear_semifused",
           "spear_set_wait_limit", "spear_workspace_timeouts", "spear_stream_read",
           "spear_slo_predict", "spear_slo_pick_chunk", "spear_status_string",
           "spear_abi_version")


class SpearError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: status {status} ({msg})")
        self.status = status


class _W4(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("zeros", ctypes.c_void_p), ("N", ctypes.c_int64), ("K", ctypes.c_int64)]


class _EC(ctypes.Structure):
    _fields_ = [("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("w_gate", ctypes.c_void_p),
                ("b", ctypes.c_float), ("tau", ctypes.c_float), ("hard", ctypes.c_int32),
                ("r", ctypes.c_int32), ("g_out", ctypes.c_void_p), ("idx_out", ctypes.c_void_p),
                ("n_active_out", ctypes.c_void_p), ("gate_h", ctypes.c_int32),
                ("alpha", ctypes.c_float), ("gate_w1", ctypes.c_void_p),
                ("gate_c1", ctypes.c_void_p), ("gate_w2", ctypes.c_void_p),
                ("gate_c2", ctypes.c_void_p)]


class _LUT(ctypes.Structure):
    _fields_ = [("npoints", ctypes.c_int32), ("tokens", ctypes.c_void_p),
                ("nkinds", ctypes.c_int32), ("us", ctypes.c_void_p), ("count", ctypes.c_void_p),
                ("overhead_us", ctypes.c_float)]


_lib = None


def load():
    """Open libspear.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libspear.so not found at {LIB_PATH}; build it with "
                           "quantized_gemm_w4a16_amd.build.build()")
    lib = ctypes.CDLL(LIB_PATH)
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.spear_pack_w4.argtypes = [P, i32, i64, i64, P, P, P]
    lib.spear_gate.argtypes = [P, i64, i64, P, ctypes.c_float, ctypes.c_float, i32, P, P, P, P]
    lib.spear_w4_linear_workspace_size.argtypes = [i64, i64, i64, i32]
    lib.spear_w4_linear_workspace_size.restype = ctypes.c_size_t
    lib.spear_workspace_init.argtypes = [P, ctypes.c_size_t, P]
    lin = [P, i64, ctypes.POINTER(_W4), ctypes.POINTER(_EC), P, i32, P, ctypes.c_size_t]
    lib.spear_w4_linear.argtypes = lin + [P]
    lib.spear_w4_linear_path.argtypes = lin + [i32, P]
    lib.spear_w4_linear_noalloc.argtypes = [P, i64, ctypes.POINTER(_W4), ctypes.POINTER(_EC), P,
                                            i32, i32, P]
    lib.spear_w4_linear_semifused.argtypes = [P, i64, ctypes.POINTER(_W4), ctypes.POINTER(_EC), P,
                                              P, ctypes.c_size_t, P, P, P, P]
    lib.spear_set_wait_limit.argtypes = [ctypes.c_uint32]
    lib.spear_set_wait_limit.restype = None
    lib.spear_workspace_timeouts.argtypes = [P, ctypes.POINTER(i32), P]
    lib.spear_stream_read.argtypes = [P, ctypes.c_size_t, P, P]
    lib.spear_slo_predict.argtypes = [ctypes.POINTER(_LUT), i32, ctypes.POINTER(ctypes.c_float)]
    lib.spear_slo_pick_chunk.argtypes = [ctypes.POINTER(_LUT), i32, i32, i32, ctypes.c_float,
                                         ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_float)]
    lib.spear_status_string.argtypes = [i32]
    lib.spear_status_string.restype = ctypes.c_char_p
    lib.spear_abi_version.restype = i32
    for name in ("spear_pack_w4", "spear_gate", "spear_workspace_init", "spear_w4_linear",
                 "spear_w4_linear_path", "spear_w4_linear_noalloc", "spear_w4_linear_semifused",
                 "spear_workspace_timeouts",
                 "spear_stream_read", "spear_slo_predict", "spear_slo_pick_chunk"):
        getattr(lib, name).restype = i32
    _lib = lib
    return lib


def _check(fn: str, st: int):
    if st != SPEAR_OK:
        raise SpearError(fn, st, load().spear_status_string(st).decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


@dataclass
class W4:
    """Packed weights on the device: packed [N][K/2] uint8, scales [N] fp32,
    zeros [N] uint8 or None (zero point 8)."""
    packed: torch.Tensor
    scales: torch.Tensor
    zeros: Optional[torch.Tensor]
    N: int
    K: int

    def _c(self):
        return _W4(_ptr(self.packed), _ptr(self.scales), _ptr(self.zeros), self.N, self.K)


@dataclass
class EC:
    """Error compensator on the device: A [r][K], B [N][r], w_gate [K] as bf16
    (torch.bfloat16 or int16 bit tensors), gate bias b, threshold tau, hard flag.
    Optional outputs g_out [M] fp32, idx_out [M] int32, n_active_out [1] int32.
    Optional vector gate (fp32): gate_w1 [h][r], gate_c1 [h], gate_w2 [r][h],
    gate_c2 [r] and its scale alpha."""
    A: torch.Tensor
    B: torch.Tensor
    w_gate: torch.Tensor
    b: float = 0.0
    tau: float = 0.0
    hard: int = 0
    g_out: Optional[torch.Tensor] = None
    idx_out: Optional[torch.Tensor] = None
    n_active_out: Optional[torch.Tensor] = None
    gate_w1: Optional[torch.Tensor] = None
    gate_c1: Optional[torch.Tensor] = None
    gate_w2: Optional[torch.Tensor] = None
    gate_c2: Optional[torch.Tensor] = None
    alpha: float = 1.0

    @property
    def r(self) -> int:
        return int(self.A.shape[0])

    @property
    def gate_h(self) -> int:
        return 0 if self.gate_w1 is None else int(self.gate_w1.shape[0])

    def _c(self):
        return _EC(_ptr(self.A), _ptr(self.B), _ptr(self.w_gate), float(self.b), float(self.tau),
                   int(self.hard), self.r, _ptr(self.g_out), _ptr(self.idx_out),
                   _ptr(self.n_active_out), self.gate_h, float(self.alpha), _ptr(self.gate_w1),
                   _ptr(self.gate_c1), _ptr(self.gate_w2), _ptr(self.gate_c2))


def spear_abi_version() -> int:
    return int(load().spear_abi_version())


def spear_status_string(st: int) -> str:
    return load().spear_status_string(st).decode()


def spear_pack_w4(codes: torch.Tensor, kind: int, packed: Optional[torch.Tensor] = None,
                  bad_codes: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    N, K = codes.shape
    if packed is None:
        packed = torch.empty((N, K // 2), dtype=torch.uint8, device=codes.device)
    _check("spear_pack_w4", load().spear_pack_w4(_ptr(codes), kind, N, K, _ptr(packed),
                                                 _ptr(bad_codes), _stream(stream)))
    return packed


def spear_gate(x: torch.Tensor, w_gate: torch.Tensor, b: float, tau: float, hard: int,
               g=None, idx=None, n_active=None, stream=None):
    M, K = x.shape
    dev = x.device
    g = torch.empty(M, dtype=torch.float32, device=dev) if g is None else g
    idx = torch.empty(max(M, 1), dtype=torch.int32, device=dev) if idx is None else idx
    n_active = torch.empty(1, dtype=torch.int32, device=dev) if n_active is None else n_active
    _check("spear_gate", load().spear_gate(_ptr(x), M, K, _ptr(w_gate), float(b), float(tau),
                                           int(hard), _ptr(g), _ptr(idx), _ptr(n_active),
                                           _stream(stream)))
    return g, idx, n_active


def spear_w4_linear_workspace_size(M: int, N: int, K: int, r: int) -> int:
    return int(load().spear_w4_linear_workspace_size(M, N, K, r))


def spear_workspace_init(ws: torch.Tensor, stream=None):
    _check("spear_workspace_init", load().spear_workspace_init(_ptr(ws), ws.numel(),
                                                               _stream(stream)))


def new_workspace(M: int, N: int, K: int, r: int, device="cuda") -> torch.Tensor:
    """A zero-filled workspace tensor of the required size (torch allocation)."""
    n = max(spear_w4_linear_workspace_size(M, N, K, r), 256)
    return torch.zeros(n, dtype=torch.uint8, device=device)


def spear_w4_linear(x: torch.Tensor, w: W4, ec: Optional[EC] = None,
                    y: Optional[torch.Tensor] = None, out_dtype: int = OUT_F32,
                    workspace: Optional[torch.Tensor] = None, path: int = PATH_AUTO,
                    stream=None) -> torch.Tensor:
    M = int(x.shape[0])
    if y is None:
        dt = torch.float32 if out_dtype == OUT_F32 else torch.bfloat16
        y = torch.empty((M, w.N), dtype=dt, device=x.device)
    if workspace is None:
        workspace = new_workspace(M, w.N, w.K, ec.r if ec is not None else 0, x.device)
    wc = w._c()
    ecc = ec._c() if ec is not None else None
    st = load().spear_w4_linear_path(_ptr(x), M, ctypes.byref(wc),
                                     ctypes.byref(ecc) if ecc is not None else None,
                                     _ptr(y), out_dtype, _ptr(workspace), workspace.numel(),
                                     path, _stream(stream))
    _check("spear_w4_linear", st)
    return y


class SemiFused:
    """The second stream and the two events of the semi-fused prefill (torch
    objects; the events are recorded once so that their HIP handles exist)."""

    def __init__(self, device="cuda"):
        self.aux = torch.cuda.Stream(device=device)
        self.ev_fork = torch.cuda.Event()
        self.ev_join = torch.cuda.Event()
        self.ev_fork.record(self.aux)
        self.ev_join.record(self.aux)
        self.aux.synchronize()


def spear_w4_linear_semifused(x: torch.Tensor, w: W4, ec: Optional[EC], sf: SemiFused,
                              y: Optional[torch.Tensor] = None,
                              workspace: Optional[torch.Tensor] = None,
                              stream=None) -> torch.Tensor:
    """The prefill layer with the EC as a separate kernel on sf.aux (fp32 y)."""
    M = int(x.shape[0])
    if y is None:
        y = torch.empty((M, w.N), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = new_workspace(M, w.N, w.K, ec.r if ec is not None else 0, x.device)
    wc = w._c()
    ecc = ec._c() if ec is not None else None
    st = load().spear_w4_linear_semifused(_ptr(x), M, ctypes.byref(wc),
                                          ctypes.byref(ecc) if ecc is not None else None,
                                          _ptr(y), _ptr(workspace), workspace.numel(),
                                          _stream(stream), sf.aux.cuda_stream,
                                          sf.ev_fork.cuda_event, sf.ev_join.cuda_event)
    _check("spear_w4_linear_semifused", st)
    return y


NOALLOC_MAX_WORKSPACE = 48 << 20


def spear_w4_linear_noalloc(x: torch.Tensor, w: W4, ec: Optional[EC] = None,
                            y: Optional[torch.Tensor] = None, out_dtype: int = OUT_F32,
                            path: int = PATH_AUTO, stream=None) -> torch.Tensor:
    """The layer through the allocation-free entry point (the library's own
    scratch stands in for the workspace).  y must be given by callers that
    cannot allocate; it is allocated here only for convenience when None."""
    M = int(x.shape[0])
    if y is None:
        dt = torch.float32 if out_dtype == OUT_F32 else torch.bfloat16
        y = torch.empty((M, w.N), dtype=dt, device=x.device)
    wc = w._c()
    ecc = ec._c() if ec is not None else None
    st = load().spear_w4_linear_noalloc(_ptr(x), M, ctypes.byref(wc),
                                        ctypes.byref(ecc) if ecc is not None else None,
                                        _ptr(y), out_dtype, path, _stream(stream))
    _check("spear_w4_linear_noalloc", st)
    return y


def spear_set_wait_limit(rounds: int):
    load().spear_set_wait_limit(int(rounds))


def spear_workspace_timeouts(ws: torch.Tensor, stream=None) -> int:
    out = ctypes.c_int32(0)
    _check("spear_workspace_timeouts", load().spear_workspace_timeouts(_ptr(ws), ctypes.byref(out),
                                                                       _stream(stream)))
    return int(out.value)


def spear_stream_read(buf: torch.Tensor, sink: torch.Tensor, nbytes: Optional[int] = None,
                      stream=None):
    """Measurement helper: read every byte of buf once (the plain read floor)."""
    n = buf.numel() * buf.element_size() if nbytes is None else nbytes
    _check("spear_stream_read", load().spear_stream_read(_ptr(buf), n, _ptr(sink),
                                                         _stream(stream)))


class SloLut:
    """Kernel-latency table for the chunk picker (host memory): tokens [P]
    ascending, us [kinds][P] microseconds per call, count [kinds] calls per
    step, overhead_us per step."""

    def __init__(self, tokens, us, count, overhead_us=0.0):
        import numpy as np
        self.tokens = np.ascontiguousarray(tokens, dtype=np.int32)
        self.us = np.ascontiguousarray(us, dtype=np.float32)
        self.count = np.ascontiguousarray(count, dtype=np.int32)
        assert self.us.shape == (self.count.shape[0], self.tokens.shape[0])
        self._c = _LUT(self.tokens.shape[0], self.tokens.ctypes.data, self.count.shape[0],
                       self.us.ctypes.data, self.count.ctypes.data, float(overhead_us))

    def predict(self, tokens: int) -> float:
        out = ctypes.c_float(0)
        _check("spear_slo_predict", load().spear_slo_predict(ctypes.byref(self._c), int(tokens),
                                                             ctypes.byref(out)))
        return float(out.value)

    def pick_chunk(self, n_decode: int, pending: int, slo_us: float, align: int = 1):
        c, p = ctypes.c_int32(0), ctypes.c_float(0)
        _check("spear_slo_pick_chunk", load().spear_slo_pick_chunk(
            ctypes.byref(self._c), int(n_decode), int(pending), int(align), float(slo_us),
            ctypes.byref(c), ctypes.byref(p)))
        return int(c.value), float(p.value)
