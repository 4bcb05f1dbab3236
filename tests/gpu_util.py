"""Helpers shared by the GPU tests: move seeded numpy inputs to the device, run
the HIP path through the C ABI, run the oracle on the same bits, compare."""
import numpy as np
import torch

import oracle
from quantized_gemm_w4a16_amd import spear as sp

RTOL_L2 = 1e-3      # relative L2 error bound for fp32 outputs
ATOL_MAX = 2e-2     # max absolute error bound for fp32 outputs


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def host(t):
    return t.detach().cpu().numpy()


def gpu_weights(d, pack_on_gpu=True):
    if pack_on_gpu:
        packed = sp.spear_pack_w4(dev(d["codes"]), d["kind"])
    else:
        packed = dev(oracle.pack_w4(d["codes"], d["kind"])[0])
    z = dev(d["zeros"]) if d["zeros"] is not None else None
    return sp.W4(packed, dev(d["scales"]), z, d["N"], d["K"])


def gpu_ec(ec, M, outputs=True):
    if ec is None:
        return None
    e = sp.EC(dev(ec["A"]), dev(ec["B"]), dev(ec["w_g"]), ec["b"], ec["tau"], ec["hard"])
    if ec.get("gate_h", 0):
        e.gate_w1 = dev(np.asarray(ec["gate_w1"], np.float32))
        e.gate_c1 = dev(np.asarray(ec["gate_c1"], np.float32))
        e.gate_w2 = dev(np.asarray(ec["gate_w2"], np.float32))
        e.gate_c2 = dev(np.asarray(ec["gate_c2"], np.float32))
        e.alpha = float(ec.get("alpha", 1.0))
    if outputs:
        e.g_out = torch.full((max(M, 1),), -1.0, dtype=torch.float32, device="cuda")
        e.idx_out = torch.full((max(M, 1),), -1, dtype=torch.int32, device="cuda")
        e.n_active_out = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    return e


def run_gpu(d, path=sp.PATH_AUTO, out=sp.OUT_F32, ec=None, w=None, outputs=True, ws=None):
    """-> (y numpy, ec device object or None)."""
    w = gpu_weights(d) if w is None else w
    e = gpu_ec(d["ec"] if ec is None else ec, d["M"], outputs) if (ec is not False) else None
    y = sp.spear_w4_linear(dev(d["x"]), w, e, out_dtype=out, path=path, workspace=ws)
    torch.cuda.synchronize()
    if out == sp.OUT_BF16:
        yh = host(y.view(torch.int16)).view(np.uint16)
        yh = (yh.astype(np.uint32) << 16).view(np.float32)
    else:
        yh = host(y)
    return yh, e


def run_oracle(d, ec="cfg"):
    packed, bad = oracle.pack_w4(d["codes"], d["kind"])
    assert bad == 0
    e = d["ec"] if ec == "cfg" else ec
    return oracle.w4_linear(d["x"], packed, d["scales"], d["zeros"], e)


def errors(y, ref):
    y = y.astype(np.float64)
    diff = y - ref
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300))
    return rel, float(np.max(np.abs(diff))) if diff.size else 0.0


# Two GPU kernels that add the same fp32 products in a different order (the
# fused decode's 4 stream waves against the 8 of a plain decode over a long K
# range) differ by a few fp32 roundings of the partial sums: far below the
# parity bound.
RTOL_REORDER = 1e-5


def assert_reordered(y, other, what=""):
    rel, mx = errors(y, other.astype(np.float64))
    print(f"[reorder] {what} rel_l2={rel:.3e} max_abs={mx:.3e}", flush=True)
    assert rel <= RTOL_REORDER, (what, rel, mx)


def assert_close(y, ref, what=""):
    rel, mx = errors(y, ref)
    print(f"[parity] {what} rel_l2={rel:.3e} max_abs={mx:.3e}", flush=True)
    assert rel <= RTOL_L2 and mx <= ATOL_MAX, (what, rel, mx)
    return rel, mx
