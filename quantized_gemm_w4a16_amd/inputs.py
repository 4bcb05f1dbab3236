"""Seeded synthetic inputs for the W4A16 + gated-EC linear layer.

This module only draws numbers and rounds them to bf16; it holds none of the
layer's arithmetic, so the HIP path and the CPU oracle can both be fed from it.
Every array is numpy; bf16 tensors are carried as their raw uint16 bits.

Workloads (shapes and value distributions):
  C1  M=16, K=N=1024; signed codes U{-8..7}, fp32 scales U[0.005,0.02];
      x ~ N(0,1); EC rank 16, A,B ~ N(0, 0.02); w_g ~ N(0, 1/sqrt(K)), b=0, soft.
  C2  M in {1,4,8}, K=N=4096 (7B-class attention projection); unsigned codes
      U{0..15} with zero point U{6..9}, bf16 scales; x ~ N(0,1); EC rank 32, soft.
  C3  M=64, K=4096, N=14336 (MLP up-projection); unsigned codes; x ~ N(0,1) with
      1% of input channels scaled x20; EC rank 64, hard gate, ~40% of tokens skip.
  C4  M=N=K=4096 (prefill); signed codes as C1; x Student-t (nu=4); EC rank 32, soft.
  C5  28-layer stack of a 1.5B-class decoder's linears (d=2048, MLP 8192: q,k,v,o
      2048->2048, gate,up 2048->8192, down 8192->2048); unsigned codes; x ~ N(0,1)
      with 0.5% of channels x30; ECs (rank 32, hard, ~50% skip) on 4 of the 28
      layers; M in {1,16,128,2048}.
The standard deviation is the second parameter of N(.,.).
"""
from __future__ import annotations

import math
from statistics import NormalDist

import numpy as np

SEED_BASE = 20260600
CODES_S4 = 0
CODES_U4 = 1

C5_D = 2048
C5_FF = 8192
C5_LAYERS = 28
C5_LINEARS = ("q", "k", "v", "o", "gate", "up", "down")
C5_EC_LAYERS_COUNT = 4


def bf16_bits(a) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest even (finite inputs)."""
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(list(key)))


def _weights(rng, N, K, kind, scale_dtype):
    if kind == CODES_S4:
        codes = rng.integers(-8, 8, size=(N, K), dtype=np.int8)
        zeros = None
    else:
        codes = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
        zeros = rng.integers(6, 10, size=N, dtype=np.uint8)
    scales = rng.uniform(0.005, 0.02, size=N).astype(np.float32)
    if scale_dtype == "bf16":
        scales = bf16_to_f32(bf16_bits(scales))
    return codes, scales, zeros


def _ec(rng, N, K, r, hard, tau):
    A = bf16_bits(rng.normal(0.0, 0.02, size=(r, K)).astype(np.float32))
    B = bf16_bits(rng.normal(0.0, 0.02, size=(N, r)).astype(np.float32))
    w_g = bf16_bits(rng.normal(0.0, 1.0 / math.sqrt(K), size=K).astype(np.float32))
    return {"A": A, "B": B, "w_g": w_g, "b": 0.0, "tau": tau, "hard": hard, "r": r}


def _activations(rng, M, K, dist, outlier_frac, outlier_gain):
    if dist == "t4":
        x = rng.standard_t(4, size=(M, K)).astype(np.float32)
    else:
        x = rng.normal(0.0, 1.0, size=(M, K)).astype(np.float32)
    chans = np.zeros(0, dtype=np.int64)
    if outlier_frac:
        n_out = int(round(outlier_frac * K))
        chans = np.sort(rng.choice(K, size=n_out, replace=False))
        x[:, chans] *= np.float32(outlier_gain)
    return bf16_bits(x), chans


def tau_for_skip(w_g_bits, K, chans, outlier_gain, skip_frac, b=0.0) -> float:
    """Hard-gate threshold from the input recipe alone: the gate logit of a token
    is b + x.w_g with x drawn as above, i.e. normal with variance
    sum_k w_g[k]^2 var(x_k); tau is the sigmoid of that law's skip_frac quantile."""
    w = bf16_to_f32(w_g_bits).astype(np.float64)
    var = np.ones(K)
    var[chans] = float(outlier_gain) ** 2
    sd = math.sqrt(float(np.sum(w * w * var)))
    t = b + sd * NormalDist().inv_cdf(skip_frac)
    return float(np.float32(1.0 / (1.0 + math.exp(-t))))


def make(cfg: int, M: int | None = None, seed: int | None = None) -> dict:
    """Inputs of one linear call for workload C1..C4 (C5 via make_c5)."""
    seed = SEED_BASE + cfg if seed is None else seed
    rw = _rng(seed, 0)
    if cfg == 1:
        M = 16 if M is None else M
        K = N = 1024
        codes, scales, zeros = _weights(rw, N, K, CODES_S4, "f32")
        ec = _ec(rw, N, K, 16, 0, 0.0)
        x, chans = _activations(_rng(seed, 1, M), M, K, "normal", 0.0, 1.0)
        kind = CODES_S4
    elif cfg == 2:
        M = 1 if M is None else M
        K = N = 4096
        codes, scales, zeros = _weights(rw, N, K, CODES_U4, "bf16")
        ec = _ec(rw, N, K, 32, 0, 0.0)
        x, chans = _activations(_rng(seed, 1, M), M, K, "normal", 0.0, 1.0)
        kind = CODES_U4
    elif cfg == 3:
        M = 64 if M is None else M
        K, N = 4096, 14336
        codes, scales, zeros = _weights(rw, N, K, CODES_U4, "bf16")
        ec = _ec(rw, N, K, 64, 1, 0.0)
        x, chans = _activations(_rng(seed, 1, M), M, K, "normal", 0.01, 20.0)
        ec["tau"] = tau_for_skip(ec["w_g"], K, chans, 20.0, 0.40)
        kind = CODES_U4
    elif cfg == 4:
        M = 4096 if M is None else M
        K = N = 4096
        codes, scales, zeros = _weights(rw, N, K, CODES_S4, "f32")
        ec = _ec(rw, N, K, 32, 0, 0.0)
        x, chans = _activations(_rng(seed, 1, M), M, K, "t4", 0.0, 1.0)
        kind = CODES_S4
    else:
        raise ValueError(f"unknown workload C{cfg}")
    return {"name": f"C{cfg}", "M": M, "K": K, "N": N, "kind": kind, "codes": codes,
            "scales": scales, "zeros": zeros, "x": x, "ec": ec, "outlier_channels": chans}


def c5_shape(lin: str):
    """(K, N) of one linear of the C5 stack."""
    if lin in ("q", "k", "v", "o"):
        return C5_D, C5_D
    if lin in ("gate", "up"):
        return C5_D, C5_FF
    if lin == "down":
        return C5_FF, C5_D
    raise ValueError(lin)


def c5_ec_layers(seed: int | None = None):
    seed = SEED_BASE + 5 if seed is None else seed
    return sorted(int(i) for i in _rng(seed, 99).choice(C5_LAYERS, C5_EC_LAYERS_COUNT,
                                                         replace=False))


def make_c5(layer: int, lin: str, M: int, seed: int | None = None) -> dict:
    """Inputs of one linear of the C5 stack (layer 0..27, lin in C5_LINEARS)."""
    seed = SEED_BASE + 5 if seed is None else seed
    K, N = c5_shape(lin)
    li = C5_LINEARS.index(lin)
    rw = _rng(seed, 0, layer, li)
    codes, scales, zeros = _weights(rw, N, K, CODES_U4, "bf16")
    ec = None
    if layer in c5_ec_layers(seed):
        ec = _ec(rw, N, K, 32, 1, 0.5)   # logit(0.5) = 0 = median of a centred logit
    x, chans = _activations(_rng(seed, 1, layer, li, M), M, K, "normal", 0.005, 30.0)
    return {"name": f"C5.L{layer}.{lin}", "M": M, "K": K, "N": N, "kind": CODES_U4,
            "codes": codes, "scales": scales, "zeros": zeros, "x": x, "ec": ec,
            "outlier_channels": chans}
