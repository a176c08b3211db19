"""Seeded synthetic inputs for the TTR hybrid-attention forward.

This module only draws random numbers and rounds them to the IO dtype; it
holds none of the method's arithmetic. Both the fp64 oracle (through the
tests) and the HIP path consume exactly the arrays it returns.

Workloads (shapes and distributions follow the Flux attention shapes the
TTR trainer page targets -- "Flux2TTRTrainer", sections "Why this exists" and
"Inputs worth setting" -- and the linear-attention layer page,
"NNT Define Linear Attention", section "The inputs"):

  tiny_fp32   B=1 H=2  N=256   D=64  F=256 fp32, L=16 (every 16th token), b=0
  flux_512    B=1 H=24 N=1536  D=128 F=256 bf16, L=64   (1024 image + 512 text)
  flux_1024   B=1 H=24 N=4608  D=128 F=256 bf16, L=128  (4096 image + 512 text)
  flux_2048   B=1 H=24 N=16896 D=128 F=256 bf16, L=256  (16384 image + 512 text)
  causal      B=8 H=8  N=32768 D=64  (identity map, F=D) bf16, causal, chunk 256
  flux_1024_h3  flux_1024 at H=3: one GPU's share when the 24 heads are spread
                over 8 GPUs (its own seed)

Distributions: Q, K, V ~ N(0, 1); W_h ~ N(0, 1/D) (variance notation, so the
standard deviation is 1/sqrt(D)); b_h ~ N(0, 0.01) (std 0.1) except the tiny
config where b_h = 0; g_h ~ N(0, 1); eps = 1e-6 (the fp32 value).

NNT layer workloads ("NNT Define Linear Attention", section "The inputs":
embed_dim 512, num_heads 8; the page fixes no sequence length, so N = 4096
tokens, B = 8 are chosen): x ~ N(0, 1) [B, N, E]; Wq, Wk, Wv, Wo ~ N(0, 1/E)
[E, E]; bq, bk, bv, bo ~ N(0, 0.01) [E]; drawn in that order; bf16 rounds x
and the four W (the biases stay fp32).

  nnt_layer         B=8 N=4096 E=512 H=8 bf16, elu + 1, not causal
  nnt_layer_causal  the same, causal

Draw order: Q, K, V, W, b, g from numpy's PCG64 ``default_rng(seed)`` with
``standard_normal(dtype=float32)`` scaled by the std. bf16 workloads round
every IO tensor (Q, K, V, W) to bfloat16 with round-to-nearest-even; b and g
stay fp32. The rounded values are the canonical inputs for both sides.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = ["Workload", "WORKLOADS", "make_inputs", "bf16_round_bits", "bf16_bits_to_f32",
           "LayerWorkload", "LAYER_WORKLOADS", "make_layer_inputs", "make_grad_output", "query_subsample"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    D: int
    F: int
    dtype: str  # "fp32" or "bf16"
    L: int  # landmark count (0 = none)
    causal: bool
    proj: bool  # True: phi(x) = elu(x W_h + b_h) + 1;  False: phi(x) = elu(x) + 1 (F = D)
    w_std: float
    b_std: float
    seed: int
    chunk: int = 128
    eps: float = 1e-6

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def tokens(self) -> int:
        return self.B * self.N


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 1, 2, 256, 64, 256, "fp32", 16, False, True,
                          1 / 8.0, 0.0, 1000),
    "flux_512": Workload("flux_512", 1, 24, 1536, 128, 256, "bf16", 64, False, True,
                         1 / np.sqrt(128.0), 0.1, 1001),
    "flux_1024": Workload("flux_1024", 1, 24, 4608, 128, 256, "bf16", 128, False, True,
                          1 / np.sqrt(128.0), 0.1, 1002),
    "flux_2048": Workload("flux_2048", 1, 24, 16896, 128, 256, "bf16", 256, False, True,
                          1 / np.sqrt(128.0), 0.1, 1003),
    # one GPU's share of flux_1024 when its 24 heads are spread over 8 GPUs
    "flux_1024_h3": Workload("flux_1024_h3", 1, 3, 4608, 128, 256, "bf16", 128, False, True,
                             1 / np.sqrt(128.0), 0.1, 1007),
    "causal": Workload("causal", 8, 8, 32768, 64, 64, "bf16", 0, True, False,
                       0.0, 0.0, 1004, chunk=256),
}


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exactly equal fp32 values."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def make_inputs(w: Workload, seed: Optional[int] = None) -> dict:
    """Draw one seeded input set for workload ``w``.

    Returns a dict with fp32 arrays ``Q, K, V`` [B,H,N,D], ``W`` [H,D,F] or
    None, ``b`` [H,F] or None, ``g`` [H], the fp32 ``eps`` and, for bf16
    workloads, the uint16 bit patterns ``Q_bits`` ... ``W_bits``. The fp32
    arrays hold the values after rounding to the IO dtype.
    """
    rng = np.random.default_rng(w.seed if seed is None else seed)
    shp = (w.B, w.H, w.N, w.D)
    out: dict = {}
    out["Q"] = rng.standard_normal(shp, dtype=np.float32)
    out["K"] = rng.standard_normal(shp, dtype=np.float32)
    out["V"] = rng.standard_normal(shp, dtype=np.float32)
    if w.proj:
        out["W"] = rng.standard_normal((w.H, w.D, w.F), dtype=np.float32) * np.float32(w.w_std)
        out["b"] = rng.standard_normal((w.H, w.F), dtype=np.float32) * np.float32(w.b_std)
    else:
        out["W"] = None
        out["b"] = None
    out["g"] = rng.standard_normal((w.H,), dtype=np.float32)
    out["eps"] = np.float32(w.eps)
    if w.dtype == "bf16":
        for k in ("Q", "K", "V", "W"):
            if out[k] is None:
                out[k + "_bits"] = None
                continue
            bits = bf16_round_bits(out[k])
            out[k + "_bits"] = bits
            out[k] = bf16_bits_to_f32(bits)
    elif w.dtype != "fp32":
        raise ValueError(f"unknown dtype {w.dtype!r}")
    return out


@dataclasses.dataclass(frozen=True)
class LayerWorkload:
    name: str
    B: int
    N: int
    E: int
    H: int
    dtype: str  # "fp32" or "bf16"
    causal: bool
    fmap: str  # "elu1", "relu" or "softmax"
    seed: int
    b_std: float = 0.1
    eps: float = 1e-6

    def with_(self, **kw) -> "LayerWorkload":
        return dataclasses.replace(self, **kw)

    @property
    def tokens(self) -> int:
        return self.B * self.N


LAYER_WORKLOADS = {
    "nnt_layer": LayerWorkload("nnt_layer", 8, 4096, 512, 8, "bf16", False, "elu1", 1005),
    "nnt_layer_causal": LayerWorkload("nnt_layer_causal", 8, 4096, 512, 8, "bf16", True, "elu1", 1006),
}


def make_layer_inputs(w: LayerWorkload, seed: Optional[int] = None, bias: bool = True) -> dict:
    """Draw one seeded input set for layer workload ``w``: fp32 arrays ``x``
    [B,N,E], ``Wq Wk Wv Wo`` [E,E], ``bq bk bv bo`` [E] (None without bias),
    ``eps`` and, for bf16, the uint16 bit patterns ``x_bits`` and ``W*_bits``.
    The fp32 arrays hold the values after rounding to the IO dtype."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    out: dict = {"x": rng.standard_normal((w.B, w.N, w.E), dtype=np.float32)}
    ws = np.float32(1.0 / np.sqrt(w.E))
    for k in ("Wq", "Wk", "Wv", "Wo"):
        out[k] = rng.standard_normal((w.E, w.E), dtype=np.float32) * ws
    for k in ("bq", "bk", "bv", "bo"):
        out[k] = rng.standard_normal((w.E,), dtype=np.float32) * np.float32(w.b_std) if bias else None
    out["eps"] = np.float32(w.eps)
    if w.dtype == "bf16":
        for k in ("x", "Wq", "Wk", "Wv", "Wo"):
            bits = bf16_round_bits(out[k])
            out[k + "_bits"] = bits
            out[k] = bf16_bits_to_f32(bits)
    elif w.dtype != "fp32":
        raise ValueError(f"unknown dtype {w.dtype!r}")
    return out


def make_grad_output(w: Workload, seed: int) -> np.ndarray:
    """A seeded upstream gradient dLoss/dout for workload ``w``: fp32 [B,H,N,D] ~ N(0, 1)."""
    return np.random.default_rng(seed).standard_normal((w.B, w.H, w.N, w.D), dtype=np.float32)


def query_subsample(N: int, Nq: int, seed: int) -> np.ndarray:
    """Seeded subset of Nq of the N token positions, strictly increasing int32
    (the query rows a replay sample keeps)."""
    if not 1 <= Nq <= N:
        raise ValueError("need 1 <= Nq <= N")
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(N, size=Nq, replace=False)).astype(np.int32)
