"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This module holds no attention arithmetic. It draws q, k, v and dO from a
seeded generator, rounds them once to the storage dtype (round-to-nearest-even)
and hands out the exact stored values twice: as the storage arrays the GPU
receives and as float64 arrays for the oracle, decoded bit-exactly.

Workloads (the five shapes the method is measured on):
  0  fp32  B=1 Hq=Hkv=2  L=16    D=32   full attention
  1  fp16  B=2 Hq=Hkv=8  L=256   D=64   causal
  2  bf16  B=4 Hq=32 Hkv=8  L=2048  D=128  causal (GQA 4:1)
  3  bf16  B=1 Hq=16 Hkv=2  L=8192  D=256  causal + sliding window 1024 (GQA 8:1)
  4  bf16  B=1 Hq=32 Hkv=4  L=32768 D=128  causal, dO ~ N(0, 0.01) (GQA 8:1)
Every workload uses scale = 1/sqrt(D), the default softmax scale of the ggmlR
wrapper (ggmlR R/ag_flash_attn.R, ag_flash_attention, argument `scale`).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

DTYPES = ("f32", "f16", "bf16")


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str
    B: int
    Hq: int
    Hkv: int
    Lq: int
    Lkv: int
    D: int
    causal: bool
    window: int
    sigma_qkv: float
    sigma_do: float
    tol: float
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)


# Parity tolerance on max|gpu - ref| / max|ref| per output tensor.
TOL = {"f32": 1e-5, "f16": 5e-3, "bf16": 2e-2}

WORKLOADS = [
    Workload("tiny_f32_mha_L16_D32", "f32", 1, 2, 2, 16, 16, 32, False, 0, 1.0, 1.0, TOL["f32"], 1000),
    Workload("f16_causal_mha_L256_D64", "f16", 2, 8, 8, 256, 256, 64, True, 0, 1.0, 1.0, TOL["f16"], 1001),
    Workload("bf16_causal_gqa4_L2048_D128", "bf16", 4, 32, 8, 2048, 2048, 128, True, 0, 1.0, 1.0, TOL["bf16"], 1002),
    Workload("bf16_causal_gqa8_win1024_L8192_D256", "bf16", 1, 16, 2, 8192, 8192, 256, True, 1024, 1.0, 1.0, TOL["bf16"], 1003),
    Workload("bf16_causal_gqa8_L32768_D128", "bf16", 1, 32, 4, 32768, 32768, 128, True, 0, 1.0, 0.01, TOL["bf16"], 1004),
    # short queries against a long key range (the short-sequence path: 8 query
    # rows per head, every key visible), the bandwidth-bound case
    Workload("bf16_gqa4_q8_kv4096_D128", "bf16", 8, 32, 8, 8, 4096, 128, False, 0, 1.0, 1.0, TOL["bf16"], 1005),
]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); return the uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    bias = ((u >> 16) & 1) + 0x7FFF
    out = ((u + bias) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Decode bfloat16 bit patterns exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def encode(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 -> storage array: float32, float16 (RNE) or bf16 bits as uint16 (RNE)."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return np.ascontiguousarray(x.astype(np.float16))
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def decode(s: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array -> exact float64 values."""
    if dtype == "bf16":
        return bf16_bits_to_f64(s)
    return np.asarray(s).astype(np.float64)


def draw(shape, dtype: str, sigma: float, rng: np.random.Generator) -> np.ndarray:
    """One N(0, sigma) tensor, drawn in float32 and rounded once to the storage dtype."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x = x * np.float32(sigma)
    return encode(x, dtype)


def make_inputs(B, Hq, Hkv, Lq, Lkv, D, dtype, seed, sigma_qkv=1.0, sigma_do=1.0, Dv=None):
    """Storage arrays for q, k, v, dO drawn in that order from PCG64(seed);
    v and dO have head dim Dv (default D)."""
    Dv = D if Dv is None else Dv
    rng = np.random.Generator(np.random.PCG64(seed))
    q = draw((B, Hq, Lq, D), dtype, sigma_qkv, rng)
    k = draw((B, Hkv, Lkv, D), dtype, sigma_qkv, rng)
    v = draw((B, Hkv, Lkv, Dv), dtype, sigma_qkv, rng)
    do = draw((B, Hq, Lq, Dv), dtype, sigma_do, rng)
    return {"q": q, "k": k, "v": v, "do": do}


def make_spiked_inputs(B, Hq, Hkv, Lq, Lkv, D, dtype, seed, period=100, offset=100, height=6.5, sigma_qk=0.35,
                       Dv=None):
    """Inputs whose scores (under the default scale 1/sqrt(D)) have a flat floor
    and isolated high keys, for exercising a running maximum that grows.

    q, k, v and dO are drawn as in make_inputs (q and k with sigma_qk, v and dO
    with sigma 1); then component 0 of every q row is set to 1 and component 0
    of key j to height * sqrt(D) for the keys j = offset, offset + period, ...
    (else 0), so the score of those keys stands about `height` (natural-log
    units) above the others, whose spread is about sigma_qk**2. Values are
    rounded to the storage dtype after the change, like every other input."""
    Dv = D if Dv is None else Dv
    rng = np.random.Generator(np.random.PCG64(seed))
    x = {}
    for name, shape, sigma in (("q", (B, Hq, Lq, D), sigma_qk), ("k", (B, Hkv, Lkv, D), sigma_qk),
                               ("v", (B, Hkv, Lkv, Dv), 1.0), ("do", (B, Hq, Lq, Dv), 1.0)):
        x[name] = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(sigma)
    x["q"][..., 0] = 1.0
    j = np.arange(Lkv)
    spike = (j >= offset) & ((j - offset) % period == 0)
    x["k"][..., 0] = np.where(spike, np.float32(height * math.sqrt(D)), np.float32(0.0))
    return {name: encode(val, dtype) for name, val in x.items()}


def workload_inputs(w: Workload):
    return make_inputs(w.B, w.Hq, w.Hkv, w.Lq, w.Lkv, w.D, w.dtype, w.seed, w.sigma_qkv, w.sigma_do)


def to_torch(a: np.ndarray, dtype: str):
    """Storage array -> CPU torch tensor of the matching dtype (no value change)."""
    import torch

    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a))


def from_torch(t, dtype: str) -> np.ndarray:
    """CPU or GPU torch tensor -> exact float64 values."""
    import torch

    t = t.detach().to("cpu").contiguous()
    if dtype == "bf16":
        return bf16_bits_to_f64(t.view(torch.int16).numpy().view(np.uint16))
    if t.dtype == torch.float16:
        return t.numpy().astype(np.float64)
    return t.to(torch.float64).numpy()
