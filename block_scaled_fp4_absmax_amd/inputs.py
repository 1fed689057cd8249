"""Seeded synthetic inputs for the five workloads (numpy PCG64, float64 draws).

This module holds none of the quantization arithmetic: it only draws random
tensors and rounds them to bfloat16 bit patterns. Both the HIP path's tests and
the CPU oracle's tests take their inputs from here.

Recipe (each stands in for LLM weights or activations; no model is loaded):

* ``c1`` MXFP4 256x4096: 0.02*N(0,1); round(0.1% * N) distinct flat positions
  (``rng.choice(N, k, replace=False)``) multiplied by 20. Seed 0.
* ``c2`` NVFP4+RaZeR 4096x4096: 0.02*N(0,1); round(0.5% * N) distinct positions
  get ``rng.laplace(0, 0.3)`` added. Seed 1.
* ``c3`` MXFP4 + Hadamard, 8192 tokens x 8192 hidden: 0.5*Student-t(3); 16 fixed
  channels (``rng.choice(cols, 16, replace=False)``) multiplied by 50. Seed 2.
* ``c4`` two-level rotation + MXFP4, 16384x8192: per 32-channel block variance
  exp(1.5*z), z ~ N(0,1), shared by all tokens; Gaussian within. Seed 3.
* ``c5`` Llama-70B-shaped decoder-layer weights ``[out, in]``: q, k, v, o, gate,
  up, down; each 0.02*N(0,1) with round(0.1% * N) distinct positions x20.
  Tensor t (in that order) uses seed 400 + t.

Every draw is float64, cast to float32, then rounded to bfloat16 with
round-to-nearest-even. The draw order inside each recipe is fixed, so a recipe
with fewer rows is not a prefix of the full tensor; parity tests that need a
small case generate the small case directly.
"""
from __future__ import annotations

from typing import Dict, List, Tuple

import numpy as np

C5_SHAPES: List[Tuple[str, int, int]] = [
    ("q", 8192, 8192),
    ("k", 1024, 8192),
    ("v", 1024, 8192),
    ("o", 8192, 8192),
    ("gate", 28672, 8192),
    ("up", 28672, 8192),
    ("down", 8192, 28672),
]

FULL_SHAPES: Dict[str, Tuple[int, int]] = {
    "c1": (256, 4096),
    "c2": (4096, 4096),
    "c3": (8192, 8192),
    "c4": (16384, 8192),
}


def f64_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float64 -> float32 -> bfloat16 bits (round-to-nearest-even), uint16."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    out = np.empty(u.shape, np.uint16)
    chunk = 1 << 24
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)
    for s in range(0, flat_u.size, chunk):
        v = flat_u[s:s + chunk].astype(np.uint64)
        v = (v + 0x7FFF + ((v >> 16) & 1)) >> 16
        flat_o[s:s + chunk] = v.astype(np.uint16)
    return out


def _outliers_scaled(rng, x: np.ndarray, frac: float, factor: float) -> None:
    n = x.size
    k = int(round(frac * n))
    pos = rng.choice(n, k, replace=False)
    x.reshape(-1)[pos] *= factor


def gen_c1(rows: int = 256, cols: int = 4096, seed: int = 0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    x = 0.02 * rng.standard_normal((rows, cols))
    _outliers_scaled(rng, x, 0.001, 20.0)
    return f64_to_bf16_bits(x)


def gen_c2(rows: int = 4096, cols: int = 4096, seed: int = 1) -> np.ndarray:
    rng = np.random.default_rng(seed)
    x = 0.02 * rng.standard_normal((rows, cols))
    n = x.size
    k = int(round(0.005 * n))
    pos = rng.choice(n, k, replace=False)
    x.reshape(-1)[pos] += rng.laplace(0.0, 0.3, k)
    return f64_to_bf16_bits(x)


def gen_c3(rows: int = 8192, cols: int = 8192, seed: int = 2) -> np.ndarray:
    rng = np.random.default_rng(seed)
    x = 0.5 * rng.standard_t(3, (rows, cols))
    ch = rng.choice(cols, 16, replace=False)
    x[:, ch] *= 50.0
    return f64_to_bf16_bits(x)


def c3_outlier_channels(cols: int = 8192, rows: int = 8192, seed: int = 2) -> np.ndarray:
    """The 16 channels ``gen_c3`` scales, re-drawn from the same stream."""
    rng = np.random.default_rng(seed)
    rng.standard_t(3, (rows, cols))
    return np.sort(rng.choice(cols, 16, replace=False))


def gen_c4(rows: int = 16384, cols: int = 8192, seed: int = 3) -> np.ndarray:
    assert cols % 32 == 0
    rng = np.random.default_rng(seed)
    z = rng.standard_normal(cols // 32)
    std = np.repeat(np.sqrt(np.exp(1.5 * z)), 32)
    x = rng.standard_normal((rows, cols)) * std[None, :]
    return f64_to_bf16_bits(x)


def gen_c5(t: int, rows: int = None, cols: int = None) -> np.ndarray:
    """Tensor t of the layer (0=q .. 6=down); rows/cols override the shape."""
    name, r0, c0 = C5_SHAPES[t]
    rows = r0 if rows is None else rows
    cols = c0 if cols is None else cols
    rng = np.random.default_rng(400 + t)
    x = 0.02 * rng.standard_normal((rows, cols))
    _outliers_scaled(rng, x, 0.001, 20.0)
    return f64_to_bf16_bits(x)


def generate(name: str, rows: int = None, cols: int = None) -> np.ndarray:
    """bf16 bits of workload ``name`` ('c1'..'c4', or 'c5_<t>'), optionally resized."""
    if name.startswith("c5"):
        t = int(name.split("_")[1])
        return gen_c5(t, rows, cols)
    r, c = FULL_SHAPES[name]
    rows = r if rows is None else rows
    cols = c if cols is None else cols
    return {"c1": gen_c1, "c2": gen_c2, "c3": gen_c3, "c4": gen_c4}[name](rows, cols)


def bf16_bits_to_f32(x: np.ndarray) -> np.ndarray:
    return (x.astype(np.uint32) << 16).view(np.float32)
