"""Seeded synthetic workloads for the Prox sparse SwiGLU FFN decode path.

This module only draws random numbers and rounds them to bf16.  It holds none
of the method's arithmetic (no quantisation, selection, SiLU or products), so
both the CPU oracle's tests and the GPU path's tests and bench can take their
inputs from it without sharing any of the computation under test.

Shapes and distributions follow the five workloads the path is measured on:

  c1  tiny SwiGLU FFN      d=512,  F=1376,  B=1,         int8 proxy,  keep 50 %, sparsity 50 %
  c2  Llama-2-7B layer     d=4096, F=11008, B=1,         int8 proxy,  keep 60 %, sparsity 50/70/90 %
  c3  Llama-3-8B stack     d=4096, F=14336, 32 layers,   int4 g128,   keep 60 %, sparsity 70 %, B in {1,4,16}
  c4  70B layer            d=8192, F=28672, B in {1,8},  int8 proxy,  keep 60 %, sparsity 50/70 %
  c5  mixed stack          64 layers alternating (3584, 18944) / (5120, 13824), B=32, int4 g128,
                           keep 60 %, sparsity 80 %
  c2_p512  prefill         the c2 layer over 512 tokens in one call (sparsity 70 %)

Weights are N(0, 0.02) in fp32 rounded to bf16 (round to nearest even).
Activations x are Laplace(0, 1) in fp32; c1/c2 scale 4 fixed outlier dims by
20, c4 scales round(0.5 % of d) = 41 outlier dims by 30, c3/c5 divide each
token by its RMS.  Everything is rounded to bf16 at the end.

Random streams are numpy ``default_rng([seed, config, layer, tensor])`` (weight
matrices: one stream per chunk of 1024 rows, ``[..., tensor, chunk]``) so any
tensor can be regenerated on its own.  Layout: ``wg_t`` and ``wu_t`` are
[F][d] (row j = intermediate channel j, i.e. the gate/up weight of a
bias-free linear layer stored output-major); ``wd`` is [F][d] as in the
SwiGLU definition, where row j of W_down is the output direction of channel j.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

ROOT_SEED = 0

# tensor ids inside one (config, layer) stream family
_T_GATE, _T_UP, _T_DOWN, _T_X, _T_OUTLIER = 1, 2, 3, 4, 99


def bf16_round(a: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16), round to nearest even.

    Inputs are finite by construction (normal / Laplace draws)."""
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp32 values."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def pct_count(n: int, pct: int) -> int:
    """Integer count of ``pct`` percent of ``n``, rounded half up, no floats."""
    return (n * pct + 50) // 100


@dataclass(frozen=True)
class LayerShape:
    d: int
    F: int


@dataclass(frozen=True)
class Workload:
    """One measured workload: shapes, batch and the method's settings."""

    name: str
    config_id: int
    layers: Tuple[LayerShape, ...]
    batch: int
    proxy: str                      # "int8" | "int4"
    keep_pct: int                   # input keep, percent of d
    sparsity_pct: int               # FFN sparsity, percent of F inactive
    x_kind: str                     # "outlier" | "rmsnorm"
    outlier_count: int = 0          # 0 -> derived from d for "outlier"
    outlier_scale: float = 1.0

    def k_in(self, layer: int = 0) -> int:
        return pct_count(self.layers[layer].d, self.keep_pct)

    def k_ff(self, layer: int = 0) -> int:
        return pct_count(self.layers[layer].F, 100 - self.sparsity_pct)

    @property
    def n_layers(self) -> int:
        return len(self.layers)


def _stack(shapes: List[LayerShape], n: int) -> Tuple[LayerShape, ...]:
    return tuple(shapes[i % len(shapes)] for i in range(n))


def workloads() -> Dict[str, Workload]:
    """Every (config, sweep point) of the five workloads, by name."""
    w: Dict[str, Workload] = {}
    s1 = LayerShape(512, 1376)
    w["c1"] = Workload("c1", 1, (s1,), 1, "int8", 50, 50, "outlier", 4, 20.0)
    s2 = LayerShape(4096, 11008)
    for sp in (50, 70, 90):
        w[f"c2_s{sp}"] = Workload(f"c2_s{sp}", 2, (s2,), 1, "int8", 60, sp, "outlier", 4, 20.0)
    # every channel kept (sparsity 0): the dense FFN through the same path
    # (exact mode with k_ff = d_ff is the dense layer on the library's kernels)
    w["c2_s0"] = Workload("c2_s0", 2, (s2,), 1, "int8", 60, 0, "outlier", 4, 20.0)
    # prefill: the Llama-2-7B layer over 512 tokens at once (every token its
    # own mask; the union of the masks covers nearly every channel)
    w["c2_p512"] = Workload("c2_p512", 2, (s2,), 512, "int8", 60, 70, "outlier", 4, 20.0)
    s3 = LayerShape(4096, 14336)
    for b in (1, 4, 16):
        w[f"c3_b{b}"] = Workload(f"c3_b{b}", 3, _stack([s3], 32), b, "int4", 60, 70, "rmsnorm")
    s4 = LayerShape(8192, 28672)
    for b in (1, 8):
        for sp in (50, 70):
            w[f"c4_b{b}_s{sp}"] = Workload(f"c4_b{b}_s{sp}", 4, (s4,), b, "int8", 60, sp,
                                           "outlier", 41, 30.0)
    w["c4_b1_s0"] = Workload("c4_b1_s0", 4, (s4,), 1, "int8", 60, 0, "outlier", 41, 30.0)
    s5a, s5b = LayerShape(3584, 18944), LayerShape(5120, 13824)
    w["c5"] = Workload("c5", 5, _stack([s5a, s5b], 64), 32, "int4", 60, 80, "rmsnorm")
    return w


def _rng(config_id: int, layer: int, tensor: int, seed: int = ROOT_SEED, *more: int) -> np.random.Generator:
    return np.random.default_rng([seed, config_id, layer, tensor, *more])


_CHUNK_ROWS = 1024          # rows of a weight matrix drawn from one stream
_THREADS = min(8, os.cpu_count() or 1)


def _normal_bf16(config_id: int, layer: int, tensor: int, rows: int, cols: int, std: float,
                 seed: int) -> np.ndarray:
    """N(0, std) fp32 -> bf16 bits [rows][cols]; rows drawn in chunks of
    _CHUNK_ROWS, chunk c from stream (seed, config, layer, tensor, c), so the
    chunks can be filled by several threads and the result does not depend on
    how many."""
    out = np.empty((rows, cols), dtype=np.uint16)

    def fill(c):
        r0, r1 = c * _CHUNK_ROWS, min(rows, (c + 1) * _CHUNK_ROWS)
        a = np.empty((r1 - r0, cols), dtype=np.float32)
        _rng(config_id, layer, tensor, seed, c).standard_normal(out=a, dtype=np.float32)
        a *= np.float32(std)
        out[r0:r1] = bf16_round(a)

    n = (rows + _CHUNK_ROWS - 1) // _CHUNK_ROWS
    if n <= 1:
        for c in range(n):
            fill(c)
    else:
        with ThreadPoolExecutor(max_workers=_THREADS) as ex:
            list(ex.map(fill, range(n)))
    return out


def gen_weights(config_id: int, layer: int, d: int, F: int, std: float = 0.02,
                seed: int = ROOT_SEED) -> Dict[str, np.ndarray]:
    """bf16 bit patterns: wg_t, wu_t [F][d] and wd [F][d]."""
    return {name: _normal_bf16(config_id, layer, tid, F, d, std, seed)
            for name, tid in (("wg_t", _T_GATE), ("wu_t", _T_UP), ("wd", _T_DOWN))}


def outlier_dims(config_id: int, d: int, count: int, seed: int = ROOT_SEED) -> np.ndarray:
    r = _rng(config_id, 0, _T_OUTLIER, seed)
    return np.sort(r.choice(d, size=count, replace=False))


def gen_x(wl: Workload, layer: int, batch: Optional[int] = None, step: int = 0,
          seed: int = ROOT_SEED) -> np.ndarray:
    """Activations as bf16 bit patterns [B][d] for ``layer`` of ``wl``.

    ``step`` selects an independent draw (a later decode step)."""
    B = wl.batch if batch is None else batch
    d = wl.layers[layer].d
    r = _rng(wl.config_id, layer, _T_X + 16 * step, seed)
    x = r.laplace(0.0, 1.0, size=(B, d)).astype(np.float32)
    if wl.x_kind == "outlier":
        dims = outlier_dims(wl.config_id, d, wl.outlier_count, seed)
        x[:, dims] *= np.float32(wl.outlier_scale)
    elif wl.x_kind == "rmsnorm":
        rms = np.sqrt(np.mean(x.astype(np.float64) ** 2, axis=1, keepdims=True))
        x = (x / rms).astype(np.float32)
    else:
        raise ValueError(wl.x_kind)
    return bf16_round(x)


def gen_small(d: int, F: int, B: int, seed: int, std: float = 0.02,
              x_kind: str = "outlier", outliers: int = 2, outlier_scale: float = 20.0,
              ) -> Dict[str, np.ndarray]:
    """Free-form small case (tests): weights and x as bf16 bit patterns."""
    r = np.random.default_rng([seed, 7777, d, F, B])
    out = {}
    for name in ("wg_t", "wu_t", "wd"):
        a = r.standard_normal((F, d), dtype=np.float32) * np.float32(std)
        out[name] = bf16_round(a)
    x = r.laplace(0.0, 1.0, size=(B, d)).astype(np.float32)
    if x_kind == "outlier" and outliers > 0:
        dims = r.choice(d, size=min(outliers, d), replace=False)
        x[:, dims] *= np.float32(outlier_scale)
    elif x_kind == "rmsnorm":
        rms = np.sqrt(np.mean(x.astype(np.float64) ** 2, axis=1, keepdims=True))
        x = (x / rms).astype(np.float32)
    out["x"] = bf16_round(x)
    return out


def gen_ties(d: int, F: int, B: int, seed: int, levels: int = 5) -> Dict[str, np.ndarray]:
    """Tie-heavy small case: x and weights drawn from a few small dyadic levels,
    so many |x| and many proxy codes coincide exactly."""
    r = np.random.default_rng([seed, 8888, d, F, B])
    lv = np.float32(2.0) ** -np.arange(levels, dtype=np.float32)
    out = {}
    for name in ("wg_t", "wu_t", "wd"):
        a = r.choice(lv, size=(F, d)) * r.choice(np.float32([-1, 1]), size=(F, d))
        out[name] = bf16_round((a * np.float32(0.03125)).astype(np.float32))
    x = r.choice(lv, size=(B, d)) * r.choice(np.float32([-1, 1]), size=(B, d))
    out["x"] = bf16_round(x.astype(np.float32))
    return out
