"""Seeded synthetic workloads for Nystrom kernel attention (forward).

This module only *draws inputs*: it holds none of the method's arithmetic
(no pooling, no kernel, no solver).  The HIP path and the CPU oracle both
consume the arrays it returns, so both see bit-identical inputs.

Shapes follow vision-transformer stages: tokens live on a ``grid_h x grid_w``
patch grid in raster order (token n = row * grid_w + col), one ``[N, d]``
matrix per head, laid out ``[B, H, N, d]`` C-contiguous.  Landmarks come from a
non-overlapping ``pool_h x pool_w`` average pool of that grid (SOFT review,
"method" bullets: average pooling of bottleneck tokens, m about 49;
LaplacianFormer summaries, Nystrom paragraph: landmark keys chosen by average
pooling).

Random streams: NumPy PCG64 ``default_rng(seed)``; draws happen in the order
Q, K, V, each as one ``[B, H, N, d]`` fp64 array, then scaled, then cast to the
I/O dtype.  When Q and K are shared (the Gaussian variant's shared projection)
K is not drawn.  bf16 values are produced by round-to-nearest-even from fp32
and handed out as their raw 16-bit patterns (``numpy.uint16``), because NumPy
has no bf16 type.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

LAPLACIAN = "laplacian"
GAUSSIAN = "gaussian"
F32 = "f32"
BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention-layer problem: shapes, method constants and input recipe."""

    name: str
    B: int
    H: int
    grid_h: int
    grid_w: int
    d: int
    pool_h: int
    pool_w: int
    lam: float
    eps: float
    iters: int
    kernel: str = LAPLACIAN
    dtype: str = F32
    shared_qk: bool = False
    qk_dist: str = "normal"      # "normal" or "student_t3"
    qk_scale: float = 1.0
    v_scale: float = 1.0
    seed: int = 0
    note: str = ""

    @property
    def N(self) -> int:
        return self.grid_h * self.grid_w

    @property
    def m(self) -> int:
        return (self.grid_h // self.pool_h) * (self.grid_w // self.pool_w)

    @property
    def heads(self) -> int:
        return self.B * self.H

    @property
    def tokens(self) -> int:
        """Tokens per forward call (B * N, heads of one token counted once)."""
        return self.B * self.N

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


_SQRT64 = math.sqrt(64.0)

# The five reference workloads.  Seeds are 1000 + position in this list.
WORKLOADS: List[Workload] = [
    Workload(
        name="lap_f32_n196_d32_m49", B=1, H=1, grid_h=14, grid_w=14, d=32,
        pool_h=2, pool_w=2, lam=32.0, eps=1e-3, iters=20, seed=1000,
        note="tiny Laplacian case, lambda = d"),
    Workload(
        name="lap_f32_pvt1_b8_n3136_d64_m49", B=8, H=1, grid_h=56, grid_w=56,
        d=64, pool_h=8, pool_w=8, lam=2.0 * _SQRT64, eps=1e-3, iters=20,
        qk_scale=4.0 / _SQRT64, v_scale=4.0 / _SQRT64, seed=1001,
        note="PVT stage-1 shape; inputs N(0,1)/sqrt(d)*4 = N(0, 0.5^2)"),
    Workload(
        name="lap_bf16_b32h5_n784_d64_m49", B=32, H=5, grid_h=28, grid_w=28,
        d=64, pool_h=4, pool_w=4, lam=2.0 * _SQRT64, eps=1e-3, iters=20,
        dtype=BF16, seed=1002, note="mid-stage shape, bf16 I/O, fp32 compute"),
    Workload(
        name="lap_f32_h2_n16384_d64_m64_t3", B=1, H=2, grid_h=128, grid_w=128,
        d=64, pool_h=16, pool_w=16, lam=2.0 * _SQRT64, eps=1e-2, iters=30,
        qk_dist="student_t3", qk_scale=0.5, seed=1003,
        note="high-resolution heavy-tailed case: Q,K = 0.5 * t(nu=3)"),
    Workload(
        name="gauss_f32_b16h2_n3136_d64_m49_qk", B=16, H=2, grid_h=56,
        grid_w=56, d=64, pool_h=8, pool_w=8, lam=2.0 * _SQRT64, eps=1e-3,
        iters=20, kernel=GAUSSIAN, shared_qk=True, seed=1004,
        note="SOFT Gaussian variant exp(-|q-k|^2/(2 sqrt d)) with Q = K"),
]

BY_NAME: Dict[str, Workload] = {w.name: w for w in WORKLOADS}

# Throughput is quoted on the PVT stage-1 shape.
HEADLINE = WORKLOADS[1]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 round-to-nearest-even, returned as uint16 bit patterns."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _draw(rng: np.random.Generator, dist: str, shape, scale: float) -> np.ndarray:
    if dist == "normal":
        a = rng.standard_normal(shape)
    elif dist == "student_t3":
        a = rng.standard_t(3.0, size=shape)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return a * scale


def _cast(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == F32:
        return np.ascontiguousarray(a, dtype=np.float32)
    if dtype == BF16:
        return f32_to_bf16_bits(a.astype(np.float32))
    raise ValueError(f"unknown dtype {dtype!r}")


def make_inputs(w: Workload, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Draw Q, K, V for workload ``w``.

    Returns a dict with ``q``, ``k``, ``v`` in the I/O representation
    (float32 arrays, or uint16 bf16 bit patterns).  When ``w.shared_qk`` the
    ``k`` entry *is* the ``q`` array (same object), mirroring the shared
    projection of the Gaussian variant.
    """
    rng = np.random.default_rng(w.seed if seed is None else seed)
    shape = (w.B, w.H, w.N, w.d)
    q = _cast(_draw(rng, w.qk_dist, shape, w.qk_scale), w.dtype)
    if w.shared_qk:
        k = q
    else:
        k = _cast(_draw(rng, w.qk_dist, shape, w.qk_scale), w.dtype)
    v = _cast(_draw(rng, "normal", shape, w.v_scale), w.dtype)
    return {"q": q, "k": k, "v": v}


def small_case(grid_h: int, grid_w: int, d: int, pool_h: int, pool_w: int,
               B: int = 1, H: int = 1, kernel: str = LAPLACIAN,
               dtype: str = F32, shared_qk: bool = False, iters: int = 20,
               eps: float = 1e-3, lam: Optional[float] = None,
               qk_dist: str = "normal", qk_scale: float = 1.0,
               seed: int = 7) -> Workload:
    """A custom-sized workload for parity sweeps (ragged tiles, edge cases)."""
    if lam is None:
        lam = 2.0 * math.sqrt(d)
    return Workload(
        name=f"custom_{kernel}_{dtype}_b{B}h{H}_{grid_h}x{grid_w}_d{d}_p{pool_h}x{pool_w}",
        B=B, H=H, grid_h=grid_h, grid_w=grid_w, d=d, pool_h=pool_h,
        pool_w=pool_w, lam=lam, eps=eps, iters=iters, kernel=kernel,
        dtype=dtype, shared_qk=shared_qk, qk_dist=qk_dist, qk_scale=qk_scale,
        seed=seed)


@dataclasses.dataclass(frozen=True)
class BlockWorkload:
    """One attention block on the tokens of a pyramid stage: x [B, N, C],
    projections [C, H d] (query and key shared when ``shared_qk``) and
    [H d, C], the Nystrom attention in between."""

    name: str
    B: int
    H: int
    d: int
    C: int
    grid_h: int
    grid_w: int
    pool_h: int
    pool_w: int
    lam: float
    eps: float = 1e-3
    iters: int = 20
    kernel: str = LAPLACIAN
    dtype: str = F32
    shared_qk: bool = False
    seed: int = 2000

    @property
    def N(self) -> int:
        return self.grid_h * self.grid_w

    @property
    def m(self) -> int:
        return (self.grid_h // self.pool_h) * (self.grid_w // self.pool_w)

    def replace(self, **kw) -> "BlockWorkload":
        return dataclasses.replace(self, **kw)


# The four stages of a PVT-small-like pyramid (tokens 56^2, 28^2, 14^2, 7^2;
# widths 64, 128, 320, 512; heads of 64 columns), 49 landmarks each; the
# first stage also as SOFT's Gaussian layer with the shared projection.
BLOCKS: List[BlockWorkload] = [
    BlockWorkload("block_lap_s1_b8_n3136_c64", B=8, H=1, d=64, C=64, grid_h=56, grid_w=56,
                  pool_h=8, pool_w=8, lam=2.0 * _SQRT64, seed=2000),
    BlockWorkload("block_lap_s2_b8_n784_c128", B=8, H=2, d=64, C=128, grid_h=28, grid_w=28,
                  pool_h=4, pool_w=4, lam=2.0 * _SQRT64, seed=2001),
    BlockWorkload("block_lap_s3_b8_n196_c320", B=8, H=5, d=64, C=320, grid_h=14, grid_w=14,
                  pool_h=2, pool_w=2, lam=2.0 * _SQRT64, seed=2002),
    BlockWorkload("block_lap_s4_b8_n49_c512", B=8, H=8, d=64, C=512, grid_h=7, grid_w=7,
                  pool_h=1, pool_w=1, lam=2.0 * _SQRT64, seed=2003),
    BlockWorkload("block_gauss_s1_b8_n3136_c64_qk", B=8, H=1, d=64, C=64, grid_h=56, grid_w=56,
                  pool_h=8, pool_w=8, lam=2.0 * _SQRT64, kernel=GAUSSIAN, shared_qk=True,
                  seed=2004),
]
BLOCK_BY_NAME: Dict[str, BlockWorkload] = {b.name: b for b in BLOCKS}


def make_block_inputs(w: BlockWorkload, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """x ~ N(0, 1) [B, N, C]; Wq, Wk, Wv ~ N(0, 1/C) [C, H d] (so projected
    coordinates are about N(0, 1)); Wo ~ N(0, 1/(H d)) [H d, C]; drawn in that
    order (Wk skipped when shared, the entry is then None) and cast to the
    I/O type."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    hd = w.H * w.d
    x = _cast(rng.standard_normal((w.B, w.N, w.C)), w.dtype)
    wq = _cast(rng.standard_normal((w.C, hd)) / math.sqrt(w.C), w.dtype)
    wk = None if w.shared_qk else _cast(rng.standard_normal((w.C, hd)) / math.sqrt(w.C), w.dtype)
    wv = _cast(rng.standard_normal((w.C, hd)) / math.sqrt(w.C), w.dtype)
    wo = _cast(rng.standard_normal((hd, w.C)) / math.sqrt(hd), w.dtype)
    return {"x": x, "wq": wq, "wk": wk, "wv": wv, "wo": wo}
