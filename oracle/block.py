"""fp64 CPU oracle for one attention block around the Nystrom attention.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite may import or run
this module.  It shares no code with the HIP path.

The SOFT review instantiates SOFT as one attention layer of a pyramid vision
transformer backbone ("proposed method", last bullet), with a symmetric
kernel S = exp(Q (-) K) (so queries and keys share one projection) and no
normalisation after the kernel.  The block computed here, on tokens
X [B, N, C] of one stage:

1. Q = X Wq; K = Q when the projection is shared, else K = X Wk; V = X Wv
   (weights [C, H d], no bias), each split into H heads of d columns
   (columns h d .. h d + d - 1 are head h), stored in the block's I/O type;
2. per head, O_h = the Nystrom attention of :mod:`oracle.nystrom`;
3. Y = concat_h(O_h) Wo (Wo [H d, C]), the heads' columns in head order.

Reading (the pages give no layer code): the intermediate Q, K, V and O are
materialised in the I/O type (fp32 or bf16, rounded to nearest even), as a
layer with activations of that type stores them; every product is exact
fp64 on those values.  Library primitives used as steps: numpy matrix
products.
"""
from __future__ import annotations

import numpy as np

from .nystrom import forward, widen


def _round_io(a: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 -> the I/O type -> fp64 (round to nearest even)."""
    f = np.asarray(a, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return f.astype(np.float64)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint32) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def _to_io(a: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 values already representable in the I/O type -> its storage."""
    if dtype == "f32":
        return a.astype(np.float32)
    return (a.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def block_forward(x, wq, wk, wv, wo, *, H: int, d: int, grid_h: int, grid_w: int,
                  pool_h: int, pool_w: int, lam: float, eps: float, iters: int,
                  kernel: str = "laplacian", dtype: str = "f32"):
    """Y [B, N, C] of the block for inputs in their I/O representation
    (x [B, N, C]; wq, wk, wv [C, H d]; wo [H d, C]; wk None = shared)."""
    X = widen(x, dtype)
    B, N, C = X.shape
    Wq, Wv, Wo = widen(wq, dtype), widen(wv, dtype), widen(wo, dtype)

    def heads(m):  # [B, N, H d] -> [B, H, N, d]
        return m.reshape(B, N, H, d).transpose(0, 2, 1, 3)
    Q = heads(_round_io(X @ Wq, dtype))
    K = Q if wk is None else heads(_round_io(X @ widen(wk, dtype), dtype))
    V = heads(_round_io(X @ Wv, dtype))
    res = forward(_to_io(Q, dtype), _to_io(K, dtype), _to_io(V, dtype), grid_h=grid_h,
                  grid_w=grid_w, pool_h=pool_h, pool_w=pool_w, lam=lam, eps=eps,
                  iters=iters, kernel=kernel, dtype=dtype)
    O = np.empty((B, H, N, d))
    for (b, h), r in res.items():
        O[b, h] = r["O"]
    O = _round_io(O, dtype)
    cat = O.transpose(0, 2, 1, 3).reshape(B, N, H * d)
    return cat @ Wo
