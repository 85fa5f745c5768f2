"""fp64 CPU oracle for Nystrom-approximated, softmax-free kernel attention.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the package smoke
check and the benchmark's CPU-baseline leg may import or run this module.  It
shares no code with the HIP path (no kernels, headers, helpers or tables) and
never imports it; the only thing both sides share is the seeded input arrays.

What it computes, step by step and in the pages' order, per head (b, h):

1. Landmarks L (m x d): the mean of the key tokens over each non-overlapping
   pool_h x pool_w window of the token grid, windows in raster order.
   (SOFT review, "method" bullets: bottleneck tokens sampled by average
   pooling; LaplacianFormer summaries, Nystrom paragraph: a small set of
   landmark keys picked by average pooling.)
2. Kernel maps against the landmarks: K_QL = k(Q, L) (N x m),
   K_LK = k(L, K) (m x N) and the landmark matrix k(L, L) (m x m).
   Laplacian kernel k(x, y) = exp(-||x - y||_1 / lambda)
   (LaplacianFormer summaries, "Methodologie" / section 2a, kernel formula);
   Gaussian variant exp(-||x - y||_2^2 / lambda) (SOFT review, "method"
   bullets, S = exp(Q (-) K), with the scale lambda = 2 sqrt(d) supplied by the
   caller).  Distances are formed by direct coordinate differences.
3. A = k(L, L) + eps * I, the small diagonal perturbation that makes the
   landmark matrix strictly positive definite (LaplacianFormer summaries,
   Newton-Schulz paragraph).
4. Newton-Schulz inverse: X_0 = alpha * A, X_{t+1} = 2 X_t - X_t A X_t for
   exactly `iters` steps, alpha = 1 / (||A||_1 * ||A||_inf)
   (SOFT review, "method" bullets, the A_0 / A_{k+1} recursion; the alpha
   choice is the standard one that guarantees convergence and is not printed
   on the pages).
5. O = K_QL (X (K_LK V)): the low-rank product P^T A^+ P applied to V
   (SOFT review, "method" bullets, S_hat = P^T A^+ P), evaluated right to
   left, without any further normalisation (SOFT abstract: no normalisation
   after the kernel).

Inputs arrive in their I/O representation (float32, or bf16 as uint16 bit
patterns) and are widened exactly to fp64; every step then runs in fp64.
Library primitives used as steps: numpy sums, exp and matrix products.

Every function here is pinned by tests that check it against closed forms,
library routines (SciPy cdist, LAPACK inverse/eigendecomposition),
invariants the pages state, and brute force at tiny sizes.
"""
from __future__ import annotations

from typing import Dict, Iterable, Optional, Sequence, Tuple

import numpy as np

LAPLACIAN = "laplacian"
GAUSSIAN = "gaussian"


def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """I/O representation -> fp64 (exact for both fp32 and bf16)."""
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def landmarks_avg_pool(k: np.ndarray, grid_h: int, grid_w: int,
                       pool_h: int, pool_w: int) -> np.ndarray:
    """Average-pool the key tokens of one head into landmarks.

    ``k`` is [N, d] with token n = row * grid_w + col.  Landmark
    j = R * (grid_w // pool_w) + C is the mean of the tokens in rows
    [R*pool_h, (R+1)*pool_h) and columns [C*pool_w, (C+1)*pool_w).
    """
    n, d = k.shape
    if n != grid_h * grid_w or grid_h % pool_h or grid_w % pool_w:
        raise ValueError("grid / pool mismatch")
    mh, mw = grid_h // pool_h, grid_w // pool_w
    out = np.empty((mh * mw, d), dtype=np.float64)
    for R in range(mh):
        for C in range(mw):
            rows = [r * grid_w + c
                    for r in range(R * pool_h, (R + 1) * pool_h)
                    for c in range(C * pool_w, (C + 1) * pool_w)]
            out[R * mw + C] = k[rows].mean(axis=0)
    return out


def distance_matrix(x: np.ndarray, y: np.ndarray, kernel: str) -> np.ndarray:
    """D[i, j] = ||x_i - y_j||_1 (Laplacian) or ||x_i - y_j||_2^2 (Gaussian)."""
    out = np.empty((x.shape[0], y.shape[0]), dtype=np.float64)
    for j in range(y.shape[0]):
        diff = x - y[j]
        if kernel == LAPLACIAN:
            out[:, j] = np.abs(diff).sum(axis=1)
        elif kernel == GAUSSIAN:
            out[:, j] = (diff * diff).sum(axis=1)
        else:
            raise ValueError(f"unknown kernel {kernel!r}")
    return out


def kernel_map(x: np.ndarray, y: np.ndarray, lam: float, kernel: str) -> np.ndarray:
    """k(x_i, y_j) = exp(-D[i, j] / lambda)."""
    return np.exp(-distance_matrix(x, y, kernel) / lam)


def landmark_matrix(l: np.ndarray, lam: float, eps: float, kernel: str) -> np.ndarray:
    """A = k(L, L) + eps * I."""
    return kernel_map(l, l, lam, kernel) + eps * np.eye(l.shape[0])


def ns_alpha(a: np.ndarray) -> float:
    """alpha = 1 / (max column abs-sum * max row abs-sum)."""
    col = np.abs(a).sum(axis=0).max()
    row = np.abs(a).sum(axis=1).max()
    return 1.0 / (col * row)


def newton_schulz(a: np.ndarray, iters: int) -> np.ndarray:
    """X_0 = alpha A; X_{t+1} = 2 X_t - X_t (A X_t), exactly ``iters`` times."""
    x = ns_alpha(a) * a
    for _ in range(iters):
        x = 2.0 * x - x @ (a @ x)
    return x


def nystrom_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, *,
                 grid_h: int, grid_w: int, pool_h: int, pool_w: int,
                 lam: float, eps: float, iters: int,
                 kernel: str = LAPLACIAN) -> Dict[str, np.ndarray]:
    """All intermediates and the output of one head, in fp64."""
    L = landmarks_avg_pool(k, grid_h, grid_w, pool_h, pool_w)
    kql = kernel_map(q, L, lam, kernel)          # [N, m]
    klk = kernel_map(L, k, lam, kernel)          # [m, N]
    A = landmark_matrix(L, lam, eps, kernel)     # [m, m]
    X = newton_schulz(A, iters)                  # [m, m]
    W = klk @ v                                  # [m, d]
    Y = X @ W                                    # [m, d]
    O = kql @ Y                                  # [N, d]
    return {"L": L, "KQL": kql, "KLK": klk, "A": A, "X": X, "W": W,
            "Y": Y, "O": O}


def forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, *,
            grid_h: int, grid_w: int, pool_h: int, pool_w: int,
            lam: float, eps: float, iters: int, kernel: str = LAPLACIAN,
            dtype: str = "f32",
            heads: Optional[Iterable[Tuple[int, int]]] = None,
            stages: bool = False):
    """Oracle forward over [B, H, N, d] inputs in their I/O representation.

    Returns ``{(b, h): result}`` for the requested heads (all heads by
    default); each result holds ``O`` and, when ``stages`` is set, every
    intermediate of :func:`nystrom_head`.
    """
    B, H = q.shape[0], q.shape[1]
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(H)]
    out = {}
    for (b, h) in heads:
        res = nystrom_head(widen(q[b, h], dtype), widen(k[b, h], dtype),
                           widen(v[b, h], dtype), grid_h=grid_h,
                           grid_w=grid_w, pool_h=pool_h, pool_w=pool_w,
                           lam=lam, eps=eps, iters=iters, kernel=kernel)
        out[(b, h)] = res if stages else {"O": res["O"]}
    return out


def forward_workload(w, inputs: Dict[str, np.ndarray],
                     heads: Optional[Sequence[Tuple[int, int]]] = None,
                     stages: bool = False):
    """Convenience wrapper taking a workload description and its inputs."""
    return forward(inputs["q"], inputs["k"], inputs["v"], grid_h=w.grid_h,
                   grid_w=w.grid_w, pool_h=w.pool_h, pool_w=w.pool_w,
                   lam=w.lam, eps=w.eps, iters=w.iters, kernel=w.kernel,
                   dtype=w.dtype, heads=heads, stages=stages)


def full_kernel_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                          lam: float, kernel: str = LAPLACIAN) -> np.ndarray:
    """Exact (non-approximated) kernel attention k(Q, K) V, fp64, O(N^2).

    Used only as a sanity reference for approximation quality.
    """
    return kernel_map(q, k, lam, kernel) @ v


def normalized_feature_map(kql: np.ndarray, delta: float) -> np.ndarray:
    """Z = (K_QL - mu) / sqrt(var + delta), per column j (landmark): mu_j and
    var_j the mean and the population variance of column j over the queries.

    LaplacianFormer summaries (Arabic summary, section 2(b); Dutch summary,
    "Methodologie" item 1): each query's similarity vector is centred and
    whitened, the covariance's inverse square root replaced by a diagonal
    estimator that normalises each feature dimension on its own across the
    batch of queries.  Reading: the similarity vector of query i is row i of
    K_QL (its kernel values against the landmarks); the batch is the head's
    N queries; delta is the whitening's stabiliser (not printed on the pages).
    """
    mu = kql.mean(axis=0)
    var = ((kql - mu) ** 2).mean(axis=0)
    return (kql - mu) / np.sqrt(var + delta)


def nystrom_head_normalized(q, k, v, *, grid_h, grid_w, pool_h, pool_w, lam, eps,
                            iters, delta, kernel=LAPLACIAN):
    """One head with the normalised feature map in place of K_QL:
    O = Z (X (K_LK V)), Z = normalized_feature_map(K_QL, delta)."""
    res = nystrom_head(q, k, v, grid_h=grid_h, grid_w=grid_w, pool_h=pool_h,
                       pool_w=pool_w, lam=lam, eps=eps, iters=iters, kernel=kernel)
    Z = normalized_feature_map(res["KQL"], delta)
    res["Z"] = Z
    res["O"] = Z @ res["Y"]
    return res


def forward_normalized(q, k, v, *, grid_h, grid_w, pool_h, pool_w, lam, eps, iters,
                       delta, kernel=LAPLACIAN, dtype="f32", heads=None):
    """forward() with the normalised feature map; returns {(b, h): O}."""
    B, H = q.shape[0], q.shape[1]
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(H)]
    return {(b, h): nystrom_head_normalized(
        widen(q[b, h], dtype), widen(k[b, h], dtype), widen(v[b, h], dtype),
        grid_h=grid_h, grid_w=grid_w, pool_h=pool_h, pool_w=pool_w, lam=lam, eps=eps,
        iters=iters, delta=delta, kernel=kernel)["O"] for (b, h) in heads}
