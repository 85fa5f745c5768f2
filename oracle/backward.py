"""fp64 CPU oracle for the backward pass of Nystrom kernel attention.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite may import or run
this module.  It shares no code with the HIP path.

The pages state that the method's custom kernels serve the backward pass as
well as the forward pass (LaplacianFormer summaries, implementation and
results paragraphs), but give no formulas for it.  The backward pass here is
therefore the plain reverse-mode derivative of the forward oracle
(:mod:`oracle.nystrom`), taken step by step in reverse order:

    O = K_QL Y,  Y = X W,  W = K_LK V
    X = X_T,  X_{t+1} = 2 X_t - X_t A X_t,  X_0 = alpha A
    alpha = 1 / (c r),  c = max column abs-sum of A,  r = max row abs-sum
    A = k(L, L) + eps I,  K_QL = k(Q, L),  K_LK = k(L, K)
    k(x, y) = exp(-D(x, y) / lambda)
    L = average pool of K over the landmark windows

Readings where the forward is not differentiable:

* |t| at t = 0 (Laplacian distance): the subgradient 0 is taken, i.e.
  d|t|/dt = sign(t) with sign(0) = 0.
* alpha's maxima: the derivative flows through the first column (row) of
  largest abs-sum, as numpy.argmax picks it; with a tie any choice is a valid
  subgradient.  alpha is part of the function at a fixed iteration count (X_T
  depends on it), so its derivative is kept.
* Q and K given as one tensor (shared projection): the caller adds dQ and dK.

Every function is pinned by central finite differences of the fp64 forward
oracle, by a brute-force explicit-matrix check of dV, and by planted-mistake
tests.  Library primitives used as steps: numpy sums, sign, exp and matrix
products.
"""
from __future__ import annotations

from typing import Dict

import numpy as np

from .nystrom import (GAUSSIAN, LAPLACIAN, kernel_map, landmark_matrix,
                      landmarks_avg_pool, ns_alpha)


def avg_pool_backward(d_l: np.ndarray, grid_h: int, grid_w: int,
                      pool_h: int, pool_w: int) -> np.ndarray:
    """Gradient of the landmark average pool: each key token in window j
    receives d_l[j] / (pool_h * pool_w)."""
    mh, mw = grid_h // pool_h, grid_w // pool_w
    d_k = np.zeros((grid_h * grid_w, d_l.shape[1]), dtype=np.float64)
    for R in range(mh):
        for C in range(mw):
            for r in range(R * pool_h, (R + 1) * pool_h):
                for c in range(C * pool_w, (C + 1) * pool_w):
                    d_k[r * grid_w + c] += d_l[R * mw + C] / (pool_h * pool_w)
    return d_k


def distance_backward(x: np.ndarray, y: np.ndarray, d_dist: np.ndarray,
                      kernel: str):
    """Gradients of D[i, j] = ||x_i - y_j||_1 (Laplacian) or
    ||x_i - y_j||_2^2 (Gaussian) with respect to x and y, given dL/dD."""
    d_x = np.zeros_like(x)
    d_y = np.zeros_like(y)
    for j in range(y.shape[0]):
        diff = x - y[j]                         # [n, d]
        if kernel == LAPLACIAN:
            s = np.sign(diff)                   # sign(0) = 0
        elif kernel == GAUSSIAN:
            s = 2.0 * diff
        else:
            raise ValueError(f"unknown kernel {kernel!r}")
        g = d_dist[:, j:j + 1] * s              # dL/dx_i from column j
        d_x += g
        d_y[j] -= g.sum(axis=0)
    return d_x, d_y


def kernel_map_backward(x: np.ndarray, y: np.ndarray, kmap: np.ndarray,
                        d_kmap: np.ndarray, lam: float, kernel: str):
    """Gradients of k(x_i, y_j) = exp(-D[i, j] / lambda) with respect to x
    and y, given the forward values ``kmap`` and dL/dk."""
    d_dist = -d_kmap * kmap / lam
    return distance_backward(x, y, d_dist, kernel)


def ns_alpha_backward(a: np.ndarray, d_alpha: float) -> np.ndarray:
    """Gradient of alpha = 1 / (c r) with respect to A, where c is the largest
    column abs-sum and r the largest row abs-sum."""
    absa = np.abs(a)
    jc = int(np.argmax(absa.sum(axis=0)))
    ir = int(np.argmax(absa.sum(axis=1)))
    c = absa[:, jc].sum()
    r = absa[ir, :].sum()
    alpha = 1.0 / (c * r)
    d_c = -d_alpha * alpha / c
    d_r = -d_alpha * alpha / r
    d_a = np.zeros_like(a)
    d_a[:, jc] += d_c * np.sign(a[:, jc])
    d_a[ir, :] += d_r * np.sign(a[ir, :])
    return d_a


def newton_schulz_backward(a: np.ndarray, iters: int,
                           d_x: np.ndarray) -> np.ndarray:
    """Gradient with respect to A of X_T, the Newton-Schulz iterate after
    ``iters`` steps from X_0 = alpha A, given dL/dX_T.

    Step X_{t+1} = 2 X_t - X_t A X_t, taken back from t = T - 1 to 0 with
    G = dL/dX_{t+1}:
        dL/dX_t  = 2 G - G (A X_t)^T - (X_t A)^T G
        dL/dA   += -X_t^T G X_t^T
    then X_0 = alpha A gives dL/dA += alpha dL/dX_0 and
    dL/dalpha = <dL/dX_0, A>, which flows through alpha's maxima.
    """
    alpha = ns_alpha(a)
    xs = [alpha * a]
    for _ in range(iters):
        x = xs[-1]
        xs.append(2.0 * x - x @ (a @ x))
    d_a = np.zeros_like(a)
    g = d_x
    for t in range(iters - 1, -1, -1):
        x = xs[t]
        d_a -= x.T @ g @ x.T
        g = 2.0 * g - g @ (a @ x).T - (x @ a).T @ g
    d_a += alpha * g
    d_a += ns_alpha_backward(a, float((g * a).sum()))
    return d_a


def nystrom_head_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                          d_out: np.ndarray, *, grid_h: int, grid_w: int,
                          pool_h: int, pool_w: int, lam: float, eps: float,
                          iters: int, kernel: str = LAPLACIAN
                          ) -> Dict[str, np.ndarray]:
    """dL/dQ, dL/dK, dL/dV of one head for dL/dO = ``d_out`` (all fp64), plus
    the gradients of the intermediates (L, K_QL, K_LK, A, X, W, Y)."""
    # forward, keeping what the backward needs
    L = landmarks_avg_pool(k, grid_h, grid_w, pool_h, pool_w)
    kql = kernel_map(q, L, lam, kernel)            # [N, m]
    klk = kernel_map(L, k, lam, kernel)            # [m, N]
    A = landmark_matrix(L, lam, eps, kernel)       # [m, m]
    alpha = ns_alpha(A)
    X = alpha * A
    for _ in range(iters):
        X = 2.0 * X - X @ (A @ X)
    W = klk @ v                                    # [m, d]
    Y = X @ W                                      # [m, d]

    # O = K_QL Y
    d_kql = d_out @ Y.T
    d_y = kql.T @ d_out
    # Y = X W
    d_x = d_y @ W.T
    d_w = X.T @ d_y
    # W = K_LK V
    d_klk = d_w @ v.T
    d_v = klk.T @ d_w
    # X = NS(A)
    d_a = newton_schulz_backward(A, iters, d_x)
    # A = k(L, L) + eps I: both arguments are L
    kll = A - eps * np.eye(A.shape[0])
    d_l1, d_l2 = kernel_map_backward(L, L, kll, d_a, lam, kernel)
    # K_QL = k(Q, L), K_LK = k(L, K)
    d_q, d_l3 = kernel_map_backward(q, L, kql, d_kql, lam, kernel)
    d_l4, d_k_direct = kernel_map_backward(L, k, klk, d_klk, lam, kernel)
    d_l = d_l1 + d_l2 + d_l3 + d_l4
    # L = pool(K)
    d_k = d_k_direct + avg_pool_backward(d_l, grid_h, grid_w, pool_h, pool_w)
    return {"dQ": d_q, "dK": d_k, "dV": d_v, "dL": d_l, "dKQL": d_kql,
            "dKLK": d_klk, "dA": d_a, "dX": d_x, "dW": d_w, "dY": d_y}
