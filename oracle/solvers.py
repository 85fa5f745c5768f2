"""fp64 CPU oracle for the landmark solve Y = A^{-1} W by two methods.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite and the
benchmark's solver comparison may import or run this module.  It shares no
code with the HIP path.

The LaplacianFormer summaries report that the Newton-Schulz iteration is more
stable and converges better than conjugate-gradient solvers, above all on
ill-conditioned landmark matrices (Arabic summary, section 4, efficiency
analysis, solver robustness), without giving numbers.  The comparison needs
both solvers run the same way:

* Newton-Schulz: X_T from :func:`oracle.nystrom.newton_schulz`, then
  Y = X_T W.
* Conjugate gradient (the textbook method of Hestenes and Stiefel for a
  symmetric positive definite A), on A Y = W, every column of W its own
  system, started from Y = 0, exactly ``iters`` steps:
      r = w, p = r
      each step: q = A p; a = (r.r) / (p.q); y += a p; r -= a q;
                 b = (r_new.r_new) / (r_old.r_old); p = r + b p
  A column whose residual is exactly zero stops changing (a = 0).

Pinned by the solution of numpy.linalg.solve after m steps on a
well-conditioned matrix (finite termination), the first step's closed form
(steepest descent), Krylov optimality of every iterate against brute-force
least squares in the A-norm over an explicit Krylov basis, and planted
mistakes.  Library primitives used as steps: numpy matrix products and sums.
"""
from __future__ import annotations

import numpy as np

from .nystrom import newton_schulz


def conjugate_gradient(a: np.ndarray, w: np.ndarray, iters: int) -> np.ndarray:
    """Y after ``iters`` conjugate-gradient steps on A Y = W (columns
    independent), from Y = 0."""
    w = np.asarray(w, dtype=np.float64)
    y = np.zeros_like(w)
    r = w.copy()
    p = r.copy()
    rr = (r * r).sum(axis=0)
    for _ in range(iters):
        q = a @ p
        pq = (p * q).sum(axis=0)
        alpha = np.divide(rr, pq, out=np.zeros_like(rr), where=pq != 0)
        y += alpha * p
        r -= alpha * q
        rr_new = (r * r).sum(axis=0)
        beta = np.divide(rr_new, rr, out=np.zeros_like(rr), where=rr != 0)
        p = r + beta * p
        rr = rr_new
    return y


def newton_schulz_solve(a: np.ndarray, w: np.ndarray, iters: int) -> np.ndarray:
    """Y = X_T W with X_T the Newton-Schulz iterate after ``iters`` steps."""
    return newton_schulz(a, iters) @ np.asarray(w, dtype=np.float64)


def relative_residual(a: np.ndarray, w: np.ndarray, y: np.ndarray) -> float:
    """||A Y - W||_F / ||W||_F."""
    return float(np.linalg.norm(a @ y - w) / np.linalg.norm(w))
