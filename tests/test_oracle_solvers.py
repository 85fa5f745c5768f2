"""Pins of the conjugate-gradient oracle (oracle/solvers.py) against things
that do not come from it: LAPACK's solve at finite termination, the first
step's closed form, Krylov optimality against brute-force least squares, and
planted mistakes that each of them catches.  CPU only."""
import numpy as np
import pytest

import oracle
from oracle import solvers as s


def _spd(n, seed, shift):
    r = np.random.default_rng(seed)
    m = r.standard_normal((n, n))
    return m @ m.T / n + shift * np.eye(n)


def pin_finite_termination(cg):
    """In exact arithmetic CG on an n x n SPD system ends in n steps; on a
    well-conditioned matrix fp64 gets there to rounding."""
    a = _spd(12, 1, 1.0)
    w = np.random.default_rng(2).standard_normal((12, 3))
    y = cg(a, w, 12)
    ref = np.linalg.solve(a, w)
    assert np.abs(y - ref).max() / np.abs(ref).max() < 1e-10, "no termination in n steps"


def pin_first_step_closed_form(cg):
    """Step 1 from y = 0 is steepest descent: y = (w.w / w.Aw) w per column."""
    a = _spd(9, 3, 0.5)
    w = np.random.default_rng(4).standard_normal((9, 4))
    expect = (w * w).sum(0) / (w * (a @ w)).sum(0) * w
    assert np.allclose(cg(a, w, 1), expect, rtol=1e-13, atol=1e-15), "first step"


def pin_krylov_optimality(cg):
    """Iterate k minimises the A-norm of the error over the Krylov space
    span(w, Aw, .., A^{k-1} w): the minimiser is found here by brute force
    (least squares in the A-inner product over an explicit basis)."""
    a = _spd(10, 5, 0.3)
    w = np.random.default_rng(6).standard_normal((10, 2))
    chol = np.linalg.cholesky(a)
    for k in (1, 2, 3, 5):
        y = cg(a, w, k)
        for c in range(w.shape[1]):
            basis = np.stack([np.linalg.matrix_power(a, i) @ w[:, c] for i in range(k)], 1)
            # minimise ||L^T (V z) - L^T x*|| with x* = A^{-1} w: A-norm error
            xs = np.linalg.solve(a, w[:, c])
            z, *_ = np.linalg.lstsq(chol.T @ basis, chol.T @ xs, rcond=None)
            best = basis @ z
            assert np.abs(y[:, c] - best).max() / np.abs(best).max() < 1e-8, f"k={k} col {c}"


def pin_zero_rhs(cg):
    """A zero right-hand side stays zero (no division by a zero residual)."""
    a = _spd(6, 7, 0.5)
    w = np.zeros((6, 2))
    w[:, 1] = 1.0
    y = cg(a, w, 4)
    assert np.all(y[:, 0] == 0.0) and np.all(np.isfinite(y))


PINS = [pin_finite_termination, pin_first_step_closed_form, pin_krylov_optimality,
        pin_zero_rhs]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_cg_pin(pin):
    pin(s.conjugate_gradient)


def _cg_mutant(kind):
    def cg(a, w, iters):
        y = np.zeros_like(w)
        r = w.copy()
        p = r.copy()
        rr = (r * r).sum(0)
        for it in range(iters):
            q = a @ p
            alpha = rr / (p * q).sum(0)
            if kind == "alpha from p.p":
                alpha = rr / (p * p).sum(0)
            y = y + alpha * p
            r = r - alpha * q if kind != "residual sign" else r + alpha * q
            rr_new = (r * r).sum(0)
            beta = rr_new / rr
            if kind == "no conjugation":
                beta = 0.0 * beta
            p = r + beta * p
            rr = rr_new
        if kind == "one step short":
            return cg_ref_short(a, w, iters)
        return y

    def cg_ref_short(a, w, iters):
        return s.conjugate_gradient(a, w, max(iters - 1, 0))
    return cg


@pytest.mark.parametrize("kind", ["alpha from p.p", "residual sign", "no conjugation",
                                  "one step short"])
def test_cg_mutation_is_caught(kind):
    bad = _cg_mutant(kind)
    failed = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(bad)
        except (AssertionError, np.linalg.LinAlgError):
            failed.append(pin.__name__)
    assert failed, kind


def test_ns_solve_is_x_times_w():
    """The Newton-Schulz solve is the oracle's iterate times W (and reaches
    LAPACK's solve once converged)."""
    a = _spd(8, 9, 0.8)
    w = np.random.default_rng(10).standard_normal((8, 3))
    assert np.allclose(s.newton_schulz_solve(a, w, 5), oracle.newton_schulz(a, 5) @ w)
    assert np.allclose(s.newton_schulz_solve(a, w, 60), np.linalg.solve(a, w), rtol=1e-9)
    assert s.relative_residual(a, w, np.linalg.solve(a, w)) < 1e-13
