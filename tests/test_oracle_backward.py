"""Pins for the fp64 backward oracle (oracle/backward.py), CPU only.

The backward oracle is pinned against things that do not come from it:

* central finite differences of the fp64 forward oracle, element by element
  over Q, K and V, at points kept away from the forward's kinks (|t| at 0 and
  ties in alpha's maxima), for both kernels and several iteration counts;
* dV against the explicit N x N matrix K_QL X K_LK (brute force: O is linear
  in V, so dL/dV = (K_QL X K_LK)^T dL/dO);
* planted mistakes in the backward oracle (a dropped alpha term, a wrong
  sign, an off-by-one iterate, a missing pool or Gaussian factor), each of
  which the finite-difference pin must catch.
"""
import numpy as np
import pytest

import oracle.backward as ob
import oracle.nystrom as o

H_FD = 1e-6
RTOL = 2e-6


def _case(seed, grid_h=4, grid_w=4, d=3, pool_h=2, pool_w=2, kernel=o.LAPLACIAN,
          iters=3, lam=2.0, eps=1e-2, scale=0.7):
    """Random inputs whose forward stays at least 1e-4 away from every kink:
    no coordinate difference of a (token, landmark) or (landmark, landmark)
    pair near zero, and a clear largest column / row abs-sum of A."""
    geom = dict(grid_h=grid_h, grid_w=grid_w, pool_h=pool_h, pool_w=pool_w,
                lam=lam, eps=eps, iters=iters, kernel=kernel)
    n = grid_h * grid_w
    for s in range(seed, seed + 1000):
        rng = np.random.default_rng(s)
        q = scale * rng.standard_normal((n, d))
        k = scale * rng.standard_normal((n, d))
        v = rng.standard_normal((n, d))
        g = rng.standard_normal((n, d))
        L = o.landmarks_avg_pool(k, grid_h, grid_w, pool_h, pool_w)
        m = L.shape[0]
        gaps = [np.abs(q[:, None, :] - L[None]).min(),
                np.abs(L[:, None, :] - k[None]).min()]
        if m > 1:
            off = ~np.eye(m, dtype=bool)
            gaps.append(np.abs(L[:, None, :] - L[None])[off].min())
            sums = np.sort(np.abs(o.landmark_matrix(L, lam, eps, kernel)).sum(axis=0))
            gaps.append(sums[-1] - sums[-2])
        if min(gaps) > 1e-4:
            return q, k, v, g, geom
    raise RuntimeError("no kink-free case found")


def _loss(q, k, v, g, geom):
    return float((o.nystrom_head(q, k, v, **geom)["O"] * g).sum())


def _fd(f, x):
    out = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        xp = x.copy()
        xm = x.copy()
        xp[idx] += H_FD
        xm[idx] -= H_FD
        out[idx] = (f(xp) - f(xm)) / (2 * H_FD)
    return out


def _rel(a, b):
    return np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)


def _check_fd(q, k, v, g, geom):
    grads = ob.nystrom_head_backward(q, k, v, g, **geom)
    fd_q = _fd(lambda x: _loss(x, k, v, g, geom), q)
    fd_k = _fd(lambda x: _loss(q, x, v, g, geom), k)
    fd_v = _fd(lambda x: _loss(q, k, x, g, geom), v)
    for name, fd in (("dQ", fd_q), ("dK", fd_k), ("dV", fd_v)):
        err = _rel(grads[name], fd)
        assert err <= RTOL, f"{name}: normwise error {err:.3e} against finite differences"


CASES = [
    dict(seed=1, kernel=o.LAPLACIAN, iters=3),
    dict(seed=2, kernel=o.LAPLACIAN, iters=0),      # X = alpha A: the alpha path alone
    dict(seed=3, kernel=o.LAPLACIAN, iters=8),
    dict(seed=4, kernel=o.GAUSSIAN, iters=3),
    dict(seed=5, kernel=o.GAUSSIAN, iters=0),
    dict(seed=6, kernel=o.LAPLACIAN, iters=3, grid_h=6, grid_w=4, pool_h=3, pool_w=2, d=2),
    dict(seed=7, kernel=o.LAPLACIAN, iters=2, grid_h=4, grid_w=4, pool_h=4, pool_w=4),  # m = 1
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c['kernel']}-it{c['iters']}-s{c['seed']}")
def test_backward_matches_finite_differences(case):
    case = dict(case)
    seed = case.pop("seed")
    _check_fd(*_case(seed, **case))


def test_shared_qk_gradient_is_sum():
    """Q and K as one tensor Z: dL/dZ = dQ + dK (finite differences in Z)."""
    q, _, v, g, geom = _case(11, kernel=o.GAUSSIAN, iters=3)
    grads = ob.nystrom_head_backward(q, q, v, g, **geom)
    fd = _fd(lambda z: _loss(z, z, v, g, geom), q)
    assert _rel(grads["dQ"] + grads["dK"], fd) <= RTOL


def test_dv_brute_force_matrix():
    """dV = (K_QL X K_LK)^T dO with the N x N matrix formed explicitly."""
    q, k, v, g, geom = _case(21, grid_h=8, grid_w=8, d=5, iters=20, lam=4.0, eps=1e-3)
    fwd = o.nystrom_head(q, k, v, **geom)
    M = fwd["KQL"] @ fwd["X"] @ fwd["KLK"]          # [N, N]
    grads = ob.nystrom_head_backward(q, k, v, g, **geom)
    assert _rel(grads["dV"], M.T @ g) <= 1e-12


def test_directional_derivative_larger_case():
    """m = 16 landmarks, 20 steps: <grad, U> against a central difference of
    the loss along a random direction U, for Q, K and V together."""
    q, k, v, g, geom = _case(31, grid_h=8, grid_w=8, d=6, iters=20, lam=4.0, eps=1e-3)
    grads = ob.nystrom_head_backward(q, k, v, g, **geom)
    rng = np.random.default_rng(5)
    for _ in range(3):
        uq, uk, uv = (rng.standard_normal(q.shape) for _ in range(3))
        h = 1e-6
        fp = _loss(q + h * uq, k + h * uk, v + h * uv, g, geom)
        fm = _loss(q - h * uq, k - h * uk, v - h * uv, g, geom)
        fd = (fp - fm) / (2 * h)
        an = (grads["dQ"] * uq).sum() + (grads["dK"] * uk).sum() + (grads["dV"] * uv).sum()
        assert abs(an - fd) <= 1e-5 * max(abs(fd), 1e-3), (an, fd)


# ----------------------------------------------------------------------------
# Planted mistakes: each must be caught by the finite-difference pin.
# ----------------------------------------------------------------------------

orig_alpha = ob.ns_alpha_backward
orig_dist = ob.distance_backward
orig_pool = ob.avg_pool_backward


def _no_alpha(a, d_alpha):
    return np.zeros_like(a)


def _dist_y_wrong_sign(x, y, d_dist, kernel):
    d_x, d_y = orig_dist(x, y, d_dist, kernel)
    return d_x, -d_y


def _dist_no_gauss_factor(x, y, d_dist, kernel):
    d_x, d_y = orig_dist(x, y, d_dist, kernel)
    if kernel == o.GAUSSIAN:
        return d_x / 2, d_y / 2
    return d_x, d_y


def _pool_sum(d_l, gh, gw, ph, pw):
    return orig_pool(d_l, gh, gw, ph, pw) * (ph * pw)


def _ns_off_by_one(a, iters, d_x):
    # step t taken back with X_{t+1} in place of X_t.  (Transposing A X_t
    # would not be a mistake here: X_t is a polynomial in the symmetric A, so
    # A X_t is symmetric.)
    alpha = o.ns_alpha(a)
    xs = [alpha * a]
    for _ in range(iters):
        x = xs[-1]
        xs.append(2.0 * x - x @ (a @ x))
    d_a = np.zeros_like(a)
    g = d_x
    for t in range(iters - 1, -1, -1):
        x = xs[t + 1]
        d_a -= x.T @ g @ x.T
        g = 2.0 * g - g @ (a @ x).T - (x @ a).T @ g
    d_a += alpha * g
    d_a += orig_alpha(a, float((g * a).sum()))
    return d_a


MUTANTS = [
    ("ns_alpha_backward", _no_alpha, dict(seed=2, kernel=o.LAPLACIAN, iters=0)),
    ("distance_backward", _dist_y_wrong_sign, dict(seed=1, kernel=o.LAPLACIAN, iters=3)),
    ("distance_backward", _dist_no_gauss_factor, dict(seed=4, kernel=o.GAUSSIAN, iters=3)),
    ("avg_pool_backward", _pool_sum, dict(seed=1, kernel=o.LAPLACIAN, iters=3)),
    ("newton_schulz_backward", _ns_off_by_one, dict(seed=3, kernel=o.LAPLACIAN, iters=8)),
]


@pytest.mark.parametrize("name,fn,case", MUTANTS, ids=[f"{m[0]}:{m[1].__name__}" for m in MUTANTS])
def test_planted_mistake_is_caught(monkeypatch, name, fn, case):
    monkeypatch.setattr(ob, name, fn)
    case = dict(case)
    seed = case.pop("seed")
    with pytest.raises(AssertionError):
        _check_fd(*_case(seed, **case))
