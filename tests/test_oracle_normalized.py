"""Pins of the normalised feature map (oracle.nystrom.normalized_feature_map
and nystrom_head_normalized) against things that do not come from it:
closed forms of its column moments, invariances of centring and diagonal
whitening, a loops-only brute force, and planted mistakes.  CPU only."""
import math

import numpy as np
import pytest

import oracle.nystrom as o
from pins import _pure_python_head


def _kql(seed=1, n=40, m=7):
    r = np.random.default_rng(seed)
    return np.exp(-np.abs(r.standard_normal((n, m))) * r.uniform(0.5, 2.0, m))


def pin_column_moments(f):
    """Every column of Z has mean 0 and population variance var / (var +
    delta) (= 1 with delta = 0)."""
    k = _kql()
    var = k.var(axis=0)
    for delta in (0.0, 1e-2):
        z = f(k, delta)
        assert np.abs(z.mean(axis=0)).max() < 1e-12, "columns not centred"
        assert np.allclose(z.var(axis=0), var / (var + delta), rtol=1e-12), "column variance"


def pin_shift_and_scale_invariance(f):
    """Adding a constant to a column changes nothing; with delta = 0 neither
    does scaling a column by a positive factor (the diagonal estimator
    normalises each dimension on its own)."""
    k = _kql(2)
    r = np.random.default_rng(3)
    shift = r.standard_normal(k.shape[1])
    scale = r.uniform(0.1, 10.0, k.shape[1])
    assert np.allclose(f(k + shift, 1e-3), f(k, 1e-3), atol=1e-12), "shift"
    assert np.allclose(f(k * scale, 0.0), f(k, 0.0), atol=1e-10), "scale"


def pin_brute_force(f):
    """Loops only, on a 5 x 3 similarity matrix."""
    k = _kql(4, n=5, m=3)
    delta = 0.05
    n, m = k.shape
    ref = [[0.0] * m for _ in range(n)]
    for j in range(m):
        mu = sum(k[i][j] for i in range(n)) / n
        var = sum((k[i][j] - mu) ** 2 for i in range(n)) / n
        for i in range(n):
            ref[i][j] = (k[i][j] - mu) / math.sqrt(var + delta)
    assert np.allclose(f(k, delta), np.array(ref), rtol=1e-13, atol=1e-15), "brute force"


PINS = [pin_column_moments, pin_shift_and_scale_invariance, pin_brute_force]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(o.normalized_feature_map)


def _mutant(kind):
    def f(k, delta):
        mu = k.mean(axis=0)
        if kind == "sample variance":
            var = k.var(axis=0, ddof=1)
        elif kind == "row statistics":
            mu = k.mean(axis=1, keepdims=True)
            var = k.var(axis=1, keepdims=True)
        else:
            var = k.var(axis=0)
        if kind == "divide by variance":
            return (k - mu) / (var + delta)
        if kind == "delta outside the root":
            return (k - mu) / (np.sqrt(var) + delta)
        if kind == "not centred":
            return k / np.sqrt(var + delta)
        return (k - mu) / np.sqrt(var + delta)
    return f


@pytest.mark.parametrize("kind", ["sample variance", "row statistics", "divide by variance",
                                  "delta outside the root", "not centred"])
def test_mutation_is_caught(kind):
    failed = []
    for pin in PINS:
        try:
            pin(_mutant(kind))
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, kind


def test_head_with_normalised_map_brute_force():
    """The whole head: loops-only forward, then Z from its K_QL, then Z Y."""
    r = np.random.default_rng(12)
    gh, gw, ph, pw, d = 4, 6, 2, 3, 3
    n = gh * gw
    q, k, v = (r.standard_normal((n, d)) for _ in range(3))
    ref = _pure_python_head(q.tolist(), k.tolist(), v.tolist(), gh, gw, ph, pw, 1.7, 0.1, 5,
                            "laplacian")
    kql = ref["KQL"]
    m = len(kql[0])
    delta = 1e-3
    Z = [[0.0] * m for _ in range(n)]
    for j in range(m):
        mu = sum(kql[i][j] for i in range(n)) / n
        var = sum((kql[i][j] - mu) ** 2 for i in range(n)) / n
        for i in range(n):
            Z[i][j] = (kql[i][j] - mu) / math.sqrt(var + delta)
    Y = [[sum(ref["X"][a][b] * ref["W"][b][c] for b in range(m)) for c in range(d)]
         for a in range(m)]
    O = [[sum(Z[i][j] * Y[j][c] for j in range(m)) for c in range(d)] for i in range(n)]
    got = o.nystrom_head_normalized(q, k, v, grid_h=gh, grid_w=gw, pool_h=ph, pool_w=pw,
                                    lam=1.7, eps=0.1, iters=5, delta=delta)["O"]
    assert np.abs(got - np.array(O)).max() / np.abs(np.array(O)).max() < 1e-10
