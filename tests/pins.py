"""Independent pins for the fp64 oracle.

Each ``pin_*`` function takes the oracle module (``oracle.nystrom``) and raises
``AssertionError`` when the oracle disagrees with something that does not come
from the oracle itself: a closed form, a SciPy / LAPACK routine, an invariant
the pages state, or brute force at a tiny size.  The same functions run on the
real oracle (test_oracle_pins.py) and on deliberately broken copies of it
(test_oracle_mutations.py), which shows each planted mistake is caught.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.spatial.distance import cdist

RNG_SEED = 20240611


def _rng(k=0):
    return np.random.default_rng(RNG_SEED + k)


def _close(a, b, rtol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    scale = max(np.abs(b).max(), 1e-300)
    err = np.abs(a - b).max() / scale
    assert err <= rtol, f"{what}: normwise error {err:.3e} > {rtol:.1e}"


# ----------------------------------------------------------------------------
# Landmark pooling
# ----------------------------------------------------------------------------

def pin_pool_identity(o):
    """A 1x1 pool returns every token as its own landmark, bit for bit."""
    k = _rng(1).standard_normal((5 * 7, 6))
    L = o.landmarks_avg_pool(k, 5, 7, 1, 1)
    assert L.shape == k.shape and np.array_equal(L, k), "1x1 pool is not the identity"


def pin_pool_raster_geometry(o):
    """Tokens carrying their own (row, col) pool to the window centres.

    Non-square grid and non-square window, so a swap of rows and columns or
    of the raster order moves a landmark and fails the check.
    """
    for gh, gw, ph, pw in ((6, 12, 3, 4), (12, 12, 3, 4), (8, 4, 4, 1)):
        k = np.array([[r, c] for r in range(gh) for c in range(gw)], dtype=np.float64)
        L = o.landmarks_avg_pool(k, gh, gw, ph, pw)
        mw = gw // pw
        expect = np.array([[R * ph + (ph - 1) / 2.0, C * pw + (pw - 1) / 2.0]
                           for R in range(gh // ph) for C in range(mw)])
        assert L.shape == expect.shape, f"landmark count {L.shape} vs {expect.shape}"
        assert np.array_equal(L, expect), "landmarks are not the raster-ordered window means"


def pin_pool_reshape_mean(o):
    """Second path: NumPy reshape + mean over the window axes."""
    gh, gw, ph, pw, d = 8, 10, 4, 2, 5
    k = _rng(2).standard_normal((gh * gw, d))
    L = o.landmarks_avg_pool(k, gh, gw, ph, pw)
    ref = k.reshape(gh // ph, ph, gw // pw, pw, d).mean(axis=(1, 3)).reshape(-1, d)
    _close(L, ref, 1e-15, "avg-pool vs reshape-mean")


def pin_pool_constant_windows(o):
    """Windows filled with one constant pool to that constant."""
    gh, gw, ph, pw, d = 4, 6, 2, 3, 3
    k = np.zeros((gh * gw, d))
    for r in range(gh):
        for c in range(gw):
            k[r * gw + c] = 10.0 * (r // ph) + (c // pw) + np.arange(d) * 0.25
    L = o.landmarks_avg_pool(k, gh, gw, ph, pw)
    for R in range(gh // ph):
        for C in range(gw // pw):
            assert np.array_equal(L[R * (gw // pw) + C], 10.0 * R + C + np.arange(d) * 0.25)


# ----------------------------------------------------------------------------
# Distances and kernels
# ----------------------------------------------------------------------------

def pin_distance_vs_scipy(o):
    """L1 and squared-L2 distances against scipy.spatial.distance.cdist."""
    r = _rng(3)
    x = r.standard_normal((37, 9))
    y = r.standard_normal((11, 9)) * 2.0
    _close(o.distance_matrix(x, y, o.LAPLACIAN), cdist(x, y, metric="cityblock"),
           1e-14, "L1 distance vs cdist(cityblock)")
    _close(o.distance_matrix(x, y, o.GAUSSIAN), cdist(x, y, metric="sqeuclidean"),
           1e-13, "squared L2 vs cdist(sqeuclidean)")


def pin_kernel_closed_form(o):
    """Hand-computed values: x=(0,0), y=(1,-2): L1 = 3, squared L2 = 5."""
    x = np.array([[0.0, 0.0]])
    y = np.array([[1.0, -2.0]])
    for lam in (0.5, 2.0, 16.0):
        kl = o.kernel_map(x, y, lam, o.LAPLACIAN)[0, 0]
        kg = o.kernel_map(x, y, lam, o.GAUSSIAN)[0, 0]
        assert abs(kl - math.exp(-3.0 / lam)) <= 1e-15, f"Laplacian k at lambda={lam}"
        assert abs(kg - math.exp(-5.0 / lam)) <= 1e-15, f"Gaussian k at lambda={lam}"


def pin_kernel_invariants(o):
    """Symmetric, in (0, 1], unit diagonal (SOFT: symmetric, values in [0,1])."""
    r = _rng(4)
    pts = r.standard_normal((23, 16))
    for kern in (o.LAPLACIAN, o.GAUSSIAN):
        kk = o.kernel_map(pts, pts, 8.0, kern)
        assert np.array_equal(kk, kk.T), f"{kern}: k(L, L) not symmetric"
        assert np.all(kk > 0.0) and np.all(kk <= 1.0), f"{kern}: values outside (0, 1]"
        assert np.array_equal(np.diag(kk), np.ones(23)), f"{kern}: diagonal is not 1"


def pin_landmark_matrix_structure(o):
    """A - k(L, L) is exactly eps * I, and A is positive definite (min eig >= eps)."""
    r = _rng(5)
    L = r.standard_normal((49, 64)) * 0.1
    for kern, eps in ((o.LAPLACIAN, 1e-3), (o.GAUSSIAN, 1e-2)):
        A = o.landmark_matrix(L, 16.0, eps, kern)
        K = o.kernel_map(L, L, 16.0, kern)
        _close(A - K, eps * np.eye(49), 1e-12, f"{kern}: A - k(L,L) vs eps I")
        w = np.linalg.eigvalsh(A)
        assert w.min() >= eps * (1 - 1e-6), f"{kern}: min eigenvalue {w.min()} < eps"
        np.linalg.cholesky(A)


# ----------------------------------------------------------------------------
# Newton-Schulz
# ----------------------------------------------------------------------------

def _spd(n, seed, cond_shift=0.05):
    r = _rng(seed)
    m = r.standard_normal((n, n))
    return m @ m.T / n + cond_shift * np.eye(n)


def pin_ns_alpha(o):
    """alpha = 1 / (||A||_1 ||A||_inf) via numpy.linalg.norm, on a non-symmetric matrix."""
    r = _rng(6)
    a = r.standard_normal((7, 7))
    a[0, :] *= 5.0  # make row and column norms differ
    ref = 1.0 / (np.linalg.norm(a, 1) * np.linalg.norm(a, np.inf))
    got = o.ns_alpha(a)
    assert abs(got - ref) <= 1e-15 * ref, f"alpha {got} vs {ref}"


def pin_ns_converges_to_inverse(o):
    """Run long enough to converge: ||A X - I||_F < 1e-6 and X = LAPACK inv(A)."""
    for n, seed in ((49, 7), (64, 8), (5, 9)):
        A = _spd(n, seed)
        X = o.newton_schulz(A, 100)
        res = np.linalg.norm(A @ X - np.eye(n), "fro")
        assert res < 1e-6, f"NS residual {res:.3e} at n={n}"
        _close(X, np.linalg.inv(A), 1e-9, f"NS vs inv at n={n}")


def pin_ns_spectral_fixed_iters(o):
    """Fixed iteration count against the eigen-decomposition closed form.

    With A = V diag(mu) V^T every iterate is V diag(x_t(mu)) V^T where the
    scalar map is x_0 = alpha mu, x_{t+1} = 2 x_t - mu x_t^2.  Checked at
    iteration counts short of convergence, where an off-by-one or a wrong
    alpha changes the result.
    """
    A = _spd(40, 10, cond_shift=1e-3)
    mu, V = np.linalg.eigh(A)
    alpha = 1.0 / (np.linalg.norm(A, 1) * np.linalg.norm(A, np.inf))
    for iters in (0, 1, 3, 8, 15):
        x = alpha * mu
        for _ in range(iters):
            x = 2.0 * x - mu * x * x
        ref = (V * x) @ V.T
        _close(o.newton_schulz(A, iters), ref, 1e-9, f"NS spectral, iters={iters}")


# ----------------------------------------------------------------------------
# Whole-head forward
# ----------------------------------------------------------------------------

def pin_single_landmark_closed_form(o):
    """m = 1 (pool = whole grid): A = 1 + eps, X = 1/(1+eps) for any iters.

    O_i = k(q_i, l) / (1 + eps) * sum_j k(l, k_j) v_j with l = mean(K);
    evaluated with math.exp in plain loops.
    """
    r = _rng(11)
    gh, gw, d = 3, 5, 4
    n = gh * gw
    q = r.standard_normal((n, d))
    k = r.standard_normal((n, d))
    v = r.standard_normal((n, d))
    lam, eps = 2.5, 0.05
    l = [sum(k[t, c] for t in range(n)) / n for c in range(d)]
    for kern in ("laplacian", "gaussian"):
        def kv(a, b):
            if kern == "laplacian":
                dist = sum(abs(a[c] - b[c]) for c in range(d))
            else:
                dist = sum((a[c] - b[c]) ** 2 for c in range(d))
            return math.exp(-dist / lam)
        w = [sum(kv(l, k[t]) * v[t, c] for t in range(n)) for c in range(d)]
        ref = np.array([[kv(q[i], l) / (1.0 + eps) * w[c] for c in range(d)]
                        for i in range(n)])
        for iters in (0, 1, 20):
            res = o.nystrom_head(q, k, v, grid_h=gh, grid_w=gw, pool_h=gh,
                                 pool_w=gw, lam=lam, eps=eps, iters=iters,
                                 kernel=kern)
            _close(res["O"], ref, 1e-13, f"m=1 closed form ({kern}, iters={iters})")


def pin_nystrom_exact_all_landmarks(o):
    """Landmarks = all tokens (1x1 pool), eps = 0, converged NS: the Nystrom
    product reproduces exact kernel attention k(Q, K) V (brute force, N = 36).

    Q != K, so swapping which map feeds W, or dropping the inverse, fails.
    """
    r = _rng(12)
    gh, gw, d = 6, 6, 8
    n = gh * gw
    q = r.standard_normal((n, d))
    k = r.standard_normal((n, d))
    v = r.standard_normal((n, d))
    lam = 2.0 * math.sqrt(d)
    for kern in ("laplacian", "gaussian"):
        ref = _brute_full_attention(q, k, v, lam, kern)
        res = o.nystrom_head(q, k, v, grid_h=gh, grid_w=gw, pool_h=1, pool_w=1,
                             lam=lam, eps=0.0, iters=80, kernel=kern)
        _close(res["O"], ref, 1e-9, f"Nystrom exactness ({kern})")


def _brute_full_attention(q, k, v, lam, kern):
    """sum_j k(q_i, k_j) v_j with scalar loops only (no oracle code)."""
    n, d = len(q), len(q[0])

    def kv(a, b):
        diff = [a[c] - b[c] for c in range(d)]
        dist = sum(abs(x) for x in diff) if kern == "laplacian" else sum(x * x for x in diff)
        return math.exp(-dist / lam)
    return np.array([[sum(kv(q[i], k[j]) * v[j][c] for j in range(len(k)))
                      for c in range(len(v[0]))] for i in range(n)])


def pin_full_kernel_attention_brute_force(o):
    """Exact kernel attention k(Q, K) V against loops-only brute force, with
    Q != K, different query and key counts and d_v != d, so a transposed
    kernel matrix, swapped arguments or a wrong contraction fails."""
    r = _rng(19)
    nq, nk, d, dv = 7, 11, 5, 3
    q = r.standard_normal((nq, d))
    k = r.standard_normal((nk, d)) + 0.3
    v = r.standard_normal((nk, dv))
    for kern, lam in (("laplacian", 3.0), ("gaussian", 4.5)):
        got = o.full_kernel_attention(q, k, v, lam, kern)
        _close(got, _brute_full_attention(q, k, v, lam, kern), 1e-13,
               f"full kernel attention ({kern})")
    # square and Q != K: the reversed map k(K, Q) has the same shape
    qs = r.standard_normal((9, d))
    ks = r.standard_normal((9, d)) - 0.2
    vs = r.standard_normal((9, dv))
    _close(o.full_kernel_attention(qs, ks, vs, 3.0, "laplacian"),
           _brute_full_attention(qs, ks, vs, 3.0, "laplacian"), 1e-13,
           "full kernel attention (square)")


def _pure_python_head(q, k, v, gh, gw, ph, pw, lam, eps, iters, kern):
    """Brute-force forward for a tiny head, lists and loops only."""
    n, d = len(q), len(q[0])
    mh, mw = gh // ph, gw // pw
    L = []
    for R in range(mh):
        for C in range(mw):
            toks = [r * gw + c for r in range(R * ph, R * ph + ph)
                    for c in range(C * pw, C * pw + pw)]
            L.append([sum(k[t][c] for t in toks) / len(toks) for c in range(d)])
    m = len(L)

    def kv(a, b):
        diff = [a[c] - b[c] for c in range(d)]
        dist = sum(abs(x) for x in diff) if kern == "laplacian" else sum(x * x for x in diff)
        return math.exp(-dist / lam)

    def mm(a, b):
        return [[sum(a[i][t] * b[t][j] for t in range(len(b))) for j in range(len(b[0]))]
                for i in range(len(a))]

    kql = [[kv(q[i], L[j]) for j in range(m)] for i in range(n)]
    klk = [[kv(L[j], k[i]) for i in range(n)] for j in range(m)]
    A = [[kv(L[i], L[j]) + (eps if i == j else 0.0) for j in range(m)] for i in range(m)]
    n1 = max(sum(abs(A[i][j]) for i in range(m)) for j in range(m))
    ninf = max(sum(abs(A[i][j]) for j in range(m)) for i in range(m))
    X = [[A[i][j] / (n1 * ninf) for j in range(m)] for i in range(m)]
    for _ in range(iters):
        XAX = mm(X, mm(A, X))
        X = [[2.0 * X[i][j] - XAX[i][j] for j in range(m)] for i in range(m)]
    W = mm(klk, v)
    O = mm(kql, mm(X, W))
    return {"L": L, "KQL": kql, "KLK": klk, "A": A, "X": X, "W": W, "O": O}


def pin_brute_force_tiny(o):
    """Every stage against a loops-only forward on a 4x6 grid, 2x3 pool."""
    r = _rng(13)
    gh, gw, ph, pw, d = 4, 6, 2, 3, 3
    n = gh * gw
    q = r.standard_normal((n, d))
    k = r.standard_normal((n, d))
    v = r.standard_normal((n, d))
    for kern in ("laplacian", "gaussian"):
        ref = _pure_python_head(q.tolist(), k.tolist(), v.tolist(), gh, gw, ph,
                                pw, 1.7, 0.1, 5, kern)
        got = o.nystrom_head(q, k, v, grid_h=gh, grid_w=gw, pool_h=ph,
                             pool_w=pw, lam=1.7, eps=0.1, iters=5, kernel=kern)
        for key in ("L", "KQL", "KLK", "A", "X", "W", "O"):
            _close(got[key], np.array(ref[key]), 1e-12, f"brute force {key} ({kern})")


def pin_association(o):
    """K_QL (X (K_LK V)) equals ((K_QL X) K_LK) V, the full N x N product."""
    r = _rng(14)
    gh, gw, d = 16, 16, 8
    q, k, v = (r.standard_normal((gh * gw, d)) for _ in range(3))
    res = o.nystrom_head(q, k, v, grid_h=gh, grid_w=gw, pool_h=4, pool_w=4,
                         lam=4.0, eps=1e-3, iters=20)
    full = ((res["KQL"] @ res["X"]) @ res["KLK"]) @ v
    _close(res["O"], full, 1e-10, "association of the Nystrom product")


def pin_shared_qk_transpose(o):
    """With Q = K the two maps are transposes of each other."""
    r = _rng(15)
    x = r.standard_normal((64, 16))
    v = r.standard_normal((64, 16))
    for kern in ("laplacian", "gaussian"):
        res = o.nystrom_head(x, x, v, grid_h=8, grid_w=8, pool_h=2, pool_w=4,
                             lam=8.0, eps=1e-3, iters=10, kernel=kern)
        assert np.array_equal(res["KQL"], res["KLK"].T), f"{kern}: K_QL != K_LK^T for Q = K"


def pin_bf16_widening(o):
    """bf16 bit patterns widen exactly: 0x3F80 = 1, 0xC000 = -2, 0x3F81 = 1 + 2^-7."""
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x4B80], dtype=np.uint16)
    got = o.widen(bits, "bf16")
    ref = np.array([1.0, -2.0, 1.0 + 2.0 ** -7, 0.0, 2.0 ** 24])
    assert np.array_equal(got, ref), f"bf16 widening {got} vs {ref}"


def pin_heads_independent(o):
    """Batched forward equals per-head evaluation (heads do not mix)."""
    r = _rng(16)
    B, H, gh, gw, d = 2, 2, 4, 4, 4
    q, k, v = (r.standard_normal((B, H, gh * gw, d)).astype(np.float32) for _ in range(3))
    out = o.forward(q, k, v, grid_h=gh, grid_w=gw, pool_h=2, pool_w=2,
                    lam=3.0, eps=1e-2, iters=6)
    for b in range(B):
        for h in range(H):
            one = o.nystrom_head(q[b, h].astype(np.float64), k[b, h].astype(np.float64),
                                 v[b, h].astype(np.float64), grid_h=gh, grid_w=gw,
                                 pool_h=2, pool_w=2, lam=3.0, eps=1e-2, iters=6)
            assert np.array_equal(out[(b, h)]["O"], one["O"]), f"head ({b},{h}) mixes"


ALL_PINS = [
    pin_full_kernel_attention_brute_force,
    pin_pool_identity,
    pin_pool_raster_geometry,
    pin_pool_reshape_mean,
    pin_pool_constant_windows,
    pin_distance_vs_scipy,
    pin_kernel_closed_form,
    pin_kernel_invariants,
    pin_landmark_matrix_structure,
    pin_ns_alpha,
    pin_ns_converges_to_inverse,
    pin_ns_spectral_fixed_iters,
    pin_single_landmark_closed_form,
    pin_nystrom_exact_all_landmarks,
    pin_brute_force_tiny,
    pin_association,
    pin_shared_qk_transpose,
    pin_bf16_widening,
    pin_heads_independent,
]
