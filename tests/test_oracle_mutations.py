"""Plant plausible mistakes in the oracle (on the CPU, via monkeypatch) and
check that at least one independent pin fails for each of them.

This is what makes the pins meaningful: a dropped term, a wrong sign, a wrong
index order or a swapped operand anywhere in the oracle is caught.
"""
import numpy as np
import pytest

import oracle.nystrom as o
import pins

orig_pool = o.landmarks_avg_pool
orig_dist = o.distance_matrix
orig_ns = o.newton_schulz
orig_head = o.nystrom_head


def pool_column_major(k, gh, gw, ph, pw):
    L = orig_pool(k, gh, gw, ph, pw)
    mh, mw = gh // ph, gw // pw
    return L.reshape(mh, mw, -1).transpose(1, 0, 2).reshape(mh * mw, -1)


def pool_sum(k, gh, gw, ph, pw):
    return orig_pool(k, gh, gw, ph, pw) * (ph * pw)


def pool_swapped_window(k, gh, gw, ph, pw):
    # window height/width exchanged wherever the grid still tiles that way
    if gh % pw or gw % ph:
        return orig_pool(k, gh, gw, ph, pw)
    return orig_pool(k, gh, gw, pw, ph)


def dist_l2_for_laplacian(x, y, kernel):
    if kernel == o.LAPLACIAN:
        return np.sqrt(orig_dist(x, y, o.GAUSSIAN))
    return orig_dist(x, y, kernel)


def dist_signed(x, y, kernel):
    if kernel == o.LAPLACIAN:
        return np.stack([(x - y[j]).sum(axis=1) for j in range(y.shape[0])], axis=1)
    return orig_dist(x, y, kernel)


def dist_gauss_not_squared(x, y, kernel):
    if kernel == o.GAUSSIAN:
        return np.sqrt(orig_dist(x, y, kernel))
    return orig_dist(x, y, kernel)


def kmap_positive_exponent(x, y, lam, kernel):
    return np.exp(o.distance_matrix(x, y, kernel) / lam)


def kmap_times_lambda(x, y, lam, kernel):
    return np.exp(-o.distance_matrix(x, y, kernel) * lam)


def lmat_no_eps(l, lam, eps, kernel):
    return o.kernel_map(l, l, lam, kernel)


def lmat_eps_everywhere(l, lam, eps, kernel):
    return o.kernel_map(l, l, lam, kernel) + eps


def alpha_one_norm_only(a):
    return 1.0 / (np.abs(a).sum(axis=0).max() ** 2)


def alpha_frobenius(a):
    return 1.0 / np.linalg.norm(a, "fro") ** 2


def ns_dropped_factor(a, iters):
    x = o.ns_alpha(a) * a
    for _ in range(iters):
        x = 2.0 * x - x @ a
    return x


def ns_one_short(a, iters):
    return orig_ns(a, max(iters - 1, 0))


def ns_wrong_sign(a, iters):
    x = o.ns_alpha(a) * a
    for _ in range(iters):
        x = 2.0 * x + x @ (a @ x)
    return x


def head_pools_queries(q, k, v, **kw):
    return _head_variant(q, k, v, pool_src="q", **kw)


def _head_variant(q, k, v, *, grid_h, grid_w, pool_h, pool_w, lam, eps, iters,
                  kernel=o.LAPLACIAN, pool_src="k", w_map="klk", skip_x=False,
                  out_map="kql"):
    L = o.landmarks_avg_pool(q if pool_src == "q" else k, grid_h, grid_w, pool_h, pool_w)
    kql = o.kernel_map(q, L, lam, kernel)
    klk = o.kernel_map(L, k, lam, kernel)
    A = o.landmark_matrix(L, lam, eps, kernel)
    X = o.newton_schulz(A, iters)
    W = (klk if w_map == "klk" else kql.T) @ v
    Y = W if skip_x else X @ W
    O = (kql if out_map == "kql" else klk.T) @ Y
    return {"L": L, "KQL": kql, "KLK": klk, "A": A, "X": X, "W": W, "Y": Y, "O": O}


def head_w_from_kql(q, k, v, **kw):
    return _head_variant(q, k, v, w_map="kqlT", **kw)


def head_skip_inverse(q, k, v, **kw):
    return _head_variant(q, k, v, skip_x=True, **kw)


def head_out_from_klk(q, k, v, **kw):
    return _head_variant(q, k, v, out_map="klkT", **kw)


def widen_bf16_as_f16(x, dtype):
    if dtype == "bf16":
        return np.asarray(x, dtype=np.uint16).view(np.float16).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def full_attention_reversed(q, k, v, lam, kernel="laplacian"):
    # k(K, Q) V only type-checks when there are as many queries as keys;
    # elsewhere the mutant computes the right thing, so only a square case
    # can catch it
    if q.shape[0] != k.shape[0]:
        return o.kernel_map(q, k, lam, kernel) @ v
    return o.kernel_map(k, q, lam, kernel) @ v


def full_attention_no_v(q, k, v, lam, kernel="laplacian"):
    return o.kernel_map(q, k, lam, kernel).sum(axis=1, keepdims=True) * v.mean(axis=0)


MUTATIONS = {
    "full attention uses k(K, Q)": ("full_kernel_attention", full_attention_reversed),
    "full attention drops V's rows": ("full_kernel_attention", full_attention_no_v),
    "pool raster order column-major": ("landmarks_avg_pool", pool_column_major),
    "pool sums instead of averaging": ("landmarks_avg_pool", pool_sum),
    "pool window height/width swapped": ("landmarks_avg_pool", pool_swapped_window),
    "L1 replaced by L2": ("distance_matrix", dist_l2_for_laplacian),
    "abs dropped in L1": ("distance_matrix", dist_signed),
    "Gaussian distance not squared": ("distance_matrix", dist_gauss_not_squared),
    "kernel exponent sign flipped": ("kernel_map", kmap_positive_exponent),
    "lambda multiplies instead of divides": ("kernel_map", kmap_times_lambda),
    "eps I dropped": ("landmark_matrix", lmat_no_eps),
    "eps added to every entry": ("landmark_matrix", lmat_eps_everywhere),
    "alpha from the 1-norm only": ("ns_alpha", alpha_one_norm_only),
    "alpha from the Frobenius norm": ("ns_alpha", alpha_frobenius),
    "NS drops the trailing X": ("newton_schulz", ns_dropped_factor),
    "NS one iteration short": ("newton_schulz", ns_one_short),
    "NS sign flipped": ("newton_schulz", ns_wrong_sign),
    "landmarks pooled from queries": ("nystrom_head", head_pools_queries),
    "W uses K_QL^T instead of K_LK": ("nystrom_head", head_w_from_kql),
    "inverse skipped": ("nystrom_head", head_skip_inverse),
    "output uses K_LK^T instead of K_QL": ("nystrom_head", head_out_from_klk),
    "bf16 widened as fp16": ("widen", widen_bf16_as_f16),
}


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, bad = MUTATIONS[name]
    monkeypatch.setattr(o, attr, bad)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(o)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin catches the planted mistake: {name}"
