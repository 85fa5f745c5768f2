"""Parity of the HIP backward pass (lapattn_backward, through the C ABI)
against the fp64 backward oracle (oracle/backward.py).

Bar, per head and per gradient g in (dQ, dK, dV):
    |g_gpu - g_ref| <= tol * max|g_ref| + allowance      elementwise,
tol = 2e-3 with fp32 I/O and 2e-2 with bf16 I/O (the forward's bar).

The allowance is zero except at the kinks of the L1 distance.  Its
derivative takes sign(x_k - l_k); where a coordinate of a query or key lies
within rounding of a landmark's, the GPU (fp32 landmark) and the oracle
(fp64 landmark) may take opposite signs, and both are valid subgradients of
the same function.  The test finds exactly those terms, comparing
sign(x - l_gpu) with sign(x - l_ref) (the GPU's landmarks come from the same
pool kernel through lapattn_forward_stages), and allows 2 |w| for each in the
elements the term feeds: dQ or the direct part of dK, dL and through the
pool dK.  Gaussian gradients have no kinks.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_common import device_inputs, tol_for
from nystr_linear_attention_amd import api
from nystr_linear_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _dout(w, seed_off=0):
    """dO drawn from its own stream (N(0,1), cast to the I/O dtype)."""
    rng = np.random.default_rng(w.seed + 7000 + seed_off)
    a = rng.standard_normal((w.B, w.H, w.N, w.d))
    if w.dtype == wl.BF16:
        return wl.f32_to_bf16_bits(a.astype(np.float32))
    return a.astype(np.float32)


def _sign_flips(x, l_gpu, l_ref):
    """[n, m, d] booleans: sign(x - l) differs between the two landmark sets."""
    return np.sign(x[:, None, :] - l_gpu[None, :, :]) != np.sign(x[:, None, :] - l_ref[None, :, :])


def _allowances(w, q, k, res, l_gpu):
    """Elementwise allowances (dQ, dK) for the L1 kinks; see the module doc."""
    N, d, m = w.N, w.d, w.m
    zq, zk = np.zeros((N, d)), np.zeros((N, d))
    if w.kernel != wl.LAPLACIAN:
        return zq, zk
    L = res["L"]
    kql = oracle.kernel_map(q, L, w.lam, w.kernel)
    klk = oracle.kernel_map(L, k, w.lam, w.kernel)
    wq = np.abs(res["dKQL"] * kql / w.lam)          # [N, m]
    wk = np.abs(res["dKLK"] * klk / w.lam).T        # [N, m]
    a_dL = np.zeros((m, d))
    for x, wx, out in ((q, wq, zq), (k, wk, zk)):
        for n0 in range(0, N, 512):
            f = _sign_flips(x[n0:n0 + 512], l_gpu, L)          # [b, m, d]
            contrib = 2.0 * wx[n0:n0 + 512, :, None] * f
            out[n0:n0 + 512] += contrib.sum(axis=1)
            a_dL += contrib.sum(axis=0)
    kll = oracle.kernel_map(L, L, w.lam, w.kernel)
    dd = np.abs(res["dA"] * kll / w.lam)
    f = np.sign(l_gpu[:, None, :] - l_gpu[None, :, :]) != np.sign(L[:, None, :] - L[None, :, :])
    a_dL += 2.0 * ((dd + dd.T)[:, :, None] * f).sum(axis=1)
    # through the pool: dK of window j gains dL[j] / (ph pw)
    mw = w.grid_w // w.pool_w
    for n in range(N):
        r, c = divmod(n, w.grid_w)
        zk[n] += a_dL[(r // w.pool_h) * mw + c // w.pool_w] / (w.pool_h * w.pool_w)
    return zq, zk


def _alpha_margin(A):
    cs = np.sort(np.abs(A).sum(axis=0))
    return (cs[-1] - cs[-2]) / cs[-1] if len(cs) > 1 else 1.0


def run_backward_case(w, heads=None, seed_off=0):
    x = wl.make_inputs(w)
    dO = _dout(w, seed_off)
    q, k, v = device_inputs(w, x)
    g = torch.from_numpy(dO.view(np.int16) if w.dtype == wl.BF16 else dO).cuda()
    if w.dtype == wl.BF16:
        g = g.view(torch.bfloat16)
    kw = dict(grid_h=w.grid_h, grid_w=w.grid_w, pool_h=w.pool_h, pool_w=w.pool_w,
              lam=w.lam, eps=w.eps, iters=w.iters, kernel=w.kernel)
    desc = api.make_desc(w.B, w.H, w.grid_h, w.grid_w, w.d, w.pool_h, w.pool_w, w.kernel, q.dtype)
    ws = torch.full((api.backward_workspace_bytes(desc, w.iters),), 0xFF, dtype=torch.uint8,
                    device="cuda")  # poisoned: contents on entry must not matter
    dq, dk, dv = api.backward(q, k, v, g, workspace=ws, **kw)
    l_gpu = api.forward_stages(q, k, v, **kw)["L"].double().cpu().numpy()
    torch.cuda.synchronize()
    got = {n: t.float().cpu().numpy().astype(np.float64) for n, t in (("dQ", dq), ("dK", dk), ("dV", dv))}
    if heads is None:
        heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    tol = tol_for(w)
    worst = {"dQ": 0.0, "dK": 0.0, "dV": 0.0}
    for (b, h) in heads:
        qq = oracle.widen(x["q"][b, h], w.dtype)
        kk = oracle.widen(x["k"][b, h], w.dtype)
        vv = oracle.widen(x["v"][b, h], w.dtype)
        gg = oracle.widen(dO[b, h], w.dtype)
        res = oracle.backward.nystrom_head_backward(
            qq, kk, vv, gg, grid_h=w.grid_h, grid_w=w.grid_w, pool_h=w.pool_h,
            pool_w=w.pool_w, lam=w.lam, eps=w.eps, iters=w.iters, kernel=w.kernel)
        res["L"] = oracle.landmarks_avg_pool(kk, w.grid_h, w.grid_w, w.pool_h, w.pool_w)
        A = oracle.landmark_matrix(res["L"], w.lam, w.eps, w.kernel)
        assert _alpha_margin(A) > 1e-5, "alpha's maxima nearly tied: test input not usable"
        aq, ak = _allowances(w, qq, kk, res, l_gpu[b, h])
        for name, allow in (("dQ", aq), ("dK", ak), ("dV", 0.0)):
            ref, gv = res[name], got[name][b, h]
            assert np.isfinite(gv).all(), f"{name} head ({b},{h}): non-finite"
            scale = max(np.abs(ref).max(), 1e-300)
            excess = np.abs(gv - ref) - allow
            err = float(max(excess.max(), 0.0) / scale)
            worst[name] = max(worst[name], err)
            assert err <= tol, f"{w.name} {name} head ({b},{h}): error {err:.3e} beyond allowance"
    return worst


def _print_case(w, extra=""):
    print(f"\n[case] backward {w.name} B={w.B} H={w.H} N={w.N} d={w.d} m={w.m} "
          f"kernel={w.kernel} dtype={w.dtype} iters={w.iters} {extra}", flush=True)


# heads checked per workload: all of the small-head ones, four of the others
def _heads(w):
    if w.heads <= 8:
        return None
    return [(0, 0), (w.B - 1, w.H - 1), (w.B // 2, 0), (1 % w.B, (w.H - 1) // 2)]


@pytest.mark.parametrize("idx", range(len(wl.WORKLOADS)), ids=[w.name for w in wl.WORKLOADS])
def test_backward_full_size_workloads(idx):
    w = wl.WORKLOADS[idx]
    _print_case(w)
    worst = run_backward_case(w, heads=_heads(w))
    print(f"[case] worst errors beyond allowance: "
          + ", ".join(f"{n} {e:.2e}" for n, e in worst.items()), flush=True)


SMALL = [
    wl.small_case(10, 14, 32, 2, 2, B=2, H=3),                   # ragged tiles, m=35
    wl.small_case(9, 9, 16, 3, 3, B=1, H=2),                     # d=16, m=9
    wl.small_case(4, 4, 16, 1, 1),                               # N=16 < one tile, pool 1x1
    wl.small_case(8, 8, 64, 1, 1, B=2),                          # m=64
    wl.small_case(7, 9, 32, 7, 9, B=3),                          # m=1
    wl.small_case(12, 12, 64, 2, 2, iters=0),                    # X = alpha A
    wl.small_case(8, 12, 64, 2, 2, B=2, iters=1),                # one Newton-Schulz step
    wl.small_case(12, 20, 32, 3, 4, kernel=wl.GAUSSIAN, B=2),    # Gaussian, Q != K
    wl.small_case(16, 16, 64, 2, 2, shared_qk=True),             # Laplacian, Q = K
    wl.small_case(10, 10, 64, 2, 2, kernel=wl.GAUSSIAN, dtype=wl.BF16, B=2, shared_qk=True),
    wl.small_case(10, 14, 64, 2, 2, dtype=wl.BF16, B=2, H=2),    # bf16, ragged
    wl.small_case(12, 16, 32, 2, 2, B=2, eps=0.0),               # no diagonal perturbation
    wl.small_case(40, 40, 64, 5, 5, iters=64),                   # N=1600, the most steps
    wl.small_case(64, 128, 64, 16, 16),                          # 128 tiles: 2 per partial WG
]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_backward_small_and_edge_cases(w):
    _print_case(w)
    run_backward_case(w)


def test_backward_is_deterministic():
    """Every reduction runs in a fixed order: two calls give the same bits."""
    w = wl.HEADLINE
    x = wl.make_inputs(w)
    q, k, v = device_inputs(w, x)
    g = torch.from_numpy(_dout(w)).cuda()
    kw = dict(grid_h=w.grid_h, grid_w=w.grid_w, pool_h=w.pool_h, pool_w=w.pool_w,
              lam=w.lam, eps=w.eps, iters=w.iters)
    a = api.backward(q, k, v, g, **kw)
    b = api.backward(q, k, v, g, **kw)
    torch.cuda.synchronize()
    for ta, tb in zip(a, b):
        assert torch.equal(ta, tb)


def test_backward_rejects_bad_arguments():
    q = torch.randn(1, 1, 196, 32, device="cuda")
    g = torch.randn_like(q)
    kw = dict(grid_h=14, grid_w=14, pool_h=2, pool_w=2, lam=32.0, eps=1e-3, iters=3)
    with pytest.raises(ValueError):
        api.backward(q, q, q, g[..., :16].contiguous(), **kw)
    with pytest.raises(api._lib.LapattnError) as e:
        api.backward(q, q, q, g, **dict(kw, lam=0.0))
    assert e.value.status == api._lib.ERR_PARAM
