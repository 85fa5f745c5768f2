"""Parity of the normalised-feature-map forward (lapattn_forward_normalized,
through the C ABI) against the fp64 oracle (oracle.nystrom.forward_normalized):
per head, max|O_gpu - O_ref| / max|O_ref| <= 2e-3 (fp32 I/O), 2e-2 (bf16 I/O)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_common import device_inputs, normwise, poisoned_workspace, tol_for
from nystr_linear_attention_amd import api
from nystr_linear_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu

DELTA = 1e-5


def run_normalized(w, heads=None, delta=DELTA):
    x = wl.make_inputs(w)
    q, k, v = device_inputs(w, x)
    desc = api.make_desc(w.B, w.H, w.grid_h, w.grid_w, w.d, w.pool_h, w.pool_w, w.kernel, q.dtype)
    ws = poisoned_workspace(desc)
    out = api.forward_normalized(q, k, v, grid_h=w.grid_h, grid_w=w.grid_w, pool_h=w.pool_h,
                                 pool_w=w.pool_w, lam=w.lam, eps=w.eps, iters=w.iters,
                                 delta=delta, kernel=w.kernel, workspace=ws)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    ref = oracle.nystrom.forward_normalized(x["q"], x["k"], x["v"], grid_h=w.grid_h,
                                            grid_w=w.grid_w, pool_h=w.pool_h, pool_w=w.pool_w,
                                            lam=w.lam, eps=w.eps, iters=w.iters, delta=delta,
                                            kernel=w.kernel, dtype=w.dtype, heads=heads)
    worst = 0.0
    for (b, h), r in ref.items():
        err = normwise(got[b, h], r)
        worst = max(worst, err)
        assert np.isfinite(got[b, h]).all()
        assert err <= tol_for(w), f"{w.name} head ({b},{h}): {err:.3e}"
    return worst


def _heads(w):
    if w.heads <= 8:
        return None
    return [(0, 0), (w.B - 1, w.H - 1), (w.B // 2, 0)]


@pytest.mark.parametrize("idx", range(len(wl.WORKLOADS)), ids=[w.name for w in wl.WORKLOADS])
def test_normalized_full_size_workloads(idx):
    w = wl.WORKLOADS[idx]
    print(f"\n[case] normalized {w.name}", flush=True)
    worst = run_normalized(w, heads=_heads(w))
    print(f"[case] worst normwise error {worst:.3e}", flush=True)


SMALL = [
    wl.small_case(10, 14, 32, 2, 2, B=2, H=3),              # ragged tiles, m=35
    wl.small_case(9, 9, 16, 3, 3, B=1, H=2),                # d=16, m=9
    wl.small_case(8, 8, 64, 1, 1, B=2),                     # m=64
    wl.small_case(7, 9, 32, 7, 9, B=3),                     # m=1: one column of Z
    wl.small_case(12, 20, 32, 3, 4, kernel=wl.GAUSSIAN, B=2),
    wl.small_case(16, 16, 64, 2, 2, shared_qk=True),
    wl.small_case(10, 14, 64, 2, 2, dtype=wl.BF16, B=2, H=2),
]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_normalized_small_cases(w):
    run_normalized(w)


def test_normalized_rejects_bad_delta():
    q = torch.randn(1, 1, 196, 32, device="cuda")
    with pytest.raises(api._lib.LapattnError):
        api.forward_normalized(q, q, q, grid_h=14, grid_w=14, pool_h=2, pool_w=2, lam=32.0,
                               eps=1e-3, iters=3, delta=-1.0)
