"""Parity of the attention block (lapattn_block_forward, through the C ABI)
against the fp64 block oracle (oracle/block.py): per batch item,
max|Y_gpu - Y_ref| / max|Y_ref| <= 2e-3 with fp32 I/O, 2e-2 with bf16 I/O."""
import numpy as np
import pytest
import torch

import oracle
from gpu_common import normwise
from nystr_linear_attention_amd import api
from nystr_linear_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _dev(a, dtype):
    if a is None:
        return None
    if dtype == wl.BF16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run_block(w, batch_items=None):
    inp = wl.make_block_inputs(w)
    t = {k: _dev(v, w.dtype) for k, v in inp.items()}
    kw = dict(H=w.H, d=w.d, grid_h=w.grid_h, grid_w=w.grid_w, pool_h=w.pool_h, pool_w=w.pool_w,
              lam=w.lam, eps=w.eps, iters=w.iters, kernel=w.kernel)
    desc = api.make_desc(w.B, w.H, w.grid_h, w.grid_w, w.d, w.pool_h, w.pool_w, w.kernel,
                         t["x"].dtype)
    ws = torch.full((api._lib.lib().lapattn_block_workspace_bytes(desc, w.C),), 0xFF,
                    dtype=torch.uint8, device="cuda")
    y = api.block_forward(t["x"], t["wq"], t["wk"], t["wv"], t["wo"], workspace=ws, **kw)
    torch.cuda.synchronize()
    got = y.float().cpu().numpy().astype(np.float64)
    items = range(w.B) if batch_items is None else batch_items
    sl = lambda a: None if a is None else a[list(items)] if a.ndim == 3 else a  # noqa: E731
    ref = oracle.block.block_forward(sl(inp["x"]), inp["wq"], inp["wk"], inp["wv"], inp["wo"],
                                     H=w.H, d=w.d, grid_h=w.grid_h, grid_w=w.grid_w,
                                     pool_h=w.pool_h, pool_w=w.pool_w, lam=w.lam, eps=w.eps,
                                     iters=w.iters, kernel=w.kernel, dtype=w.dtype)
    tol = 2e-2 if w.dtype == wl.BF16 else 2e-3
    worst = 0.0
    for i, b in enumerate(items):
        err = normwise(got[b], ref[i])
        worst = max(worst, err)
        assert np.isfinite(got[b]).all()
        assert err <= tol, f"{w.name} item {b}: {err:.3e}"
    return worst


@pytest.mark.parametrize("w", wl.BLOCKS, ids=[b.name for b in wl.BLOCKS])
def test_block_stages(w):
    print(f"\n[case] block {w.name}", flush=True)
    worst = run_block(w, batch_items=[0, w.B - 1])
    print(f"[case] worst normwise error {worst:.3e}", flush=True)


SMALL = [
    wl.BLOCKS[0].replace(name="block_small_bf16", B=2, grid_h=16, grid_w=16, pool_h=2, pool_w=2,
                         dtype=wl.BF16),
    wl.BLOCKS[0].replace(name="block_small_d32_h2_c96", B=2, H=2, d=32, C=96, grid_h=12,
                         grid_w=10, pool_h=2, pool_w=2),
    wl.BLOCKS[0].replace(name="block_small_ragged_rows", B=3, H=1, d=32, C=32, grid_h=9,
                         grid_w=7, pool_h=3, pool_w=7),
    wl.BLOCKS[4].replace(name="block_small_gauss_qk_bf16", B=2, grid_h=12, grid_w=12,
                         pool_h=2, pool_w=2, dtype=wl.BF16),
]


@pytest.mark.parametrize("w", SMALL, ids=[b.name for b in SMALL])
def test_block_small_cases(w):
    run_block(w)


def test_block_rejects_bad_shapes():
    x = torch.zeros(1, 196, 48, device="cuda")
    w = torch.zeros(48, 64, device="cuda")
    with pytest.raises(ValueError):
        api.block_forward(x, w, None, w, w.t().contiguous(), H=1, d=64, grid_h=14, grid_w=14,
                          pool_h=2, pool_w=2, lam=16.0, eps=1e-3, iters=5)
