"""lapattn_forward_noalloc (workspace in the library's static device scratch)
against lapattn_forward (caller-owned workspace), through the C ABI.

Four calls in a row on the one scratch, each on a smaller input than the one
before, so that each call runs over what the previous one left behind: the
outputs must equal lapattn_forward's bit for bit (same plan, same kernels)
and be within the parity bar of the oracle; every call's status word must
read zero.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from gpu_common import device_inputs, normwise, tol_for
from nystr_linear_attention_amd import _lib, api
from nystr_linear_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu

# largest first: bf16 160 heads (~73 MiB of scratch), Gaussian Q = K (output
# launch), the PVT stage-1 headline, the 196-token case
SEQUENCE = ["lap_bf16_b32h5_n784_d64_m49", "gauss_f32_b16h2_n3136_d64_m49_qk",
            "lap_f32_pvt1_b8_n3136_d64_m49", "lap_f32_n196_d32_m49"]


def _desc(w, q):
    return api.make_desc(w.B, w.H, w.grid_h, w.grid_w, w.d, w.pool_h, w.pool_w, w.kernel, q.dtype)


def test_noalloc_matches_forward_on_successively_smaller_calls():
    lib = _lib.lib()
    assert lib.lapattn_init() == _lib.OK
    sizes = []
    for name in SEQUENCE:
        w = wl.BY_NAME[name]
        print(f"\n[case] noalloc {w.name}", flush=True)
        x = wl.make_inputs(w)
        q, k, v = device_inputs(w, x)
        desc = _desc(w, q)
        sizes.append(api.workspace_bytes(desc))
        assert sizes[-1] <= _lib.NOALLOC_SCRATCH_BYTES
        ref = api.forward(q, k, v, grid_h=w.grid_h, grid_w=w.grid_w, pool_h=w.pool_h,
                          pool_w=w.pool_w, lam=w.lam, eps=w.eps, iters=w.iters, kernel=w.kernel)
        out = torch.full_like(q, float("nan"))
        status = torch.full((1,), 0x7777, dtype=torch.int32, device=q.device)
        st = lib.lapattn_forward_noalloc(ctypes.byref(desc), q.data_ptr(), k.data_ptr(),
                                         v.data_ptr(), w.lam, w.eps, w.iters, out.data_ptr(),
                                         status.data_ptr(), torch.cuda.current_stream().cuda_stream)
        assert st == _lib.OK, _lib.strerror(st)
        torch.cuda.synchronize()
        assert int(status.item()) == 0, "timed-out waits"
        a = ref.float().cpu().numpy()
        b = out.float().cpu().numpy()
        assert np.array_equal(a, b), f"{name}: noalloc differs from lapattn_forward"
        got = b.astype(np.float64)
        for (bb, h), r in oracle.forward_workload(w, x, heads=[(0, 0), (w.B - 1, w.H - 1)]).items():
            assert normwise(got[bb, h], r["O"]) <= tol_for(w), f"{name} head ({bb},{h})"
    assert sizes == sorted(sizes, reverse=True) and len(set(sizes)) == len(sizes)


def test_noalloc_status_may_be_null_and_oversize_is_rejected():
    lib = _lib.lib()
    w = wl.WORKLOADS[0]
    x = wl.make_inputs(w)
    q, k, v = device_inputs(w, x)
    desc = _desc(w, q)
    out = torch.empty_like(q)
    st = lib.lapattn_forward_noalloc(ctypes.byref(desc), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                     w.lam, w.eps, w.iters, out.data_ptr(), None,
                                     torch.cuda.current_stream().cuda_stream)
    assert st == _lib.OK
    torch.cuda.synchronize()
    ref = oracle.forward_workload(w, x)[(0, 0)]["O"]
    assert normwise(out.cpu().numpy()[0, 0].astype(np.float64), ref) <= tol_for(w)
    # a descriptor whose workspace exceeds the scratch: rejected, nothing enqueued
    big = api.make_desc(1024, 8, 56, 56, 64, 8, 8)
    assert api.workspace_bytes(big) > _lib.NOALLOC_SCRATCH_BYTES
    st = lib.lapattn_forward_noalloc(ctypes.byref(big), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                     w.lam, w.eps, w.iters, out.data_ptr(), None, None)
    assert st == _lib.ERR_SCRATCH
