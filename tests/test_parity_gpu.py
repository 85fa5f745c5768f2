"""Parity of the HIP path (through the C ABI) against the fp64 oracle.

Bar: per head, max|O_gpu - O_ref| / max|O_ref| <= 2e-3 with fp32 I/O and
<= 2e-2 with bf16 I/O (fp32 compute in both cases); at full size the worst
head must also stay within the precision guard of gpu_common (2e-4 / 6e-3).
Stage checks use the bounds stated next to each one.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_common import compare_output, guard_for, normwise, run_gpu, tol_for
from nystr_linear_attention_amd import api
from nystr_linear_attention_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _print_case(w, extra=""):
    print(f"\n[case] {w.name} B={w.B} H={w.H} N={w.N} d={w.d} m={w.m} "
          f"kernel={w.kernel} dtype={w.dtype} iters={w.iters} {extra}", flush=True)


# Each workload at its own seed (1000 + position) and two more.
SEED_OFFSETS = (0, 1, 2)


@pytest.mark.parametrize("off", SEED_OFFSETS, ids=[f"seed+{o}" for o in SEED_OFFSETS])
@pytest.mark.parametrize("idx", range(len(wl.WORKLOADS)), ids=[w.name for w in wl.WORKLOADS])
def test_full_size_workloads(idx, off):
    """All heads of every reference workload, default (overlapped) launch plan."""
    w = wl.WORKLOADS[idx]
    w = w.replace(seed=w.seed + 100 * off)
    _print_case(w, f"seed={w.seed}")
    x = wl.make_inputs(w)
    got = run_gpu(w, x)
    worst = compare_output(w, x, got["O"])
    print(f"[case] worst normwise error {worst:.3e} (tol {tol_for(w):.0e})", flush=True)
    assert worst <= guard_for(w), f"{w.name}: {worst:.3e} beyond the precision guard"


SMALL = [
    wl.small_case(10, 14, 32, 2, 2, B=2, H=3),                    # ragged tiles, m=35
    wl.small_case(9, 9, 16, 3, 3, B=1, H=2),                      # d=16, m=9
    wl.small_case(4, 4, 16, 1, 1),                                # N=16 < one tile, m=16
    wl.small_case(8, 8, 64, 1, 1, B=2),                           # m=64 (maximum), pool 1x1
    wl.small_case(7, 9, 32, 7, 9, B=3),                           # m=1
    wl.small_case(12, 12, 64, 2, 2, iters=0),                     # no NS steps
    wl.small_case(12, 20, 32, 3, 4, kernel=wl.GAUSSIAN, B=2),     # Gaussian, Q != K
    wl.small_case(16, 16, 64, 2, 2, shared_qk=True),              # Laplacian, Q = K
    wl.small_case(10, 14, 64, 2, 2, dtype=wl.BF16, B=2, H=2),     # bf16, ragged
    wl.small_case(24, 24, 64, 3, 3, qk_dist="student_t3", qk_scale=0.5, eps=1e-2, iters=30),
    wl.small_case(40, 40, 64, 5, 5, B=1, H=1, iters=64),          # N=1600, max iters
    wl.small_case(64, 128, 64, 16, 16),                           # 128 tiles, 3 per key WG: 43 W partials
    wl.small_case(128, 192, 32, 16, 32),                          # 384 tiles: 128 W partials (the most), m=48
    wl.small_case(9, 9, 16, 3, 3, B=2, shared_qk=True),           # Q = K: output launch, m=9 (mpad 16)
    wl.small_case(10, 14, 32, 2, 2, H=2, shared_qk=True),         # Q = K, m=35 (mpad 48), ragged tiles
    wl.small_case(10, 10, 64, 2, 2, kernel=wl.GAUSSIAN, dtype=wl.BF16, B=2, shared_qk=True),
    wl.small_case(7, 7, 32, 1, 1, B=64),                          # 64 heads: pool takes 4 landmarks per WG
    wl.small_case(10, 14, 32, 2, 2, B=150),                       # grid not resident: output launch, key WGs take 3 tiles
    wl.small_case(12, 16, 32, 2, 2, B=2, eps=0.0),                # no diagonal perturbation (kernel matrix alone is PD)
    wl.small_case(8, 12, 64, 2, 2, B=2, iters=1),                 # a single Newton-Schulz step
    wl.small_case(20, 20, 32, 4, 4, B=300),                       # output launch of 600 workgroups, ragged last tile
    # m = 16 k + 1: Newton-Schulz on a 16 k interior plus a border row / column
    wl.small_case(17, 8, 32, 1, 8, B=2),                          # m=17, ragged tiles
    wl.small_case(6, 22, 32, 2, 2, H=2),                          # m=33
    wl.small_case(14, 14, 16, 2, 2),                              # m=49, d=16
    wl.small_case(14, 14, 32, 2, 2, iters=0),                     # m=49, no steps (X_0 with its border)
    wl.small_case(14, 14, 32, 2, 2, iters=1),                     # m=49, one step
    wl.small_case(14, 14, 64, 2, 2, kernel=wl.GAUSSIAN, shared_qk=True, B=2),  # m=49, output launch
    wl.small_case(14, 14, 32, 2, 2, B=150),                       # m=49, grid not resident
    wl.small_case(17, 4, 64, 1, 4, eps=1e-5, iters=30),           # m=17, nearly singular A
]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_small_and_edge_cases(w):
    _print_case(w)
    x = wl.make_inputs(w)
    got = run_gpu(w, x)
    compare_output(w, x, got["O"])


STAGE_CASES = [wl.WORKLOADS[0], wl.small_case(10, 14, 32, 2, 2, B=2, H=1),
               wl.small_case(12, 20, 32, 3, 4, kernel=wl.GAUSSIAN),
               wl.small_case(8, 8, 64, 1, 1),
               wl.small_case(64, 128, 64, 16, 16),
               wl.small_case(7, 7, 32, 1, 1, B=64),
               wl.small_case(17, 8, 32, 1, 8, B=2),                # border: m = 17, 33, 49
               wl.small_case(6, 22, 32, 2, 2),
               wl.small_case(14, 14, 64, 2, 2, iters=7)]


@pytest.mark.parametrize("w", STAGE_CASES, ids=[w.name for w in STAGE_CASES])
def test_stages(w):
    """Every intermediate against the oracle's same-named one."""
    _print_case(w, "stages")
    x = wl.make_inputs(w)
    got = run_gpu(w, x, stages=True)
    ref = oracle.forward_workload(w, x, stages=True)
    for (b, h), r in ref.items():
        assert normwise(got["L"][b, h], r["L"]) <= 1e-6, "landmarks"
        for key, ref_key in (("KQL", "KQL"), ("KLK", "KLK"), ("A", "A")):
            rel = np.abs(got[key][b, h] - r[ref_key]) / np.abs(r[ref_key])
            assert rel.max() <= 1e-4, f"{key}: elementwise relative error {rel.max():.3e}"
        assert normwise(got["X"][b, h], r["X"]) <= 2e-3, "Newton-Schulz result"
        assert normwise(got["W"][b, h], r["W"]) <= 1e-5, "W = K_LK V"
        assert normwise(got["O"][b, h], r["O"]) <= tol_for(w), "output"


def test_serial_and_fused_plans_are_bitwise_equal():
    w = wl.HEADLINE
    _print_case(w, "serial vs fused")
    x = wl.make_inputs(w)
    a = run_gpu(w, x, serial=False)["O"]
    b = run_gpu(w, x, serial=True)["O"]
    c = run_gpu(w, x, serial=False)["O"]
    assert np.array_equal(a, b) and np.array_equal(a, c)


LINEAR_CASES = [wl.HEADLINE, wl.WORKLOADS[4],
                wl.small_case(10, 14, 64, 2, 2, dtype=wl.BF16, B=2, H=2),   # bf16 I/O
                wl.small_case(12, 20, 32, 3, 4, kernel=wl.GAUSSIAN, B=2),    # Gaussian, Q != K
                wl.small_case(10, 14, 32, 2, 2, B=150)]                      # output-launch plan


@pytest.mark.parametrize("w", LINEAR_CASES, ids=[w.name for w in LINEAR_CASES])
def test_output_scales_exactly_with_v(w):
    """O is linear in V, and every scale the kernels choose (the split
    operands' powers of two, the row scales of W^T and Y^T) follows a power of
    two through exactly: O(2^k V) equals 2^k O(V) bit for bit (no value
    leaves the normal range at k = +-40)."""
    _print_case(w, "O(2^k V) = 2^k O(V)")
    x = wl.make_inputs(w)
    base = run_gpu(w, x)["O"]
    for k in (40, -40):
        xs = dict(x)
        if w.dtype == wl.BF16:
            # bf16 bits: scale the widened values and take the (exact) high half
            f = (x["v"].astype(np.uint32) << 16).view(np.float32) * np.float32(2.0 ** k)
            xs["v"] = (f.view(np.uint32) >> 16).astype(np.uint16)
        else:
            xs["v"] = x["v"] * np.float32(2.0 ** k)
        got = run_gpu(w, xs)["O"]
        assert np.array_equal(got, base * 2.0 ** k), f"k={k}: O does not scale exactly"


TICKET_CASES = [wl.HEADLINE, wl.WORKLOADS[3], wl.WORKLOADS[4],
                wl.small_case(10, 14, 32, 2, 2, B=3, H=1),     # BH % 8 != 0: three queues
                wl.small_case(10, 14, 32, 2, 2, B=150),        # output-launch plan, 8 queues
                wl.small_case(20, 20, 32, 4, 4, B=9)]          # 9 heads over 8 queues


@pytest.mark.parametrize("w", TICKET_CASES, ids=[w.name for w in TICKET_CASES])
def test_ticket_roles_are_bitwise_equal(w):
    """Roles handed out by ticket (LAPATTN_FLAG_TICKETS) give the same bits as
    roles by workgroup index, and pass the parity bar."""
    _print_case(w, "tickets")
    x = wl.make_inputs(w)
    a = run_gpu(w, x)["O"]
    b = run_gpu(w, x, tickets=True)["O"]
    assert np.array_equal(a, b)
    compare_output(w, x, b, heads=[(0, 0), (w.B - 1, w.H - 1)])


def test_device_errors_are_reported():
    q = torch.zeros(1, 1, 196, 32, device="cuda")
    with pytest.raises(ValueError):
        api.forward(q, q, q, grid_h=14, grid_w=13, pool_h=2, pool_w=2, lam=1.0, eps=0.0, iters=1)
    with pytest.raises(api._lib.LapattnError) as e:
        api.forward(q, q, q, grid_h=14, grid_w=14, pool_h=2, pool_w=2, lam=-1.0, eps=0.0, iters=1)
    assert e.value.status == api._lib.ERR_PARAM
    with pytest.raises(api._lib.LapattnError) as e:
        api.forward(q, q, q, grid_h=14, grid_w=14, pool_h=2, pool_w=2, lam=1.0, eps=0.0,
                    iters=1, out=q)
    assert e.value.status == api._lib.ERR_ALIAS


def test_bad_out_and_workspace_are_rejected_before_launch():
    """A caller-supplied out or workspace that the library would write out of
    bounds or in the wrong layout raises ValueError before any launch."""
    q = torch.randn(1, 2, 196, 32, device="cuda")
    kw = dict(grid_h=14, grid_w=14, pool_h=2, pool_w=2, lam=32.0, eps=1e-3, iters=3)
    bad_outs = {
        "undersized": torch.empty(1, 1, 196, 32, device="cuda"),
        "flat": torch.empty(2 * 196 * 32, device="cuda"),
        "fp64": torch.empty(1, 2, 196, 32, device="cuda", dtype=torch.float64),
        "bf16": torch.empty(1, 2, 196, 32, device="cuda", dtype=torch.bfloat16),
        "host": torch.empty(1, 2, 196, 32),
        "strided": torch.empty(1, 2, 32, 196, device="cuda").transpose(2, 3),
    }
    for name, o in bad_outs.items():
        o.fill_(7.0)
        with pytest.raises(ValueError):
            api.forward(q, q.clone(), q.clone(), out=o, **kw)
        assert bool((o == 7.0).all()), f"{name}: written although rejected"
    desc = api.make_desc(1, 2, 14, 14, 32, 2, 2)
    n = api.workspace_bytes(desc)
    for ws in (torch.empty(n - 256, dtype=torch.uint8, device="cuda"),
               torch.empty(n // 4 + 1, dtype=torch.float32, device="cuda"),
               torch.empty(n, dtype=torch.uint8)):
        with pytest.raises(ValueError):
            api.forward(q, q.clone(), q.clone(), workspace=ws, **kw)
    torch.cuda.synchronize()


def test_status_word_is_cleared_by_every_call():
    """The status word reads zero after a call even when the workspace held
    garbage on entry (it is set by the call's first launch)."""
    w = wl.WORKLOADS[0].replace(B=2, H=2)
    x = wl.make_inputs(w)
    q, k, v = (torch.from_numpy(x[n]).cuda() for n in "qkv")
    desc = api.make_desc(w.B, w.H, w.grid_h, w.grid_w, w.d, w.pool_h, w.pool_w)
    ws = api.alloc_workspace(desc, q.device)
    off = api.status_offset(desc)
    assert off % 4 == 0 and off + 4 <= ws.numel()
    ws.fill_(0xA5)
    api.forward(q, k, v, grid_h=w.grid_h, grid_w=w.grid_w, pool_h=w.pool_h, pool_w=w.pool_w,
                lam=w.lam, eps=w.eps, iters=w.iters, workspace=ws, check=False)
    assert api.status(desc, ws) == 0


@pytest.mark.parametrize("serial", [False, True], ids=["fused", "serial"])
def test_kernel_event_hook(serial):
    """Events bound to each launch time the kernels and change no result."""
    import ctypes

    from nystr_linear_attention_amd import _lib
    w = wl.WORKLOADS[0].replace(B=2, H=2)
    _print_case(w, f"event hook serial={serial}")
    x = wl.make_inputs(w)
    plain = run_gpu(w, x, serial=serial)["O"]
    rt = ctypes.CDLL("libamdhip64.so")
    rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                       ctypes.c_void_p]
    rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
    n = 2 * len(_lib.STAGES)
    evs = (ctypes.c_void_p * n)()
    for i in range(n):
        e = ctypes.c_void_p()
        assert rt.hipEventCreate(ctypes.byref(e)) == 0
        evs[i] = e.value
    lib = _lib.lib()
    try:
        assert lib.lapattn_set_stage_events(evs, n) == _lib.OK
        timed = run_gpu(w, x, serial=serial)["O"]
        assert lib.lapattn_set_stage_events(None, 0) == _lib.OK
        torch.cuda.synchronize()
        desc = api.make_desc(w.B, w.H, w.grid_h, w.grid_w, w.d, w.pool_h, w.pool_w, w.kernel,
                             torch.float32, serial=serial)
        used = api.launches(desc, w.shared_qk)
        for s, name in enumerate(_lib.STAGES):
            if name not in used:
                continue            # slots without a launch in this call
            ms = ctypes.c_float()
            assert rt.hipEventElapsedTime(ctypes.byref(ms), evs[2 * s], evs[2 * s + 1]) == 0, name
            assert 0.0 < ms.value < 1000.0, (name, ms.value)
    finally:
        lib.lapattn_set_stage_events(None, 0)
        for i in range(n):
            rt.hipEventDestroy(evs[i])
    assert np.array_equal(plain, timed)
