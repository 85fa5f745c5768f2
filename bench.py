#!/usr/bin/env python3
"""Benchmark: attention-layer forward tokens/s on one MI355X.

Default workload: Laplacian Nystrom attention, PVT stage-1 shape
(B=8, H=1, 56x56 grid -> N=3136 tokens, d=64, 8x8 average-pool landmarks ->
m=49, lambda=2*sqrt(d)=16, eps=1e-3, 20 Newton-Schulz steps), fp32 I/O,
synthetic seeded inputs N(0,1)/sqrt(d)*4 already resident in HBM.

One step = one lapattn_forward call over the whole batch (landmark pool,
solver, kernel maps, W reduction, output).  Prints one JSON line on stdout;
progress goes to stderr.  `value` is the warm rate (the same buffers every
step); `cold` repeats the steps rotating over copies of the buffers larger
than the Infinity Cache, so that every step reads its inputs from HBM.
Per-kernel times carry the 10th, 50th and 90th percentiles over the launches
of the kernel-event pass.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published peaks used as roofline denominators.
PEAK_HBM_GBS = 8000.0
PEAK_FP32_VALU_TFLOPS = 157.3
PEAK_FP32_MFMA_TFLOPS = 157.3
PEAK_FP16_MFMA_TFLOPS = 2500.0   # dense fp16 / bf16 MFMA


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """Timing events from the HIP runtime.  The library binds a start/stop
    pair to each kernel launch (hipExtLaunchKernel), so their elapsed time is
    that kernel's own duration."""

    def __init__(self):
        self.rt = ctypes.CDLL("libamdhip64.so")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                ctypes.c_void_p, ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.owned = []

    def create(self, n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            if self.rt.hipEventCreate(ctypes.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            arr[i] = ev.value
            self.owned.append(ev.value)
        return arr

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.rt.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def close(self):
        for ev in self.owned:
            self.rt.hipEventDestroy(ev)
        self.owned = []


def work(w):
    """Algorithmic work of the launches of one forward call.

    Flops: 3 per coordinate pair of an L1 or squared-L2 distance (difference,
    |.| or square, accumulate); 2 per multiply-add of a contraction.  Bytes:
    what the step must read and write at least (inputs once, outputs once)."""
    BH, N, d, m = w.heads, w.N, w.d, w.m
    e = 2 if w.dtype == "bf16" else 4
    sides = 1 if w.shared_qk else 2
    map_pairs = BH * sides * N * m * d          # K_QL and K_LK
    amat_pairs = BH * m * m * d                 # A = k(L, L)
    ns = BH * 4 * m ** 3 * w.iters              # Newton-Schulz
    klkv = BH * 2 * m * N * d                   # W = K_LK V
    y = BH * 2 * m * m * d                      # Y = X W
    out = BH * 2 * N * m * d                    # O = K_QL Y
    return {
        "map_pairs": map_pairs,
        "amat_pairs": amat_pairs,
        "ns": ns,
        "klkv": klkv,
        "pool": {"bytes": BH * (N * d * e + m * d * 4)},
        # solver launch of the serial plan: A, alpha, Newton-Schulz
        "solver": {"flops": 3 * amat_pairs + ns},
        # map launch of the serial plan: maps, W, Y and O
        "maps": {"flops": 3 * map_pairs + klkv + y + out},
        "fused": {"flops": 3 * (map_pairs + amat_pairs) + ns + klkv + y + out},
        "out": {"bytes": BH * (m * N * 4 + N * d * e)},
    }


def backward_work(w):
    """Algorithmic work of the backward launches of one call (per the
    definitions of `work`).  Distance stages count 3 flops per coordinate
    pair for the kernel map recomputed and 6 for its derivative (difference,
    sign, two multiply-adds: one into dQ or dK, one into dL); the
    Newton-Schulz backward counts the 6 products per step of its definition
    (X_t^T G X_t^T, G (A X_t)^T, (X_t A)^T G), 2 m^3 flops each."""
    BH, N, d, m, T = w.heads, w.N, w.d, w.m, w.iters
    e = 2 if w.dtype == "bf16" else 4
    pairs = BH * 2 * N * m * d                    # K_QL and K_LK
    return {
        "part": {"flops": 3 * pairs + BH * 4 * m ** 3 * T + BH * 2 * 2 * m * N * d,
                 "bound": "alu"},
        "head": {"flops": BH * (12 * m ** 3 * T + 3 * 2 * m * m * d), "bound": "mfma"},
        "grad": {"flops": 9 * pairs + BH * 3 * 2 * N * m * d, "bound": "alu",
                 "pairs": pairs},
        "dk": {"bytes": BH * (N * d * 4 + 2 * ((N + 63) // 64) * 64 * d * 4 + N * d * e),
               "bound": "hbm"},
    }


def cpu_baseline(w, inputs, seconds):
    """The fp64 oracle on the host, one thread, over whole heads of the same
    workload until `seconds` of CPU time have been spent."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle

    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    done = 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        while True:
            bh = heads[done % len(heads)]
            oracle.forward_workload(w, inputs, heads=[bh])
            done += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    tokens = done * w.N
    return {
        "value": tokens / el,
        "unit": "tokens/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{done} whole heads of {w.name} (N={w.N} tokens each, "
                  f"round-robin over its {len(heads)} heads), fp64 NumPy, "
                  f"BLAS limited to 1 thread, {el:.1f} s",
        "numpy": np.__version__,
    }


def _oracle_worker(job):
    """Pool worker: the fp64 oracle with one BLAS thread over whole heads of a
    workload (round-robin from `offset`) for `seconds`; returns (heads, s).
    Imports no GPU code: only the input generator and the oracle."""
    name, seconds, offset = job
    from threadpoolctl import threadpool_limits

    import oracle
    from nystr_linear_attention_amd import workloads as wl
    w = wl.BY_NAME[name]
    x = wl.make_inputs(w)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    done = 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        while True:
            oracle.forward_workload(w, x, heads=[heads[(offset + done) % len(heads)]])
            done += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                return done, el


def cpu_baseline_pool(w, seconds, workers):
    """The same oracle in `workers` spawned processes at once (heads are
    independent), each with one BLAS thread; the rate is the sum of the
    workers' rates.  Run before the GPU is initialised."""
    import multiprocessing as mp
    with mp.get_context("spawn").Pool(workers) as pool:
        res = pool.map(_oracle_worker, [(w.name, seconds, i) for i in range(workers)])
    heads = sum(d for d, _ in res)
    return {
        "value": sum(d * w.N / el for d, el in res),
        "unit": "tokens/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"{heads} whole heads of {w.name} over {workers} processes "
                  f"(one BLAS thread each), {seconds:.0f} s each",
    }


def host_info():
    """CPU model, usable cores and the BLAS NumPy calls (name, version,
    threading layer) of the host the CPU baseline ran on."""
    import numpy as np
    from threadpoolctl import threadpool_info
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = [{k: i.get(k) for k in ("internal_api", "version", "threading_layer",
                                    "architecture", "num_threads")}
            for i in threadpool_info() if i.get("user_api") == "blas"]
    return {"cpu_model": model, "usable_cores": len(os.sched_getaffinity(0)),
            "numpy": np.__version__, "blas": blas}


def source_digest():
    """sha256 of the kernel sources, to tie stored counter figures to a build."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "nystr_linear_attention_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload, kernel):
    """HBM bytes per launch from the committed counter summary of `kernel` on
    `workload`, or None if there is none or the kernel sources changed since."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ":" in line:
                k, v = line[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("source digest") != source_digest():
        return None
    try:
        return int(fields["bytes per launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(mib):
    """A plain device copy of known size, for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: 5 copies of {mib} MiB ({n * 4} bytes read and written each)")
    return 0


def bench_backward(w, x, q, k, v, dev, stream, lib, hip, timed, pct, args):
    """lapattn_backward on the same inputs and a seeded dO: K warm steps for
    the step time, K more with events bound to each launch for the kernels'
    own durations, each against the roofline of the unit that bounds it."""
    import numpy as np
    import torch

    from nystr_linear_attention_amd import _lib, api
    from nystr_linear_attention_amd import workloads as wl
    rng = np.random.default_rng(w.seed + 7000)
    g = rng.standard_normal((w.B, w.H, w.N, w.d))
    if w.dtype == wl.BF16:
        dout = torch.from_numpy(wl.f32_to_bf16_bits(g.astype(np.float32)).view(np.int16)).to(dev)
        dout = dout.view(torch.bfloat16)
    else:
        dout = torch.from_numpy(g.astype(np.float32)).to(dev)
    desc = api.make_desc(w.B, w.H, w.grid_h, w.grid_w, w.d, w.pool_h, w.pool_w, w.kernel, q.dtype)
    ws = torch.empty(api.backward_workspace_bytes(desc, w.iters), dtype=torch.uint8, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    call = (ctypes.byref(desc), q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(), w.lam,
            w.eps, w.iters, dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), ws.numel(),
            stream)

    def step():
        st = lib.lapattn_backward(*call)
        if st != 0:
            raise _lib.LapattnError(st, _lib.strerror(st))
    # the status word of the forward steps does not exist here: nothing waits
    step.status = torch.zeros(4, dtype=torch.uint8, device=dev)
    for _ in range(max(2, args.warmup // 2)):
        step()
    torch.cuda.synchronize()
    ms, _ = timed(step, args.steps, False)
    used = ("bwd_part", "bwd_head", "bwd_grad", "bwd_dk", "pool")
    ms_ev, kern = timed(step, args.steps, True, tuple(n for n in _lib.STAGES if n not in used))
    log(f"[bench] backward: {ms * 1e3:.2f} us/step; kernels (us): "
        + ", ".join(f"{n}={t * 1e3:.2f}" for n, t in kern.items()))
    bw = backward_work(w)
    peaks = {"alu": (PEAK_FP32_VALU_TFLOPS, "TFLOP/s", "FP32 VALU"),
             "mfma": (PEAK_FP32_MFMA_TFLOPS, "TFLOP/s", "fp32 MFMA"),
             "hbm": (PEAK_HBM_GBS, "GB/s", "HBM")}
    kernels = {}
    for name, t in kern.items():
        e = {"us": round(t * 1e3, 3)}
        if name in pct:
            e.update({f"p{p}_us": round(t_ * 1e3, 3) for p, t_ in zip((10, 50, 90), pct[name])})
        key = name[4:] if name.startswith("bwd_") else None
        if key in bw:
            b = bw[key]
            peak, unit, pipe = peaks[b["bound"]]
            amount = b.get("flops", b.get("bytes"))
            rate = amount / (t * 1e-3) / (1e12 if unit == "TFLOP/s" else 1e9)
            e.update({"bound": b["bound"], "pipe": pipe, "algorithmic": amount,
                      "achieved": round(rate, 3), "unit": unit, "frac": round(rate / peak, 4)})
        kernels[name] = e
    dom = max((n for n in kern if n.startswith("bwd_")), key=lambda n: kern[n])
    d = kernels[dom]
    return {
        "ms_per_step": round(ms, 5),
        "value": round(w.B * w.N / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "ms_per_step_kernel_event_pass": round(ms_ev, 5),
        "kernels": kernels,
        "roofline": {"kernel": dom, "bound": d["bound"], "pipe": d["pipe"],
                     "achieved": d["achieved"], "peak": peaks[d["bound"]][0], "unit": d["unit"],
                     "frac": d["frac"], "traffic": None},
        "note": "dO seeded N(0,1); dQ, dK, dV written; flops and bytes are algorithmic "
                "(see backward_work in bench.py)",
    }


def solver_compare(args):
    """Newton-Schulz against conjugate gradient on the landmark systems of
    the workloads: for each step count, the relative residual
    ||A Y - W|| / ||W|| and the error max|Y - Y*| / max|Y*| against LAPACK's
    solve Y* of the same fp32 A and W (the GPU's own, from
    lapattn_forward_stages), median and worst over the heads; and the GPU time
    of one solve launch over all heads at the workload's step count."""
    import numpy as np
    import torch

    from nystr_linear_attention_amd import api
    from nystr_linear_attention_amd import workloads as wl
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    out = {"metric": "landmark solve Y = A^-1 W: Newton-Schulz vs conjugate gradient",
           "unit": "relative residual / error vs LAPACK solve; us per solve launch",
           "workloads": {}}
    names = args.solver_workloads.split(",")
    for name in names:
        w = wl.BY_NAME[name]
        x = wl.make_inputs(w)

        def to_dev(a):
            if w.dtype == wl.BF16:
                return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
            return torch.from_numpy(a).to(dev)
        q = to_dev(x["q"])
        k = q if w.shared_qk else to_dev(x["k"])
        v = to_dev(x["v"])
        kw = dict(grid_h=w.grid_h, grid_w=w.grid_w, pool_h=w.pool_h, pool_w=w.pool_w,
                  lam=w.lam, eps=w.eps, kernel=w.kernel)
        st = api.forward_stages(q, k, v, iters=w.iters, **kw)
        L, W = st["L"].contiguous(), st["W"].contiguous()
        A = st["A"].double().cpu().numpy().reshape(w.heads, w.m, w.m)
        Wn = W.double().cpu().numpy().reshape(w.heads, w.m, w.d)
        ystar = np.stack([np.linalg.solve(A[i], Wn[i]) for i in range(w.heads)])
        kappa = [float(np.linalg.cond(A[i])) for i in range(w.heads)]
        rows = []
        for T in (5, 10, 15, 20, 25, 30, 40, 64):
            row = {"iters": T}
            for solver in ("ns", "cg"):
                y = api.landmark_solve(L, W, iters=T, solver=solver, **kw)
                y = y.double().cpu().numpy().reshape(w.heads, w.m, w.d)
                res = [float(np.linalg.norm(A[i] @ y[i] - Wn[i]) / np.linalg.norm(Wn[i]))
                       for i in range(w.heads)]
                err = [float(np.abs(y[i] - ystar[i]).max() / np.abs(ystar[i]).max())
                       for i in range(w.heads)]
                row[solver] = {"residual_median": float(np.median(res)), "residual_max": max(res),
                               "error_median": float(np.median(err)), "error_max": max(err)}
            rows.append(row)
        times = {}
        for solver in ("ns", "cg"):
            for _ in range(5):
                api.landmark_solve(L, W, iters=w.iters, solver=solver, **kw)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(50):
                api.landmark_solve(L, W, iters=w.iters, solver=solver, **kw)
            e1.record()
            torch.cuda.synchronize()
            times[solver] = round(e0.elapsed_time(e1) / 50 * 1e3, 2)
        out["workloads"][name] = {"heads": w.heads, "m": w.m, "d": w.d, "iters": w.iters,
                                  "kappa_median": float(np.median(kappa)),
                                  "kappa_max": max(kappa), "steps": rows,
                                  "us_per_launch_at_iters": times}
        log(f"[solver] {name}: kappa {np.median(kappa):.3g}; us per launch {times}")
        for r in rows:
            log(f"[solver]   T={r['iters']:3d}  ns res {r['ns']['residual_median']:.2e} "
                f"err {r['ns']['error_median']:.2e}   cg res {r['cg']['residual_median']:.2e} "
                f"err {r['cg']['error_median']:.2e}")
    print(json.dumps(out), flush=True)
    return 0


def bench_block(bw, steps, warmup):
    """One attention block (lapattn_block_forward: the projections into the
    heads, the Nystrom attention, the projection back) on seeded tokens and
    weights resident in HBM: mean time of `steps` calls after `warmup`."""
    import numpy as np
    import torch

    from nystr_linear_attention_amd import _lib, api
    from nystr_linear_attention_amd import workloads as wl
    dev = torch.device("cuda:0")
    inp = wl.make_block_inputs(bw)

    def to_dev(a):
        if a is None:
            return None
        if bw.dtype == wl.BF16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)
    t = {k: to_dev(v) for k, v in inp.items()}
    desc = api.make_desc(bw.B, bw.H, bw.grid_h, bw.grid_w, bw.d, bw.pool_h, bw.pool_w, bw.kernel,
                         t["x"].dtype)
    lib = _lib.lib()
    ws = torch.empty(lib.lapattn_block_workspace_bytes(ctypes.byref(desc), bw.C),
                     dtype=torch.uint8, device=dev)
    y = torch.empty_like(t["x"])
    stream = torch.cuda.current_stream().cuda_stream
    call = (ctypes.byref(desc), bw.C, t["x"].data_ptr(), t["wq"].data_ptr(),
            None if t["wk"] is None else t["wk"].data_ptr(), t["wv"].data_ptr(),
            t["wo"].data_ptr(), bw.lam, bw.eps, bw.iters, y.data_ptr(), ws.data_ptr(),
            ws.numel(), stream)

    def step():
        st = lib.lapattn_block_forward(*call)
        if st != 0:
            raise _lib.LapattnError(st, _lib.strerror(st))
    for _ in range(warmup):
        step()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    timeouts = int(ws[:4].cpu().view(torch.int32).item())
    hd = bw.H * bw.d
    proj_flops = 2 * bw.B * bw.N * bw.C * hd * (3 if not bw.shared_qk else 2) \
        + 2 * bw.B * bw.N * hd * bw.C
    return {"workload": bw.name, "B": bw.B, "N": bw.N, "C": bw.C, "H": bw.H, "d": bw.d,
            "m": bw.m, "kernel": bw.kernel, "shared_qk": bw.shared_qk,
            "ms_per_step": round(ms, 5), "value": round(bw.B * bw.N / (ms * 1e-3), 1),
            "unit": "tokens/s", "projection_flops": proj_flops, "timeouts": timeouts}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--serial", action="store_true",
                    help="time the serial launch plan (solver, then maps) instead of the fused one")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="processes of the pooled CPU baseline (default: the usable cores, "
                         "at most 16; 1 skips it)")
    ap.add_argument("--no-other-plan", action="store_true",
                    help="skip the pass over the other launch plan (its fields become null)")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache pass (steps rotating over copies of the inputs)")
    ap.add_argument("--cold-mib", type=int, default=640,
                    help="total size of the input copies the cold pass rotates over")
    ap.add_argument("--solver-compare", action="store_true",
                    help="only compare Newton-Schulz and conjugate gradient on the landmark "
                         "systems (its own JSON line)")
    ap.add_argument("--solver-workloads", default="lap_f32_pvt1_b8_n3136_d64_m49,"
                    "gauss_f32_b16h2_n3136_d64_m49_qk,lap_f32_h2_n16384_d64_m64_t3")
    ap.add_argument("--blocks", action="store_true",
                    help="only time the attention block of every pyramid stage (its own JSON line)")
    ap.add_argument("--no-block", action="store_true",
                    help="skip the stage-1 attention block measurement")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward pass measurement")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: the library runs on one "
              "GPU only (heads are independent, so B*H would shard across GPUs with no "
              "exchange).", file=sys.stderr)
        return 2
    if args.copy_calibration:
        return copy_calibration(args.copy_calibration)
    if args.solver_compare:
        return solver_compare(args)
    if args.blocks:
        import torch
        from nystr_linear_attention_amd import workloads as wl
        torch.cuda.set_device(0)
        rows = [bench_block(bw, args.steps, args.warmup) for bw in wl.BLOCKS]
        for r in rows:
            log(f"[bench] block {r['workload']}: {r['ms_per_step'] * 1e3:.2f} us/step, "
                f"{r['value']:.3g} tokens/s")
        print(json.dumps({"metric": "attention-block tokens/sec (fwd) per pyramid stage",
                          "unit": "tokens/s", "blocks": rows}), flush=True)
        return 3 if any(r["timeouts"] for r in rows) else 0

    import numpy as np
    import torch

    from nystr_linear_attention_amd import _lib, api
    from nystr_linear_attention_amd import workloads as wl

    w = wl.BY_NAME[args.workload] if args.workload else wl.HEADLINE
    log(f"[bench] workload {w.name}: B={w.B} H={w.H} N={w.N} d={w.d} m={w.m} "
        f"kernel={w.kernel} dtype={w.dtype} iters={w.iters}")
    x = wl.make_inputs(w)
    # The pooled CPU baseline runs first, before anything touches the GPU
    # (torch.cuda.set_device already starts the runtime's initialisation).
    pooled = None
    if not args.no_cpu_baseline:
        workers = args.cpu_workers or min(16, len(os.sched_getaffinity(0)))
        if workers > 1:
            log(f"[bench] cpu baseline: oracle in {workers} processes for ~{args.cpu_seconds:.0f} s")
            pooled = cpu_baseline_pool(w, args.cpu_seconds, workers)
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")

    def to_dev(a):
        if w.dtype == wl.BF16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    q = to_dev(x["q"])
    k = q if w.shared_qk else to_dev(x["k"])
    v = to_dev(x["v"])
    out = torch.empty_like(q)
    lib = _lib.lib()
    api.init()
    stream = torch.cuda.current_stream().cuda_stream

    def make_step(serial, bufs=None):
        qq, kk, vv, oo = bufs if bufs is not None else (q, k, v, out)
        desc = api.make_desc(w.B, w.H, w.grid_h, w.grid_w, w.d, w.pool_h, w.pool_w,
                             w.kernel, q.dtype, serial=serial)
        ws = api.alloc_workspace(desc, dev)
        call = (ctypes.byref(desc), qq.data_ptr(), kk.data_ptr(), vv.data_ptr(), w.lam, w.eps,
                w.iters, oo.data_ptr(), ws.data_ptr(), ws.numel(), stream)

        def step():
            st = lib.lapattn_forward(*call)
            if st != 0:
                raise _lib.LapattnError(st, _lib.strerror(st))
        step.keep = (desc, ws, qq, kk, vv, oo)
        step.status = ws[api.status_offset(desc):api.status_offset(desc) + 4]
        step.nbytes = ws.numel() + sum(t.numel() * t.element_size()
                                       for t in {id(t): t for t in (qq, kk, vv, oo)}.values())
        return step

    hip = HipEvents()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)

    pct = {}  # slot -> (p10, p50, p90) kernel ms of the last kernel-event pass

    timeouts = [0]  # timed-out in-launch waits seen in any checked call

    def read_status(steps_list):
        for st in steps_list:
            timeouts[0] += int(st.status.cpu().view(torch.int32).item())

    def timed(step, steps, kernel_events, unused=()):
        """Times `steps` calls; with kernel_events, also every kernel's own
        duration (start/stop events bound to each launch).  Returns
        (ms per step, {slot: mean kernel ms}); the kernel-event pass also
        leaves each slot's 10th, 50th and 90th percentiles in `pct`.
        `step` may be a list of steps, called in turn.  The status word of
        the last call on each workspace is read afterwards; the kernel-event
        pass (not used for `value`) also copies every call's status word to
        the device right after the call, so that each of them is checked."""
        steps_list = step if isinstance(step, list) else [step]
        nev = 2 * len(_lib.STAGES)
        evsets = [hip.create(nev) for _ in range(steps)] if kernel_events else []
        every = torch.zeros(steps, 4, dtype=torch.uint8, device=dev) if kernel_events else None
        torch.cuda.synchronize()
        t0.record()
        for i in range(steps):
            if kernel_events:
                lib.lapattn_set_stage_events(evsets[i], nev)
            st = steps_list[i % len(steps_list)]
            st()
            if kernel_events:
                every[i].copy_(st.status)
        t1.record()
        lib.lapattn_set_stage_events(None, 0)
        torch.cuda.synchronize()
        read_status(steps_list)
        if every is not None:
            timeouts[0] += int(every.view(torch.int32).sum().item())
        ms = t0.elapsed_time(t1) / steps
        per = {}
        for s, name in enumerate(_lib.STAGES):
            if evsets and name not in unused:
                vals = [hip.elapsed_ms(evs[2 * s], evs[2 * s + 1]) for evs in evsets]
                per[name] = sum(vals) / len(vals)
                pct[name] = tuple(float(np.percentile(vals, p)) for p in (10, 50, 90))
        return ms, per

    fused = make_step(serial=False)
    serial = make_step(serial=True)
    main_step = serial if args.serial else fused
    for _ in range(args.warmup):
        main_step()
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} done")

    # Timed region: K steps, plain launches -> value.
    ms_step, _ = timed(main_step, args.steps, False)
    log(f"[bench] timed {args.steps} steps: {ms_step * 1e3:.2f} us/step")
    # Kernel durations: K more steps, each kernel launched with its own
    # start/stop events (hipExtLaunchKernel).  Binding events to launches
    # slows the step (each launch then completes with a timestamped signal),
    # not the kernels; the step time of this pass is reported separately.
    # The fused plan has no map-only launch: its MAPS slot stays unrecorded.
    def unused_slots(serial_plan):
        desc = api.make_desc(w.B, w.H, w.grid_h, w.grid_w, w.d, w.pool_h, w.pool_w, w.kernel,
                             q.dtype, serial=serial_plan)
        used = api.launches(desc, w.shared_qk)
        return tuple(n for n in _lib.STAGES if n not in used)
    unused = unused_slots(args.serial)
    ms_ev, kern = timed(main_step, args.steps, True, unused)
    pct_main = dict(pct)
    log(f"[bench] kernel-event pass: {ms_ev * 1e3:.2f} us/step; kernels (us): "
        + ", ".join(f"{n}={t * 1e3:.2f}" for n, t in kern.items()))
    # The other launch plan, for the L1 stage on its own (serial) or fused.
    kern_other = {}
    if not args.no_other_plan:
        other = fused if args.serial else serial
        for _ in range(max(2, args.warmup // 4)):
            other()
        ms_other, kern_other = timed(other, args.steps, True, unused_slots(not args.serial))
        log(f"[bench] {'fused' if args.serial else 'serial'} plan: {ms_other * 1e3:.2f} us/step; "
            "kernels (us): " + ", ".join(f"{n}={t * 1e3:.2f}" for n, t in kern_other.items()))
    # Cold caches: the same steps rotating over copies of the inputs, output
    # and workspace that together exceed the 256 MB Infinity Cache, so that
    # every step reads its inputs from HBM.  Reported beside `value`.
    cold = None
    if not args.no_cold:
        nsets = max(2, -(-(args.cold_mib << 20) // main_step.nbytes))

        def copy_set():
            qq = q.clone()
            return (qq, qq if w.shared_qk else k.clone(), v.clone(), torch.empty_like(out))
        cold_steps = [make_step(args.serial, copy_set()) for _ in range(nsets)]
        for st in cold_steps:
            st()
        csteps = max(args.steps, 2 * nsets)
        ms_cold, _ = timed(cold_steps, csteps, False)
        cold = {"ms_per_step": round(ms_cold, 5),
                "value": round(w.B * w.N / (ms_cold * 1e-3), 1),
                "unit": "tokens/s", "steps": csteps, "sets": nsets,
                "MB_rotated": round(nsets * main_step.nbytes / 1e6, 1)}
        log(f"[bench] cold pass ({nsets} copies, {cold['MB_rotated']} MB): "
            f"{ms_cold * 1e3:.2f} us/step")
        del cold_steps
        torch.cuda.empty_cache()
    kf = kern_other if args.serial else kern      # fused-plan kernels (may be empty)
    ks = kern if args.serial else kern_other      # serial-plan kernels (may be empty)

    tokens = w.B * w.N
    value = tokens / (ms_step * 1e-3)
    wk = work(w)
    peak = PEAK_FP32_VALU_TFLOPS
    # Dominant kernel: main (the fused launch; in the serial plan, whichever
    # of its two launches is longer).  Its roofline is the distance stage the
    # metric names: the L1 map pairs (K_QL, K_LK) and the pairs of A, 3 flops
    # per coordinate pair, on FP32 VALU; the Gaussian variant's distances
    # run on fp16 MFMA instead (X L^T as scaled hi + lo parts, three products
    # per block; 2 flops per multiply-add of X L^T, against the fp16 peak).
    if args.serial:
        dom_ms = max(ks["maps"], ks["main"])
        dom_desc = ("main_kernel, map workgroups only (serial plan)" if ks["maps"] >= ks["main"]
                    else "main_kernel, solver workgroups only (serial plan)")
    else:
        dom_ms = kf["main"]
        dom_desc = "main_kernel (fused: solver, map and output workgroups in one launch)"
    l1_pairs = wk["map_pairs"] + wk["amat_pairs"]
    if w.kernel == wl.GAUSSIAN:
        dom_flops = 2 * wk["map_pairs"]
        bound, dpeak, stage = "mfma", PEAK_FP16_MFMA_TFLOPS, (
            "Gaussian distance stage: X L^T of K_QL (and K_LK when K != Q) on fp16 MFMA as "
            "scaled hi + lo parts (3 products), 2 flops per multiply-add, over the launch's time")
    else:
        dom_flops = 3 * l1_pairs
        bound, dpeak, stage = "alu", PEAK_FP32_VALU_TFLOPS, (
            "L1 stage: |q - l| terms of K_QL, K_LK and A on FP32 VALU, 3 flops per "
            "coordinate pair, over the launch's time")
    ach = dom_flops / (dom_ms * 1e-3) / 1e12
    traffic = stored_traffic(w.name, "main_kernel") if not args.serial else None
    roofline = {
        "kernel": dom_desc,
        "stage": stage,
        "bound": bound,
        "pipe": "fp16 MFMA" if bound == "mfma" else "FP32 VALU",
        "achieved": round(ach, 3),
        "peak": dpeak,
        "unit": "TFLOP/s",
        "frac": round(ach / dpeak, 4),
        "traffic": traffic,
        "kernel_us": round(dom_ms * 1e3, 3),
        "flops_per_launch": dom_flops,
    }
    # L1 stage: the distance maps and A, 3 flops per coordinate pair
    def frac_of(flops, t_ms):
        return round(flops / (t_ms * 1e-3) / 1e12 / peak, 4)
    l1 = {"pairs": l1_pairs,
          "note": "fused: maps and A over the whole fused main launch (conservative); "
                  "maps_only: the K_QL / K_LK pairs over the map launch of the serial plan "
                  "(which also forms W, Y and O)"}
    if kf:
        t = kf["main"]
        l1.update(fused_us=round(t * 1e3, 3), frac_fused=frac_of(3 * l1_pairs, t))
    if ks:
        t = ks["maps"]
        l1.update(maps_only_us=round(t * 1e3, 3), frac_maps_only=frac_of(3 * wk["map_pairs"], t))
    kernels = {}
    for name, t in kern.items():
        e = {"us": round(t * 1e3, 3)}
        if name in pct_main:
            e.update({f"p{p}_us": round(t_ * 1e3, 3) for p, t_ in zip((10, 50, 90), pct_main[name])})
        if name in ("pool", "out") and name in wk:
            e["GB/s"] = round(wk[name]["bytes"] / (t * 1e-3) / 1e9, 1)
            e["hbm_frac"] = round(e["GB/s"] / PEAK_HBM_GBS, 4)
        kernels[name] = e
    # The main launch as an HBM stream: the bytes it must move (inputs once,
    # output once, landmarks) and, when counters for these sources are
    # stored, the bytes it did move.
    if kf:
        t = kf["main"]
        e = 2 if w.dtype == wl.BF16 else 4
        ins = (2 if w.shared_qk else 3) * w.heads * w.N * w.d * e
        alg = ins + w.heads * w.N * w.d * e + w.heads * w.m * w.d * 4
        hbm = {"algorithmic_bytes": alg,
               "algorithmic_GB/s": round(alg / (t * 1e-3) / 1e9, 1)}
        hbm["algorithmic_frac"] = round(hbm["algorithmic_GB/s"] / PEAK_HBM_GBS, 4)
        if traffic:
            hbm.update({"counter_bytes": traffic,
                        "counter_GB/s": round(traffic / (t * 1e-3) / 1e9, 1),
                        "counter_over_algorithmic": round(traffic / alg, 3)})
        kernels.setdefault("main", {})["hbm"] = hbm
    # Contractions, each against the peak of the matrix-core dtype it runs
    # on, over the fused main launch that holds them all.
    n16 = 16 * ((w.m + 15) // 16)
    contractions = None
    if kf:
        t = kf["main"] * 1e-3
        ns_issued = w.heads * w.iters * 2 * 3 * 2 * n16 ** 3
        yo = 2 * w.m * w.m * w.d + 2 * w.N * w.m * w.d
        mpad = 16 * ((w.m + 15) // 16)
        yo_issued = 3 * w.heads * (2 * w.d * 64 * 64 + 2 * w.N * 64 * w.d)
        klkv_issued = w.heads * 2 * w.d * mpad * 64 * -(-w.N // 64)
        contractions = {
            "note": "algorithmic flops (2 per multiply-add at the unpadded sizes) and the "
                    "flops the matrix cores issue (split-fp16 products run 3 fp16 MFMAs; "
                    "padding to 16-wide blocks), both over the fused main launch",
            "newton_schulz": {
                "unit": "fp16 MFMA (hi*hi + lo*hi + hi*lo)", "algorithmic_flops": wk["ns"],
                "issued_flops": ns_issued, "peak_TFLOP/s": PEAK_FP16_MFMA_TFLOPS,
                "issued_frac": round(ns_issued / t / 1e12 / PEAK_FP16_MFMA_TFLOPS, 5)},
            "y_and_out": {
                "unit": "fp16 MFMA (hi*hi + lo*hi + hi*lo)",
                "algorithmic_flops": w.heads * yo, "issued_flops": yo_issued,
                "peak_TFLOP/s": PEAK_FP16_MFMA_TFLOPS,
                "issued_frac": round(yo_issued / t / 1e12 / PEAK_FP16_MFMA_TFLOPS, 5)},
            "klk_v": ({
                "unit": "fp16 MFMA (hi*hi + lo*hi + hi*lo)", "algorithmic_flops": wk["klkv"],
                "issued_flops": 3 * klkv_issued, "peak_TFLOP/s": PEAK_FP16_MFMA_TFLOPS,
                "issued_frac": round(3 * klkv_issued / t / 1e12 / PEAK_FP16_MFMA_TFLOPS, 5)}
                if w.kernel == wl.GAUSSIAN else {
                "unit": "fp32 MFMA 16x16x4", "algorithmic_flops": wk["klkv"],
                "issued_flops": klkv_issued, "peak_TFLOP/s": PEAK_FP32_MFMA_TFLOPS,
                "issued_frac": round(klkv_issued / t / 1e12 / PEAK_FP32_MFMA_TFLOPS, 5)}),
        }
    mfma = None
    if ks:
        # The solver launch of the serial plan: one workgroup (one CU) per
        # head.  MFMA utilisation of the Newton-Schulz stage as 4 m^3 iters
        # flops per head at the unpadded m over that launch, against the
        # fp32 matrix peak, device-wide and per CU that holds a solver; and
        # the fp16 work its steps issue (3 fp16 products, hi*hi, lo*hi,
        # hi*lo, for each of the 2 matrix products per step, on the matrix
        # zero padded to n = 16 ceil(m / 16)) against the fp16 peak per CU.
        solver_ms = ks["main"]
        f32eq = wk["ns"]
        dev_frac = f32eq / (solver_ms * 1e-3) / 1e12 / PEAK_FP32_MFMA_TFLOPS
        f16 = w.heads * w.iters * 2 * 3 * 2 * n16 ** 3
        tf = f16 / (solver_ms * 1e-3) / 1e12
        per_cu_peak = PEAK_FP16_MFMA_TFLOPS / 256
        mfma = {"solver_only_us": round(solver_ms * 1e3, 3),
                "ns_flops": f32eq,
                "utilisation_device": round(dev_frac, 5),
                "utilisation_per_active_cu": round(dev_frac * 256 / min(256, w.heads), 4),
                "fp16_mfma_flops_issued": f16,
                "fp16_TFLOP/s": round(tf, 3),
                "fp16_per_active_cu_frac": round(tf / (per_cu_peak * min(256, w.heads)), 4),
                "note": "utilisation = 4 m^3 iters B H / t(solver launch) / 157.3 TFLOP/s "
                        "(unpadded m; device-wide, and per CU that holds a solver); the fp16 "
                        "figures count the split products the steps issue on the padded matrix"}

    res = {
        "metric": "attention-layer tokens/sec (fwd) at N=3136,d=64,m=49; % FP32 VALU peak of L1 stage",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if w.dtype == wl.F32 else "bf16 I/O, f32 compute",
        "arithmetic": "L1 maps on FP32 VALU; squared-L2 maps as |x|^2 + |l|^2 - 2 x.l with "
                      "x.l as power-of-two scaled fp16 hi+lo splits on fp16 MFMA; Newton-Schulz "
                      "products as fp16 hi+lo splits on fp16 MFMA (about 22 significant bits); "
                      "Y and O as scaled fp16 hi+lo splits on fp16 MFMA; K_LK V on fp32 MFMA "
                      "(Laplacian) or as scaled fp16 hi+lo splits (Gaussian); fp32 accumulation "
                      "throughout",
        "data": "synthetic (seeded, shapes and distributions of the workload; resident in HBM)",
        "config": {
            "workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "m": w.m,
            "pool": f"{w.pool_h}x{w.pool_w}", "lambda": w.lam, "eps": w.eps,
            "iters": w.iters, "kernel": w.kernel,
            "launch": "serial (solver, then maps)" if args.serial
                      else "fused (solver and map workgroups in one launch)",
        },
        "roofline": roofline,
        "l1_stage": l1,
        "contractions": contractions,
        "solver_mfma": mfma,
        "kernels": kernels,
        "ms_per_step_kernel_event_pass": round(ms_ev, 5),
        "cold": cold,
    }
    if not args.no_backward:
        res["backward"] = bench_backward(w, x, q, k, v, dev, stream, lib, hip, timed, pct, args)
    if not args.no_backward:
        # the normalised feature map variant on the same inputs (its own plan:
        # K_QL stored, a statistics launch, the output launch)
        ws_n = api.alloc_workspace(api.make_desc(w.B, w.H, w.grid_h, w.grid_w, w.d, w.pool_h,
                                                 w.pool_w, w.kernel, q.dtype), dev)
        out_n = torch.empty_like(q)
        dn = api.make_desc(w.B, w.H, w.grid_h, w.grid_w, w.d, w.pool_h, w.pool_w, w.kernel, q.dtype)
        calln = (ctypes.byref(dn), q.data_ptr(), k.data_ptr(), v.data_ptr(), w.lam, w.eps,
                 w.iters, 1e-5, out_n.data_ptr(), ws_n.data_ptr(), ws_n.numel(), stream)

        def step_n():
            st = lib.lapattn_forward_normalized(*calln)
            if st != 0:
                raise _lib.LapattnError(st, _lib.strerror(st))
        step_n.status = ws_n[api.status_offset(dn):api.status_offset(dn) + 4]
        for _ in range(args.warmup):
            step_n()
        ms_n, _ = timed(step_n, args.steps, False)
        res["normalized"] = {"ms_per_step": round(ms_n, 5),
                             "value": round(w.B * w.N / (ms_n * 1e-3), 1), "unit": "tokens/s",
                             "delta": 1e-5,
                             "note": "normalised feature map Z = (K_QL - mu) / sqrt(var + delta) "
                                     "in place of K_QL; output-launch plan plus a statistics "
                                     "launch"}
        log(f"[bench] normalized map: {ms_n * 1e3:.2f} us/step")
    if not args.no_block:
        res["block"] = bench_block(wl.BLOCKS[0], args.steps, args.warmup)
        timeouts[0] += res["block"]["timeouts"]
        log(f"[bench] block {wl.BLOCKS[0].name}: {res['block']['ms_per_step'] * 1e3:.2f} us/step")
    res["timeouts"] = timeouts[0]
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline: oracle for ~{args.cpu_seconds:.0f} s")
        res["cpu_baseline"] = cpu_baseline(w, x, args.cpu_seconds)
        res["cpu_baseline"]["pooled"] = pooled
        res["cpu_baseline"]["host"] = host_info()
    hip.close()
    print(json.dumps(res), flush=True)
    if timeouts[0]:
        log(f"[bench] ERROR: {timeouts[0]} in-launch wait(s) timed out: outputs were invalid")
        return 3
    return 0


if __name__ == "__main__":
    sys.exit(main())
