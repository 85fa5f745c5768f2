"""PyTorch-facing binding of the C ABI: argument marshalling only.

Tensors supply device pointers and the current HIP stream; every step of the
computation runs in the library's kernels.  Names mirror the C entry points.
"""
from __future__ import annotations

import ctypes
from typing import Dict, Optional

import torch

from . import _lib
from ._lib import Desc

_KERNELS = {"laplacian": _lib.KERNEL_LAPLACIAN, "gaussian": _lib.KERNEL_GAUSSIAN}
_DTYPES = {torch.float32: _lib.DTYPE_F32, torch.bfloat16: _lib.DTYPE_BF16}


def make_desc(B: int, H: int, grid_h: int, grid_w: int, d: int, pool_h: int,
              pool_w: int, kernel: str = "laplacian", dtype=torch.float32,
              serial: bool = False, tickets: bool = False) -> Desc:
    if kernel not in _KERNELS:
        raise ValueError(f"kernel must be one of {sorted(_KERNELS)}")
    if dtype not in _DTYPES:
        raise ValueError("dtype must be torch.float32 or torch.bfloat16")
    flags = (_lib.FLAG_SERIAL if serial else 0) | (_lib.FLAG_TICKETS if tickets else 0)
    return Desc(B, H, grid_h, grid_w, d, pool_h, pool_w, _KERNELS[kernel],
                _DTYPES[dtype], flags)


def version() -> int:
    return _lib.lib().lapattn_version()


def init() -> None:
    _lib.check(_lib.lib().lapattn_init())


def check(desc: Desc, lam: float, eps: float, iters: int) -> int:
    return _lib.lib().lapattn_check(ctypes.byref(desc), lam, eps, iters)


def workspace_bytes(desc: Desc) -> int:
    return int(_lib.lib().lapattn_workspace_bytes(ctypes.byref(desc)))


def alloc_workspace(desc: Desc, device) -> torch.Tensor:
    n = workspace_bytes(desc)
    if n == 0:
        raise ValueError("invalid descriptor")
    return torch.empty(n, dtype=torch.uint8, device=device)


def _desc_for(q: torch.Tensor, grid_h: int, grid_w: int, pool_h: int, pool_w: int,
              kernel: str, serial: bool, tickets: bool = False) -> Desc:
    if q.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, H, N, d = q.shape
    if N != grid_h * grid_w:
        raise ValueError(f"N={N} does not match the {grid_h}x{grid_w} grid")
    return make_desc(B, H, grid_h, grid_w, d, pool_h, pool_w, kernel, q.dtype, serial, tickets)


def _check_io(q, k, v):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dtype != q.dtype or t.shape != q.shape:
            raise ValueError("q, k and v must share shape and dtype")


def _check_out(out, q):
    """The library writes B*H*N*d elements of q's dtype through out's pointer:
    anything but a contiguous tensor of q's shape, dtype and device would be
    written out of bounds or in the wrong layout."""
    if not isinstance(out, torch.Tensor):
        raise ValueError("out must be a tensor")
    if out.shape != q.shape or out.dtype != q.dtype or out.device != q.device:
        raise ValueError(f"out must match q: shape {tuple(q.shape)}, dtype {q.dtype}, "
                         f"device {q.device} (got {tuple(out.shape)}, {out.dtype}, {out.device})")
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")


def _check_workspace(ws, desc, device):
    if not isinstance(ws, torch.Tensor) or ws.dtype != torch.uint8:
        raise ValueError("workspace must be a torch.uint8 tensor (its numel is the byte count)")
    if ws.device != device or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    need = workspace_bytes(desc)
    if ws.numel() < need:
        raise ValueError(f"workspace holds {ws.numel()} bytes, {need} needed")


def status_offset(desc: Desc) -> int:
    off = int(_lib.lib().lapattn_status_offset(ctypes.byref(desc)))
    if off == ctypes.c_size_t(-1).value:
        raise ValueError("invalid descriptor")
    return off


def status(desc: Desc, workspace: torch.Tensor) -> int:
    """Timed-out in-launch waits of the last call on `workspace` (0 when its
    output is valid).  Synchronises with the device."""
    off = status_offset(desc)
    word = workspace[off:off + 4].cpu()
    return int(word.view(torch.int32).item())


def _stream_ptr(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, grid_h: int,
            grid_w: int, pool_h: int, pool_w: int, lam: float, eps: float,
            iters: int, kernel: str = "laplacian", out: Optional[torch.Tensor] = None,
            workspace: Optional[torch.Tensor] = None, serial: bool = False,
            tickets: bool = False, stream=None, check: bool = True) -> torch.Tensor:
    """O = K_QL (X (K_LK V)) per head; see include/lapattn.h.

    With `check` (the default) the call's status word is read back after the
    launch, which waits for the call to finish, and LapattnTimeout is raised
    if any of its in-launch waits ran out of time.  With check=False nothing
    synchronises; read `status(desc, workspace)` before reusing the workspace.
    """
    _check_io(q, k, v)
    desc = _desc_for(q, grid_h, grid_w, pool_h, pool_w, kernel, serial, tickets)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_out(out, q)
    if workspace is None:
        workspace = alloc_workspace(desc, q.device)
    else:
        _check_workspace(workspace, desc, q.device)
    st = _lib.lib().lapattn_forward(
        ctypes.byref(desc), q.data_ptr(), k.data_ptr(), v.data_ptr(), lam, eps, iters,
        out.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream_ptr(stream))
    _lib.check(st)
    if check:
        with torch.cuda.stream(stream) if stream is not None else _nullctx():
            n = status(desc, workspace)
        if n:
            raise _lib.LapattnTimeout(n)
    return out


class _nullctx:
    def __enter__(self):
        return self

    def __exit__(self, *a):
        return False


def forward_stages(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, grid_h: int,
                   grid_w: int, pool_h: int, pool_w: int, lam: float, eps: float,
                   iters: int, kernel: str = "laplacian", serial: bool = False,
                   stream=None) -> Dict[str, torch.Tensor]:
    """forward() plus fp32 copies of L, K_QL, K_LK, A, X and W."""
    _check_io(q, k, v)
    desc = _desc_for(q, grid_h, grid_w, pool_h, pool_w, kernel, serial)
    B, H, N, d = q.shape
    m = (grid_h // pool_h) * (grid_w // pool_w)
    dev = q.device
    f32 = torch.float32
    res = {
        "O": torch.empty_like(q),
        "L": torch.empty(B, H, m, d, dtype=f32, device=dev),
        "KQL": torch.empty(B, H, N, m, dtype=f32, device=dev),
        "KLK": torch.empty(B, H, m, N, dtype=f32, device=dev),
        "A": torch.empty(B, H, m, m, dtype=f32, device=dev),
        "X": torch.empty(B, H, m, m, dtype=f32, device=dev),
        "W": torch.empty(B, H, m, d, dtype=f32, device=dev),
    }
    ws = alloc_workspace(desc, dev)
    st = _lib.lib().lapattn_forward_stages(
        ctypes.byref(desc), q.data_ptr(), k.data_ptr(), v.data_ptr(), lam, eps, iters,
        res["O"].data_ptr(), ws.data_ptr(), ws.numel(), _stream_ptr(stream),
        res["L"].data_ptr(), res["KQL"].data_ptr(), res["KLK"].data_ptr(),
        res["A"].data_ptr(), res["X"].data_ptr(), res["W"].data_ptr())
    _lib.check(st)
    with torch.cuda.stream(stream) if stream is not None else _nullctx():
        n = status(desc, ws)
    if n:
        raise _lib.LapattnTimeout(n)
    return res


def launches(desc: Desc, q_is_k: bool) -> tuple:
    """Names of the launch slots a forward call with this descriptor uses."""
    mask = _lib.lib().lapattn_launches(ctypes.byref(desc), 1 if q_is_k else 0)
    if mask < 0:
        raise _lib.LapattnError(mask, _lib.strerror(mask))
    return tuple(name for s, name in enumerate(_lib.STAGES) if mask >> s & 1)


def backward_workspace_bytes(desc: Desc, iters: int) -> int:
    return int(_lib.lib().lapattn_backward_workspace_bytes(ctypes.byref(desc), iters))


def backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, dout: torch.Tensor, *,
             grid_h: int, grid_w: int, pool_h: int, pool_w: int, lam: float, eps: float,
             iters: int, kernel: str = "laplacian", workspace: Optional[torch.Tensor] = None,
             stream=None):
    """(dQ, dK, dV) of a loss with gradient dout at O = forward(q, k, v, ...);
    see include/lapattn.h.  With k the same tensor as q, the gradient with
    respect to that tensor is dQ + dK."""
    _check_io(q, k, v)
    _check_out(dout, q)
    desc = _desc_for(q, grid_h, grid_w, pool_h, pool_w, kernel, False)
    n = backward_workspace_bytes(desc, iters)
    if n == 0:
        raise ValueError("invalid descriptor or iters")
    if workspace is None:
        workspace = torch.empty(n, dtype=torch.uint8, device=q.device)
    elif (workspace.dtype != torch.uint8 or workspace.device != q.device
          or not workspace.is_contiguous() or workspace.numel() < n):
        raise ValueError(f"workspace must be a contiguous uint8 tensor of >= {n} bytes on q's device")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    st = _lib.lib().lapattn_backward(
        ctypes.byref(desc), q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(), lam, eps,
        iters, dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
        workspace.numel(), _stream_ptr(stream))
    _lib.check(st)
    return dq, dk, dv


def landmark_solve(L: torch.Tensor, W: torch.Tensor, *, grid_h: int, grid_w: int, pool_h: int,
                   pool_w: int, lam: float, eps: float, iters: int, solver: str = "ns",
                   kernel: str = "laplacian", stream=None) -> torch.Tensor:
    """Y = A^{-1} W per head, A = k(L, L) + eps I, by Newton-Schulz ("ns") or
    conjugate gradient ("cg"); L and W fp32 [B, H, m, d] on the GPU."""
    if solver not in ("ns", "cg"):
        raise ValueError("solver must be 'ns' or 'cg'")
    for name, t in (("L", L), ("W", W)):
        if not t.is_cuda or t.dtype != torch.float32 or not t.is_contiguous() or t.dim() != 4:
            raise ValueError(f"{name} must be a contiguous fp32 [B, H, m, d] GPU tensor")
    B, H, m, d = L.shape
    if W.shape != L.shape or m != (grid_h // pool_h) * (grid_w // pool_w):
        raise ValueError("L and W must be [B, H, m, d] with m the landmark count of the grid")
    desc = make_desc(B, H, grid_h, grid_w, d, pool_h, pool_w, kernel, torch.float32)
    y = torch.empty_like(W)
    st = _lib.lib().lapattn_landmark_solve(
        ctypes.byref(desc), L.data_ptr(), W.data_ptr(), lam, eps, iters,
        _lib.SOLVER_CG if solver == "cg" else _lib.SOLVER_NEWTON_SCHULZ, y.data_ptr(),
        _stream_ptr(stream))
    _lib.check(st)
    return y


def block_forward(x: torch.Tensor, wq: torch.Tensor, wk: Optional[torch.Tensor], wv: torch.Tensor,
                  wo: torch.Tensor, *, H: int, d: int, grid_h: int, grid_w: int, pool_h: int,
                  pool_w: int, lam: float, eps: float, iters: int, kernel: str = "laplacian",
                  workspace: Optional[torch.Tensor] = None, stream=None,
                  check: bool = True) -> torch.Tensor:
    """Y = concat_h(attention(X Wq, X Wk or X Wq, X Wv)_h) Wo; see
    include/lapattn.h.  x [B, N, C]; wq, wk, wv [C, H d]; wo [H d, C]."""
    if x.dim() != 3 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous [B, N, C] GPU tensor")
    B, N, C = x.shape
    if N != grid_h * grid_w:
        raise ValueError(f"N={N} does not match the {grid_h}x{grid_w} grid")
    for name, t, shape in (("wq", wq, (C, H * d)), ("wk", wk, (C, H * d)),
                           ("wv", wv, (C, H * d)), ("wo", wo, (H * d, C))):
        if t is None and name == "wk":
            continue
        if tuple(t.shape) != shape or t.dtype != x.dtype or t.device != x.device \
                or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {shape} tensor like x")
    desc = make_desc(B, H, grid_h, grid_w, d, pool_h, pool_w, kernel, x.dtype)
    n = int(_lib.lib().lapattn_block_workspace_bytes(ctypes.byref(desc), C))
    if n == 0:
        raise ValueError("invalid descriptor (C and H d must be multiples of 32)")
    if workspace is None:
        workspace = torch.empty(n, dtype=torch.uint8, device=x.device)
    elif (workspace.dtype != torch.uint8 or workspace.device != x.device
          or not workspace.is_contiguous() or workspace.numel() < n):
        raise ValueError(f"workspace must be a contiguous uint8 tensor of >= {n} bytes on x's device")
    y = torch.empty_like(x)
    st = _lib.lib().lapattn_block_forward(
        ctypes.byref(desc), C, x.data_ptr(), wq.data_ptr(), None if wk is None else wk.data_ptr(),
        wv.data_ptr(), wo.data_ptr(), lam, eps, iters, y.data_ptr(), workspace.data_ptr(),
        workspace.numel(), _stream_ptr(stream))
    _lib.check(st)
    if check:
        with torch.cuda.stream(stream) if stream is not None else _nullctx():
            cnt = int(workspace[:4].cpu().view(torch.int32).item())
        if cnt:
            raise _lib.LapattnTimeout(cnt)
    return y


def forward_normalized(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, grid_h: int,
                       grid_w: int, pool_h: int, pool_w: int, lam: float, eps: float,
                       iters: int, delta: float, kernel: str = "laplacian",
                       workspace: Optional[torch.Tensor] = None, stream=None,
                       check: bool = True) -> torch.Tensor:
    """O = Z (X (K_LK V)) with the normalised feature map Z of K_QL; see
    include/lapattn.h."""
    _check_io(q, k, v)
    desc = _desc_for(q, grid_h, grid_w, pool_h, pool_w, kernel, False)
    out = torch.empty_like(q)
    if workspace is None:
        workspace = alloc_workspace(desc, q.device)
    else:
        _check_workspace(workspace, desc, q.device)
    st = _lib.lib().lapattn_forward_normalized(
        ctypes.byref(desc), q.data_ptr(), k.data_ptr(), v.data_ptr(), lam, eps, iters, delta,
        out.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream_ptr(stream))
    _lib.check(st)
    if check:
        with torch.cuda.stream(stream) if stream is not None else _nullctx():
            n = status(desc, workspace)
        if n:
            raise _lib.LapattnTimeout(n)
    return out
