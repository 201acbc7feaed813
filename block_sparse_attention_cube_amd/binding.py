"""PyTorch binding of libvsa.so: the same entry points, tensors in, tensors out.

Only marshalling happens here: shape checks, output/workspace allocation with
torch (device memory), and the call with the current HIP stream.  Every step
of the computation runs in the library's HIP kernels; tensors must already
live on the GPU.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence, Tuple

import torch

from . import _lib as L

Grid = Tuple[int, int, int]


def cube_counts(grid: Grid) -> Tuple[int, int]:
    """(C, Np): number of 4x4x4 cubes and padded token count of a (T, Hh, Ww) grid."""
    T, Hh, Ww = grid
    C = (-(-T // 4)) * (-(-Hh // 4)) * (-(-Ww // 4))
    return C, 64 * C


def _code(dtype: torch.dtype) -> int:
    if dtype == torch.bfloat16:
        return L.VSA_BF16
    if dtype == torch.float32:
        return L.VSA_F32
    raise TypeError(f"VSA supports bfloat16 and float32 tensors, got {dtype}")


def make_problem(B: int, H: int, grid: Grid, d: int, topk: int, dtype: torch.dtype) -> L.VSAProblem:
    T, Hh, Ww = grid
    return L.VSAProblem(B, H, T, Hh, Ww, d, 4, 4, 4, topk, _code(dtype))


def _device_tensor(t: torch.Tensor, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (got device {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _expect(t: torch.Tensor, shape: Sequence[int], dtype: torch.dtype, name: str) -> None:
    _device_tensor(t, name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _workspace(prob: L.VSAProblem, op: int, device) -> Tuple[Optional[torch.Tensor], int]:
    n = int(L.lib().vsa_workspace_bytes(ctypes.byref(prob), op))
    if n == 0:
        return None, 0
    return torch.empty(n, dtype=torch.uint8, device=device), n


def workspace_bytes(B: int, H: int, grid: Grid, d: int, topk: int, dtype: torch.dtype,
                    op: int = L.VSA_OP_FORWARD) -> int:
    prob = make_problem(B, H, grid, d, topk, dtype)
    return int(L.lib().vsa_workspace_bytes(ctypes.byref(prob), op))


def check_problem(B: int, H: int, grid: Grid, d: int, topk: int, dtype: torch.dtype) -> int:
    prob = make_problem(B, H, grid, d, topk, dtype)
    return int(L.lib().vsa_check_problem(ctypes.byref(prob)))


def _means(means: Optional[torch.Tensor], B: int, H: int, C: int, d: int) -> None:
    """Checks an optional per-cube means buffer [3,B,H,C,d] fp32 (q, k, v)."""
    if means is not None:
        _expect(means, (3, B, H, C, d), torch.float32, "means")


def _raster_inputs(q, k, v, grid):
    _device_tensor(q, "q")
    B, H, N, d = q.shape
    if N != grid[0] * grid[1] * grid[2]:
        raise ValueError(f"q has {N} tokens, grid {grid} has {grid[0] * grid[1] * grid[2]}")
    _expect(k, q.shape, q.dtype, "k")
    _expect(v, q.shape, q.dtype, "v")
    return B, H, N, d


def reorder(x: torch.Tensor, grid: Grid, inverse: bool = False) -> torch.Tensor:
    """Raster [B,H,N,d] -> cube order [B,H,Np,d] (pads zero), or back if inverse."""
    _device_tensor(x, "x")
    B, H, n, d = x.shape
    C, Np = cube_counts(grid)
    N = grid[0] * grid[1] * grid[2]
    if n != (Np if inverse else N):
        raise ValueError(f"x has {n} rows, expected {Np if inverse else N}")
    y = torch.empty((B, H, N if inverse else Np, d), dtype=x.dtype, device=x.device)
    prob = make_problem(B, H, grid, d, 1, x.dtype)
    L.check(L.lib().vsa_reorder(ctypes.byref(prob), _ptr(x), _ptr(y), int(inverse),
                                _stream(x.device)), "vsa_reorder")
    return y


def coarse(qcube: torch.Tensor, kcube: torch.Tensor, vcube: torch.Tensor, grid: Grid,
           topk: int, return_scores: bool = False):
    """Coarse stage on cube-order inputs: (o_coarse [B,H,C,d], idx [B,H,C,K][, scores])."""
    _device_tensor(qcube, "qcube")
    B, H, Np_in, d = qcube.shape
    C, Np = cube_counts(grid)
    if Np_in != Np:
        raise ValueError(f"qcube has {Np_in} rows, expected {Np}")
    _expect(kcube, qcube.shape, qcube.dtype, "kcube")
    _expect(vcube, qcube.shape, qcube.dtype, "vcube")
    prob = make_problem(B, H, grid, d, topk, qcube.dtype)
    L.check(L.lib().vsa_check_problem(ctypes.byref(prob)), "vsa_coarse")
    dev = qcube.device
    oc = torch.empty((B, H, C, d), dtype=qcube.dtype, device=dev)
    idx = torch.empty((B, H, C, topk), dtype=torch.int32, device=dev)
    sc = torch.empty((B, H, C, C), dtype=torch.float32, device=dev) if return_scores else None
    ws, nws = _workspace(prob, L.VSA_OP_COARSE, dev)
    L.check(L.lib().vsa_coarse(ctypes.byref(prob), _ptr(qcube), _ptr(kcube), _ptr(vcube),
                               _ptr(oc), _ptr(idx), _ptr(sc), _ptr(ws), nws, _stream(dev)),
            "vsa_coarse")
    return (oc, idx, sc) if return_scores else (oc, idx)


def fine(qcube: torch.Tensor, kcube: torch.Tensor, vcube: torch.Tensor, idx: torch.Tensor,
         grid: Grid, return_lse: bool = True, out: Optional[torch.Tensor] = None):
    """Fine stage on cube-order inputs: (o_fine cube order [B,H,Np,d], lse [B,H,Np])."""
    _device_tensor(qcube, "qcube")
    B, H, Np_in, d = qcube.shape
    C, Np = cube_counts(grid)
    if Np_in != Np:
        raise ValueError(f"qcube has {Np_in} rows, expected {Np}")
    _expect(kcube, qcube.shape, qcube.dtype, "kcube")
    _expect(vcube, qcube.shape, qcube.dtype, "vcube")
    _device_tensor(idx, "idx")
    if idx.dtype != torch.int32 or idx.dim() != 4 or tuple(idx.shape[:3]) != (B, H, C):
        raise ValueError(f"idx must be int32 [B,H,C,K], got {idx.dtype} {tuple(idx.shape)}")
    topk = idx.shape[3]
    prob = make_problem(B, H, grid, d, topk, qcube.dtype)
    dev = qcube.device
    o = out if out is not None else torch.empty_like(qcube)
    _expect(o, qcube.shape, qcube.dtype, "out")
    lse = torch.empty((B, H, Np), dtype=torch.float32, device=dev) if return_lse else None
    ws, nws = _workspace(prob, L.VSA_OP_FINE, dev)
    L.check(L.lib().vsa_fine(ctypes.byref(prob), _ptr(qcube), _ptr(kcube), _ptr(vcube),
                             _ptr(idx), _ptr(o), _ptr(lse), _ptr(ws), nws, _stream(dev)),
            "vsa_fine")
    return o, lse


def fine_raster(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, idx: torch.Tensor, grid: Grid,
                oc: Optional[torch.Tensor] = None, return_lse: bool = True, out=None):
    """The fine stage of the forward on raster tensors (bf16): returns
    (o_fine [B,H,N,d], lse [B,H,Np] or None, o_coarse [B,H,N,d] or None); with
    oc (per-cube [B,H,C,d]) each valid token also receives its cube's row in
    o_coarse.  out: optional preallocated (o_fine, o_coarse)."""
    B, H, N, d = _raster_inputs(q, k, v, grid)
    C, Np = cube_counts(grid)
    _device_tensor(idx, "idx")
    if idx.dtype != torch.int32 or idx.dim() != 4 or tuple(idx.shape[:3]) != (B, H, C):
        raise ValueError(f"idx must be int32 [B,H,C,K], got {idx.dtype} {tuple(idx.shape)}")
    prob = make_problem(B, H, grid, d, idx.shape[3], q.dtype)
    dev = q.device
    o, o_coarse = out if out is not None else (torch.empty_like(q),
                                               torch.empty_like(q) if oc is not None else None)
    _expect(o, q.shape, q.dtype, "o_fine")
    if oc is not None:
        _expect(oc, (B, H, C, d), q.dtype, "oc")
        _expect(o_coarse, q.shape, q.dtype, "o_coarse")
    lse = torch.empty((B, H, Np), dtype=torch.float32, device=dev) if return_lse else None
    L.check(L.lib().vsa_fine_raster(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(idx),
                                    _ptr(o), _ptr(lse), _ptr(oc),
                                    _ptr(o_coarse if oc is not None else None), _stream(dev)),
            "vsa_fine_raster")
    return o, lse, (o_coarse if oc is not None else None)


def dense(qcube: torch.Tensor, kcube: torch.Tensor, vcube: torch.Tensor, grid: Grid,
          return_lse: bool = True, out: Optional[torch.Tensor] = None):
    """Dense attention over every cube (cube order, bf16): (o [B,H,Np,d], lse [B,H,Np])."""
    _device_tensor(qcube, "qcube")
    B, H, Np_in, d = qcube.shape
    C, Np = cube_counts(grid)
    if Np_in != Np:
        raise ValueError(f"qcube has {Np_in} rows, expected {Np}")
    _expect(kcube, qcube.shape, qcube.dtype, "kcube")
    _expect(vcube, qcube.shape, qcube.dtype, "vcube")
    prob = make_problem(B, H, grid, d, C, qcube.dtype)
    dev = qcube.device
    o = out if out is not None else torch.empty_like(qcube)
    _expect(o, qcube.shape, qcube.dtype, "out")
    lse = torch.empty((B, H, Np), dtype=torch.float32, device=dev) if return_lse else None
    L.check(L.lib().vsa_dense(ctypes.byref(prob), _ptr(qcube), _ptr(kcube), _ptr(vcube), _ptr(o),
                              _ptr(lse), _stream(dev)), "vsa_dense")
    return o, lse


class ForwardPlan:
    """Preallocated outputs and workspace for repeated vsa_forward calls on one shape.
    keep_means: also write the per-cube means of q, k, v into self.means
    [3,B,H,C,d] fp32, for a later backward."""

    def __init__(self, B: int, H: int, grid: Grid, d: int, topk: int, dtype: torch.dtype,
                 device, return_lse: bool = True, op: int = L.VSA_OP_FORWARD,
                 keep_means: bool = False):
        self.prob = make_problem(B, H, grid, d, topk, dtype)
        L.check(L.lib().vsa_check_problem(ctypes.byref(self.prob)), "vsa_forward")
        C, Np = cube_counts(grid)
        N = grid[0] * grid[1] * grid[2]
        self.shape = (B, H, N, d)
        self.dtype = dtype
        self.device = torch.device(device)
        self.o_fine = torch.empty(self.shape, dtype=dtype, device=device)
        self.o_coarse = torch.empty(self.shape, dtype=dtype, device=device)
        self.idx = torch.empty((B, H, C, topk), dtype=torch.int32, device=device)
        self.lse = torch.empty((B, H, Np), dtype=torch.float32, device=device) if return_lse else None
        self.means = (torch.empty((3, B, H, C, d), dtype=torch.float32, device=device)
                      if keep_means else None)
        self.ws, self.nws = _workspace(self.prob, op, device)

    def run(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor):
        for t, n in ((q, "q"), (k, "k"), (v, "v")):
            _expect(t, self.shape, self.dtype, n)
        L.check(L.lib().vsa_forward(ctypes.byref(self.prob), _ptr(q), _ptr(k), _ptr(v),
                                    _ptr(self.o_fine), _ptr(self.o_coarse), _ptr(self.idx),
                                    _ptr(self.lse), _ptr(self.means), _ptr(self.ws), self.nws,
                                    _stream(self.device)), "vsa_forward")
        return self.o_fine, self.o_coarse, self.idx, self.lse


class BackwardPlan:
    """Preallocated gradients and workspace for repeated vsa_backward calls on one shape."""

    def __init__(self, B: int, H: int, grid: Grid, d: int, topk: int, dtype: torch.dtype,
                 device):
        self.prob = make_problem(B, H, grid, d, topk, dtype)
        L.check(L.lib().vsa_check_problem(ctypes.byref(self.prob)), "vsa_backward")
        C, Np = cube_counts(grid)
        N = grid[0] * grid[1] * grid[2]
        self.shape = (B, H, N, d)
        self.lse_shape = (B, H, Np)
        self.idx_shape = (B, H, C, topk)
        self.means_shape = (3, B, H, C, d)
        self.dtype = dtype
        self.device = torch.device(device)
        self.dq, self.dk, self.dv = (torch.empty(self.shape, dtype=dtype, device=device)
                                     for _ in range(3))
        self.ws, self.nws = _workspace(self.prob, L.VSA_OP_BACKWARD, device)

    def run(self, q, k, v, o_fine, lse, idx, do_fine, do_coarse=None, means=None):
        """means: the forward's per-cube means (ForwardPlan(keep_means=True).means),
        or None to recompute them from q, k, v."""
        for t, n in ((q, "q"), (k, "k"), (v, "v"), (o_fine, "o_fine"), (do_fine, "do_fine")):
            _expect(t, self.shape, self.dtype, n)
        if do_coarse is not None:
            _expect(do_coarse, self.shape, self.dtype, "do_coarse")
        _expect(lse, self.lse_shape, torch.float32, "lse")
        _expect(idx, self.idx_shape, torch.int32, "idx")
        if means is not None:
            _expect(means, self.means_shape, torch.float32, "means")
        L.check(L.lib().vsa_backward(ctypes.byref(self.prob), _ptr(q), _ptr(k), _ptr(v),
                                     _ptr(o_fine), _ptr(lse), _ptr(idx), _ptr(means), _ptr(do_fine),
                                     _ptr(do_coarse), _ptr(self.dq), _ptr(self.dk), _ptr(self.dv),
                                     _ptr(self.ws), self.nws, _stream(self.device)),
                "vsa_backward")
        return self.dq, self.dk, self.dv


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, grid: Grid, topk: int,
            return_lse: bool = True, means: Optional[torch.Tensor] = None):
    """Whole VSA forward on raster tensors: (o_fine, o_coarse, idx, lse).
    means: optional [3,B,H,C,d] fp32 tensor that receives the per-cube means
    of q, k, v (hand it to backward)."""
    B, H, N, d = _raster_inputs(q, k, v, grid)
    _means(means, B, H, cube_counts(grid)[0], d)
    plan = ForwardPlan(B, H, grid, d, topk, q.dtype, q.device, return_lse)
    plan.means = means
    return plan.run(q, k, v)


def forward_static(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, grid: Grid, topk: int,
                   out=None, return_lse: bool = True, means: Optional[torch.Tensor] = None):
    """vsa_forward_static: the whole forward with the library's own device
    scratch (no workspace).  out: optional preallocated (o_fine, o_coarse, idx,
    lse) to write into, so that the call itself allocates nothing; means as
    for forward."""
    B, H, N, d = _raster_inputs(q, k, v, grid)
    C, Np = cube_counts(grid)
    _means(means, B, H, C, d)
    prob = make_problem(B, H, grid, d, topk, q.dtype)
    L.check(L.lib().vsa_check_problem(ctypes.byref(prob)), "vsa_forward_static")
    dev = q.device
    if out is None:
        out = (torch.empty_like(q), torch.empty_like(q),
               torch.empty((B, H, C, topk), dtype=torch.int32, device=dev),
               torch.empty((B, H, Np), dtype=torch.float32, device=dev) if return_lse else None)
    o_fine, o_coarse, idx, lse = out
    _expect(o_fine, q.shape, q.dtype, "o_fine")
    _expect(o_coarse, q.shape, q.dtype, "o_coarse")
    _expect(idx, (B, H, C, topk), torch.int32, "idx")
    if lse is not None:
        _expect(lse, (B, H, Np), torch.float32, "lse")
    L.check(L.lib().vsa_forward_static(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v),
                                       _ptr(o_fine), _ptr(o_coarse), _ptr(idx), _ptr(lse),
                                       _ptr(means), _stream(dev)), "vsa_forward_static")
    return o_fine, o_coarse, idx, lse


def backward(q, k, v, o_fine, lse, idx, do_fine, do_coarse, grid: Grid,
             means: Optional[torch.Tensor] = None):
    """Gradients (dq, dk, dv) of sum(o_fine*do_fine) + sum(o_coarse*do_coarse).
    means: the forward's per-cube means, or None to recompute them."""
    B, H, N, d = _raster_inputs(q, k, v, grid)
    C, Np = cube_counts(grid)
    _means(means, B, H, C, d)
    _expect(o_fine, q.shape, q.dtype, "o_fine")
    _expect(do_fine, q.shape, q.dtype, "do_fine")
    if do_coarse is not None:
        _expect(do_coarse, q.shape, q.dtype, "do_coarse")
    _expect(lse, (B, H, Np), torch.float32, "lse")
    _device_tensor(idx, "idx")
    if idx.dtype != torch.int32 or tuple(idx.shape[:3]) != (B, H, C):
        raise ValueError("idx must be int32 [B,H,C,K]")
    topk = idx.shape[3]
    prob = make_problem(B, H, grid, d, topk, q.dtype)
    dev = q.device
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws, nws = _workspace(prob, L.VSA_OP_BACKWARD, dev)
    L.check(L.lib().vsa_backward(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(o_fine),
                                 _ptr(lse), _ptr(idx), _ptr(means), _ptr(do_fine), _ptr(do_coarse),
                                 _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), nws, _stream(dev)),
            "vsa_backward")
    return dq, dk, dv


def _cube_inputs(qcube, kcube, vcube, grid):
    _device_tensor(qcube, "qcube")
    B, H, Np_in, d = qcube.shape
    C, Np = cube_counts(grid)
    if Np_in != Np:
        raise ValueError(f"qcube has {Np_in} rows, expected {Np}")
    _expect(kcube, qcube.shape, qcube.dtype, "kcube")
    _expect(vcube, qcube.shape, qcube.dtype, "vcube")
    return B, H, C, Np, d


def forward_cube(qcube: torch.Tensor, kcube: torch.Tensor, vcube: torch.Tensor, grid: Grid,
                 topk: int, return_lse: bool = True, means: Optional[torch.Tensor] = None):
    """Whole forward on cube-order tensors: (o_fine [B,H,Np,d] cube order,
    o_coarse [B,H,C,d] per cube, idx [B,H,C,K], lse [B,H,Np]); means as for
    forward."""
    B, H, C, Np, d = _cube_inputs(qcube, kcube, vcube, grid)
    _means(means, B, H, C, d)
    prob = make_problem(B, H, grid, d, topk, qcube.dtype)
    L.check(L.lib().vsa_check_problem(ctypes.byref(prob)), "vsa_forward_cube")
    dev = qcube.device
    o = torch.empty_like(qcube)
    oc = torch.empty((B, H, C, d), dtype=qcube.dtype, device=dev)
    idx = torch.empty((B, H, C, topk), dtype=torch.int32, device=dev)
    lse = torch.empty((B, H, Np), dtype=torch.float32, device=dev) if return_lse else None
    ws, nws = _workspace(prob, L.VSA_OP_FORWARD_CUBE, dev)
    L.check(L.lib().vsa_forward_cube(ctypes.byref(prob), _ptr(qcube), _ptr(kcube), _ptr(vcube),
                                     _ptr(o), _ptr(oc), _ptr(idx), _ptr(lse), _ptr(means),
                                     _ptr(ws), nws, _stream(dev)), "vsa_forward_cube")
    return o, oc, idx, lse


def backward_cube(qcube, kcube, vcube, o_fine, lse, idx, do_fine, do_coarse, grid: Grid,
                  means: Optional[torch.Tensor] = None):
    """Gradients (dq, dk, dv) in cube order of sum(o_fine*do_fine) +
    sum(o_coarse*do_coarse) for the outputs of forward_cube (do_coarse per
    cube [B,H,C,d] or None; means from forward_cube or None)."""
    B, H, C, Np, d = _cube_inputs(qcube, kcube, vcube, grid)
    _means(means, B, H, C, d)
    _expect(o_fine, qcube.shape, qcube.dtype, "o_fine")
    _expect(do_fine, qcube.shape, qcube.dtype, "do_fine")
    if do_coarse is not None:
        _expect(do_coarse, (B, H, C, d), qcube.dtype, "do_coarse")
    _expect(lse, (B, H, Np), torch.float32, "lse")
    _device_tensor(idx, "idx")
    if idx.dtype != torch.int32 or tuple(idx.shape[:3]) != (B, H, C):
        raise ValueError("idx must be int32 [B,H,C,K]")
    prob = make_problem(B, H, grid, d, idx.shape[3], qcube.dtype)
    dev = qcube.device
    dq, dk, dv = (torch.empty_like(qcube) for _ in range(3))
    ws, nws = _workspace(prob, L.VSA_OP_BACKWARD_CUBE, dev)
    L.check(L.lib().vsa_backward_cube(ctypes.byref(prob), _ptr(qcube), _ptr(kcube), _ptr(vcube),
                                      _ptr(o_fine), _ptr(lse), _ptr(idx), _ptr(means),
                                      _ptr(do_fine), _ptr(do_coarse), _ptr(dq), _ptr(dk),
                                      _ptr(dv), _ptr(ws), nws, _stream(dev)), "vsa_backward_cube")
    return dq, dk, dv


def quantize_fp8(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, grid: Grid):
    """E4M3 copies of bf16 raster q, k, v (d = 128) for fine_fp8.

    Returns (q8, k8, vt8, exps): q8, k8 uint8 [B,H,Np,128] cube order, vt8
    uint8 [B,H,C,128,64] (per-cube transposed V tiles), exps int32 [3,B,H,C].
    """
    B, H, N, d = _raster_inputs(q, k, v, grid)
    C, Np = cube_counts(grid)
    prob = make_problem(B, H, grid, d, 1, q.dtype)
    dev = q.device
    q8 = torch.empty((B, H, Np, d), dtype=torch.uint8, device=dev)
    k8 = torch.empty_like(q8)
    vt8 = torch.empty((B, H, C, d, 64), dtype=torch.uint8, device=dev)
    exps = torch.empty((3, B, H, C), dtype=torch.int32, device=dev)
    L.check(L.lib().vsa_quantize_fp8(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(q8),
                                     _ptr(k8), _ptr(vt8), _ptr(exps), _stream(dev)),
            "vsa_quantize_fp8")
    return q8, k8, vt8, exps


def fine_fp8(q8: torch.Tensor, k8: torch.Tensor, vt8: torch.Tensor, exps: torch.Tensor,
             idx: torch.Tensor, grid: Grid, return_lse: bool = True,
             out: Optional[torch.Tensor] = None):
    """FP8 fine stage: (o_fine bf16 cube order [B,H,Np,128], lse [B,H,Np])."""
    _device_tensor(q8, "q8")
    B, H, Np_in, d = q8.shape
    C, Np = cube_counts(grid)
    if Np_in != Np:
        raise ValueError(f"q8 has {Np_in} rows, expected {Np}")
    _expect(k8, q8.shape, torch.uint8, "k8")
    _expect(vt8, (B, H, C, d, 64), torch.uint8, "vt8")
    _expect(exps, (3, B, H, C), torch.int32, "exps")
    _device_tensor(idx, "idx")
    if idx.dtype != torch.int32 or idx.dim() != 4 or tuple(idx.shape[:3]) != (B, H, C):
        raise ValueError(f"idx must be int32 [B,H,C,K], got {idx.dtype} {tuple(idx.shape)}")
    prob = make_problem(B, H, grid, d, idx.shape[3], torch.bfloat16)
    dev = q8.device
    o = out if out is not None else torch.empty((B, H, Np, d), dtype=torch.bfloat16, device=dev)
    _expect(o, (B, H, Np, d), torch.bfloat16, "out")
    lse = torch.empty((B, H, Np), dtype=torch.float32, device=dev) if return_lse else None
    L.check(L.lib().vsa_fine_fp8(ctypes.byref(prob), _ptr(q8), _ptr(k8), _ptr(vt8), _ptr(exps),
                                 _ptr(idx), _ptr(o), _ptr(lse), _stream(dev)), "vsa_fine_fp8")
    return o, lse


class ForwardFp8Plan(ForwardPlan):
    """Preallocated outputs and workspace for repeated vsa_forward_fp8 calls."""

    def __init__(self, B: int, H: int, grid: Grid, d: int, topk: int, device,
                 return_lse: bool = True):
        prob = make_problem(B, H, grid, d, topk, torch.bfloat16)
        if L.lib().vsa_workspace_bytes(ctypes.byref(prob), L.VSA_OP_FORWARD_FP8) == 0:
            L.check(L.VSA_ERR_UNSUPPORTED, "vsa_forward_fp8")   # d != 128 or invalid
        super().__init__(B, H, grid, d, topk, torch.bfloat16, device, return_lse,
                         op=L.VSA_OP_FORWARD_FP8)

    def run(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor):
        for t, n in ((q, "q"), (k, "k"), (v, "v")):
            _expect(t, self.shape, self.dtype, n)
        L.check(L.lib().vsa_forward_fp8(ctypes.byref(self.prob), _ptr(q), _ptr(k), _ptr(v),
                                        _ptr(self.o_fine), _ptr(self.o_coarse), _ptr(self.idx),
                                        _ptr(self.lse), _ptr(self.ws), self.nws,
                                        _stream(self.device)), "vsa_forward_fp8")
        return self.o_fine, self.o_coarse, self.idx, self.lse


def forward_fp8(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, grid: Grid, topk: int,
                return_lse: bool = True):
    """VSA forward with the FP8 fine stage (bf16 raster in, d = 128)."""
    B, H, N, d = _raster_inputs(q, k, v, grid)
    if q.dtype != torch.bfloat16:
        raise TypeError("forward_fp8 takes bfloat16 q, k, v")
    plan = ForwardFp8Plan(B, H, grid, d, topk, q.device, return_lse)
    return plan.run(q, k, v)


class VSAFunction(torch.autograd.Function):
    """Trainable VSA: (o_fine, o_coarse) = VSA(q, k, v); the selection is constant."""

    @staticmethod
    def forward(ctx, q, k, v, grid, topk):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        B, H, N, d = q.shape
        means = torch.empty((3, B, H, cube_counts(grid)[0], d), dtype=torch.float32,
                            device=q.device)
        o_fine, o_coarse, idx, lse = forward(q, k, v, grid, topk, return_lse=True, means=means)
        o_fine, o_coarse = o_fine.clone(), o_coarse.clone()
        ctx.save_for_backward(q, k, v, o_fine, lse, idx, means)
        ctx.grid = grid
        ctx.mark_non_differentiable(idx)
        return o_fine, o_coarse, idx.clone()

    @staticmethod
    def backward(ctx, do_fine, do_coarse, _didx):
        q, k, v, o_fine, lse, idx, means = ctx.saved_tensors
        do_fine = torch.zeros_like(o_fine) if do_fine is None else do_fine.contiguous()
        do_coarse = None if do_coarse is None else do_coarse.contiguous()
        dq, dk, dv = backward(q, k, v, o_fine, lse, idx, do_fine, do_coarse, ctx.grid, means)
        return dq, dk, dv, None, None


def vsa_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, grid: Grid, topk: int):
    """Autograd entry: returns (o_fine, o_coarse, idx)."""
    return VSAFunction.apply(q, k, v, grid, topk)
