"""Python binding of libdsa3d.so (C ABI in include/dsa3d.h).

Argument marshalling only: torch supplies device memory and the current stream, every
step of the computation runs in the library's HIP kernels.  There is no CPU fallback:
the calls raise if the library is missing or the tensors are not on the GPU.

Tensors: q, k, v, out, dout, dq, dk, dv are contiguous [N, heads, head_dim] (float32 or
bfloat16, one dtype per call); lse is float32 [heads, N]; offsets int32 [N, 3] (dt, dy, dx);
token n = (t * Hp + y) * Wp + x on the grid (F, Hp, Wp).
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBPATH = os.path.join(_HERE, "libdsa3d.so")
_lib = None

F32, BF16 = 0, 1


class DSA3DError(RuntimeError):
    pass


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIBPATH):
            raise DSA3DError(f"{LIBPATH} is missing: build it with __graft_entry__.build()")
        lib = ctypes.CDLL(LIBPATH)
        i32, vp, sz, f32 = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_float
        lib.dsa3d_workspace_bytes.argtypes = [i32] * 8
        lib.dsa3d_workspace_bytes.restype = sz
        lib.dsa3d_window_starts.argtypes = [vp, i32, i32, i32, i32, i32, i32, vp, vp]
        lib.dsa3d_window_starts.restype = i32
        lib.dsa3d_forward.argtypes = [vp, vp, vp, vp] + [i32] * 8 + [f32, i32, vp, vp, vp, sz, vp]
        lib.dsa3d_forward.restype = i32
        lib.dsa3d_backward.argtypes = [vp] * 7 + [i32] * 8 + [f32, i32, vp, vp, vp, vp, sz, vp]
        lib.dsa3d_backward.restype = i32
        lib.dsa3d_status_string.argtypes = [i32]
        lib.dsa3d_status_string.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def status_string(code):
    return load().dsa3d_status_string(code).decode()


def _check(code, what):
    if code != 0:
        raise DSA3DError(f"{what}: {status_string(code)} (status {code})")


def _dtype_code(t):
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise DSA3DError(f"unsupported dtype {t.dtype}: float32 or bfloat16")


def _dev(t, name):
    if not t.is_cuda:
        raise DSA3DError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise DSA3DError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def workspace_bytes(grid, heads, window, backward):
    return int(load().dsa3d_workspace_bytes(*grid, heads, *window, int(bool(backward))))


def workspace(grid, heads, window, backward, device="cuda"):
    n = max(workspace_bytes(grid, heads, window, backward), 256)
    return torch.empty(n, dtype=torch.uint8, device=device)


def window_starts(offsets, grid, window):
    """int32 [N, 3] window starts (st, sy, sx) computed on the GPU."""
    N = grid[0] * grid[1] * grid[2]
    starts = torch.empty((N, 3), dtype=torch.int32, device=offsets.device)
    _check(load().dsa3d_window_starts(_dev(offsets, "offsets"), *grid, *window, starts.data_ptr(), _stream()),
           "dsa3d_window_starts")
    return starts


def _shape(q, grid):
    N, H, D = q.shape
    if N != grid[0] * grid[1] * grid[2]:
        raise DSA3DError(f"q has {N} tokens, grid {grid} has {grid[0] * grid[1] * grid[2]}")
    return N, H, D


def forward(q, k, v, offsets, grid, window, scale=None, out=None, lse=None, ws=None):
    """Returns (out [N, H, D], lse [H, N] float32)."""
    N, H, D = _shape(q, grid)
    for t, name in ((k, "k"), (v, "v")):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise DSA3DError(f"{name} must match q in shape and dtype")
    if scale is None:
        scale = D ** -0.5
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    ws = workspace(grid, H, window, False, q.device) if ws is None else ws
    _check(load().dsa3d_forward(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(offsets, "offsets"), *grid, H, D,
                                *window, float(scale), _dtype_code(q), _dev(out, "out"), _dev(lse, "lse"),
                                _dev(ws, "workspace"), ws.numel(), _stream()), "dsa3d_forward")
    return out, lse


def backward(q, k, v, offsets, out, lse, dout, grid, window, scale=None, dq=None, dk=None, dv=None, ws=None):
    """Returns (dq, dk, dv), each [N, H, D] in q's dtype."""
    N, H, D = _shape(q, grid)
    for t, name in ((k, "k"), (v, "v"), (out, "out"), (dout, "dout")):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise DSA3DError(f"{name} must match q in shape and dtype")
    if scale is None:
        scale = D ** -0.5
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    ws = workspace(grid, H, window, True, q.device) if ws is None else ws
    _check(load().dsa3d_backward(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(offsets, "offsets"),
                                 _dev(out, "out"), _dev(lse, "lse"), _dev(dout, "dout"), *grid, H, D, *window,
                                 float(scale), _dtype_code(q), _dev(dq, "dq"), _dev(dk, "dk"), _dev(dv, "dv"),
                                 _dev(ws, "workspace"), ws.numel(), _stream()), "dsa3d_backward")
    return dq, dk, dv


class DSA3DFunction(torch.autograd.Function):
    """autograd wrapper: forward and backward both run in the HIP library."""

    @staticmethod
    def forward(ctx, q, k, v, offsets, grid, window, scale):
        out, lse = forward(q, k, v, offsets, grid, window, scale)
        ctx.save_for_backward(q, k, v, offsets, out, lse)
        ctx.cfg = (grid, window, scale)
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, offsets, out, lse = ctx.saved_tensors
        grid, window, scale = ctx.cfg
        dq, dk, dv = backward(q, k, v, offsets, out, lse, dout.contiguous(), grid, window, scale)
        return dq, dk, dv, None, None, None, None


def dsa3d_attention(q, k, v, offsets, grid, window, scale=None):
    """Differentiable 3D-DSA attention term (integer offsets)."""
    if scale is None:
        scale = q.shape[-1] ** -0.5
    return DSA3DFunction.apply(q, k, v, offsets, tuple(grid), tuple(window), float(scale))
