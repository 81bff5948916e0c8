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


FLAG_GENERIC_KERNELS = 1  # DSA3D_FLAG_GENERIC_KERNELS
FLAG_REUSE_PREP = 2  # DSA3D_FLAG_REUSE_PREP


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIBPATH):
            raise DSA3DError(f"{LIBPATH} is missing: build it with __graft_entry__.build()")
        lib = ctypes.CDLL(LIBPATH)
        i32, u32, vp, sz, f32 = ctypes.c_int, ctypes.c_uint, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_float
        lib.dsa3d_workspace_bytes.argtypes = [i32] * 8
        lib.dsa3d_workspace_bytes.restype = sz
        lib.dsa3d_workspace_bytes_heads.argtypes = [i32] * 8
        lib.dsa3d_workspace_bytes_heads.restype = sz
        lib.dsa3d_window_starts.argtypes = [vp, i32, i32, i32, i32, i32, i32, vp, vp]
        lib.dsa3d_window_starts.restype = i32
        fwd = [vp, vp, vp, vp] + [i32] * 8 + [f32, i32, vp, vp, vp, sz, vp]
        bwd = [vp] * 7 + [i32] * 8 + [f32, i32, vp, vp, vp, vp, sz, vp]
        lib.dsa3d_forward.argtypes = fwd
        lib.dsa3d_backward.argtypes = bwd
        lib.dsa3d_forward_ex.argtypes = fwd + [u32, vp]
        lib.dsa3d_backward_ex.argtypes = bwd + [u32, vp]
        lib.dsa3d_forward_static.argtypes = [vp, vp, vp, vp] + [i32] * 8 + [f32, i32, vp, vp, vp]
        i64 = ctypes.c_longlong
        lib.dsa3d_sampled_workspace_bytes.argtypes = [i32] * 9
        lib.dsa3d_sampled_workspace_bytes.restype = sz
        lib.dsa3d_sampled_forward.argtypes = [vp, vp, vp, vp, i64, i64, i64] + [i32] * 9 + [f32, i32, vp, vp, vp]
        lib.dsa3d_sampled_backward.argtypes = ([vp, vp, vp, vp, i64, i64, i64, i32, vp, vp, vp] + [i32] * 8 +
                                               [f32, i32, vp, vp, vp, vp, vp, sz, vp])
        lib.dsa3d_dwconv3d_forward.argtypes = [vp, vp, vp] + [i32] * 8 + [vp, i32, vp]
        lib.dsa3d_dwconv3d_workspace_bytes.argtypes = [i32] * 7
        lib.dsa3d_dwconv3d_workspace_bytes.restype = sz
        lib.dsa3d_dwconv3d_backward.argtypes = [vp, vp, vp] + [i32] * 8 + [vp, vp, vp, vp, sz, vp]
        lib.dsa3d_linear_forward.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp, vp]
        lib.dsa3d_linear_workspace_bytes.argtypes = [i32] * 4
        lib.dsa3d_linear_workspace_bytes.restype = sz
        lib.dsa3d_linear_backward.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, sz, vp]
        lib.dsa3d_forward_heads.argtypes = fwd + [u32]
        lib.dsa3d_backward_heads.argtypes = bwd + [u32]
        for f in ("dsa3d_forward", "dsa3d_backward", "dsa3d_forward_ex", "dsa3d_backward_ex", "dsa3d_forward_static",
                  "dsa3d_forward_heads", "dsa3d_backward_heads", "dsa3d_sampled_forward", "dsa3d_sampled_backward",
                  "dsa3d_dwconv3d_forward", "dsa3d_dwconv3d_backward", "dsa3d_linear_forward",
                  "dsa3d_linear_backward"):
            getattr(lib, f).restype = i32
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


def _want(t, name, shape, dtype):
    """Shape and dtype of an argument (checked before anything touches the GPU)."""
    if not isinstance(t, torch.Tensor):
        raise DSA3DError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise DSA3DError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise DSA3DError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _dev(t, name, device=None):
    if not t.is_cuda:
        raise DSA3DError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise DSA3DError(f"{name} is on {t.device}, the other tensors on {device}")
    if not t.is_contiguous():
        raise DSA3DError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def workspace_bytes(grid, heads, window, backward, per_head=False):
    """Workspace of dsa3d_forward / dsa3d_backward; per_head=True: the size with which
    the per-head-offset calls bucket every head at once (dsa3d_workspace_bytes_heads)."""
    fn = load().dsa3d_workspace_bytes_heads if per_head else load().dsa3d_workspace_bytes
    return int(fn(*grid, heads, *window, int(bool(backward))))


def workspace(grid, heads, window, backward, device="cuda", per_head=False):
    n = max(workspace_bytes(grid, heads, window, backward, per_head), 256)
    return torch.empty(n, dtype=torch.uint8, device=device)


def window_starts(offsets, grid, window):
    """int32 [N, 3] window starts (st, sy, sx) computed on the GPU."""
    N = grid[0] * grid[1] * grid[2]
    _want(offsets, "offsets", (N, 3), torch.int32)
    starts = torch.empty((N, 3), dtype=torch.int32, device=offsets.device)
    _check(load().dsa3d_window_starts(_dev(offsets, "offsets"), *grid, *window, starts.data_ptr(), _stream()),
           "dsa3d_window_starts")
    return starts


def _shape(q, grid):
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise DSA3DError("q must be a [N, heads, head_dim] tensor")
    N, H, D = q.shape
    if N != grid[0] * grid[1] * grid[2]:
        raise DSA3DError(f"q has {N} tokens, grid {grid} has {grid[0] * grid[1] * grid[2]}")
    _dtype_code(q)
    return N, H, D


def _workspace_arg(ws, grid, H, window, backward, device, per_head=False):
    if ws is None:
        return workspace(grid, H, window, backward, device, per_head)
    if not isinstance(ws, torch.Tensor) or ws.dtype != torch.uint8 or ws.dim() != 1:
        raise DSA3DError("ws must be a 1-D uint8 tensor")
    return ws


def _offsets_shape(offsets, N, H):
    """(N, 3) shared by the heads, or (H, N, 3) per head."""
    return (H, N, 3) if isinstance(offsets, torch.Tensor) and offsets.dim() == 3 else (N, 3)


def forward(q, k, v, offsets, grid, window, scale=None, out=None, lse=None, ws=None, generic=False):
    """Returns (out [N, H, D], lse [H, N] float32).  offsets: int32 [N, 3] shared by the
    heads, or [H, N, 3] per head (dsa3d_forward_heads).  generic=True runs the per-group
    kernels (DSA3D_FLAG_GENERIC_KERNELS) whatever the geometry."""
    N, H, D = _shape(q, grid)
    for t, name in ((k, "k"), (v, "v")):
        _want(t, name, q.shape, q.dtype)
    per_head = _offsets_shape(offsets, N, H) == (H, N, 3)
    _want(offsets, "offsets", _offsets_shape(offsets, N, H), torch.int32)
    if out is not None:
        _want(out, "out", q.shape, q.dtype)
    if lse is not None:
        _want(lse, "lse", (H, N), torch.float32)
    if scale is None:
        scale = D ** -0.5
    dev = q.device
    ptrs = [_dev(t, n, dev) for t, n in ((q, "q"), (k, "k"), (v, "v"), (offsets, "offsets"))]
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((H, N), dtype=torch.float32, device=dev) if lse is None else lse
    ws = _workspace_arg(ws, grid, H, window, False, dev, per_head)
    flags = FLAG_GENERIC_KERNELS if generic else 0
    args = (*ptrs, *grid, H, D, *window, float(scale), _dtype_code(q), _dev(out, "out", dev), _dev(lse, "lse", dev),
            _dev(ws, "workspace", dev), ws.numel(), _stream(), flags)
    if per_head:
        _check(load().dsa3d_forward_heads(*args), "dsa3d_forward_heads")
    else:
        _check(load().dsa3d_forward_ex(*args, None), "dsa3d_forward")
    return out, lse


def forward_static(q, k, v, offsets, grid, window, scale=None, out=None, lse=None):
    """The forward through dsa3d_forward_static: no workspace, the library's static scratch
    array instead (geometries up to DSA3D_STATIC_SCRATCH_BYTES of scratch).  Returns
    (out, lse); out and lse are allocated here only when not given."""
    N, H, D = _shape(q, grid)
    for t, name in ((k, "k"), (v, "v")):
        _want(t, name, q.shape, q.dtype)
    _want(offsets, "offsets", (N, 3), torch.int32)
    if out is not None:
        _want(out, "out", q.shape, q.dtype)
    if lse is not None:
        _want(lse, "lse", (H, N), torch.float32)
    if scale is None:
        scale = D ** -0.5
    dev = q.device
    ptrs = [_dev(t, n, dev) for t, n in ((q, "q"), (k, "k"), (v, "v"), (offsets, "offsets"))]
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((H, N), dtype=torch.float32, device=dev) if lse is None else lse
    _check(load().dsa3d_forward_static(*ptrs, *grid, H, D, *window, float(scale), _dtype_code(q),
                                       _dev(out, "out", dev), _dev(lse, "lse", dev), _stream()),
           "dsa3d_forward_static")
    return out, lse


def backward(q, k, v, offsets, out, lse, dout, grid, window, scale=None, dq=None, dk=None, dv=None, ws=None,
             generic=False, reuse_prep=False):
    """Returns (dq, dk, dv), each [N, H, D] in q's dtype.  offsets as in forward().
    reuse_prep=True (DSA3D_FLAG_REUSE_PREP) uses the buckets and schedules that forward()
    just built in the same `ws` (a workspace sized for the backward) with the same offsets,
    geometry and `generic`."""
    if reuse_prep and ws is None:
        raise DSA3DError("reuse_prep needs the workspace the forward used")
    N, H, D = _shape(q, grid)
    for t, name in ((k, "k"), (v, "v"), (out, "out"), (dout, "dout")):
        _want(t, name, q.shape, q.dtype)
    per_head = _offsets_shape(offsets, N, H) == (H, N, 3)
    _want(offsets, "offsets", _offsets_shape(offsets, N, H), torch.int32)
    _want(lse, "lse", (H, N), torch.float32)
    for t, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        if t is not None:
            _want(t, name, q.shape, q.dtype)
    if scale is None:
        scale = D ** -0.5
    dev = q.device
    ptrs = [_dev(t, n, dev) for t, n in ((q, "q"), (k, "k"), (v, "v"), (offsets, "offsets"), (out, "out"),
                                         (lse, "lse"), (dout, "dout"))]
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    ws = _workspace_arg(ws, grid, H, window, True, dev, per_head)
    flags = (FLAG_GENERIC_KERNELS if generic else 0) | (FLAG_REUSE_PREP if reuse_prep else 0)
    args = (*ptrs, *grid, H, D, *window, float(scale), _dtype_code(q), _dev(dq, "dq", dev), _dev(dk, "dk", dev),
            _dev(dv, "dv", dev), _dev(ws, "workspace", dev), ws.numel(), _stream(), flags)
    if per_head:
        _check(load().dsa3d_backward_heads(*args), "dsa3d_backward_heads")
    else:
        _check(load().dsa3d_backward_ex(*args, None), "dsa3d_backward")
    return dq, dk, dv


# ---- sampled windows (real offsets, trilinear sampling) ---------------------------------
SAMPLE_MODES = {"box": 0, "free": 1}


def _sampled_layout(offsets, N, H, K, mode):
    """Element strides (token, head, sample) of float32 offsets broadcastable to (N, H, 3)
    (box) or (N, H, K, 3) (free); the last axis must be contiguous."""
    if not isinstance(offsets, torch.Tensor) or offsets.dtype != torch.float32:
        raise DSA3DError("offsets must be a float32 tensor")
    want = (N, H, 3) if mode == "box" else (N, H, K, 3)
    if offsets.dim() != len(want):
        raise DSA3DError(f"{mode} offsets must have {len(want)} axes, broadcastable to {want}")
    try:
        full = offsets.expand(*want)
    except RuntimeError as e:
        raise DSA3DError(f"offsets of shape {tuple(offsets.shape)} do not broadcast to {want}") from e
    st = full.stride()
    if st[-1] != 1:
        raise DSA3DError("offsets: the (dt, dy, dx) axis must be contiguous")
    return st[0], st[1], (st[2] if mode == "free" else 0)


def sampled_workspace_bytes(grid, heads, window, mode, backward=True):
    return int(load().dsa3d_sampled_workspace_bytes(*grid, heads, *window, SAMPLE_MODES[mode], int(bool(backward))))


def sampled_forward(q, k, v, offsets, grid, window, mode, scale=None, out=None, lse=None):
    """Sampled windows (dsa3d_sampled_forward).  mode "box" (one offset per (query, head),
    offsets broadcastable to [N, H, 3]) or "free" (per-sample offsets broadcastable to
    [N, H, K, 3]); offsets float32.  Returns (out [N, H, D], lse [H, N] float32)."""
    N, H, D = _shape(q, grid)
    if mode not in SAMPLE_MODES:
        raise DSA3DError(f"mode must be one of {list(SAMPLE_MODES)}")
    K = window[0] * window[1] * window[2]
    for t, name in ((k, "k"), (v, "v")):
        _want(t, name, q.shape, q.dtype)
    sn, sh, ss = _sampled_layout(offsets, N, H, K, mode)
    if out is not None:
        _want(out, "out", q.shape, q.dtype)
    if lse is not None:
        _want(lse, "lse", (H, N), torch.float32)
    if scale is None:
        scale = D ** -0.5
    dev = q.device
    ptrs = [_dev(t, n, dev) for t, n in ((q, "q"), (k, "k"), (v, "v"))]
    if not offsets.is_cuda or offsets.device != dev:
        raise DSA3DError("offsets must be on q's GPU")
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((H, N), dtype=torch.float32, device=dev) if lse is None else lse
    _check(load().dsa3d_sampled_forward(*ptrs, offsets.data_ptr(), sn, sh, ss, SAMPLE_MODES[mode], *grid, H, D,
                                        *window, float(scale), _dtype_code(q), _dev(out, "out", dev),
                                        _dev(lse, "lse", dev), _stream()), "dsa3d_sampled_forward")
    return out, lse


def sampled_backward(q, k, v, offsets, out, lse, dout, grid, window, mode, scale=None, ws=None):
    """Returns (dq, dk, dv, doffsets); doffsets has the shape and strides of `offsets`, each
    entry the gradient summed over the heads / samples that share it."""
    N, H, D = _shape(q, grid)
    if mode not in SAMPLE_MODES:
        raise DSA3DError(f"mode must be one of {list(SAMPLE_MODES)}")
    K = window[0] * window[1] * window[2]
    for t, name in ((k, "k"), (v, "v"), (out, "out"), (dout, "dout")):
        _want(t, name, q.shape, q.dtype)
    _want(lse, "lse", (H, N), torch.float32)
    sn, sh, ss = _sampled_layout(offsets, N, H, K, mode)
    if scale is None:
        scale = D ** -0.5
    dev = q.device
    ptrs = [_dev(t, n, dev) for t, n in ((q, "q"), (k, "k"), (v, "v"))]
    if not offsets.is_cuda or offsets.device != dev:
        raise DSA3DError("offsets must be on q's GPU")
    rest = [_dev(t, n, dev) for t, n in ((out, "out"), (lse, "lse"), (dout, "dout"))]
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    doff = torch.empty_strided(offsets.shape, offsets.stride(), dtype=torch.float32, device=dev)
    if ws is None:
        n = sampled_workspace_bytes(grid, H, window, mode, True)
        if n == 0:
            raise DSA3DError("sampled backward: geometry past the limits (N * heads * K < 2^31)")
        ws = torch.empty(n, dtype=torch.uint8, device=dev)
    _check(load().dsa3d_sampled_backward(*ptrs, offsets.data_ptr(), sn, sh, ss, SAMPLE_MODES[mode], *rest, *grid, H,
                                         D, *window, float(scale), _dtype_code(q), dq.data_ptr(), dk.data_ptr(),
                                         dv.data_ptr(), doff.data_ptr(), _dev(ws, "workspace", dev), ws.numel(),
                                         _stream()), "dsa3d_sampled_backward")
    return dq, dk, dv, doff


# ---- the DWConv3D term and the offset predictor ------------------------------------------

def _ptr_or_none(t, name, dev):
    return None if t is None else _dev(t, name, dev)


def _conv_shape(x, weight, grid):
    """(N, C) of x [N, C] on the grid, with weight float32 [C, ct, cy, cx]."""
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise DSA3DError("x must be a [N, C] tensor")
    N, C = x.shape
    if N != grid[0] * grid[1] * grid[2]:
        raise DSA3DError(f"x has {N} tokens, grid {grid} has {grid[0] * grid[1] * grid[2]}")
    if not isinstance(weight, torch.Tensor) or weight.dim() != 4 or weight.shape[0] != C:
        raise DSA3DError("weight must be float32 [C, ct, cy, cx]")
    _want(weight, "weight", weight.shape, torch.float32)
    return N, C


def dwconv3d_forward(x, weight, bias, grid, out=None, accumulate=False):
    """Depthwise 3-D convolution of x [N, C] (float32 or bfloat16) with weight float32
    [C, ct, cy, cx] and bias float32 [C] or None.  accumulate=True adds into `out` (e.g.
    the attention output seen as [N, C]); otherwise `out` (or a new tensor) is overwritten."""
    N, C = _conv_shape(x, weight, grid)
    if bias is not None:
        _want(bias, "bias", (C,), torch.float32)
    if accumulate and out is None:
        raise DSA3DError("accumulate needs out")
    if out is not None:
        _want(out, "out", x.shape, x.dtype)
    dev = x.device
    out = torch.empty_like(x) if out is None else out
    ct, cy, cx = weight.shape[1:]
    _check(load().dsa3d_dwconv3d_forward(_dev(x, "x", dev), _dev(weight, "weight", dev), _ptr_or_none(bias, "bias", dev),
                                         *grid, C, ct, cy, cx, _dtype_code(x), _dev(out, "out", dev), int(accumulate),
                                         _stream()), "dsa3d_dwconv3d_forward")
    return out


def dwconv3d_backward(x, weight, dy, grid, need_bias=True):
    """Returns (dx [N, C] in x's dtype, dweight float32 like weight, dbias float32 [C] or None)."""
    N, C = _conv_shape(x, weight, grid)
    _want(dy, "dy", x.shape, x.dtype)
    dev = x.device
    ct, cy, cx = weight.shape[1:]
    dx = torch.empty_like(x)
    dw = torch.empty_like(weight)
    db = torch.empty(C, dtype=torch.float32, device=dev) if need_bias else None
    n = load().dsa3d_dwconv3d_workspace_bytes(*grid, C, ct, cy, cx)
    if n == 0:
        raise DSA3DError("dsa3d_dwconv3d_backward: invalid geometry")
    ws = torch.empty(n, dtype=torch.uint8, device=dev)
    _check(load().dsa3d_dwconv3d_backward(_dev(x, "x", dev), _dev(weight, "weight", dev), _dev(dy, "dy", dev), *grid,
                                          C, ct, cy, cx, _dtype_code(x), dx.data_ptr(), dw.data_ptr(),
                                          None if db is None else db.data_ptr(), ws.data_ptr(), ws.numel(),
                                          _stream()), "dsa3d_dwconv3d_backward")
    return dx, dw, db


def linear_forward(x, weight, bias=None):
    """y float32 [M, O] = x [M, K] weight[O, K]^T + bias (x, weight: float32 or bfloat16)."""
    if not isinstance(x, torch.Tensor) or x.dim() != 2 or not isinstance(weight, torch.Tensor) or weight.dim() != 2:
        raise DSA3DError("x must be [M, K] and weight [O, K]")
    M, K = x.shape
    O = weight.shape[0]
    _want(weight, "weight", (O, K), x.dtype)
    if bias is not None:
        _want(bias, "bias", (O,), torch.float32)
    dev = x.device
    y = torch.empty((M, O), dtype=torch.float32, device=dev)
    _check(load().dsa3d_linear_forward(_dev(x, "x", dev), _dev(weight, "weight", dev), _ptr_or_none(bias, "bias", dev),
                                       M, K, O, _dtype_code(x), y.data_ptr(), _stream()), "dsa3d_linear_forward")
    return y


def linear_backward(x, weight, dy, need_bias=True):
    """Returns (dx [M, K] in x's dtype, dweight float32 [O, K], dbias float32 [O] or None)."""
    if not isinstance(x, torch.Tensor) or x.dim() != 2 or not isinstance(weight, torch.Tensor) or weight.dim() != 2:
        raise DSA3DError("x must be [M, K] and weight [O, K]")
    M, K = x.shape
    O = weight.shape[0]
    _want(weight, "weight", (O, K), x.dtype)
    _want(dy, "dy", (M, O), torch.float32)
    dev = x.device
    dx = torch.empty_like(x)
    dw = torch.empty((O, K), dtype=torch.float32, device=dev)
    db = torch.empty(O, dtype=torch.float32, device=dev) if need_bias else None
    n = load().dsa3d_linear_workspace_bytes(M, K, O, _dtype_code(x))
    if n == 0:
        raise DSA3DError("dsa3d_linear_backward: invalid sizes")
    ws = torch.empty(n, dtype=torch.uint8, device=dev)
    _check(load().dsa3d_linear_backward(_dev(x, "x", dev), _dev(weight, "weight", dev), _dev(dy, "dy", dev), M, K, O,
                                        _dtype_code(x), dx.data_ptr(), dw.data_ptr(),
                                        None if db is None else db.data_ptr(), ws.data_ptr(), ws.numel(), _stream()),
           "dsa3d_linear_backward")
    return dx, dw, db


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
