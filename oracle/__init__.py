"""CPU oracle for 3D Deformable Slide Attention (fp64).  TEST INFRASTRUCTURE ONLY.

ctypes wrapper over oracle.c (see its header for the definition and the readings of
the paper it follows).  Only the tests, the smoke check and the benchmark's CPU
baseline import this package; the HIP library never does.

Inputs are host numpy arrays: q/k/v/dout as float32, float64 or raw bf16 bits (uint16),
[N][H][D] row-major; offsets int32 [N][3] (dt, dy, dx).  Outputs are float64.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIBPATH = os.path.join(_HERE, "liboracle.so")
_lib = None


class _Cfg(ctypes.Structure):
    _fields_ = [("F", ctypes.c_int), ("Hp", ctypes.c_int), ("Wp", ctypes.c_int),
                ("H", ctypes.c_int), ("D", ctypes.c_int),
                ("kt", ctypes.c_int), ("ky", ctypes.c_int), ("kx", ctypes.c_int),
                ("scale", ctypes.c_double), ("dtype", ctypes.c_int)]


def build():
    tmp = _LIBPATH + ".tmp"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, _LIBPATH)


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIBPATH):
            raise RuntimeError(f"{_LIBPATH} is missing: run __graft_entry__.build() first")
        lib = ctypes.CDLL(_LIBPATH)
        P, vp, i64, i32 = ctypes.POINTER(_Cfg), ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.oracle_window_starts.argtypes = [vp, i32, i32, i32, i32, i32, i32, vp]
        lib.oracle_forward.argtypes = [P, vp, vp, vp, vp, vp, vp]
        lib.oracle_forward_rows.argtypes = [P, vp, vp, vp, vp, i64, vp, vp, vp]
        lib.oracle_weights.argtypes = [P, vp, vp, vp, vp, i64, i32, vp, vp]
        lib.oracle_weights.restype = ctypes.c_double
        lib.oracle_backward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.oracle_backward_q_rows.argtypes = [P, vp, vp, vp, vp, vp, i64, vp, vp]
        lib.oracle_backward_kv_rows.argtypes = [P, vp, vp, vp, vp, vp, i64, vp, vp, vp]
        lib.oracle_dwconv3d_forward.argtypes = [vp, i32, vp, vp] + [i32] * 7 + [vp]
        lib.oracle_dwconv3d_backward.argtypes = [vp, i32, vp, vp] + [i32] * 7 + [vp, vp, vp]
        lib.oracle_forward_heads.argtypes = [P, vp, vp, vp, vp, vp, vp]
        lib.oracle_backward_heads.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.oracle_sampled_forward.argtypes = [P, vp, vp, vp, vp, i64, i64, i64, i32, vp, vp]
        lib.oracle_sampled_backward.argtypes = [P, vp, vp, vp, vp, vp, i64, i64, i64, i32, vp, vp, vp, vp]
        for f in ("oracle_window_starts", "oracle_forward", "oracle_forward_rows", "oracle_backward",
                  "oracle_backward_q_rows", "oracle_backward_kv_rows", "oracle_forward_heads",
                  "oracle_backward_heads", "oracle_sampled_forward", "oracle_sampled_backward",
                  "oracle_dwconv3d_forward", "oracle_dwconv3d_backward"):
            getattr(lib, f).restype = None
        _lib = lib
    return _lib


def _dtype_code(a):
    if a.dtype == np.float32:
        return 0
    if a.dtype == np.uint16:
        return 1
    if a.dtype == np.float64:
        return 2
    raise TypeError(f"oracle inputs are float32, float64 or bf16 bits (uint16), got {a.dtype}")


def _check_window(grid, window):
    # The window is centred (odd extents) and lies inside the grid once its start is
    # clamped, which needs each extent to be at most the grid's.
    for g, k in zip(grid, window):
        if not (1 <= k <= g and k % 2 == 1):
            raise ValueError(f"window {tuple(window)} must be odd and fit the grid {tuple(grid)}")


def _cfg(q, grid, window, scale):
    F, Hp, Wp = grid
    kt, ky, kx = window
    N, H, D = q.shape
    assert N == F * Hp * Wp and D <= 256
    _check_window(grid, window)
    return _Cfg(F, Hp, Wp, H, D, kt, ky, kx, float(scale), _dtype_code(q))


def _c(a, dtype=None):
    a = np.ascontiguousarray(a if dtype is None else a.astype(dtype, copy=False))
    return a


def window_starts(offsets, grid, window):
    off = _c(offsets, np.int32)
    N = grid[0] * grid[1] * grid[2]
    assert off.shape == (N, 3)
    _check_window(grid, window)
    out = np.empty((N, 3), dtype=np.int32)
    _load().oracle_window_starts(off.ctypes.data, *grid, *window, out.ctypes.data)
    return out


def forward(q, k, v, offsets, grid, window, scale):
    """O [N][H][D] float64 and LSE [H][N] float64."""
    q, k, v, off = _c(q), _c(k), _c(v), _c(offsets, np.int32)
    cfg = _cfg(q, grid, window, scale)
    N, H, D = q.shape
    out = np.empty((N, H, D), dtype=np.float64)
    lse = np.empty((H, N), dtype=np.float64)
    _load().oracle_forward(ctypes.byref(cfg), q.ctypes.data, k.ctypes.data, v.ctypes.data, off.ctypes.data,
                           out.ctypes.data, lse.ctypes.data)
    return out, lse


def forward_rows(q, k, v, offsets, grid, window, scale, rows):
    """O and LSE for the rows r = n*H + h only: out [R][D], lse [R]."""
    q, k, v, off = _c(q), _c(k), _c(v), _c(offsets, np.int32)
    rows = _c(rows, np.int64)
    cfg = _cfg(q, grid, window, scale)
    out = np.empty((len(rows), q.shape[2]), dtype=np.float64)
    lse = np.empty(len(rows), dtype=np.float64)
    _load().oracle_forward_rows(ctypes.byref(cfg), q.ctypes.data, k.ctypes.data, v.ctypes.data, off.ctypes.data,
                                len(rows), rows.ctypes.data, out.ctypes.data, lse.ctypes.data)
    return out, lse


def weights(q, k, v, offsets, grid, window, scale, n, h):
    """(keys [K] int64, P [K] float64, lse) of one (query, head)."""
    q, k, v, off = _c(q), _c(k), _c(v), _c(offsets, np.int32)
    cfg = _cfg(q, grid, window, scale)
    K = window[0] * window[1] * window[2]
    keys = np.empty(K, dtype=np.int64)
    p = np.empty(K, dtype=np.float64)
    lse = _load().oracle_weights(ctypes.byref(cfg), q.ctypes.data, k.ctypes.data, v.ctypes.data, off.ctypes.data,
                                 int(n), int(h), keys.ctypes.data, p.ctypes.data)
    return keys, p, lse


def backward(q, k, v, dout, offsets, grid, window, scale):
    """dq, dk, dv [N][H][D] float64 (per-head scatter form)."""
    q, k, v, do, off = _c(q), _c(k), _c(v), _c(dout), _c(offsets, np.int32)
    assert do.dtype == q.dtype
    cfg = _cfg(q, grid, window, scale)
    dq = np.empty(q.shape, dtype=np.float64)
    dk = np.empty(q.shape, dtype=np.float64)
    dv = np.empty(q.shape, dtype=np.float64)
    _load().oracle_backward(ctypes.byref(cfg), q.ctypes.data, k.ctypes.data, v.ctypes.data, do.ctypes.data,
                            off.ctypes.data, dq.ctypes.data, dk.ctypes.data, dv.ctypes.data)
    return dq, dk, dv


def backward_q_rows(q, k, v, dout, offsets, grid, window, scale, rows):
    q, k, v, do, off = _c(q), _c(k), _c(v), _c(dout), _c(offsets, np.int32)
    rows = _c(rows, np.int64)
    cfg = _cfg(q, grid, window, scale)
    dq = np.empty((len(rows), q.shape[2]), dtype=np.float64)
    _load().oracle_backward_q_rows(ctypes.byref(cfg), q.ctypes.data, k.ctypes.data, v.ctypes.data, do.ctypes.data,
                                   off.ctypes.data, len(rows), rows.ctypes.data, dq.ctypes.data)
    return dq


def backward_kv_rows(q, k, v, dout, offsets, grid, window, scale, rows):
    """dk, dv for key rows r = j*H + h (key-centric gather form): [R][D] each."""
    q, k, v, do, off = _c(q), _c(k), _c(v), _c(dout), _c(offsets, np.int32)
    rows = _c(rows, np.int64)
    cfg = _cfg(q, grid, window, scale)
    dk = np.empty((len(rows), q.shape[2]), dtype=np.float64)
    dv = np.empty((len(rows), q.shape[2]), dtype=np.float64)
    _load().oracle_backward_kv_rows(ctypes.byref(cfg), q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                    do.ctypes.data, off.ctypes.data, len(rows), rows.ctypes.data, dk.ctypes.data,
                                    dv.ctypes.data)
    return dk, dv


# ---- per-head integer offsets ---------------------------------------------------------

def forward_heads(q, k, v, offsets_heads, grid, window, scale):
    """Per-head offsets int32 [H][N][3]: O [N][H][D], LSE [H][N] (float64)."""
    q, k, v, off = _c(q), _c(k), _c(v), _c(offsets_heads, np.int32)
    cfg = _cfg(q, grid, window, scale)
    N, H, D = q.shape
    assert off.shape == (H, N, 3)
    out = np.empty((N, H, D), dtype=np.float64)
    lse = np.empty((H, N), dtype=np.float64)
    _load().oracle_forward_heads(ctypes.byref(cfg), q.ctypes.data, k.ctypes.data, v.ctypes.data, off.ctypes.data,
                                 out.ctypes.data, lse.ctypes.data)
    return out, lse


def backward_heads(q, k, v, dout, offsets_heads, grid, window, scale):
    q, k, v, do, off = _c(q), _c(k), _c(v), _c(dout), _c(offsets_heads, np.int32)
    cfg = _cfg(q, grid, window, scale)
    N, H, D = q.shape
    assert off.shape == (H, N, 3) and do.dtype == q.dtype
    dq, dk, dv = (np.empty(q.shape, dtype=np.float64) for _ in range(3))
    _load().oracle_backward_heads(ctypes.byref(cfg), q.ctypes.data, k.ctypes.data, v.ctypes.data, do.ctypes.data,
                                  off.ctypes.data, dq.ctypes.data, dk.ctypes.data, dv.ctypes.data)
    return dq, dk, dv


# ---- sampled windows (real offsets, trilinear sampling) ---------------------------------
MODES = {"box": 0, "free": 1}


def _sampled_offsets(offsets, N, H, K, mode):
    """Broadcast the offsets to the canonical shape of the mode, box (N, H, 3) or free
    (N, H, K, 3), and return (float64 array, element strides (sn, sh, ss))."""
    off = np.ascontiguousarray(np.asarray(offsets, dtype=np.float64))
    if off.ndim != (3 if mode == "box" else 4):
        raise ValueError(f"{mode} offsets must be broadcastable to (N, H, 3) / (N, H, K, 3), got {off.shape}")
    if mode == "box":
        full = np.broadcast_to(off, (N, H, 3))
        sn, sh, ss = full.strides[0] // 8, full.strides[1] // 8, 0
    else:
        full = np.broadcast_to(off, (N, H, K, 3))
        sn, sh, ss = full.strides[0] // 8, full.strides[1] // 8, full.strides[2] // 8
    assert full.strides[-1] == 8
    return off, (sn, sh, ss)


def sampled_forward(q, k, v, offsets, grid, window, scale, mode):
    """Sampled windows (see oracle.c).  offsets: float, broadcastable to (N, H, 3) in box
    mode or (N, H, K, 3) in free mode.  Returns O [N][H][D], LSE [H][N] (float64)."""
    q, k, v = _c(q), _c(k), _c(v)
    cfg = _cfg(q, grid, window, scale)
    N, H, D = q.shape
    K = window[0] * window[1] * window[2]
    off, (sn, sh, ss) = _sampled_offsets(offsets, N, H, K, mode)
    out = np.empty((N, H, D), dtype=np.float64)
    lse = np.empty((H, N), dtype=np.float64)
    _load().oracle_sampled_forward(ctypes.byref(cfg), q.ctypes.data, k.ctypes.data, v.ctypes.data, off.ctypes.data,
                                   sn, sh, ss, MODES[mode], out.ctypes.data, lse.ctypes.data)
    return out, lse


def sampled_backward(q, k, v, dout, offsets, grid, window, scale, mode):
    """dq, dk, dv [N][H][D] and doffsets in the shape of `offsets` (the gradient of each
    given entry: summed over the heads / samples that share it)."""
    q, k, v, do = _c(q), _c(k), _c(v), _c(dout)
    assert do.dtype == q.dtype
    cfg = _cfg(q, grid, window, scale)
    N, H, D = q.shape
    K = window[0] * window[1] * window[2]
    off, (sn, sh, ss) = _sampled_offsets(offsets, N, H, K, mode)
    dq, dk, dv = (np.empty(q.shape, dtype=np.float64) for _ in range(3))
    full_shape = (N, H, 3) if mode == "box" else (N, H, K, 3)
    g = np.empty(full_shape, dtype=np.float64)
    _load().oracle_sampled_backward(ctypes.byref(cfg), q.ctypes.data, k.ctypes.data, v.ctypes.data, do.ctypes.data,
                                    off.ctypes.data, sn, sh, ss, MODES[mode], dq.ctypes.data, dk.ctypes.data,
                                    dv.ctypes.data, g.ctypes.data)
    # sum over the axes along which the given offsets are shared
    shape = off.shape
    axes = tuple(i for i, s in enumerate(shape) if s == 1 and full_shape[i] != 1)
    doff = g.sum(axis=axes, keepdims=True) if axes else g
    return dq, dk, dv, doff.reshape(shape)


# ---- depthwise 3-D convolution and the offset predictor ---------------------------------

def dwconv3d_forward(x, weight, bias, grid):
    """Depthwise 3-D convolution (see oracle.c): x [N][C] (float32, float64 or bf16 bits),
    weight [C][ct][cy][cx], bias [C] or None (float).  Returns y [N][C] float64."""
    x = _c(x)
    N, C = x.shape
    assert N == grid[0] * grid[1] * grid[2]
    w = _c(weight, np.float64)
    ct, cy, cx = w.shape[1:]
    assert w.shape[0] == C and ct % 2 and cy % 2 and cx % 2
    b = None if bias is None else _c(bias, np.float64)
    y = np.empty((N, C), dtype=np.float64)
    _load().oracle_dwconv3d_forward(x.ctypes.data, _dtype_code(x), w.ctypes.data,
                                    None if b is None else b.ctypes.data, *grid, C, ct, cy, cx, y.ctypes.data)
    return y


def dwconv3d_backward(x, weight, dy, grid):
    """dx [N][C], dweight [C][ct][cy][cx], dbias [C] (float64) for an output gradient dy."""
    x = _c(x)
    N, C = x.shape
    w = _c(weight, np.float64)
    ct, cy, cx = w.shape[1:]
    dy = np.asarray(dy)
    g = bf16_to_f64(dy) if dy.dtype == np.uint16 else _c(dy, np.float64)
    g = np.ascontiguousarray(g)
    dx = np.empty((N, C), dtype=np.float64)
    dw = np.empty(w.shape, dtype=np.float64)
    db = np.empty(C, dtype=np.float64)
    _load().oracle_dwconv3d_backward(x.ctypes.data, _dtype_code(x), w.ctypes.data, g.ctypes.data, *grid, C, ct, cy, cx,
                                     dx.ctypes.data, dw.ctypes.data, db.ctypes.data)
    return dx, dw, db


def linear_forward(x, weight, bias):
    """The predictor's pointwise layer (a 1 x 1 x 1 convolution, i.e. a linear map per
    token): y = x W^T + b, x [M][K], W [O][K], b [O]; float64 (one matrix product)."""
    x = np.asarray(x, dtype=np.float64)
    y = x @ np.asarray(weight, dtype=np.float64).T
    return y if bias is None else y + np.asarray(bias, dtype=np.float64)


def linear_backward(x, weight, dy):
    """dx = dy W, dW = dy^T x, db = sum over rows of dy (float64)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    return dy @ w, dy.T @ x, dy.sum(0)


def bf16_to_f64(bits):
    """bf16 bit patterns (uint16) as float64 values."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
