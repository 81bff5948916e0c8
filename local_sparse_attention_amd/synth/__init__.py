"""Seeded synthetic inputs (Q, K, V, dO, offsets) for the 3D-DSA workloads.

Thin ctypes wrapper over synth.c: host numpy arrays only.  bf16 tensors are returned
as raw uint16 bit patterns.  The same arrays feed the CPU oracle and, copied to the
device, the HIP path.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIBPATH = os.path.join(_HERE, "libdsa3d_synth.so")
_lib = None

STREAM_Q, STREAM_K, STREAM_V, STREAM_DO = 0, 1, 2, 3


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIBPATH):
            raise RuntimeError(f"{_LIBPATH} is missing: run __graft_entry__.build() first")
        lib = ctypes.CDLL(_LIBPATH)
        u64, i64, dbl, vp, i32 = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p, ctypes.c_int
        lib.synth_normal_f32.argtypes = [u64, u64, u64, i64, dbl, vp]
        lib.synth_normal_bf16.argtypes = [u64, u64, u64, i64, dbl, vp]
        lib.synth_offsets_uniform.argtypes = [u64, i64, i32, i32, vp]
        lib.synth_offsets_round_normal.argtypes = [u64, i64, dbl, i32, vp]
        lib.synth_offsets_blocks.argtypes = [u64, i32, i32, i32, i32, dbl, i32, dbl, vp]
        for f in (lib.synth_normal_f32, lib.synth_normal_bf16, lib.synth_offsets_uniform,
                  lib.synth_offsets_round_normal, lib.synth_offsets_blocks):
            f.restype = None
        _lib = lib
    return _lib


def normal(seed, stream, shape, dtype, scale=1.0, first=0):
    """N(0,1)*scale, fp32 ("f32") or bf16 bits ("bf16"); element e is generator word first+e."""
    n = int(np.prod(shape))
    lib = _load()
    if dtype == "f32":
        a = np.empty(n, dtype=np.float32)
        lib.synth_normal_f32(seed, stream, first, n, scale, a.ctypes.data)
    elif dtype == "bf16":
        a = np.empty(n, dtype=np.uint16)
        lib.synth_normal_bf16(seed, stream, first, n, scale, a.ctypes.data)
    else:
        raise ValueError(dtype)
    return a.reshape(shape)


def make_offsets(wl):
    """int32 [N][3] offsets (dt, dy, dx) for a Workload, following its recipe."""
    lib = _load()
    off = np.empty((wl.N, 3), dtype=np.int32)
    kind = wl.offsets[0]
    if kind == "uniform":
        lib.synth_offsets_uniform(wl.seed, wl.N, wl.offsets[1], wl.offsets[2], off.ctypes.data)
    elif kind == "round_normal":
        lib.synth_offsets_round_normal(wl.seed, wl.N, wl.offsets[1], wl.offsets[2], off.ctypes.data)
    elif kind == "blocks":
        _, blk, sigma, drift, lim = wl.offsets
        lib.synth_offsets_blocks(wl.seed, wl.F, wl.Hp, wl.Wp, blk, sigma, int(drift), lim, off.ctypes.data)
    elif kind == "zero":
        off[:] = 0
    else:
        raise ValueError(kind)
    return off


def make_inputs(wl, with_dout=None):
    """dict(q, k, v, [dout], offsets) of host arrays for a Workload ([N][H][D] row-major)."""
    shape = (wl.N, wl.heads, wl.head_dim)
    out = {
        "q": normal(wl.seed, STREAM_Q, shape, wl.dtype, wl.qkv_scale),
        "k": normal(wl.seed, STREAM_K, shape, wl.dtype, wl.qkv_scale),
        "v": normal(wl.seed, STREAM_V, shape, wl.dtype, wl.qkv_scale),
        "offsets": make_offsets(wl),
    }
    if with_dout is None:
        with_dout = wl.backward
    if with_dout:
        out["dout"] = normal(wl.seed, STREAM_DO, shape, wl.dtype, 1.0)
    return out


def bf16_bits_to_f32(a):
    """Exact widening of raw bf16 bits to fp32."""
    return (a.astype(np.uint32) << 16).view(np.float32)


def make_head_offsets(wl):
    """int32 [H][N][3] per-head offsets: head h follows the workload's recipe with seed
    seed + 1000 h."""
    from dataclasses import replace

    return np.stack([make_offsets(replace(wl, seed=wl.seed + 1000 * h)) for h in range(wl.heads)])


def make_real_offsets(wl, mode, jitter=0.5):
    """float32 real offsets for sampled windows: the workload's integer motion field plus
    N(0, jitter) per component (stream 7).  mode "box": [N, 1, 3] (one offset per query,
    shared by the heads); "free": [N, H, K, 3] (every sample its own offset)."""
    base = make_offsets(wl).astype(np.float32)
    if mode == "box":
        return base[:, None, :] + normal(wl.seed, 7, (wl.N, 1, 3), "f32", jitter)
    return base[:, None, None, :] + normal(wl.seed, 7, (wl.N, wl.heads, wl.K, 3), "f32", jitter)
