"""The DWConv3D term and the offset predictor (depthwise 3-D convolution, pointwise linear
layer) through the C ABI against the oracle, and Eq. (1) end to end: offsets predicted from
X, sampled attention with them, plus the convolution term added into the attention output.

Bounds (from the arithmetic; S = the same sum taken over absolute values, computed by the
oracle on |inputs|):
  - convolution output: fp32 sums of at most `taps` products (+ bias, + the accumulated
    value): |err| <= 2^-22 taps S; bf16 outputs add their rounding, 2^-8 |ref|.
  - dweight / dbias: fp32 sums of N = F Hp Wp products in some fixed order (per block and
    thread, then over threads, then over blocks): |err| <= 2^-24 (N - 1) S whatever the
    order.
  - linear: fp32 sums over K products: |err| <= 2^-22 K S; on the bf16 path dy is rounded
    to bf16 before the two backward products: + 2^-8 S; bf16 dx adds 2^-8 |ref|.
  - the end-to-end output: the sampled-window tolerance of the attention term (bf16
    2e-2 + 1e-2 |ref|), offsets taken from the GPU's predictor run through the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from local_sparse_attention_amd import synth

from _gpu_helpers import assert_close, to_dev, to_host_f64

pytestmark = pytest.mark.gpu


def assert_bound(gpu, ref, bound, what):
    gpu, ref, bound = (np.asarray(a, dtype=np.float64) for a in (gpu, ref, bound))
    assert gpu.shape == ref.shape and np.isfinite(gpu).all(), what
    excess = np.abs(gpu - ref) - bound
    i = np.unravel_index(np.argmax(excess), excess.shape)
    assert excess.max() <= 0, f"{what}: err {abs(gpu[i] - ref[i]):.3e} > bound {bound[i]:.3e} at {i}"
    return float(np.abs(gpu - ref).max())


def host(a):
    """float64 values of a host array (bf16 bits or floats)."""
    return oracle.bf16_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


CONV_CASES = [
    # grid, C, filter, dtype; filters up to 3 x 3 x 3 with C a multiple of 64 take the
    # frame-sweeping kernels (8 x 16 token tiles, 64 channels), the rest the general ones
    ((5, 9, 11), 64, (3, 3, 3), "f32"),
    ((7, 13, 35), 128, (3, 3, 3), "bf16"),   # ragged tiles in both directions, two channel blocks
    ((9, 10, 20), 192, (1, 3, 3), "bf16"),   # one frame tap
    ((4, 6, 7), 64, (3, 1, 3), "f32"),       # one row tap
    ((40, 9, 17), 64, (3, 3, 1), "bf16"),    # runs of frames (fewer tiles than blocks wanted)
    ((2, 3, 3), 64, (3, 3, 3), "bf16"),      # grid smaller than a tile and than the filter along t
    ((6, 12, 10), 128, (3, 7, 7), "bf16"),
    ((4, 5, 6), 24, (5, 5, 3), "bf16"),     # filter wider than the grid along t, C not a multiple of 64
    ((3, 8, 8), 16, (1, 1, 1), "f32"),
]


@pytest.mark.parametrize("case", CONV_CASES, ids=[f"{c[0]}-C{c[1]}-{c[2]}-{c[3]}" for c in CONV_CASES])
def test_dwconv3d(dsa3d_gpu, case):
    grid, C, k, dtype = case
    N = grid[0] * grid[1] * grid[2]
    taps = k[0] * k[1] * k[2]
    x = synth.normal(41, 0, (N, C), dtype)
    y0 = synth.normal(41, 1, (N, C), dtype)
    dy = synth.normal(41, 3, (N, C), dtype)
    w = synth.normal(41, 4, (C, *k), "f32", 0.2)
    b = synth.normal(41, 5, (C,), "f32")
    print(f"case grid={grid} C={C} filter={k} {dtype}", flush=True)
    xd, dyd, wd, bd = to_dev(x), to_dev(dy), to_dev(w), to_dev(b)
    yd = dsa3d_gpu.dwconv3d_forward(xd, wd, bd, grid)
    ya = to_dev(y0)
    dsa3d_gpu.dwconv3d_forward(xd, wd, bd, grid, out=ya, accumulate=True)
    dx, dw, db = dsa3d_gpu.dwconv3d_backward(xd, wd, dyd, grid)
    torch.cuda.synchronize()
    ref = oracle.dwconv3d_forward(x, w, b, grid)
    S = oracle.dwconv3d_forward(np.abs(host(x)), np.abs(w), np.abs(b), grid)
    out_r = 2.0**-8 if dtype == "bf16" else 0.0
    assert_bound(to_host_f64(yd), ref, 2.0**-22 * taps * S + out_r * np.abs(ref), "y")
    refa = ref + host(y0)
    assert_bound(to_host_f64(ya), refa, 2.0**-22 * taps * (S + np.abs(host(y0))) + out_r * np.abs(refa), "y+=")
    rdx, rdw, rdb = oracle.dwconv3d_backward(x, w, dy, grid)
    Sx, Sw, Sb = oracle.dwconv3d_backward(np.abs(host(x)), np.abs(w), np.abs(host(dy)), grid)
    assert_bound(to_host_f64(dx), rdx, 2.0**-22 * taps * Sx + out_r * np.abs(rdx), "dx")
    acc = 2.0**-24 * max(N - 1, 1)
    assert_bound(dw.cpu().numpy(), rdw, acc * Sw + 1e-30, "dweight")
    assert_bound(db.cpu().numpy(), rdb, acc * Sb + 1e-30, "dbias")


LIN_CASES = [
    # M, K, O, dtype
    (300, 64, 81, "bf16"),      # ragged tiles
    (1000, 256, 3 * 27 * 2, "bf16"),
    (257, 40, 130, "f32"),
    (129, 12, 7, "bf16"),        # K not a multiple of 8: element-wise loads
    (5000, 72, 260, "bf16"),     # 256-column blocks with a ragged edge; dW with K split in 4 parts
    (300, 520, 600, "bf16"),     # 256-column blocks for y and dx, K = 600 and 520 (ragged K steps)
    (4500, 300, 40, "f32"),      # fp32 dW with K split in 4 parts (the last one shorter)
]


@pytest.mark.parametrize("case", LIN_CASES, ids=[f"M{c[0]}-K{c[1]}-O{c[2]}-{c[3]}" for c in LIN_CASES])
def test_linear(dsa3d_gpu, case):
    M, K, O, dtype = case
    x = synth.normal(51, 0, (M, K), dtype)
    w = synth.normal(51, 1, (O, K), dtype, 0.1)
    b = synth.normal(51, 2, (O,), "f32")
    dy = synth.normal(51, 3, (M, O), "f32")
    print(f"case M={M} K={K} O={O} {dtype}", flush=True)
    xd, wd = to_dev(x), to_dev(w)
    y = dsa3d_gpu.linear_forward(xd, wd, to_dev(b))
    dx, dw, db = dsa3d_gpu.linear_backward(xd, wd, to_dev(dy))
    torch.cuda.synchronize()
    xh, wh = host(x), host(w)
    ref = oracle.linear_forward(xh, wh, b)
    S = np.abs(xh) @ np.abs(wh).T + np.abs(b)
    assert_bound(y.cpu().numpy(), ref, 2.0**-22 * K * S, "y")
    rdx, rdw, rdb = oracle.linear_backward(xh, wh, dy)
    Sdx, Sdw, Sdb = oracle.linear_backward(np.abs(xh), np.abs(wh), np.abs(dy))
    dyr = 2.0**-8 if dtype == "bf16" else 0.0
    out_r = 2.0**-8 if dtype == "bf16" else 0.0
    assert_bound(to_host_f64(dx), rdx, (2.0**-22 * O + dyr) * Sdx + out_r * np.abs(rdx), "dx")
    assert_bound(dw.cpu().numpy(), rdw, (2.0**-22 * M + dyr) * Sdw, "dweight")
    assert_bound(db.cpu().numpy(), rdb, 2.0**-22 * M * Sdb, "dbias")


def test_eq1_end_to_end(dsa3d_gpu):
    """Attention(X) = DWConv3D(X) + sum_j alpha_j TrilinearSample(X W_v, offsets_j), the
    offsets predicted from X by a depthwise convolution and a linear layer (per head and
    sample).  Q, K, V stand for X W_q, X W_k, X W_v (the projections are plain GEMMs
    outside the operator)."""
    grid, H, D, win = (6, 10, 12), 2, 64, (3, 3, 3)
    F, Hp, Wp = grid
    N, C, K = F * Hp * Wp, H * D, 27
    X = synth.normal(61, 0, (N, C), "bf16")
    q, k, v = (synth.normal(61, i + 1, (N, H, D), "bf16") for i in range(3))
    w_off = synth.normal(61, 4, (C, 3, 3, 3), "f32", 0.1)
    b_off = synth.normal(61, 5, (C,), "f32", 0.1)
    w_lin = synth.normal(61, 6, (H * K * 3, C), "bf16", 0.05)
    b_lin = synth.normal(61, 7, (H * K * 3,), "f32", 0.5)
    w_dw = synth.normal(61, 8, (C, 3, 3, 3), "f32", 0.1)
    b_dw = synth.normal(61, 9, (C,), "f32", 0.1)
    Xd = to_dev(X)
    # predictor: depthwise conv, then the pointwise layer to [N, H, K, 3] offsets
    hid = dsa3d_gpu.dwconv3d_forward(Xd, to_dev(w_off), to_dev(b_off), grid)
    off = dsa3d_gpu.linear_forward(hid, to_dev(w_lin), to_dev(b_lin)).reshape(N, H, K, 3)
    out, lse = dsa3d_gpu.sampled_forward(to_dev(q), to_dev(k), to_dev(v), off, grid, win, "free", D ** -0.5)
    # the convolution term added into the attention output ([N, H, D] seen as [N, C])
    dsa3d_gpu.dwconv3d_forward(Xd, to_dev(w_dw), to_dev(b_dw), grid, out=out.view(N, C), accumulate=True)
    torch.cuda.synchronize()
    # the predictor against the oracle (hidden layer and offsets)
    hid_ref = oracle.dwconv3d_forward(X, w_off, b_off, grid)
    assert_close(to_host_f64(hid), hid_ref, "bf16", "predictor hidden")
    off_gpu = off.cpu().numpy().astype(np.float64)
    off_ref = oracle.linear_forward(to_host_f64(hid), host(w_lin), b_lin).reshape(N, H, K, 3)
    assert np.abs(off_gpu - off_ref).max() <= 1e-3 * max(1.0, np.abs(off_ref).max())
    # Eq. (1) with the GPU's offsets through the oracle
    attn, _ = oracle.sampled_forward(q, k, v, off_gpu, grid, win, D ** -0.5, "free")
    ref = attn.reshape(N, C) + oracle.dwconv3d_forward(X, w_dw, b_dw, grid)
    # two bf16 roundings (attention output, then the sum)
    assert_close(to_host_f64(out).reshape(N, C), ref, "bf16", "Attention(X)")
