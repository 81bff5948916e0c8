"""Pins for the oracle's depthwise 3-D convolution (Eq. (1)'s first term and the first
stage of the offset predictor) and the predictor's pointwise layer, CPU only.

The implementation paragraph of the MegaSlide-DiT 3D Deformable Slide Attention section
builds the predictor from nn.Conv3d with groups equal to the hidden size followed by a
pointwise layer.  The oracle's plain loops are tied to torch's own conv3d / linear with
autograd (float64), to closed forms (a centre-tap filter is the identity plus bias; an
all-ones filter on ones counts the in-grid neighbours) and to exact bf16 reads."""
import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

import oracle


def torch_dwconv(x, w, b, grid):
    F, Hp, Wp = grid
    N, C = x.shape
    ct, cy, cx = w.shape[1:]
    xt = x.T.reshape(1, C, F, Hp, Wp)
    y = Fn.conv3d(xt, w.reshape(C, 1, ct, cy, cx), b, padding=((ct - 1) // 2, (cy - 1) // 2, (cx - 1) // 2), groups=C)
    return y.reshape(C, N).T


@pytest.mark.parametrize("grid,C,k", [((4, 5, 6), 3, (3, 3, 3)), ((5, 7, 4), 2, (3, 5, 1)), ((3, 9, 9), 4, (1, 7, 7)),
                                      ((2, 3, 3), 2, (5, 5, 5))])
def test_dwconv_against_torch_conv3d(grid, C, k):
    g = np.random.default_rng(1)
    N = grid[0] * grid[1] * grid[2]
    x = g.standard_normal((N, C))
    w = g.standard_normal((C, *k))
    b = g.standard_normal(C)
    dy = g.standard_normal((N, C))
    y = oracle.dwconv3d_forward(x, w, b, grid)
    dx, dw, db = oracle.dwconv3d_backward(x, w, dy, grid)
    xt, wt, bt = (torch.tensor(a, requires_grad=True) for a in (x, w, b))
    yt = torch_dwconv(xt, wt, bt, grid)
    (yt * torch.tensor(dy)).sum().backward()
    assert np.abs(y - yt.detach().numpy()).max() < 1e-12
    assert np.abs(dx - xt.grad.numpy()).max() < 1e-12
    assert np.abs(dw - wt.grad.numpy()).max() < 1e-11
    assert np.abs(db - bt.grad.numpy()).max() < 1e-11


def test_dwconv_closed_forms():
    grid, C, k = (4, 6, 5), 3, (3, 5, 3)
    N = 4 * 6 * 5
    g = np.random.default_rng(2)
    x = g.standard_normal((N, C))
    b = g.standard_normal(C)
    centre = np.zeros((C, *k))
    centre[:, 1, 2, 1] = 1.0
    assert np.abs(oracle.dwconv3d_forward(x, centre, b, grid) - (x + b)).max() == 0
    ones = oracle.dwconv3d_forward(np.ones((N, C)), np.ones((C, *k)), None, grid)
    # neighbours inside the grid along each axis, multiplied over the axes
    cnt = np.ones(grid)
    for ax, (G, kk) in enumerate(zip(grid, k)):
        r = (kk - 1) // 2
        c1 = np.array([min(p + r, G - 1) - max(p - r, 0) + 1 for p in range(G)], dtype=float)
        shape = [1, 1, 1]
        shape[ax] = G
        cnt = cnt * c1.reshape(shape)
    assert np.array_equal(ones, np.repeat(cnt.reshape(-1, 1), C, 1))


def test_dwconv_reads_bf16_bits_exactly():
    grid, C, k = (3, 4, 5), 2, (3, 3, 3)
    N = 60
    g = np.random.default_rng(3)
    x32 = g.standard_normal((N, C)).astype(np.float32)
    bits = torch.tensor(x32).bfloat16().view(torch.int16).numpy().view(np.uint16)
    w = g.standard_normal((C, *k))
    a = oracle.dwconv3d_forward(bits, w, None, grid)
    b = oracle.dwconv3d_forward(oracle.bf16_to_f64(bits), w, None, grid)
    assert np.array_equal(a, b)


def test_linear_against_torch_and_identity():
    g = np.random.default_rng(4)
    x = g.standard_normal((37, 12))
    w = g.standard_normal((9, 12))
    b = g.standard_normal(9)
    dy = g.standard_normal((37, 9))
    xt, wt, bt = (torch.tensor(a, requires_grad=True) for a in (x, w, b))
    yt = Fn.linear(xt, wt, bt)
    (yt * torch.tensor(dy)).sum().backward()
    assert np.abs(oracle.linear_forward(x, w, b) - yt.detach().numpy()).max() < 1e-12
    dx, dw, db = oracle.linear_backward(x, w, dy)
    for a, t in ((dx, xt), (dw, wt), (db, bt)):
        assert np.abs(a - t.grad.numpy()).max() < 1e-12
    assert np.array_equal(oracle.linear_forward(x, np.eye(12), np.zeros(12)), x)
