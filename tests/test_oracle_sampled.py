"""Pins for the oracle's per-head offsets and sampled windows (real offsets, trilinear
sampling, offset gradients), CPU only.

The MegaSlide-DiT 3D Deformable Slide Attention section learns offsets per token and
head, samples keys and values at real positions by trilinear interpolation, and its
implementation paragraph does the sampling with grid_sample (bilinear mode, 5-D
tensors).  These tests tie the oracle to:
  - the integer oracle (itself pinned to brute-force dense attention): box windows with
    integer offsets, per-head offsets head by head;
  - torch's own grid_sample route with autograd (float64): outputs, log-sum-exp, dq, dk,
    dv and the offset gradients, in both readings of the sample positions;
  - central finite differences of the oracle's forward for the offset gradients;
  - invariants of box windows (weights inside the grid sum to one).
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

import oracle

rng = np.random.default_rng(4321)


def rand_qkv(grid, H, D, seed):
    g = np.random.default_rng(seed)
    N = grid[0] * grid[1] * grid[2]
    return tuple(g.standard_normal((N, H, D)) for _ in range(4))


def positions(grid, window, off, mode):
    """Sample positions [N, H, K, 3] (t, y, x) as a torch float64 expression of `off`
    (box: [N, H, 3] broadcastable; free: [N, H, K, 3] broadcastable)."""
    F, Hp, Wp = grid
    kt, ky, kx = window
    t, y, x = torch.meshgrid(torch.arange(F), torch.arange(Hp), torch.arange(Wp), indexing="ij")
    p = torch.stack([t.reshape(-1), y.reshape(-1), x.reshape(-1)], 1).double()  # [N, 3]
    u, v, w = torch.meshgrid(torch.arange(kt), torch.arange(ky), torch.arange(kx), indexing="ij")
    lat = torch.stack([u.reshape(-1), v.reshape(-1), w.reshape(-1)], 1).double()  # [K, 3]
    r = torch.tensor([(kt - 1) // 2, (ky - 1) // 2, (kx - 1) // 2], dtype=torch.float64)
    G = torch.tensor(grid, dtype=torch.float64)
    k = torch.tensor(window, dtype=torch.float64)
    if mode == "box":
        s = torch.minimum(torch.maximum(p[:, None, :] + off - r, torch.zeros(3, dtype=torch.float64)), G - k)
        return s[:, :, None, :] + lat[None, None, :, :]
    return p[:, None, None, :] + lat[None, None, :, :] - r + off


def torch_route(q, k, v, dout, off, grid, window, scale, mode):
    """Attention over trilinear samples taken by grid_sample (zeros padding, align_corners),
    float64, with autograd.  Returns O, LSE and the gradients of q, k, v, off."""
    F, Hp, Wp = grid
    N, H, D = q.shape
    qt, kt_, vt = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    ot = torch.tensor(off, dtype=torch.float64, requires_grad=True)
    P = positions(grid, window, ot, mode)
    P = P.expand(N, H, P.shape[2], 3)
    K = P.shape[2]
    # grid_sample's last axis is (x, y, t), normalised to [-1, 1] over the grid points
    norm = torch.stack([2 * P[..., 2] / (Wp - 1) - 1, 2 * P[..., 1] / (Hp - 1) - 1, 2 * P[..., 0] / (F - 1) - 1], -1)
    outs, lses = [], []
    for h in range(H):
        grid_h = norm[:, h].reshape(1, N, K, 1, 3)
        kin = kt_[:, h, :].T.reshape(1, D, F, Hp, Wp)
        vin = vt[:, h, :].T.reshape(1, D, F, Hp, Wp)
        ks = Fn.grid_sample(kin, grid_h, mode="bilinear", padding_mode="zeros", align_corners=True)[0, :, :, :, 0]
        vs = Fn.grid_sample(vin, grid_h, mode="bilinear", padding_mode="zeros", align_corners=True)[0, :, :, :, 0]
        z = scale * torch.einsum("nd,dnk->nk", qt[:, h, :], ks)
        lses.append(torch.logsumexp(z, -1))
        outs.append(torch.einsum("nk,dnk->nd", torch.softmax(z, -1), vs))
    O = torch.stack(outs, 1)
    L = torch.stack(lses, 0)
    (O * torch.tensor(dout)).sum().backward()
    return O.detach().numpy(), L.detach().numpy(), qt.grad.numpy(), kt_.grad.numpy(), vt.grad.numpy(), ot.grad.numpy()


CASES = [
    # grid, H, D, window, mode, offsets shape (broadcastable), offset scale
    ((4, 5, 6), 2, 8, (3, 3, 3), "free", "per-sample", 1.3),
    ((3, 6, 5), 2, 4, (3, 3, 5), "free", "per-query", 2.0),
    ((5, 4, 7), 2, 8, (3, 3, 3), "box", "per-query", 1.7),
    ((4, 6, 6), 3, 4, (3, 5, 3), "box", "per-head", 2.5),
]


def make_offsets(g, grid, H, window, mode, kind, scale):
    N = grid[0] * grid[1] * grid[2]
    K = window[0] * window[1] * window[2]
    if mode == "box":
        shape = (N, 1, 3) if kind == "per-query" else (N, H, 3)
    else:
        shape = {"per-sample": (N, H, K, 3), "per-query": (N, 1, 1, 3)}[kind]
    return scale * g.standard_normal(shape)


@pytest.mark.parametrize("case", CASES, ids=[f"{c[4]}-{c[5]}" for c in CASES])
def test_sampled_against_grid_sample_autograd(case):
    grid, H, D, window, mode, kind, oscale = case
    g = np.random.default_rng(7)
    q, k, v, do = rand_qkv(grid, H, D, 3)
    off = make_offsets(g, grid, H, window, mode, kind, oscale)
    scale = D ** -0.5
    O, L = oracle.sampled_forward(q, k, v, off, grid, window, scale, mode)
    dq, dk, dv, doff = oracle.sampled_backward(q, k, v, do, off, grid, window, scale, mode)
    O2, L2, dq2, dk2, dv2, doff2 = torch_route(q, k, v, do, off, grid, window, scale, mode)
    for a, b, name in ((O, O2, "O"), (L, L2, "lse"), (dq, dq2, "dq"), (dk, dk2, "dk"), (dv, dv2, "dv"),
                       (doff, doff2, "doffsets")):
        assert a.shape == b.shape, name
        assert np.abs(a - b).max() <= 1e-10 * max(1.0, np.abs(b).max()), (name, np.abs(a - b).max())
    if mode == "free":
        # some samples must leave the grid, or the zero padding is not exercised
        P = positions(grid, window, torch.tensor(off), mode).expand(-1, H, -1, -1).numpy()
        G = np.array(grid)
        assert ((P < 0) | (P > G - 1)).any()


@pytest.mark.parametrize("mode", ["box", "free"])
def test_offset_gradient_finite_differences(mode):
    grid, H, D, window = (4, 5, 5), 2, 4, (3, 3, 3)
    g = np.random.default_rng(11)
    q, k, v, do = rand_qkv(grid, H, D, 5)
    N, K = grid[0] * grid[1] * grid[2], 27
    off = 1.5 * g.standard_normal((N, H, 3) if mode == "box" else (N, H, K, 3))
    scale = 0.5
    _, _, _, doff = oracle.sampled_backward(q, k, v, do, off, grid, window, scale, mode)
    eps = 1e-6
    picks = [tuple(g.integers(0, s) for s in off.shape) for _ in range(25)]
    for idx in picks:
        a, b = off.copy(), off.copy()
        a[idx] += eps
        b[idx] -= eps
        fa = (oracle.sampled_forward(q, k, v, a, grid, window, scale, mode)[0] * do).sum()
        fb = (oracle.sampled_forward(q, k, v, b, grid, window, scale, mode)[0] * do).sum()
        fd = (fa - fb) / (2 * eps)
        assert abs(fd - doff[idx]) <= 1e-6 * max(1.0, abs(fd)), (idx, fd, doff[idx])


def test_box_windows_with_integer_offsets_are_the_integer_windows():
    grid, H, D, window = (5, 7, 6), 2, 8, (3, 5, 3)
    g = np.random.default_rng(2)
    q, k, v, do = rand_qkv(grid, H, D, 9)
    N = grid[0] * grid[1] * grid[2]
    off = g.integers(-6, 7, size=(N, 3)).astype(np.int32)  # many windows clamp at the borders
    O, L = oracle.forward(q, k, v, off, grid, window, 0.3)
    O2, L2 = oracle.sampled_forward(q, k, v, off[:, None, :].astype(np.float64), grid, window, 0.3, "box")
    assert np.abs(O - O2).max() < 1e-12 and np.abs(L - L2).max() < 1e-12
    ref = oracle.backward(q, k, v, do, off, grid, window, 0.3)
    got = oracle.sampled_backward(q, k, v, do, off[:, None, :].astype(np.float64), grid, window, 0.3, "box")
    for a, b in zip(ref, got[:3]):
        assert np.abs(a - b).max() < 1e-12


def test_free_samples_with_zero_offsets_are_the_centred_window_inside_the_grid():
    # zero offsets: sample (u, v, w) sits on the grid point p + (u, v, w) - r; where the
    # centred window lies inside the grid this is the integer window of a zero offset
    grid, H, D, window = (5, 8, 8), 1, 4, (3, 3, 3)
    q, k, v, _ = rand_qkv(grid, H, D, 1)
    N = grid[0] * grid[1] * grid[2]
    zero = np.zeros((N, 1, 1, 3))
    O, _ = oracle.sampled_forward(q, k, v, zero, grid, window, 1.0, "free")
    O2, _ = oracle.forward(q, k, v, np.zeros((N, 3), np.int32), grid, window, 1.0)
    F, Hp, Wp = grid
    t, y, x = np.meshgrid(np.arange(F), np.arange(Hp), np.arange(Wp), indexing="ij")
    inner = ((t > 0) & (t < F - 1) & (y > 0) & (y < Hp - 1) & (x > 0) & (x < Wp - 1)).reshape(-1)
    assert np.abs(O[inner] - O2[inner]).max() < 1e-12
    # at the border the free reading zero-pads: a zero key row gives logit 0 and a zero value
    assert np.abs(O[~inner] - O2[~inner]).max() > 1e-3


def test_box_window_invariants():
    # box windows stay inside the grid, so each sample's weights sum to one:
    # sum_j dV_j = sum_n dO_n and sum_j dK_j = 0 per head, as for integer windows
    grid, H, D, window = (4, 6, 7), 2, 4, (3, 3, 3)
    g = np.random.default_rng(5)
    q, k, v, do = rand_qkv(grid, H, D, 2)
    N = grid[0] * grid[1] * grid[2]
    off = 3.0 * g.standard_normal((N, H, 3))
    _, dk, dv, _ = oracle.sampled_backward(q, k, v, do, off, grid, window, 0.5, "box")
    assert np.abs(dv.sum(0) - do.sum(0)).max() < 1e-10
    assert np.abs(dk.sum(0)).max() < 1e-10


def test_per_head_offsets_are_heads_of_shared_offsets():
    grid, H, D, window = (4, 7, 5), 3, 8, (3, 3, 3)
    g = np.random.default_rng(3)
    q, k, v, do = rand_qkv(grid, H, D, 4)
    N = grid[0] * grid[1] * grid[2]
    offh = g.integers(-5, 6, size=(H, N, 3)).astype(np.int32)
    O, L = oracle.forward_heads(q, k, v, offh, grid, window, 0.4)
    dq, dk, dv = oracle.backward_heads(q, k, v, do, offh, grid, window, 0.4)
    for h in range(H):
        sl = lambda a: np.ascontiguousarray(a[:, h:h + 1, :])
        Oh, Lh = oracle.forward(sl(q), sl(k), sl(v), offh[h], grid, window, 0.4)
        assert np.abs(O[:, h:h + 1] - Oh).max() < 1e-13 and np.abs(L[h] - Lh[0]).max() < 1e-13
        gh = oracle.backward(sl(q), sl(k), sl(v), sl(do), offh[h], grid, window, 0.4)
        for a, b in zip((dq, dk, dv), gh):
            assert np.abs(a[:, h:h + 1] - b).max() < 1e-13
    # the same per-head integer offsets as box windows of the sampled form
    offb = np.transpose(offh, (1, 0, 2)).astype(np.float64)
    O2, L2 = oracle.sampled_forward(q, k, v, offb, grid, window, 0.4, "box")
    assert np.abs(O - O2).max() < 1e-12 and np.abs(L - L2).max() < 1e-12
