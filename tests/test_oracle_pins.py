"""Pins for the CPU oracle, checked against what the definition fixes (CPU only).

The oracle follows the 3D Deformable Slide Attention section of the MegaSlide-DiT
paper (Eq. (1), attention term; softmax alpha; T x H' x W' reshape).  These tests tie
it to independent routes: brute-force dense attention with a mask built from a
different statement of the window rule, the library dense-attention routine, the
paper's own grid_sample route, autograd, finite differences, closed forms and
invariants, and hand-derived window starts.
"""
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(1234)


# ---- an independent statement of the window rule ---------------------------------
# The window is the k-wide box inside [0, G) whose centre is nearest to the shifted
# position p + o (written as an argmin over every valid start, not as a clamp).
def brute_start(p, o, k, G):
    r = (k - 1) // 2
    starts = np.arange(0, G - k + 1)
    return int(starts[np.argmin(np.abs(starts + r - (p + o)))])


def coords(grid):
    F, Hp, Wp = grid
    t, y, x = np.meshgrid(np.arange(F), np.arange(Hp), np.arange(Wp), indexing="ij")
    return np.stack([t.ravel(), y.ravel(), x.ravel()], 1)


def brute_mask(grid, window, offsets):
    """[N][N] boolean: key j is in the window of query n."""
    pos = coords(grid)
    N = len(pos)
    lo = np.empty((N, 3), dtype=np.int64)
    for n in range(N):
        for d in range(3):
            lo[n, d] = brute_start(pos[n, d], int(offsets[n, d]), window[d], grid[d])
    kk = np.asarray(window)
    inside = (pos[None, :, :] >= lo[:, None, :]) & (pos[None, :, :] < lo[:, None, :] + kk)
    return inside.all(-1)


def dense_attention(q, k, v, mask, scale):
    """Masked dense softmax attention in float64 torch; q,k,v [N][H][D], mask [N][N]."""
    q, k, v = (torch.as_tensor(a, dtype=torch.float64) for a in (q, k, v))
    s = torch.einsum("nhd,jhd->hnj", q, k) * scale
    s = s.masked_fill(~torch.as_tensor(mask)[None], float("-inf"))
    lse = torch.logsumexp(s, -1)
    o = torch.einsum("hnj,jhd->nhd", torch.softmax(s, -1), v)
    return o, lse


def rand_case(grid, H, D, omax, dtype=np.float64, seed=0):
    g = np.random.default_rng(seed)
    N = grid[0] * grid[1] * grid[2]
    q, k, v, do = (g.standard_normal((N, H, D)).astype(dtype) for _ in range(4))
    off = g.integers(-omax, omax + 1, size=(N, 3)).astype(np.int32)
    return q, k, v, do, off


# ---- window starts -----------------------------------------------------------------
def test_window_starts_golden():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "window_starts.txt")) if l.strip() and l[0] != "#"]
    assert len(rows) >= 8
    for r in rows:
        F, Hp, Wp, kt, ky, kx, t, y, x, dt, dy, dx, st, sy, sx = map(int, r)
        off = np.zeros((F * Hp * Wp, 3), dtype=np.int32)
        n = (t * Hp + y) * Wp + x
        off[n] = (dt, dy, dx)
        s = oracle.window_starts(off, (F, Hp, Wp), (kt, ky, kx))
        assert tuple(s[n]) == (st, sy, sx), r


@pytest.mark.parametrize("window", [(3, 3, 3), (1, 1, 1), (3, 7, 7), (5, 9, 9), (5, 1, 3)])
def test_window_starts_match_argmin_rule(window):
    grid = (6, 11, 13)
    if any(w > g for w, g in zip(window, grid)):
        window = tuple(min(w, g if g % 2 else g - 1) for w, g in zip(window, grid))
    N = grid[0] * grid[1] * grid[2]
    off = rng.integers(-15, 16, size=(N, 3)).astype(np.int32)
    off[:7] = [[2**31 - 1, -(2**31), 0], [-(2**31), 2**31 - 1, 5], [10**9, 10**9, -10**9],
               [0, 0, 0], [-1, 1, -1], [grid[0], -grid[1], grid[2]], [-grid[0] - 1, grid[1] + 1, 3]]
    s = oracle.window_starts(off, grid, window)
    pos = coords(grid)
    for n in range(N):
        for d in range(3):
            assert s[n, d] == brute_start(pos[n, d], int(off[n, d]), window[d], grid[d])
    # the window always lies inside the grid and holds the shifted position when that is inside
    assert (s >= 0).all() and (s + np.asarray(window) <= np.asarray(grid)).all()
    c = pos + off.astype(np.int64)
    ins = ((c >= 0) & (c < np.asarray(grid))).all(1)
    assert ((c[ins] >= s[ins]) & (c[ins] < s[ins] + np.asarray(window))).all()


# ---- forward -----------------------------------------------------------------------
@pytest.mark.parametrize("grid,window,omax", [((3, 4, 5), (3, 3, 3), 3), ((4, 6, 5), (1, 3, 5), 6),
                                              ((5, 5, 7), (3, 5, 3), 0), ((2, 7, 6), (1, 7, 1), 20)])
def test_forward_matches_masked_dense(grid, window, omax):
    H, D = 2, 8
    q, k, v, _, off = rand_case(grid, H, D, omax, seed=7)
    o, lse = oracle.forward(q, k, v, off, grid, window, 0.37)
    o_ref, lse_ref = dense_attention(q, k, v, brute_mask(grid, window, off), 0.37)
    np.testing.assert_allclose(o, o_ref.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_window_equal_to_grid_is_dense_attention(dtype):
    grid, H, D = (3, 5, 7), 3, 16
    q, k, v, _, off = rand_case(grid, H, D, 4, dtype=dtype, seed=3)
    scale = D ** -0.5
    for offsets in (np.zeros_like(off), off):  # whatever the offsets, the window is the whole grid
        o, lse = oracle.forward(q, k, v, offsets, grid, grid, scale)
        qt, kt_, vt = (torch.as_tensor(a.astype(np.float64)).permute(1, 0, 2) for a in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt_, vt, scale=scale).permute(1, 0, 2)
        np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-12)
        lse_ref = torch.logsumexp(torch.einsum("hnd,hjd->hnj", qt, kt_) * scale, -1)
        np.testing.assert_allclose(lse, lse_ref.numpy(), rtol=0, atol=1e-12)


def test_one_voxel_window_returns_shifted_clamped_value():
    grid, H, D = (4, 6, 5), 2, 8
    q, k, v, _, off = rand_case(grid, H, D, 7, dtype=np.float32, seed=11)
    o, lse = oracle.forward(q, k, v, off, grid, (1, 1, 1), 0.5)
    pos = coords(grid)
    c = np.clip(pos + off, 0, np.asarray(grid) - 1)
    j = (c[:, 0] * grid[1] + c[:, 1]) * grid[2] + c[:, 2]
    assert np.array_equal(o, v[j].astype(np.float64))  # exact
    logit = 0.5 * np.einsum("nhd,nhd->hn", q.astype(np.float64), k[j].astype(np.float64))
    np.testing.assert_allclose(lse, logit, rtol=0, atol=1e-12)


def test_zero_queries_average_the_window():
    grid, window, H, D = (4, 7, 6), (3, 3, 5), 2, 4
    _, k, v, _, off = rand_case(grid, H, D, 4, seed=5)
    q = np.zeros_like(k)
    o, lse = oracle.forward(q, k, v, off, grid, window, 1.0)
    mask = brute_mask(grid, window, off)
    K = np.prod(window)
    assert (mask.sum(1) == K).all()
    mean = np.einsum("nj,jhd->nhd", mask.astype(np.float64), v) / K
    np.testing.assert_allclose(o, mean, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, np.log(K), rtol=0, atol=1e-13)


def test_weights_are_a_distribution_over_the_window():
    grid, window, H, D = (5, 6, 7), (3, 5, 3), 2, 8
    q, k, v, _, off = rand_case(grid, H, D, 5, seed=9)
    mask = brute_mask(grid, window, off)
    for n in rng.integers(0, len(off), 25):
        for h in range(H):
            keys, p, _ = oracle.weights(q, k, v, off, grid, window, 0.3, n, h)
            assert len(set(keys.tolist())) == len(keys) == np.prod(window)
            assert set(keys.tolist()) == set(np.nonzero(mask[n])[0].tolist())
            assert (p > 0).all() and abs(p.sum() - 1.0) <= 1e-12


def test_grid_sample_route_matches_on_interior_windows():
    """The paper samples K and V with F.grid_sample (trilinear, 5D); at integer positions
    inside the grid that sampling is exact, so it must reproduce the oracle there."""
    grid, window, H, D = (6, 9, 11), (3, 3, 5), 2, 4
    F, Hp, Wp = grid
    q, k, v, _, off = rand_case(grid, H, D, 2, seed=21)
    o, _ = oracle.forward(q, k, v, off, grid, window, 0.45)
    pos = coords(grid)
    r = (np.asarray(window) - 1) // 2
    c = pos + off
    interior = ((c - r >= 0) & (c + r < np.asarray(grid))).all(1)
    idx = np.nonzero(interior)[0]
    assert len(idx) > 50
    u, w_, x_ = np.meshgrid(*(np.arange(kk) - rr for kk, rr in zip(window, r)), indexing="ij")
    rel = np.stack([u.ravel(), w_.ravel(), x_.ravel()], 1)  # [K][3] (t, y, x)
    samp = c[idx][:, None, :] + rel[None]  # [n][K][3]
    g = torch.empty(1, len(idx), len(rel), 1, 3, dtype=torch.float64)
    g[0, :, :, 0, 0] = torch.as_tensor(2.0 * samp[..., 2] / (Wp - 1) - 1.0)
    g[0, :, :, 0, 1] = torch.as_tensor(2.0 * samp[..., 1] / (Hp - 1) - 1.0)
    g[0, :, :, 0, 2] = torch.as_tensor(2.0 * samp[..., 0] / (F - 1) - 1.0)

    def sample(x):  # x [N][H][D] -> [n][K][H][D]
        vol = torch.as_tensor(x).reshape(F, Hp, Wp, H * D).permute(3, 0, 1, 2)[None]
        out = torch.nn.functional.grid_sample(vol, g, mode="bilinear", align_corners=True)
        return out[0, :, :, :, 0].permute(1, 2, 0).reshape(len(idx), len(rel), H, D)

    ks, vs = sample(k), sample(v)
    s = torch.einsum("nhd,nkhd->nhk", torch.as_tensor(q[idx]), ks) * 0.45
    ref = torch.einsum("nhk,nkhd->nhd", torch.softmax(s, -1), vs)
    np.testing.assert_allclose(o[idx], ref.numpy(), rtol=0, atol=1e-12)


def test_forward_invariants():
    grid, window, H, D = (5, 8, 9), (3, 3, 3), 2, 8
    q, k, v, _, off = rand_case(grid, H, D, 2, seed=31)
    o, lse = oracle.forward(q, k, v, off, grid, window, 0.3)
    # adding one vector to every key shifts each query's logits by a constant
    c = rng.standard_normal((1, H, D))
    o2, _ = oracle.forward(q, k + c, v, off, grid, window, 0.3)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-12)
    # affine values: a V + b -> a O + b
    b = rng.standard_normal((1, H, D))
    o3, _ = oracle.forward(q, k, 2.5 * v + b, off, grid, window, 0.3)
    np.testing.assert_allclose(o3, 2.5 * o + b, rtol=0, atol=1e-12)
    # a constant offset equals zero offsets on K, V shifted by it (interior windows)
    shift = np.array([1, -2, 3])
    off_c = np.broadcast_to(shift.astype(np.int32), off.shape).copy()
    oc, _ = oracle.forward(q, k, v, off_c, grid, window, 0.3)
    roll = lambda a: np.roll(a.reshape(*grid, H, D), tuple(-shift), axis=(0, 1, 2)).reshape(-1, H, D)
    oz, _ = oracle.forward(q, roll(k), roll(v), np.zeros_like(off), grid, window, 0.3)
    pos = coords(grid)
    r = (np.asarray(window) - 1) // 2
    ok = ((pos + shift - r >= 0) & (pos + shift + r < np.asarray(grid)) & (pos - r >= 0)
          & (pos + r < np.asarray(grid))).all(1)
    assert ok.sum() > 20
    np.testing.assert_allclose(oc[ok], oz[ok], rtol=0, atol=1e-12)


# ---- backward ----------------------------------------------------------------------
def test_backward_matches_autograd_on_masked_dense():
    grid, window, H, D = (3, 4, 5), (3, 3, 3), 2, 4
    q, k, v, do, off = rand_case(grid, H, D, 3, seed=41)
    dq, dk, dv = oracle.backward(q, k, v, do, off, grid, window, 0.6)
    mask = brute_mask(grid, window, off)
    qt, kt_, vt = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    s = (torch.einsum("nhd,jhd->hnj", qt, kt_) * 0.6).masked_fill(~torch.as_tensor(mask)[None], float("-inf"))
    o = torch.einsum("hnj,jhd->nhd", torch.softmax(s, -1), vt)
    o.backward(torch.as_tensor(do))
    for a, b in ((dq, qt.grad), (dk, kt_.grad), (dv, vt.grad)):
        np.testing.assert_allclose(a, b.numpy(), rtol=0, atol=1e-11)


def test_backward_finite_differences():
    """Central differences of L = sum(G * O) with h = 1e-6, offsets including clamped ones."""
    grid, window, H, D = (3, 4, 5), (3, 3, 3), 2, 4
    q, k, v, G, off = rand_case(grid, H, D, 3, seed=43)
    off[0] = (-5, 9, -9)
    dq, dk, dv = oracle.backward(q, k, v, G, off, grid, window, 0.6)

    def loss(q_, k_, v_):
        return float((oracle.forward(q_, k_, v_, off, grid, window, 0.6)[0] * G).sum())

    h = 1e-6
    g = np.random.default_rng(5)
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        for _ in range(12):
            i = tuple(int(g.integers(0, s)) for s in q.shape)
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][i] += h
            args_m[which][i] -= h
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - grad[i]) <= 1e-6 * max(1.0, abs(grad[i])), (which, i, fd, grad[i])


def test_backward_invariants():
    grid, window, H, D = (4, 7, 6), (3, 5, 3), 3, 8
    q, k, v, do, off = rand_case(grid, H, D, 4, seed=47)
    dq, dk, dv = oracle.backward(q, k, v, do, off, grid, window, 0.4)
    # every row of P sums to one, and every row of dS sums to zero
    np.testing.assert_allclose(dv.sum(0), do.sum(0), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk.sum(0), 0.0, rtol=0, atol=1e-11)
    # one-voxel window: no gradient through the logits, dV collects dO by target
    dq1, dk1, dv1 = oracle.backward(q, k, v, do, off, grid, (1, 1, 1), 0.4)
    assert np.abs(dq1).max() <= 1e-14 and np.abs(dk1).max() <= 1e-14
    pos = coords(grid)
    c = np.clip(pos + off, 0, np.asarray(grid) - 1)
    j = (c[:, 0] * grid[1] + c[:, 1]) * grid[2] + c[:, 2]
    ref = np.zeros_like(dv1)
    np.add.at(ref, j, do)
    np.testing.assert_allclose(dv1, ref, rtol=0, atol=1e-13)


@pytest.mark.parametrize("grid,window,omax", [((4, 6, 7), (3, 3, 5), 3), ((3, 9, 8), (1, 5, 7), 40),
                                              ((5, 5, 5), (5, 5, 5), 2)])
def test_row_functions_match_full(grid, window, omax):
    """Key-centric gather (dk, dv) against the per-head scatter, and the row forms of
    the forward and of dq against the full ones."""
    H, D = 2, 8
    q, k, v, do, off = rand_case(grid, H, D, omax, dtype=np.float32, seed=53)
    o, lse = oracle.forward(q, k, v, off, grid, window, 0.35)
    dq, dk, dv = oracle.backward(q, k, v, do, off, grid, window, 0.35)
    N = len(off)
    rows = np.arange(N * H)
    o_r, lse_r = oracle.forward_rows(q, k, v, off, grid, window, 0.35, rows)
    np.testing.assert_allclose(o_r, o.reshape(N * H, D), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse_r, lse.T.reshape(-1), rtol=0, atol=1e-13)
    dq_r = oracle.backward_q_rows(q, k, v, do, off, grid, window, 0.35, rows)
    np.testing.assert_allclose(dq_r, dq.reshape(N * H, D), rtol=0, atol=1e-12)
    dk_r, dv_r = oracle.backward_kv_rows(q, k, v, do, off, grid, window, 0.35, rows)
    np.testing.assert_allclose(dk_r, dk.reshape(N * H, D), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv_r, dv.reshape(N * H, D), rtol=0, atol=1e-12)


def test_bf16_inputs_are_read_exactly():
    grid, window, H, D = (3, 4, 5), (3, 3, 3), 2, 8
    q, k, v, do, off = rand_case(grid, H, D, 2, dtype=np.float32, seed=61)
    to_bits = lambda a: (torch.as_tensor(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    widen = lambda b: (b.astype(np.uint32) << 16).view(np.float32)
    qb, kb, vb, dob = map(to_bits, (q, k, v, do))
    o_b, lse_b = oracle.forward(qb, kb, vb, off, grid, window, 0.5)
    o_f, lse_f = oracle.forward(widen(qb), widen(kb), widen(vb), off, grid, window, 0.5)
    assert np.array_equal(o_b, o_f) and np.array_equal(lse_b, lse_f)
    g_b = oracle.backward(qb, kb, vb, dob, off, grid, window, 0.5)
    g_f = oracle.backward(widen(qb), widen(kb), widen(vb), widen(dob), off, grid, window, 0.5)
    for a, b in zip(g_b, g_f):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("window", [(3, 9, 9), (3, 4, 3), (5, 3, 3)])
def test_window_must_be_odd_and_fit_the_grid(window):
    """A window wider than the grid (or of even extent) has no centred, clamped
    placement: the oracle refuses it, like the library's DSA3D_ERR_WINDOW."""
    grid = (4, 8, 8)
    N = 4 * 8 * 8
    q = np.zeros((N, 1, 64), np.float32)
    off = np.zeros((N, 3), np.int32)
    with pytest.raises(ValueError):
        oracle.window_starts(off, grid, window)
    with pytest.raises(ValueError):
        oracle.forward(q, q, q, off, grid, window, 1.0)
