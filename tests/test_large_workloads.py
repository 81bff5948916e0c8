"""Parity at the full sizes of the 720p-like, full-width and 256-frame workloads, in the
launch configuration the benchmark times.

- 720p-like (grid 32 x 45 x 80, 16 heads x 128, window 3 x 9 x 9): every element of O, LSE,
  dQ, dK and dV against the full oracle.
- 5 x 9 x 9 window over 100 frames (grid 100 x 32 x 32, 8 heads x 128, drifting offsets):
  every element as well.  Its 96 start slices make three query-side work items of 32
  slices, and its 64 key-block columns x 8 heads = 512 workgroups keep the key-centric
  dK/dV pass at one run over all 100 frames, as at the 256-frame workload.
- full-width (64 x 68 x 120, 64 heads) and 256-frame (256 x 68 x 120, 16 heads x 128,
  window 5 x 9 x 9): every (query, head) row of the start slices on both sides of each
  query-side work-item boundary (slices 31 | 32, and 63 | 64 at 256 frames), grid
  corners and edge centres, and random rows, against the oracle computed row by row;
  plus properties that hold at any size, checked over every output.

- 256-frame workload with per-head offsets (16 drifting motion fields, all heads bucketed
  together, as the benchmark runs it): per head, the rows of its own work-item boundary
  slices (heads 0 and 15), corners, edge centres and random rows, against the oracle with
  that head's offsets.
- the DWConv3D term on the 256-frame grid (2048 channels, 3 x 3 x 3 filter, added into an
  existing output): every position of 32 channels spread over the 32 channel blocks and
  their lanes, forward, input gradient, filter and bias gradients, against the oracle on
  those channels (depthwise: channels are independent).
- the offset predictor at the benchmark's size (16 x 32 x 32, 1024 channels, pointwise layer to
  8 heads x 147 samples x 3 = 3528 offsets, bf16): the depthwise stages every element, the
  pointwise layer on 256 rows (outputs, input gradient) and 64 output columns (weight and
  bias gradients; both are independent per row / per column), each stage fed the GPU's
  own input so that the stages are checked one at a time.
- sampled windows on the benchmark's workloads (16 x 32 x 32, 8 heads x 128, the 3 x 7 x 7
  window, bf16; box windows with one real offset per query on the lattice kernels, and free
  per-sample offsets): every element of O, LSE, dQ, dK, dV and the offset gradient against
  the full oracle.

Properties (P = softmax weights of a query, rows sum to one; dS rows sum to zero):
  sum_j dV[j,h] = sum_n dO[n,h]        sum_j dK[j,h] = 0        all outputs finite.
"""
import numpy as np
import pytest
import torch

import oracle
from local_sparse_attention_amd import configs, synth
from local_sparse_attention_amd.configs import Workload

from _gpu_helpers import (assert_close, assert_lse_close, border_and_random_rows, gather_rows, nan_like, to_dev,
                          to_host_f64)

pytestmark = pytest.mark.gpu

SAMPLES = {"C4": (512, 96), "C5": (512, 96)}
# query-side work items are 32 start slices (the frame-sweeping kernels' QS_TS)
ITEM_SLICES = 32


def run_gpu(dsa3d, wl, inp):
    grid, window = (wl.F, wl.Hp, wl.Wp), (wl.kt, wl.ky, wl.kx)
    q, k, v, do, off = (to_dev(inp[x]) for x in ("q", "k", "v", "dout", "offsets"))
    print(f"case {wl.name}: forward + backward on the GPU", flush=True)
    # outputs start as NaN: an element the library leaves unwritten fails the checks
    out, lse = dsa3d.forward(q, k, v, off, grid, window, wl.scale, out=nan_like(q),
                             lse=torch.full((q.shape[1], q.shape[0]), float("nan"), device=q.device))
    dq, dk, dv = dsa3d.backward(q, k, v, off, out, lse, do, grid, window, wl.scale, dq=nan_like(q), dk=nan_like(q),
                                dv=nan_like(q))
    torch.cuda.synchronize()
    return do, out, lse, dq, dk, dv


def check_properties(wl, do, out, lse, dq, dk, dv):
    """Properties over every output, per head, in float64 on the device."""
    N = wl.N
    dv_sum = dv.double().sum(0)
    do_sum = do.double().sum(0)
    dk_sum = dk.double().sum(0)
    # each bf16 output carries a rounding error of at most 2^-9 relative; a sum of N of them
    # stays within a few sqrt(N) * 2^-9 * rms(value) (independent roundings)
    tol_v = 8 * np.sqrt(N) * 2.0**-9 * dv.double().pow(2).mean().sqrt().item() + 1e-6
    tol_k = 8 * np.sqrt(N) * 2.0**-9 * dk.double().pow(2).mean().sqrt().item() + 1e-6
    ev = (dv_sum - do_sum).abs().max().item()
    ek = dk_sum.abs().max().item()
    print(f"sum dV - sum dO: {ev:.3e} (tol {tol_v:.3e});  sum dK: {ek:.3e} (tol {tol_k:.3e})", flush=True)
    assert ev <= tol_v and ek <= tol_k
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    assert torch.isfinite(dq.float()).all() and torch.isfinite(dk.float()).all() and torch.isfinite(dv.float()).all()


def run_full(dsa3d, wl):
    """Every output element against the full oracle."""
    grid, window = (wl.F, wl.Hp, wl.Wp), (wl.kt, wl.ky, wl.kx)
    print(f"case {wl.name}: generating inputs N={wl.N} H={wl.heads} D={wl.head_dim}", flush=True)
    inp = synth.make_inputs(wl)
    do, out, lse, dq, dk, dv = run_gpu(dsa3d, wl, inp)
    check_properties(wl, do, out, lse, dq, dk, dv)
    args = (inp["q"], inp["k"], inp["v"])
    print(f"case {wl.name}: full oracle forward", flush=True)
    o_ref, lse_ref = oracle.forward(*args, inp["offsets"], grid, window, wl.scale)
    errs = {"out": assert_close(to_host_f64(out), o_ref, wl.dtype, "out"),
            "lse": assert_lse_close(lse.cpu().numpy(), lse_ref)}
    del o_ref, lse_ref
    print(f"case {wl.name}: full oracle backward", flush=True)
    refs = oracle.backward(*args, inp["dout"], inp["offsets"], grid, window, wl.scale)
    for name, gpu, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
        errs[name] = assert_close(to_host_f64(gpu), ref, wl.dtype, name)
    print("max abs err", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)


def boundary_rows(wl, offsets, boundaries=2):
    """Rows r = n*H + h (every head) of the queries whose window starts in a slice next to
    one of the first `boundaries` query-side work-item boundaries."""
    grid, window = (wl.F, wl.Hp, wl.Wp), (wl.kt, wl.ky, wl.kx)
    st = oracle.window_starts(offsets, grid, window)[:, 0]
    Lt = wl.F - wl.kt + 1
    slices = [s for b in range(ITEM_SLICES, Lt, ITEM_SLICES)[:boundaries] for s in (b - 1, b)]
    toks = np.nonzero(np.isin(st, slices))[0].astype(np.int64)
    rows = (toks[:, None] * wl.heads + np.arange(wl.heads)[None, :]).ravel()
    return slices, rows


def run_sampled(dsa3d, name):
    wl = configs.ALL[name]
    grid, window = (wl.F, wl.Hp, wl.Wp), (wl.kt, wl.ky, wl.kx)
    print(f"case {wl.name}: generating inputs N={wl.N} H={wl.heads} D={wl.head_dim}", flush=True)
    inp = synth.make_inputs(wl)
    do, out, lse, dq, dk, dv = run_gpu(dsa3d, wl, inp)

    nq, nk = SAMPLES[name]
    slices, brows = boundary_rows(wl, inp["offsets"])
    qrows = np.unique(np.concatenate([border_and_random_rows(grid, wl.heads, nq, seed=1), brows]))
    krows = border_and_random_rows(grid, wl.heads, nk, seed=2)
    args = (inp["q"], inp["k"], inp["v"])
    print(f"case {wl.name}: oracle on {len(qrows)} query rows ({len(brows)} in start slices {slices}) and "
          f"{len(krows)} key rows", flush=True)
    o_ref, lse_ref = oracle.forward_rows(*args, inp["offsets"], grid, window, wl.scale, qrows)
    assert_close(gather_rows(out, qrows), o_ref, wl.dtype, "out")
    lse_g = lse.T.reshape(-1)[torch.as_tensor(qrows, device=lse.device)].cpu().numpy()
    assert_lse_close(lse_g, lse_ref)
    del o_ref
    dq_ref = oracle.backward_q_rows(*args, inp["dout"], inp["offsets"], grid, window, wl.scale, qrows)
    assert_close(gather_rows(dq, qrows), dq_ref, wl.dtype, "dq")
    del dq_ref
    dk_ref, dv_ref = oracle.backward_kv_rows(*args, inp["dout"], inp["offsets"], grid, window, wl.scale, krows)
    assert_close(gather_rows(dk, krows), dk_ref, wl.dtype, "dk")
    assert_close(gather_rows(dv, krows), dv_ref, wl.dtype, "dv")
    check_properties(wl, do, out, lse, dq, dk, dv)


@pytest.mark.timeout(900)
def test_720p_like_workload_every_element(dsa3d_gpu):
    run_full(dsa3d_gpu, configs.C3)


LONG_5x9x9 = Workload("kt5-9x9-drift-100f", 100, 32, 32, 8, 128, 5, 9, 9, "bf16", True, 4, 1.0,
                      ("blocks", 8, 3.0, True, 8.0))


@pytest.mark.timeout(900)
def test_5x9x9_window_three_work_items_every_element(dsa3d_gpu):
    wl = LONG_5x9x9
    assert (wl.F - wl.kt + 1) // ITEM_SLICES == 3
    assert ((wl.Hp + 3) // 4) * ((wl.Wp + 3) // 4) * wl.heads == 512
    run_full(dsa3d_gpu, wl)


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_full_width_workload(dsa3d_gpu):
    run_sampled(dsa3d_gpu, "C4")


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_256_frame_workload(dsa3d_gpu):
    run_sampled(dsa3d_gpu, "C5")


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_256_frame_workload_per_head_offsets(dsa3d_gpu):
    wl = configs.C5
    grid, window = (wl.F, wl.Hp, wl.Wp), (wl.kt, wl.ky, wl.kx)
    H = wl.heads
    print(f"case {wl.name} per-head offsets: generating inputs", flush=True)
    inp = synth.make_inputs(wl)
    offh = synth.make_head_offsets(wl)
    q, k, v, do = (to_dev(inp[x]) for x in ("q", "k", "v", "dout"))
    ws = dsa3d_gpu.workspace(grid, H, window, True, per_head=True)  # every head bucketed together
    out, lse = dsa3d_gpu.forward(q, k, v, to_dev(offh), grid, window, wl.scale, out=nan_like(q),
                                 lse=torch.full((H, wl.N), float("nan"), device="cuda"), ws=ws)
    dq, dk, dv = dsa3d_gpu.backward(q, k, v, to_dev(offh), out, lse, do, grid, window, wl.scale, dq=nan_like(q),
                                    dk=nan_like(q), dv=nan_like(q), ws=ws)
    torch.cuda.synchronize()
    del ws
    check_properties(wl, do, out, lse, dq, dk, dv)
    args = (inp["q"], inp["k"], inp["v"])
    qall = border_and_random_rows(grid, H, 1024, seed=3)
    kall = border_and_random_rows(grid, H, 256, seed=4)
    lse_flat = lse.T.reshape(-1)
    for h in range(H):
        qrows = qall[qall % H == h]
        if h in (0, H - 1):
            _, brows = boundary_rows(wl, offh[h], boundaries=1)
            qrows = np.unique(np.concatenate([qrows, brows[brows % H == h]]))
        krows = kall[kall % H == h]
        print(f"head {h}: {len(qrows)} query rows, {len(krows)} key rows", flush=True)
        o_ref, lse_ref = oracle.forward_rows(*args, offh[h], grid, window, wl.scale, qrows)
        assert_close(gather_rows(out, qrows), o_ref, wl.dtype, f"out h{h}")
        assert_lse_close(lse_flat[torch.as_tensor(qrows, device=lse.device)].cpu().numpy(), lse_ref)
        dq_ref = oracle.backward_q_rows(*args, inp["dout"], offh[h], grid, window, wl.scale, qrows)
        assert_close(gather_rows(dq, qrows), dq_ref, wl.dtype, f"dq h{h}")
        dk_ref, dv_ref = oracle.backward_kv_rows(*args, inp["dout"], offh[h], grid, window, wl.scale, krows)
        assert_close(gather_rows(dk, krows), dk_ref, wl.dtype, f"dk h{h}")
        assert_close(gather_rows(dv, krows), dv_ref, wl.dtype, f"dv h{h}")


def _assert_bound(gpu, ref, bound, what):
    gpu, ref, bound = (np.asarray(a, dtype=np.float64) for a in (gpu, ref, bound))
    assert gpu.shape == ref.shape and np.isfinite(gpu).all(), what
    excess = np.abs(gpu - ref) - bound
    i = np.unravel_index(np.argmax(excess), excess.shape)
    assert excess.max() <= 0, f"{what}: err {abs(gpu[i] - ref[i]):.3e} > bound {bound[i]:.3e} at {i}"
    return float(np.abs(gpu - ref).max())


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_dwconv3d_term_256_frame_grid(dsa3d_gpu):
    """Bounds as for the small DWConv3D cases: outputs 2^-22 taps S + 2^-8 |ref| (bf16
    rounding), filter and bias gradients 2^-24 (N - 1) S (fp32 sums of N products in a fixed
    order), S the oracle's sum over absolute values."""
    wl = configs.C5
    grid, N, C = (wl.F, wl.Hp, wl.Wp), wl.N, wl.heads * wl.head_dim
    taps = 27
    print(f"case DWConv3D term: grid {grid}, {C} channels, 3x3x3, bf16: generating inputs", flush=True)
    x = synth.normal(43, 0, (N, C), "bf16")
    y0 = synth.normal(43, 1, (N, C), "bf16")
    dy = synth.normal(43, 3, (N, C), "bf16")
    w = synth.normal(43, 4, (C, 3, 3, 3), "f32", 0.1)
    b = synth.normal(43, 5, (C,), "f32")
    xd, wd, bd = to_dev(x), to_dev(w), to_dev(b)
    ya = to_dev(y0)
    dsa3d_gpu.dwconv3d_forward(xd, wd, bd, grid, out=ya, accumulate=True)
    dyd = to_dev(dy)
    dx, dw, db = dsa3d_gpu.dwconv3d_backward(xd, wd, dyd, grid)
    torch.cuda.synchronize()
    del xd, dyd
    # one channel of every 64-channel block, at lanes spread over the block
    cs = np.arange(32) * 64 + (np.arange(32) * 7) % 64
    cst = torch.as_tensor(cs, device="cuda")
    xs, y0s, dys = (np.ascontiguousarray(a[:, cs]) for a in (x, y0, dy))
    del x, y0, dy
    ws_, bs_ = np.ascontiguousarray(w[cs]), np.ascontiguousarray(b[cs])
    print("oracle on 32 channels", flush=True)
    ref = oracle.dwconv3d_forward(xs, ws_, bs_, grid) + oracle.bf16_to_f64(y0s)
    S = oracle.dwconv3d_forward(np.abs(oracle.bf16_to_f64(xs)), np.abs(ws_), np.abs(bs_), grid)
    S += np.abs(oracle.bf16_to_f64(y0s))
    errs = {"y+=": _assert_bound(to_host_f64(ya[:, cst]), ref, 2.0**-22 * taps * S + 2.0**-8 * np.abs(ref), "y+=")}
    del ref, S
    rdx, rdw, rdb = oracle.dwconv3d_backward(xs, ws_, dys, grid)
    Sx, Sw, Sb = oracle.dwconv3d_backward(np.abs(oracle.bf16_to_f64(xs)), np.abs(ws_),
                                          np.abs(oracle.bf16_to_f64(dys)), grid)
    errs["dx"] = _assert_bound(to_host_f64(dx[:, cst]), rdx, 2.0**-22 * taps * Sx + 2.0**-8 * np.abs(rdx), "dx")
    acc = 2.0**-24 * (N - 1)
    errs["dw"] = _assert_bound(dw[cst].cpu().numpy(), rdw, acc * Sw + 1e-30, "dweight")
    errs["db"] = _assert_bound(db[cst].cpu().numpy(), rdb, acc * Sb + 1e-30, "dbias")
    print("max abs err", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)


@pytest.mark.slow
@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,mode", [("S_BOX", "box"), ("S_FREE", "free")])
def test_sampled_windows_benchmark_workloads(dsa3d_gpu, name, mode):
    """Tolerances as for the small sampled cases (bf16: 2e-2 + 1e-2 |ref|, LSE 1e-4; the
    offset gradient, an fp32 sum over heads, samples and corners of products of bf16-derived
    values, at the bf16 form)."""
    wl = getattr(configs, name)
    grid, window = (wl.F, wl.Hp, wl.Wp), (wl.kt, wl.ky, wl.kx)
    print(f"case {wl.name} ({mode}): generating inputs", flush=True)
    inp = synth.make_inputs(wl)
    off = synth.make_real_offsets(wl, mode)
    q, k, v, do = (to_dev(inp[x]) for x in ("q", "k", "v", "dout"))
    offd = to_dev(off)
    out, lse = dsa3d_gpu.sampled_forward(q, k, v, offd, grid, window, mode, wl.scale, out=nan_like(q),
                                         lse=torch.full((wl.heads, wl.N), float("nan"), device="cuda"))
    dq, dk, dv, doff = dsa3d_gpu.sampled_backward(q, k, v, offd, out, lse, do, grid, window, mode, wl.scale)
    torch.cuda.synchronize()
    args = (inp["q"], inp["k"], inp["v"])
    off64 = off.astype(np.float64)
    print("full oracle forward", flush=True)
    o_ref, lse_ref = oracle.sampled_forward(*args, off64, grid, window, wl.scale, mode)
    errs = {"out": assert_close(to_host_f64(out), o_ref, wl.dtype, "out"),
            "lse": assert_lse_close(lse.cpu().numpy(), lse_ref)}
    del o_ref, lse_ref
    print("full oracle backward", flush=True)
    refs = oracle.sampled_backward(*args, inp["dout"], off64, grid, window, wl.scale, mode)
    for nm, gpu, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), refs[:3]):
        errs[nm] = assert_close(to_host_f64(gpu), ref, wl.dtype, nm)
    g64, r64 = doff.cpu().numpy().astype(np.float64), np.asarray(refs[3], dtype=np.float64)
    assert g64.shape == r64.shape and np.isfinite(g64).all()
    excess = np.abs(g64 - r64) - (2e-2 + 1e-2 * np.abs(r64))
    i = np.unravel_index(np.argmax(excess), excess.shape)
    assert excess.max() <= 0, f"doffsets: err {abs(g64[i] - r64[i]):.3e} at {i}"
    errs["doffsets"] = float(np.abs(g64 - r64).max())
    print("max abs err", {k_: f"{v_:.2e}" for k_, v_ in errs.items()}, flush=True)


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_offset_predictor_benchmark_workload(dsa3d_gpu):
    """Bounds of the small predictor cases: convolution outputs 2^-22 taps S + 2^-8 |ref|,
    filter / bias gradients 2^-24 (N - 1) S; the pointwise layer's outputs 2^-22 K S (fp32),
    its input gradient (2^-22 O + 2^-8) S + 2^-8 |ref| (dy rounded to bf16 first, bf16
    output), weight gradient (2^-22 M + 2^-8) S, bias gradient 2^-22 M S."""
    wl = configs.S_FREE
    grid, N = (wl.F, wl.Hp, wl.Wp), wl.N
    C, O, taps = wl.heads * wl.head_dim, wl.heads * wl.K * 3, 27
    x = synth.normal(47, 0, (N, C), "bf16")
    w1 = synth.normal(47, 1, (C, 3, 3, 3), "f32", 0.1)
    b1 = synth.normal(47, 2, (C,), "f32")
    w2 = synth.normal(47, 3, (O, C), "bf16", 0.05)
    b2 = synth.normal(47, 4, (O,), "f32")
    dy = synth.normal(47, 5, (N, O), "f32")
    print(f"case predictor N={N} C={C} O={O}", flush=True)
    xd, w1d, w2d = to_dev(x), to_dev(w1), to_dev(w2)
    h = dsa3d_gpu.dwconv3d_forward(xd, w1d, to_dev(b1), grid)
    y = dsa3d_gpu.linear_forward(h, w2d, to_dev(b2))
    dh, dw2, db2 = dsa3d_gpu.linear_backward(h, w2d, to_dev(dy))
    dx, dw1, db1 = dsa3d_gpu.dwconv3d_backward(xd, w1d, dh, grid)
    torch.cuda.synchronize()
    xh, w2h = oracle.bf16_to_f64(x), oracle.bf16_to_f64(w2)
    errs = {}
    # depthwise convolution, every element
    ref = oracle.dwconv3d_forward(x, w1, b1, grid)
    S = oracle.dwconv3d_forward(np.abs(xh), np.abs(w1), np.abs(b1), grid)
    errs["h"] = _assert_bound(to_host_f64(h), ref, 2.0**-22 * taps * S + 2.0**-8 * np.abs(ref), "h")
    # pointwise layer on rows and columns, from the GPU's h and dh
    hh = to_host_f64(h)
    rows = border_and_random_rows((N, 1, 1), 1, 256, seed=5)
    cols = np.unique(np.concatenate([[0, O - 1], np.random.default_rng(6).integers(0, O, 62)]))
    ref = oracle.linear_forward(hh[rows], w2h, b2)
    S = np.abs(hh[rows]) @ np.abs(w2h).T + np.abs(b2)
    errs["y"] = _assert_bound(y[torch.as_tensor(rows, device="cuda")].cpu().numpy(), ref, 2.0**-22 * C * S, "y")
    rdh, _, _ = oracle.linear_backward(hh[rows], w2h, dy[rows])
    Sdh, _, _ = oracle.linear_backward(np.abs(hh[rows]), np.abs(w2h), np.abs(dy[rows]))
    errs["dh"] = _assert_bound(to_host_f64(dh)[rows], rdh, (2.0**-22 * O + 2.0**-8) * Sdh + 2.0**-8 * np.abs(rdh),
                               "dh")
    _, rdw2, rdb2 = oracle.linear_backward(hh, w2h[cols], np.ascontiguousarray(dy[:, cols]))
    _, Sdw2, Sdb2 = oracle.linear_backward(np.abs(hh), np.abs(w2h[cols]), np.abs(np.ascontiguousarray(dy[:, cols])))
    cold = torch.as_tensor(cols, device="cuda")
    errs["dw2"] = _assert_bound(to_host_f64(dw2[cold]), rdw2, (2.0**-22 * N + 2.0**-8) * Sdw2, "dweight2")
    errs["db2"] = _assert_bound(db2[cold].cpu().numpy(), rdb2, 2.0**-22 * N * Sdb2, "dbias2")
    # depthwise backward from the GPU's dh, every element
    dhh = dh.view(torch.int16).cpu().numpy().view(np.uint16)
    rdx, rdw1, rdb1 = oracle.dwconv3d_backward(x, w1, dhh, grid)
    Sx, Sw, Sb = oracle.dwconv3d_backward(np.abs(xh), np.abs(w1), np.abs(oracle.bf16_to_f64(dhh)), grid)
    errs["dx"] = _assert_bound(to_host_f64(dx), rdx, 2.0**-22 * taps * Sx + 2.0**-8 * np.abs(rdx), "dx")
    acc = 2.0**-24 * (N - 1)
    errs["dw1"] = _assert_bound(dw1.cpu().numpy(), rdw1, acc * Sw + 1e-30, "dweight1")
    errs["db1"] = _assert_bound(db1.cpu().numpy(), rdb1, acc * Sb + 1e-30, "dbias1")
    print("max abs err", {k_: f"{v_:.2e}" for k_, v_ in errs.items()}, flush=True)
