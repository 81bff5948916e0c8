"""HIP path (through the C ABI) against the CPU oracle, element by element, on seeded
inputs: the tiny fp32 workload, the bf16 forward workload, and edge cases (ragged tiles,
window = grid, F = kt, 1x1x1 windows, clamped and huge offsets, one token, zero
offsets), all small enough for the full oracle."""
import sys

import numpy as np
import pytest
import torch

import oracle
from local_sparse_attention_amd import configs, synth
from local_sparse_attention_amd.configs import Workload

from _gpu_helpers import assert_close, assert_lse_close, nan_like, to_dev, to_host_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(params=["default", "generic"])
def kernels(request):
    """Run each case through the default kernels (frame-sweeping where the window allows)
    and through the per-group kernels that serve every geometry (DSA3D_FLAG_GENERIC_KERNELS)."""
    return request.param == "generic"


def run_case(dsa3d, wl, inp, backward=True, generic=False):
    grid, window = (wl.F, wl.Hp, wl.Wp), (wl.kt, wl.ky, wl.kx)
    print(f"case {wl.name} grid={grid} window={window} H={wl.heads} D={wl.head_dim} {wl.dtype} "
          f"generic={generic}", flush=True)
    q, k, v, off = (to_dev(inp[x]) for x in ("q", "k", "v", "offsets"))
    # outputs start as NaN: an element the library leaves unwritten fails the comparison
    out, lse = dsa3d.forward(q, k, v, off, grid, window, wl.scale, out=nan_like(q),
                             lse=torch.full((q.shape[1], q.shape[0]), float("nan"), device=q.device),
                             generic=generic)
    res = {"out": out, "lse": lse}
    if backward:
        do = to_dev(inp["dout"])
        res["dq"], res["dk"], res["dv"] = dsa3d.backward(q, k, v, off, out, lse, do, grid, window, wl.scale,
                                                         dq=nan_like(q), dk=nan_like(q), dv=nan_like(q),
                                                         generic=generic)
    torch.cuda.synchronize()
    return res


def check_full(dsa3d, wl, inp=None, backward=True, generic=False):
    inp = inp if inp is not None else synth.make_inputs(wl, with_dout=backward)
    res = run_case(dsa3d, wl, inp, backward, generic)
    grid, window = (wl.F, wl.Hp, wl.Wp), (wl.kt, wl.ky, wl.kx)
    o_ref, lse_ref = oracle.forward(inp["q"], inp["k"], inp["v"], inp["offsets"], grid, window, wl.scale)
    errs = {"out": assert_close(to_host_f64(res["out"]), o_ref, wl.dtype, "out"),
            "lse": assert_lse_close(res["lse"].cpu().numpy(), lse_ref)}
    if backward:
        refs = oracle.backward(inp["q"], inp["k"], inp["v"], inp["dout"], inp["offsets"], grid, window, wl.scale)
        for name, ref in zip(("dq", "dk", "dv"), refs):
            errs[name] = assert_close(to_host_f64(res[name]), ref, wl.dtype, name)
    print("max abs err", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    return res, inp


def test_tiny_fp32_workload(dsa3d_gpu, kernels):
    check_full(dsa3d_gpu, configs.C1, generic=kernels)


def test_bf16_forward_workload(dsa3d_gpu, kernels):
    check_full(dsa3d_gpu, configs.C2, backward=False, generic=kernels)


def test_bf16_forward_workload_backward_too(dsa3d_gpu, kernels):
    # the forward workload's shapes through the backward as well (dO from its stream)
    check_full(dsa3d_gpu, configs.C2.with_frames(6), backward=True, generic=kernels)


def W(name, F, Hp, Wp, H, D, kt, ky, kx, dtype, offsets, seed=11, scale=1.0):
    return Workload(name, F, Hp, Wp, H, D, kt, ky, kx, dtype, True, seed, scale, offsets)


EDGE = [
    W("ragged-blocks-bf16-128", 6, 13, 10, 3, 128, 5, 9, 9, "bf16", ("blocks", 8, 3.0, False, 0.0)),
    W("ragged-blocks-f32-128", 4, 11, 14, 2, 128, 3, 5, 7, "f32", ("blocks", 4, 2.0, True, 6.0)),
    W("window-is-grid-f32", 3, 5, 7, 2, 64, 3, 5, 7, "f32", ("uniform", -4, 4)),
    W("window-is-grid-bf16", 3, 5, 7, 2, 128, 3, 5, 7, "bf16", ("uniform", -4, 4)),
    W("F-equals-kt", 3, 12, 12, 4, 64, 3, 5, 5, "bf16", ("round_normal", 2.0, 4)),
    W("one-voxel-window", 5, 9, 11, 2, 128, 1, 1, 1, "bf16", ("uniform", -6, 6)),
    W("one-voxel-window-f32", 5, 9, 11, 2, 64, 1, 1, 1, "f32", ("uniform", -6, 6)),
    W("single-token", 1, 1, 1, 1, 64, 1, 1, 1, "f32", ("uniform", -3, 3)),
    W("zero-offsets-fixed-3x7x7", 6, 16, 16, 2, 64, 3, 7, 7, "bf16", ("zero",)),
    W("thin-axis", 7, 1, 37, 3, 64, 3, 1, 5, "f32", ("uniform", -3, 3)),
    W("odd-heads-f32-64", 5, 10, 9, 5, 64, 3, 3, 3, "f32", ("round_normal", 3.0, 6)),
    W("long-window-t", 9, 6, 6, 2, 128, 9, 3, 3, "bf16", ("uniform", -2, 2)),
    W("kt5-9x9-drift", 14, 21, 26, 2, 128, 5, 9, 9, "bf16", ("blocks", 8, 3.0, True, 8.0)),
    W("kt7-5x3-f32", 9, 11, 7, 2, 64, 7, 5, 3, "f32", ("round_normal", 2.0, 5)),
    W("crowded-slices", 8, 12, 12, 2, 128, 3, 9, 9, "bf16", ("uniform", -9, 9)),
    # few key-block columns x heads: the key-centric backward splits time into runs of
    # 5 (8 runs) and 8 frames (4 runs, kt = 7 > half a run)
    W("many-runs-kt3", 40, 9, 10, 2, 128, 3, 9, 9, "bf16", ("blocks", 4, 2.0, True, 4.0)),
    W("many-runs-kt7", 30, 8, 8, 2, 64, 7, 5, 5, "bf16", ("round_normal", 2.0, 4)),
]


@pytest.mark.parametrize("wl", EDGE, ids=[w.name for w in EDGE])
def test_edge_cases(dsa3d_gpu, wl, kernels):
    check_full(dsa3d_gpu, wl, generic=kernels)


def test_huge_offsets_pile_on_borders(dsa3d_gpu, kernels):
    """Offsets far past the grid: every window clamps to a border, so a few start cells
    hold most queries (long CSR buckets in the key-centric pass)."""
    wl = W("huge-offsets", 3, 17, 19, 2, 64, 3, 7, 7, "bf16", ("uniform", -2, 2), seed=5)
    inp = synth.make_inputs(wl)
    g = np.random.default_rng(0)
    big = np.array([-(2**31), -(10**9), -40, 40, 10**9, 2**31 - 1], dtype=np.int64)
    inp["offsets"] = big[g.integers(0, len(big), size=inp["offsets"].shape)].astype(np.int32)
    check_full(dsa3d_gpu, wl, inp, generic=kernels)


def test_window_starts_bit_exact(dsa3d_gpu):
    for wl in (configs.C1, configs.C3, configs.C5.with_frames(12)):
        off = synth.make_offsets(wl)
        off[:6] = [[2**31 - 1, -(2**31), 0], [-(2**31), 2**31 - 1, 7], [10**9, -(10**9), 3], [0, 0, 0],
                   [wl.F, -wl.Hp, wl.Wp], [-wl.F - 1, wl.Hp + 1, -wl.Wp - 1]]
        grid, window = (wl.F, wl.Hp, wl.Wp), (wl.kt, wl.ky, wl.kx)
        gpu = dsa3d_gpu.window_starts(to_dev(off), grid, window).cpu().numpy()
        assert np.array_equal(gpu, oracle.window_starts(off, grid, window)), wl.name


def test_deterministic_across_calls_and_streams(dsa3d_gpu, kernels):
    wl = configs.C3.with_frames(6)
    inp = synth.make_inputs(wl)
    a = run_case(dsa3d_gpu, wl, inp, generic=kernels)
    b = run_case(dsa3d_gpu, wl, inp, generic=kernels)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        c = run_case(dsa3d_gpu, wl, inp, generic=kernels)
    s.synchronize()
    for name in a:
        assert torch.equal(a[name].view(torch.int16) if a[name].dtype == torch.bfloat16 else a[name],
                           b[name].view(torch.int16) if b[name].dtype == torch.bfloat16 else b[name]), name
        assert torch.equal(a[name].view(torch.int16) if a[name].dtype == torch.bfloat16 else a[name],
                           c[name].view(torch.int16) if c[name].dtype == torch.bfloat16 else c[name]), name


def test_autograd_wrapper(dsa3d_gpu):
    wl = configs.C1
    inp = synth.make_inputs(wl)
    grid, window = (wl.F, wl.Hp, wl.Wp), (wl.kt, wl.ky, wl.kx)
    q, k, v = (to_dev(inp[x]).requires_grad_(True) for x in ("q", "k", "v"))
    off = to_dev(inp["offsets"])
    o = dsa3d_gpu.dsa3d_attention(q, k, v, off, grid, window)
    o.backward(to_dev(inp["dout"]))
    refs = oracle.backward(inp["q"], inp["k"], inp["v"], inp["dout"], inp["offsets"], grid, window, wl.scale)
    for t, ref, name in zip((q, k, v), refs, ("dq", "dk", "dv")):
        assert_close(to_host_f64(t.grad), ref, "f32", name)
