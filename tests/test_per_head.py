"""Per-head offsets (dsa3d_forward_heads / dsa3d_backward_heads): each head has its own
integer offsets [H][N][3].  The HIP path, through the C ABI, against the oracle's per-head
form element by element, on small and multi-work-item grids, along its three routes: all
heads bucketed together (workspace of dsa3d_workspace_bytes_heads), one head after the
other (the minimum workspace), and the per-group kernels; the first two bit for bit."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
from local_sparse_attention_amd import synth
from local_sparse_attention_amd.configs import Workload

from _gpu_helpers import assert_close, assert_lse_close, nan_like, to_dev, to_host_f64

pytestmark = pytest.mark.gpu


def W(name, F, Hp, Wp, H, D, kt, ky, kx, dtype, offsets, seed=21):
    return Workload(name, F, Hp, Wp, H, D, kt, ky, kx, dtype, True, seed, 1.0, offsets)


def head_offsets(wl):
    """int32 [H][N][3]: head h takes the workload's recipe with seed + 1000 h."""
    return np.stack([synth.make_offsets(replace(wl, seed=wl.seed + 1000 * h)) for h in range(wl.heads)])


CASES = [
    W("tiny-f32", 4, 8, 8, 3, 64, 3, 3, 3, "f32", ("uniform", -2, 2)),
    W("ragged-bf16", 6, 13, 10, 3, 128, 5, 9, 9, "bf16", ("blocks", 8, 3.0, False, 0.0)),
    W("3x7x7-bf16-64", 10, 20, 24, 4, 64, 3, 7, 7, "bf16", ("round_normal", 2.0, 4)),
    # 36 start slices over two query-side work items, drifting per-head motion fields
    W("5x9x9-drift-40f", 40, 24, 28, 4, 128, 5, 9, 9, "bf16", ("blocks", 8, 3.0, True, 8.0)),
    W("huge-and-clamped", 5, 9, 11, 2, 128, 3, 5, 5, "bf16", ("uniform", -40, 40)),
]


def run_heads(dsa3d_gpu, wl, q, k, v, do, off, route):
    """Forward + backward with per-head offsets along one route; returns (out, lse, dq, dk, dv)."""
    grid, window = (wl.F, wl.Hp, wl.Wp), (wl.kt, wl.ky, wl.kx)
    generic = route == "generic"
    wsf = wsb = None
    if route == "per-head":  # the minimum workspace: one head after the other
        wsf = dsa3d_gpu.workspace(grid, wl.heads, window, False)
        wsb = dsa3d_gpu.workspace(grid, wl.heads, window, True)
    out, lse = dsa3d_gpu.forward(q, k, v, off, grid, window, wl.scale, out=nan_like(q),
                                 lse=torch.full((wl.heads, wl.N), float("nan"), device="cuda"), ws=wsf,
                                 generic=generic)
    dq, dk, dv = dsa3d_gpu.backward(q, k, v, off, out, lse, do, grid, window, wl.scale, dq=nan_like(q),
                                    dk=nan_like(q), dv=nan_like(q), ws=wsb, generic=generic)
    torch.cuda.synchronize()
    return out, lse, dq, dk, dv


ROUTES = ["together", "per-head", "generic"]


@pytest.mark.parametrize("route", ROUTES)
@pytest.mark.parametrize("wl", CASES, ids=[w.name for w in CASES])
def test_per_head_offsets(dsa3d_gpu, wl, route):
    grid, window = (wl.F, wl.Hp, wl.Wp), (wl.kt, wl.ky, wl.kx)
    print(f"case {wl.name} grid={grid} window={window} H={wl.heads} route={route}", flush=True)
    inp = synth.make_inputs(wl)
    offh = head_offsets(wl)
    assert not all(np.array_equal(offh[0], offh[h]) for h in range(1, wl.heads))
    q, k, v, do = (to_dev(inp[x]) for x in ("q", "k", "v", "dout"))
    off = to_dev(offh)
    out, lse, dq, dk, dv = run_heads(dsa3d_gpu, wl, q, k, v, do, off, route)
    o_ref, lse_ref = oracle.forward_heads(inp["q"], inp["k"], inp["v"], offh, grid, window, wl.scale)
    errs = {"out": assert_close(to_host_f64(out), o_ref, wl.dtype, "out"),
            "lse": assert_lse_close(lse.cpu().numpy(), lse_ref)}
    refs = oracle.backward_heads(inp["q"], inp["k"], inp["v"], inp["dout"], offh, grid, window, wl.scale)
    for name, gpu, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
        errs[name] = assert_close(to_host_f64(gpu), ref, wl.dtype, name)
    print("max abs err", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)


def test_per_head_deterministic(dsa3d_gpu):
    wl = CASES[3]
    grid, window = (wl.F, wl.Hp, wl.Wp), (wl.kt, wl.ky, wl.kx)
    inp = synth.make_inputs(wl)
    q, k, v, do = (to_dev(inp[x]) for x in ("q", "k", "v", "dout"))
    off = to_dev(head_offsets(wl))
    runs = []
    for _ in range(2):
        out, lse = dsa3d_gpu.forward(q, k, v, off, grid, window, wl.scale)
        grads = dsa3d_gpu.backward(q, k, v, off, out, lse, do, grid, window, wl.scale)
        torch.cuda.synchronize()
        runs.append([out.view(torch.int16), lse.view(torch.int32)] + [g.view(torch.int16) for g in grads])
    for a, b in zip(*runs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("wl", [c for c in CASES if c.dtype == "bf16"], ids=[c.name for c in CASES if c.dtype == "bf16"])
def test_per_head_together_equals_one_by_one(dsa3d_gpu, wl):
    """All heads bucketed together and one head after the other give the same bits: the
    head-major sort keeps each head's queries in the order of its own sort."""
    print(f"case {wl.name}", flush=True)
    inp = synth.make_inputs(wl)
    q, k, v, do = (to_dev(inp[x]) for x in ("q", "k", "v", "dout"))
    off = to_dev(head_offsets(wl))
    a = run_heads(dsa3d_gpu, wl, q, k, v, do, off, "together")
    b = run_heads(dsa3d_gpu, wl, q, k, v, do, off, "per-head")
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32),
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32))
