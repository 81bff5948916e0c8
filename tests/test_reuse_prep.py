"""DSA3D_FLAG_REUSE_PREP: a backward that takes the window starts, buckets and query-side
schedules the forward just built in the same workspace gives the same bits as a backward
that builds them itself -- with shared offsets on the frame-sweeping and the per-group
kernels, in fp32 and bf16, and with per-head offsets on the all-heads-together route and on
the one-head-at-a-time route (which ignores the flag)."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from local_sparse_attention_amd import synth
from local_sparse_attention_amd.configs import Workload

from _gpu_helpers import nan_like, to_dev

pytestmark = pytest.mark.gpu


def W(name, F, Hp, Wp, H, D, kt, ky, kx, dtype, offsets, seed=71):
    return Workload(name, F, Hp, Wp, H, D, kt, ky, kx, dtype, True, seed, 1.0, offsets)


CASES = [
    (W("5x9x9-drift-40f-bf16", 40, 24, 28, 4, 128, 5, 9, 9, "bf16", ("blocks", 8, 3.0, True, 8.0)), False),
    (W("3x7x7-bf16-generic", 10, 20, 24, 2, 64, 3, 7, 7, "bf16", ("round_normal", 2.0, 4)), True),
    (W("3x3x3-f32", 6, 12, 14, 2, 64, 3, 3, 3, "f32", ("uniform", -3, 3)), False),
]


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def fwd_bwd(dsa3d, wl, q, k, v, do, off, ws, generic, reuse):
    grid, window = (wl.F, wl.Hp, wl.Wp), (wl.kt, wl.ky, wl.kx)
    out, lse = dsa3d.forward(q, k, v, off, grid, window, wl.scale, out=nan_like(q),
                             lse=torch.full((wl.heads, wl.N), float("nan"), device="cuda"), ws=ws, generic=generic)
    dq, dk, dv = dsa3d.backward(q, k, v, off, out, lse, do, grid, window, wl.scale, dq=nan_like(q), dk=nan_like(q),
                                dv=nan_like(q), ws=ws, generic=generic, reuse_prep=reuse)
    torch.cuda.synchronize()
    return out, lse, dq, dk, dv


def check_same(a, b):
    for name, x, y in zip(("out", "lse", "dq", "dk", "dv"), a, b):
        assert torch.equal(bits(x), bits(y)), name
        assert torch.isfinite(x.float()).all(), name


@pytest.mark.parametrize("wl,generic", CASES, ids=[c[0].name for c in CASES])
def test_reuse_prep_shared_offsets(dsa3d_gpu, wl, generic):
    grid, window = (wl.F, wl.Hp, wl.Wp), (wl.kt, wl.ky, wl.kx)
    print(f"case {wl.name} generic={generic}", flush=True)
    inp = synth.make_inputs(wl)
    q, k, v, do, off = (to_dev(inp[x]) for x in ("q", "k", "v", "dout", "offsets"))
    ws = dsa3d_gpu.workspace(grid, wl.heads, window, True)
    plain = fwd_bwd(dsa3d_gpu, wl, q, k, v, do, off, ws, generic, False)
    ws.fill_(0xA5)  # nothing left over from the plain run
    reused = fwd_bwd(dsa3d_gpu, wl, q, k, v, do, off, ws, generic, True)
    check_same(plain, reused)


@pytest.mark.parametrize("together", [True, False], ids=["together", "one-by-one"])
def test_reuse_prep_per_head(dsa3d_gpu, together):
    wl = CASES[0][0]
    grid, window = (wl.F, wl.Hp, wl.Wp), (wl.kt, wl.ky, wl.kx)
    inp = synth.make_inputs(wl)
    offh = np.stack([synth.make_offsets(replace(wl, seed=wl.seed + 1000 * h)) for h in range(wl.heads)])
    q, k, v, do = (to_dev(inp[x]) for x in ("q", "k", "v", "dout"))
    off = to_dev(offh)
    ws = (dsa3d_gpu.workspace(grid, wl.heads, window, True, per_head=True) if together
          else dsa3d_gpu.workspace(grid, wl.heads, window, True))
    plain = fwd_bwd(dsa3d_gpu, wl, q, k, v, do, off, ws, False, False)
    ws.fill_(0xA5)
    reused = fwd_bwd(dsa3d_gpu, wl, q, k, v, do, off, ws, False, True)
    check_same(plain, reused)
