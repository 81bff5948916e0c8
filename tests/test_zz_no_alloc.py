"""dsa3d_forward_static, the forward that allocates nothing (its scratch is the library's
static device array), called through the C ABI against dsa3d_forward on the same inputs:
the same kernels run on the same data, so the outputs must be bit-identical.  Two calls in a
row, the second on a smaller grid, so the second reads an array that still holds the first
call's contents."""
import ctypes

import numpy as np
import pytest
import torch

from local_sparse_attention_amd import configs, synth
from local_sparse_attention_amd.configs import Workload

from _gpu_helpers import nan_like, to_dev

pytestmark = pytest.mark.gpu

STATIC_BYTES = 64 * 1024 * 1024  # DSA3D_STATIC_SCRATCH_BYTES
ERR_SCRATCH = -11


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def call_static(lib, wl, dev):
    q, k, v, off = dev["q"], dev["k"], dev["v"], dev["offsets"]
    out = nan_like(q)
    lse = torch.full((wl.heads, wl.N), float("nan"), device=q.device)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = lib.dsa3d_forward_static(q.data_ptr(), k.data_ptr(), v.data_ptr(), off.data_ptr(), wl.F, wl.Hp, wl.Wp,
                                  wl.heads, wl.head_dim, wl.kt, wl.ky, wl.kx, wl.scale, 1 if wl.dtype == "bf16" else 0,
                                  out.data_ptr(), lse.data_ptr(), stream)
    assert rc == 0, rc
    return out, lse


CASES = [
    # large first: 16 x 32 x 32 tokens, window 3 x 7 x 7 (frame-sweeping kernels)
    configs.C2,
    # then a smaller, ragged grid with another window and head count
    Workload("small-ragged", 6, 13, 10, 3, 128, 5, 9, 9, "bf16", False, 11, 1.0, ("blocks", 8, 3.0, False, 0.0)),
]


def test_forward_static_matches_forward_twice(dsa3d_gpu):
    lib = dsa3d_gpu.load()
    for wl in CASES:
        grid, window = (wl.F, wl.Hp, wl.Wp), (wl.kt, wl.ky, wl.kx)
        need = dsa3d_gpu.workspace_bytes(grid, wl.heads, window, False)
        print(f"case {wl.name}: scratch {need} of {STATIC_BYTES} bytes", flush=True)
        assert 0 < need <= STATIC_BYTES
        inp = synth.make_inputs(wl, with_dout=False)
        dev = {x: to_dev(inp[x]) for x in ("q", "k", "v", "offsets")}
        out_s, lse_s = call_static(lib, wl, dev)
        out_r, lse_r = dsa3d_gpu.forward(dev["q"], dev["k"], dev["v"], dev["offsets"], grid, window, wl.scale,
                                         out=nan_like(dev["q"]),
                                         lse=torch.full((wl.heads, wl.N), float("nan"), device="cuda"))
        torch.cuda.synchronize()
        assert torch.isfinite(out_s.float()).all() and torch.isfinite(lse_s).all()
        assert torch.equal(bits(out_s), bits(out_r)), wl.name
        assert torch.equal(bits(lse_s), bits(lse_r)), wl.name


def test_forward_static_rejects_oversize_geometry(dsa3d_gpu):
    lib = dsa3d_gpu.load()
    wl = configs.C5  # about 168 MiB of scratch
    assert dsa3d_gpu.workspace_bytes((wl.F, wl.Hp, wl.Wp), wl.heads, (wl.kt, wl.ky, wl.kx), False) > STATIC_BYTES
    P = 1 << 20  # never dereferenced: the size check comes before any launch
    rc = lib.dsa3d_forward_static(P, P, P, P, wl.F, wl.Hp, wl.Wp, wl.heads, wl.head_dim, wl.kt, wl.ky, wl.kx, wl.scale,
                                  1, P, P, None)
    assert rc == ERR_SCRATCH
