"""Sampled windows (real offsets, trilinear sampling, offset gradients): the HIP path
through the C ABI against the oracle's sampled form, element by element.

Box windows with one real offset per query (shared by heads) or per (query, head), and
free per-sample offsets, some of them leaving the grid (zero padding), for fp32 and bf16,
head_dim 64 and 128; box windows up to and past the largest lattice of corner rows that the
box kernels hold per wave.  Also: box windows with integer-valued offsets equal the integer
path, and the backward is bitwise reproducible.

Tolerances: O, LSE, dQ, dK, dV as everywhere (fp32 1e-5 absolute; bf16 2e-2 + 1e-2|ref|;
LSE 1e-4).  The offset gradient is an fp32 output for both input dtypes; it sums up to
heads x samples x 8 corner terms, each carrying fp32 rounding of relative size ~2^-24 on
the product scale*dz*(q.k), so it is checked at 1e-4 + 1e-4 |ref| (fp32 inputs) and at the
bf16 form (bf16 inputs, where the inputs to the oracle are the same bf16 values)."""
import numpy as np
import pytest
import torch

import oracle
from local_sparse_attention_amd import synth
from local_sparse_attention_amd.configs import Workload

from _gpu_helpers import assert_close, assert_lse_close, nan_like, to_dev, to_host_f64

pytestmark = pytest.mark.gpu


def W(name, F, Hp, Wp, H, D, kt, ky, kx, dtype, seed=31):
    return Workload(name, F, Hp, Wp, H, D, kt, ky, kx, dtype, True, seed, 1.0, ("zero",))


def real_offsets(wl, mode, kind, sigma, seed):
    """float32 offsets, N(0, sigma) per component (seeded generator stream 7)."""
    N, H, K = wl.N, wl.heads, wl.K
    shape = {("box", "query"): (N, 1, 3), ("box", "head"): (N, H, 3), ("free", "sample"): (N, H, K, 3),
             ("free", "query"): (N, 1, 1, 3), ("box", "head-major"): (H, N, 3)}[(mode, kind)]
    return synth.normal(seed, 7, shape, "f32", sigma)


CASES = [
    (W("box-query-f32", 5, 9, 10, 2, 64, 3, 5, 5, "f32"), "box", "query", 2.0),
    (W("box-query-bf16", 6, 12, 14, 3, 128, 3, 7, 7, "bf16"), "box", "query", 2.5),
    (W("box-head-bf16", 5, 10, 12, 4, 64, 3, 5, 5, "bf16"), "box", "head", 3.0),
    (W("box-head-major-f32", 4, 8, 9, 3, 128, 3, 3, 3, "f32"), "box", "head-major", 1.5),
    (W("box-one-frame-f32", 5, 9, 11, 2, 64, 1, 3, 5, "f32"), "box", "query", 2.0),
    # the largest lattice the box kernels take ((kt+1)(ky+1)(kx+1) = 1024), and one past it,
    # which runs the per-sample corner kernels
    (W("box-lattice-1024-bf16", 5, 16, 17, 1, 64, 3, 15, 15, "bf16"), "box", "head", 3.0),
    (W("box-lattice-1536-bf16", 6, 16, 17, 1, 64, 5, 15, 15, "bf16"), "box", "query", 3.0),
    (W("free-sample-f32", 4, 7, 8, 2, 64, 3, 3, 3, "f32"), "free", "sample", 1.5),
    (W("free-sample-bf16", 5, 10, 12, 3, 128, 3, 5, 5, "bf16"), "free", "sample", 1.2),
    (W("free-query-bf16-64", 4, 9, 11, 2, 64, 3, 3, 5, "bf16"), "free", "query", 2.0),
    # the pages' 3 x 7 x 7 window, per-sample offsets, several key-side cells per key
    (W("free-3x7x7-bf16", 8, 16, 18, 4, 128, 3, 7, 7, "bf16"), "free", "sample", 1.0),
]


def check_doff(gpu, ref, dtype, what="doffsets"):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape and np.isfinite(gpu).all()
    err = np.abs(gpu - ref)
    atol, rtol = (1e-4, 1e-4) if dtype == "f32" else (2e-2, 1e-2)
    excess = err - (atol + rtol * np.abs(ref))
    i = np.unravel_index(np.argmax(excess), excess.shape)
    assert excess.max() <= 0, f"{what}: err {err[i]:.3e} at {i} (gpu {gpu[i]}, oracle {ref[i]})"
    return float(err.max())


def run(dsa3d, wl, off_host, mode, head_major=False):
    grid, window = (wl.F, wl.Hp, wl.Wp), (wl.kt, wl.ky, wl.kx)
    inp = synth.make_inputs(wl)
    q, k, v, do = (to_dev(inp[x]) for x in ("q", "k", "v", "dout"))
    off = to_dev(off_host)
    if head_major:
        off = off.permute(1, 0, 2)  # [N, H, 3] view of [H, N, 3] storage
    out, lse = dsa3d.sampled_forward(q, k, v, off, grid, window, mode, wl.scale, out=nan_like(q),
                                     lse=torch.full((wl.heads, wl.N), float("nan"), device="cuda"))
    dq, dk, dv, doff = dsa3d.sampled_backward(q, k, v, off, out, lse, do, grid, window, mode, wl.scale)
    torch.cuda.synchronize()
    return inp, (out, lse, dq, dk, dv, doff)


@pytest.mark.parametrize("case", CASES, ids=[c[0].name for c in CASES])
def test_sampled_parity(dsa3d_gpu, case):
    wl, mode, kind, sigma = case
    grid, window = (wl.F, wl.Hp, wl.Wp), (wl.kt, wl.ky, wl.kx)
    print(f"case {wl.name} grid={grid} window={window} H={wl.heads} D={wl.head_dim} {mode}/{kind}", flush=True)
    off_host = real_offsets(wl, mode, kind, sigma, wl.seed)
    head_major = kind == "head-major"
    inp, (out, lse, dq, dk, dv, doff) = run(dsa3d_gpu, wl, off_host, mode, head_major)
    off_ref = np.transpose(off_host, (1, 0, 2)) if head_major else off_host
    args = (inp["q"], inp["k"], inp["v"])
    o_ref, lse_ref = oracle.sampled_forward(*args, off_ref.astype(np.float64), grid, window, wl.scale, mode)
    errs = {"out": assert_close(to_host_f64(out), o_ref, wl.dtype, "out"),
            "lse": assert_lse_close(lse.cpu().numpy(), lse_ref)}
    refs = oracle.sampled_backward(*args, inp["dout"], off_ref.astype(np.float64), grid, window, wl.scale, mode)
    for name, gpu, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), refs[:3]):
        errs[name] = assert_close(to_host_f64(gpu), ref, wl.dtype, name)
    d = doff.permute(1, 0, 2) if head_major else doff
    errs["doffsets"] = check_doff(d.cpu().numpy(), np.transpose(refs[3], (1, 0, 2)) if head_major else refs[3],
                                  wl.dtype)
    print("max abs err", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)


def test_box_with_integer_offsets_equals_integer_path(dsa3d_gpu):
    wl = W("box-int", 6, 12, 14, 3, 128, 3, 7, 7, "bf16", seed=5)
    grid, window = (wl.F, wl.Hp, wl.Wp), (wl.kt, wl.ky, wl.kx)
    inp = synth.make_inputs(wl)
    offi = np.random.default_rng(0).integers(-6, 7, size=(wl.N, 3)).astype(np.int32)
    q, k, v = (to_dev(inp[x]) for x in ("q", "k", "v"))
    o_int, lse_int = dsa3d_gpu.forward(q, k, v, to_dev(offi), grid, window, wl.scale)
    o_s, lse_s = dsa3d_gpu.sampled_forward(q, k, v, to_dev(offi.astype(np.float32)[:, None, :]), grid, window, "box",
                                           wl.scale)
    torch.cuda.synchronize()
    # both are the same windows; the integer path rounds the weights to bf16 before P V
    assert_close(to_host_f64(o_s), to_host_f64(o_int), "bf16", "out")
    assert_lse_close(lse_s.cpu().numpy(), lse_int.cpu().numpy())


def test_sampled_backward_deterministic(dsa3d_gpu):
    wl, mode, kind, sigma = CASES[-1]
    off_host = real_offsets(wl, mode, kind, sigma, wl.seed)
    runs = [run(dsa3d_gpu, wl, off_host, mode)[1] for _ in range(2)]
    for a, b in zip(*runs):
        a = a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32)
        b = b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)
        assert torch.equal(a, b)
