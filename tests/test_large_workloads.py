"""Parity at the full sizes of the 720p-like, full-width and 256-frame workloads, in the
launch configuration the benchmark times: sampled outputs (grid corners, edge centres and
random rows) against the oracle computed row by row, plus properties that hold at any
size, checked over every output.

Properties (P = softmax weights of a query, rows sum to one; dS rows sum to zero):
  sum_j dV[j,h] = sum_n dO[n,h]        sum_j dK[j,h] = 0        all outputs finite.
"""
import numpy as np
import pytest
import torch

import oracle
from local_sparse_attention_amd import configs, synth

from _gpu_helpers import assert_close, assert_lse_close, border_and_random_rows, gather_rows, nan_like, to_dev

pytestmark = pytest.mark.gpu

SAMPLES = {"C3": (1024, 256), "C4": (512, 96), "C5": (512, 96)}


def run_sampled(dsa3d, name):
    wl = configs.ALL[name]
    grid, window = (wl.F, wl.Hp, wl.Wp), (wl.kt, wl.ky, wl.kx)
    print(f"case {wl.name}: generating inputs N={wl.N} H={wl.heads} D={wl.head_dim}", flush=True)
    inp = synth.make_inputs(wl)
    q, k, v, do, off = (to_dev(inp[x]) for x in ("q", "k", "v", "dout", "offsets"))
    print(f"case {wl.name}: forward + backward on the GPU", flush=True)
    # outputs start as NaN: an element the library leaves unwritten fails the checks
    out, lse = dsa3d.forward(q, k, v, off, grid, window, wl.scale, out=nan_like(q),
                             lse=torch.full((q.shape[1], q.shape[0]), float("nan"), device=q.device))
    dq, dk, dv = dsa3d.backward(q, k, v, off, out, lse, do, grid, window, wl.scale, dq=nan_like(q), dk=nan_like(q),
                                dv=nan_like(q))
    torch.cuda.synchronize()

    nq, nk = SAMPLES[name]
    qrows = border_and_random_rows(grid, wl.heads, nq, seed=1)
    krows = border_and_random_rows(grid, wl.heads, nk, seed=2)
    args = (inp["q"], inp["k"], inp["v"])
    print(f"case {wl.name}: oracle on {len(qrows)} query rows and {len(krows)} key rows", flush=True)
    o_ref, lse_ref = oracle.forward_rows(*args, inp["offsets"], grid, window, wl.scale, qrows)
    assert_close(gather_rows(out, qrows), o_ref, wl.dtype, "out")
    lse_g = lse.T.reshape(-1)[torch.as_tensor(qrows, device=lse.device)].cpu().numpy()
    assert_lse_close(lse_g, lse_ref)
    dq_ref = oracle.backward_q_rows(*args, inp["dout"], inp["offsets"], grid, window, wl.scale, qrows)
    assert_close(gather_rows(dq, qrows), dq_ref, wl.dtype, "dq")
    dk_ref, dv_ref = oracle.backward_kv_rows(*args, inp["dout"], inp["offsets"], grid, window, wl.scale, krows)
    assert_close(gather_rows(dk, krows), dk_ref, wl.dtype, "dk")
    assert_close(gather_rows(dv, krows), dv_ref, wl.dtype, "dv")

    # properties over every output, per head, in float64 on the device
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


def test_720p_like_workload(dsa3d_gpu):
    run_sampled(dsa3d_gpu, "C3")


@pytest.mark.slow
def test_full_width_workload(dsa3d_gpu):
    run_sampled(dsa3d_gpu, "C4")


@pytest.mark.slow
def test_256_frame_workload(dsa3d_gpu):
    run_sampled(dsa3d_gpu, "C5")
