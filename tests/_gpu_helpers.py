"""Helpers for the GPU parity tests: host <-> device copies of the generator's arrays,
the tolerance check, and row sampling for workloads too large for the full oracle."""
import numpy as np
import torch

from local_sparse_attention_amd import synth

# fp32 inputs: max |gpu - oracle| <= 1e-5.  bf16 inputs (fp32 accumulation):
# |gpu - oracle| <= 2e-2 + 1e-2 * |oracle| elementwise.
F32_ATOL = 1e-5
BF16_ATOL, BF16_RTOL = 2e-2, 1e-2


def to_dev(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def nan_like(t):
    """An output buffer shaped like t, filled with NaN (unwritten elements stay visible)."""
    return torch.full_like(t, float("nan"))


def to_host_f64(t):
    if t.dtype == torch.bfloat16:
        return synth.bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def assert_close(gpu, ref, dtype, what):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.isfinite(gpu).all(), f"{what}: non-finite values"
    err = np.abs(gpu - ref)
    if dtype == "f32":
        i = np.unravel_index(np.argmax(err), err.shape)
        assert err.max() <= F32_ATOL, f"{what}: max abs err {err.max():.3e} at {i} (gpu {gpu[i]}, oracle {ref[i]})"
    else:
        excess = err - (BF16_ATOL + BF16_RTOL * np.abs(ref))
        i = np.unravel_index(np.argmax(excess), excess.shape)
        assert excess.max() <= 0, f"{what}: err {err[i]:.3e} over tolerance at {i} (gpu {gpu[i]}, oracle {ref[i]})"
    return float(err.max())


# The log-sum-exp is an fp32 output computed from fp32 logits even for bf16 inputs, so
# it is checked tightly for every dtype: a dropped or stale product shows up there.
LSE_ATOL = 1e-4


def assert_lse_close(gpu, ref, what="lse"):
    err = np.abs(np.asarray(gpu, dtype=np.float64) - np.asarray(ref, dtype=np.float64))
    i = np.unravel_index(np.argmax(err), err.shape)
    assert err.max() <= LSE_ATOL, f"{what}: max abs err {err.max():.3e} at {i}"
    return float(err.max())


def border_and_random_rows(grid, heads, count, seed):
    """Query (or key) rows r = n*H + h: every corner and edge-centre token of the grid
    with random heads, plus random rows."""
    F, Hp, Wp = grid
    g = np.random.default_rng(seed)
    toks = []
    for t in (0, F // 2, F - 1):
        for y in (0, Hp // 2, Hp - 1):
            for x in (0, Wp // 2, Wp - 1):
                toks.append((t * Hp + y) * Wp + x)
    toks = np.array(sorted(set(toks)), dtype=np.int64)
    rows = toks * heads + g.integers(0, heads, len(toks))
    extra = g.integers(0, F * Hp * Wp * heads, max(count - len(rows), 0))
    return np.unique(np.concatenate([rows, extra]))


def gather_rows(t, rows):
    """Rows r = n*H + h of a device [N][H][D] tensor, as float64 host [R][D]."""
    N, H, D = t.shape
    idx = torch.as_tensor(rows, device=t.device)
    return to_host_f64(t.reshape(N * H, D).index_select(0, idx))
