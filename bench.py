"""Benchmark of the 3D-DSA hot path on one MI355X: forward + backward (window-start
bucketing, attention forward, dQ, dK/dV) on the 256-frame workload (grid 256 x 68 x 120,
N = 2,088,960 tokens, a 16-head slice of head_dim 128, window 5 x 9 x 9, bf16, smooth
drifting motion field), inputs resident in HBM.

One step = dsa3d_forward + dsa3d_backward over the whole grid, on one workspace: the forward
builds the window starts, buckets and query-side schedules, and the backward uses them
(DSA3D_FLAG_REUSE_PREP), as a training step does; it builds its own key-side work lists and
Delta.  Prints one JSON line.
  phases_ms  per step, from HIP events the library records on its stream: bucketing
             and work lists (the backward's: key-side lists + Delta), then each attention
             kernel
  value      query-token-heads per second (N * heads / step time)
  roofline   the dominant kernel's algorithmic bytes per launch / its mean duration,
             timed with HIP events on the library's stream, against 8 TB/s HBM (and
             against the measured streaming-read peak)
  cpu_baseline  the CPU oracle (fp64, OpenMP) on the first 5 frames of the same workload,
             forward and backward timed separately, with the host CPU model
  peaks      measured on this GPU: bf16 matrix-core loop, streaming read and copy
  linear_in_n  the same step on the first 64 and 128 frames (time linear in N)
  variants   the other forms of the operator on their own workloads, fwd+bwd: per-head
             integer offsets (256-frame workload), box windows with one real offset per
             query, free per-sample real offsets (16 x 32 x 32, 3 x 7 x 7), the DWConv3D
             term (256-frame grid) and the offset predictor (16 x 32 x 32)
"""
import argparse
import ctypes
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "3D-DSA fwd+bwd query-token-heads/s and % bf16 MFMA peak at N≈2.09M"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_F32_TFLOPS = 157.3
RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)


class Hip:
    """hipEvent timing through the HIP runtime (ctypes)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventRecord.restype = ctypes.c_int

    def events(self, n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            assert self.lib.hipEventCreate(ctypes.byref(ev)) == 0
            arr[i] = ev
        return arr

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.lib.hipEventSynchronize(b) == 0
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return float(ms.value)


# timed phase -> the attention kernel it holds on the bf16 path (rocprofv3 names)
KERNEL_OF = {"k_forward": "k_forward_qs", "k_backward_dq": "k_dq_qs", "k_backward_dkdv": "k_dkdv_tube"}


def kernel_work(wl):
    """Algorithmic flops and HBM bytes per launch of each attention kernel (per
    (query token, head) unit times N*H units):
      forward  4KD flops (QK^T, PV);            reads Q, K, V, writes O, LSE: 4Ds + 4 B
      dQ       6KD flops (S, dP, dQ);           reads Q, K, V, dO, LSE, Delta, writes dQ: 5Ds + 8 B
      dK/dV    8KD flops (S, dP, dV, dK);       reads Q, K, V, dO, LSE, Delta, writes dK, dV: 6Ds + 8 B
    (Delta = rowsum(dO * O) is its own pass, 2Ds + 4 B, timed with the backward prep.)
    """
    K, D, s, NH = wl.K, wl.head_dim, wl.elem_bytes, wl.N * wl.heads
    return {
        "k_forward": (4 * K * D * NH, (4 * D * s + 4) * NH),
        "k_backward_dq": (6 * K * D * NH, (5 * D * s + 8) * NH),
        "k_backward_dkdv": (8 * K * D * NH, (6 * D * s + 8) * NH),
    }


# the sources the integer-offset path's kernels are built from (the counters in
# profiles/traffic.json are valid while these are unchanged)
MAIN_PATH_SOURCES = ("attn_fwd.hip", "attn_dq.hip", "attn_dkdv.hip", "attn.hip", "prep.hip", "qsched.hip",
                     "common.hpp", "internal.hpp", "qs_common.hpp", "tube.hpp")


def source_hash():
    h = hashlib.sha256()
    for f in MAIN_PATH_SOURCES:
        h.update(open(os.path.join(ROOT, "local_sparse_attention_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def _short(name):
    return name.split("(")[0].split("<")[0].replace("void ", "").replace("dsa3d::", "").strip()


def _counter_means(csv_path, counter):
    """Mean value per dispatch of `counter` for each kernel in a rocprofv3 counter CSV."""
    import csv

    acc = {}
    for r in csv.DictReader(open(csv_path)):
        if r.get("Counter_Name") != counter:
            continue
        k = _short(r["Kernel_Name"])
        acc.setdefault(k, []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def write_traffic(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, workload):
    """profiles/traffic.json from two rocprofv3 --pmc runs of the benchmark (FETCH_SIZE, then
    WRITE_SIZE, KiB per dispatch) and the same two counters over a device copy of known size
    (bench.py --copy-calibration, 3 launches of 1 GiB read + 1 GiB written)."""
    fetch, write = _counter_means(fetch_csv, "FETCH_SIZE"), _counter_means(write_csv, "WRITE_SIZE")
    cf, cw = _counter_means(copy_fetch_csv, "FETCH_SIZE"), _counter_means(copy_write_csv, "WRITE_SIZE")
    copy_name = max(cf, key=cf.get)
    fs = (1 << 30) / (cf[copy_name] * 1024.0)
    ws = (1 << 30) / (cw[copy_name] * 1024.0)
    kernels = {}
    for k in sorted(set(fetch) & set(write)):
        rb, wb = fetch[k] * 1024.0 * fs, write[k] * 1024.0 * ws
        kernels[k] = {"hbm_bytes_per_launch": rb + wb, "read_bytes": rb, "write_bytes": wb}
    out = {"workload": workload, "source_hash": source_hash(), "fetch_scale": fs, "write_scale": ws,
           "copy_kernel": copy_name, "kernels": kernels, "summary": "dsa3d_256frame_fwd_bwd.md",
           "note": "bytes between L2 and the memory fabric (Infinity-Cache hits included), per dispatch"}
    json.dump(out, open(os.path.join(ROOT, "profiles", "traffic.json"), "w"), indent=1)
    return out


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken
    on the current kernel sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
        e = d["kernels"][kernel]
        if d.get("source_hash") != source_hash() or d.get("workload") != workload:
            return None
        return float(e["hbm_bytes_per_launch"])
    except (KeyError, ValueError, TypeError):
        return None


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl_full, frames=5):
    """The oracle on the first `frames` frames of the workload (same heads, head size,
    window, generator words), forward and backward timed separately, wall time on this
    host's cores."""
    import oracle
    from local_sparse_attention_amd import synth

    wl = wl_full.with_frames(frames)
    inp = synth.make_inputs(wl)
    grid, window = (wl.F, wl.Hp, wl.Wp), (wl.kt, wl.ky, wl.kx)
    t0 = time.perf_counter()
    oracle.forward(inp["q"], inp["k"], inp["v"], inp["offsets"], grid, window, wl.scale)
    t1 = time.perf_counter()
    oracle.backward(inp["q"], inp["k"], inp["v"], inp["dout"], inp["offsets"], grid, window, wl.scale)
    t2 = time.perf_counter()
    cores = len(os.sched_getaffinity(0))
    threads = min(cores, int(os.environ.get("OMP_NUM_THREADS", cores)))
    NH = wl.N * wl.heads
    return {"value": NH / (t2 - t0), "unit": "query-token-heads/s", "cores": threads, "kind": "oracle",
            "sample": f"first {frames} of {wl_full.F} frames ({wl.N} tokens x {wl.heads} heads), fwd+bwd, "
                      f"{t2 - t0:.1f} s wall",
            "fwd_s": t1 - t0, "bwd_s": t2 - t1, "fwd_value": NH / (t1 - t0), "bwd_value": NH / (t2 - t1),
            "cpu_model": cpu_model()}


def measure_peaks(lib, hip, stream_ptr):
    """Measured peaks on this GPU: bf16 matrix-core loop, streaming read and copy."""
    import torch

    lib.dsa3d_peak_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.dsa3d_peak_mfma_bf16.restype = ctypes.c_double
    lib.dsa3d_peak_mfma32_bf16.argtypes = lib.dsa3d_peak_mfma_bf16.argtypes
    lib.dsa3d_peak_mfma32_bf16.restype = ctypes.c_double
    lib.dsa3d_peak_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.dsa3d_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                    ctypes.c_void_p]
    ev = hip.events(2)
    blocks = 256 * 8
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    best = {}
    for key, fn in (("mfma_16x16x32_tflops", lib.dsa3d_peak_mfma_bf16),
                    ("mfma_32x32x16_tflops", lib.dsa3d_peak_mfma32_bf16)):
        for _ in range(3):
            hip.lib.hipEventRecord(ev[0], stream_ptr)
            flops = fn(ctypes.c_void_p(out.data_ptr()), blocks, 4096, stream_ptr)
            hip.lib.hipEventRecord(ev[1], stream_ptr)
            assert flops > 0
            best[key] = max(best.get(key, 0.0), flops / (hip.elapsed_ms(ev[0], ev[1]) / 1e3) / 1e12)
    best["mfma_bf16_tflops"] = max(best["mfma_16x16x32_tflops"], best["mfma_32x32x16_tflops"])
    nbytes = 4 << 30
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    sink = torch.empty(4096 * 256, dtype=torch.int32, device="cuda")
    for _ in range(3):
        hip.lib.hipEventRecord(ev[0], stream_ptr)
        assert lib.dsa3d_peak_read(ctypes.c_void_p(src.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()), 4096,
                                   stream_ptr) == 0
        hip.lib.hipEventRecord(ev[1], stream_ptr)
        best["read_gbs"] = max(best.get("read_gbs", 0.0), nbytes / (hip.elapsed_ms(ev[0], ev[1]) / 1e3) / 1e9)
        hip.lib.hipEventRecord(ev[0], stream_ptr)
        assert lib.dsa3d_peak_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), nbytes, 4096,
                                   stream_ptr) == 0
        hip.lib.hipEventRecord(ev[1], stream_ptr)
        best["copy_gbs"] = max(best.get("copy_gbs", 0.0), 2 * nbytes / (hip.elapsed_ms(ev[0], ev[1]) / 1e3) / 1e9)
    del src, dst, sink, out
    torch.cuda.empty_cache()
    best["note"] = ("best of 3: 2048 workgroups x 4 waves of independent bf16 MFMA chains (8 of 16x16x32, or 4 of "
                    "32x32x16); 4 GiB streaming read / copy with 16-byte loads (copy counts read + write bytes)")
    return best


def sampled_flops(wl, fwd=True, bwd=True):
    """Algorithmic fp32 VALU flops of sampled windows per launch: per (query, head, sample)
    the forward blends 8 corner rows of K and of V (2 x 16D) and takes q . K~ and
    alpha V~ (2 x 2D) = 36D; the backward takes the 8 corner dots q . k_c and dO . v_c
    (32D: every quantity of the sample, the position gradient included, is a weighted sum
    of them), dQ += scale dz w_c k_c over the corners (16D), and scatters w alpha dO and
    w scale dz q to the 8 corners (32D) = 80D."""
    per = (36 if fwd else 0) + (80 if bwd else 0)
    return float(per) * wl.head_dim * wl.K * wl.N * wl.heads


def box_flops(wl):
    """Algorithmic fp32 VALU flops of box windows (one offset per query) per fwd+bwd, in the
    lattice form the box kernels use: every sample shares the fraction, so the samples' 8
    corners are the L = (kt+1)(ky+1)(kx+1) rows of one lattice.  Per (query, head): the
    forward takes L dots q . K[l] and L updates A_l V[l] (4DL), the query-side backward the
    dots q . K[l], dO . V[l] and the dQ updates (6DL), the key side dK[l] += B_l q and
    dV[l] += A_l dO (4DL)."""
    L = (wl.kt + 1) * (wl.ky + 1) * (wl.kx + 1)
    return float(14 * L) * wl.head_dim * wl.N * wl.heads


def _timed(fn, steps, warmup):
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def dev_inputs(wl):
    import torch

    from local_sparse_attention_amd import synth

    shape = (wl.N, wl.heads, wl.head_dim)
    t = {}
    for name, sid in (("q", 0), ("k", 1), ("v", 2), ("dout", 3)):
        a = synth.normal(wl.seed, sid, shape, wl.dtype, wl.qkv_scale if name != "dout" else 1.0)
        t[name] = torch.from_numpy(a.view("int16")).cuda().view(torch.bfloat16)
        del a
    return t


def run_per_head(dsa3d, wl, t, out, lse, g, ws, steps, warmup):
    """fwd+bwd with per-head integer offsets [H][N][3] on the given workload's tensors."""
    import torch

    from local_sparse_attention_amd import synth

    grid, window = (wl.F, wl.Hp, wl.Wp), (wl.kt, wl.ky, wl.kx)
    offh = torch.from_numpy(synth.make_head_offsets(wl)).cuda()
    # the workspace with which every head is bucketed together (one launch per kernel)
    wsh = dsa3d.workspace(grid, wl.heads, window, True, per_head=True)

    def step_heads():
        dsa3d.forward(t["q"], t["k"], t["v"], offh, grid, window, wl.scale, out=out, lse=lse, ws=wsh)
        dsa3d.backward(t["q"], t["k"], t["v"], offh, out, lse, t["dout"], grid, window, wl.scale, dq=g[0], dk=g[1],
                       dv=g[2], ws=wsh, reuse_prep=True)

    ms = _timed(step_heads, steps, warmup)
    del wsh
    return {"workload": f"{wl.name} with per-head offsets [{wl.heads}][N][3] (head h: the same recipe, seed "
                        f"+ 1000 h), all heads bucketed together",
            "ms_per_step": ms, "value": wl.N * wl.heads / (ms / 1e3), "unit": "query-token-heads/s",
            "roofline": {"bound": "hbm", "achieved": wl.bytes() / (ms / 1e3) / 1e9, "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": wl.bytes() / (ms / 1e3) / 1e9 / PEAK_HBM_GBS,
                         "note": "whole step, algorithmic bytes (as the main line) over the step time"}}


def run_sampled(dsa3d, steps, warmup):
    """fwd+bwd of sampled windows (real offsets): box windows, one offset per query, and
    free per-sample offsets, each on its own workload."""
    import torch

    from local_sparse_attention_amd import configs, synth

    res = {}
    for key, wl, mode in (("box_real_offsets", configs.S_BOX, "box"),
                          ("free_per_sample_offsets", configs.S_FREE, "free")):
        grid, window = (wl.F, wl.Hp, wl.Wp), (wl.kt, wl.ky, wl.kx)
        t = dev_inputs(wl)
        off = torch.from_numpy(synth.make_real_offsets(wl, mode)).cuda()
        ws = torch.empty(dsa3d.sampled_workspace_bytes(grid, wl.heads, window, mode, True), dtype=torch.uint8,
                         device="cuda")
        box = {}

        def fwd():
            box["o"] = dsa3d.sampled_forward(t["q"], t["k"], t["v"], off, grid, window, mode, wl.scale)

        def bwd():
            dsa3d.sampled_backward(t["q"], t["k"], t["v"], off, box["o"][0], box["o"][1], t["dout"], grid, window,
                                   mode, wl.scale, ws=ws)

        ms_f = _timed(fwd, steps, warmup)
        ms_b = _timed(bwd, steps, warmup)
        ms = ms_f + ms_b
        fl = box_flops(wl) if mode == "box" else sampled_flops(wl)
        res[key] = {
            "workload": f"{wl.name}: grid {wl.F}x{wl.Hp}x{wl.Wp} (N={wl.N}), {wl.heads} heads x {wl.head_dim}, "
                        f"window {wl.kt}x{wl.ky}x{wl.kx}, {wl.dtype}, "
                        + ("one real offset per query" if mode == "box" else "one real offset per sample"),
            "ms_per_step": ms, "fwd_ms": ms_f, "bwd_ms": ms_b, "value": wl.N * wl.heads / (ms / 1e3),
            "unit": "query-token-heads/s",
            "roofline": {"bound": "alu", "achieved": fl / (ms / 1e3) / 1e12, "peak": PEAK_F32_TFLOPS,
                         "unit": "TFLOP/s", "frac": fl / (ms / 1e3) / 1e12 / PEAK_F32_TFLOPS,
                         "note": ("fp32 VALU flops of the lattice form (14DL per query-head, L = (kt+1)(ky+1)"
                                  "(kx+1))" if mode == "box" else
                                  "fp32 VALU flops of the trilinear form (36D fwd + 80D bwd per sample)")}}
        del t, off, ws, box
        torch.cuda.empty_cache()
    return res


def run_c2_warm_cold(dsa3d, steps):
    """The bf16 forward workload (16 x 32 x 32, 8 heads x 64, 3 x 7 x 7; its tensors, 16.8 MB
    each, fit the 256 MB Infinity Cache): forward time with the inputs warm from the previous
    call, and after a 1 GiB write that scrubs the caches before each call."""
    import torch

    from local_sparse_attention_amd import configs, synth

    wl = configs.C2
    grid, window = (wl.F, wl.Hp, wl.Wp), (wl.kt, wl.ky, wl.kx)
    inp = synth.make_inputs(wl, with_dout=False)
    t = {k: torch.from_numpy(inp[k].view("int16")).cuda().view(torch.bfloat16) for k in ("q", "k", "v")}
    off = torch.from_numpy(inp["offsets"]).cuda()
    out = torch.empty_like(t["q"])
    lse = torch.empty((wl.heads, wl.N), dtype=torch.float32, device="cuda")
    ws = dsa3d.workspace(grid, wl.heads, window, False)
    scrub = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")

    def fwd():
        dsa3d.forward(t["q"], t["k"], t["v"], off, grid, window, wl.scale, out=out, lse=lse, ws=ws)

    warm = _timed(fwd, steps, 3)
    cold = []
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(steps):
        scrub.fill_(1)
        a.record()
        fwd()
        b.record()
        torch.cuda.synchronize()
        cold.append(a.elapsed_time(b))
    del t, off, out, lse, ws, scrub
    torch.cuda.empty_cache()
    cold_ms = sorted(cold)[len(cold) // 2]
    return {"workload": f"{wl.name}: grid {wl.F}x{wl.Hp}x{wl.Wp}, {wl.heads} heads x {wl.head_dim}, window "
                        f"{wl.kt}x{wl.ky}x{wl.kx}, bf16, forward (prep + attention)",
            "warm_ms": warm, "cold_ms": cold_ms,
            "note": "warm: mean of back-to-back calls; cold: median over calls each preceded by a 1 GiB fill"}


def run_predictor(dsa3d, steps, warmup):
    """The DWConv3D term of Eq. (1) on the 256-frame grid (hidden 16 x 128 = 2048 channels,
    3 x 3 x 3 filter: the pages give no size), added into an attention output, forward and
    backward; and the offset predictor (3 x 3 x 3 depthwise convolution, then the pointwise
    layer from 1024 channels to 8 heads x 147 samples x 3 offsets) on the 16 x 32 x 32
    sampled-window workload, forward and backward."""
    import torch

    from local_sparse_attention_amd import configs

    res = {}
    gen = torch.Generator(device="cuda").manual_seed(7)
    wl = configs.C5
    grid, N, C = (wl.F, wl.Hp, wl.Wp), wl.N, wl.heads * wl.head_dim
    x = torch.randn((N, C), generator=gen, device="cuda").bfloat16()
    out = torch.randn((N, C), generator=gen, device="cuda").bfloat16()
    w = 0.1 * torch.randn((C, 3, 3, 3), generator=gen, device="cuda")
    b = torch.randn((C,), generator=gen, device="cuda")

    ms_f = _timed(lambda: dsa3d.dwconv3d_forward(x, w, b, grid, out=out, accumulate=True), steps, warmup)
    dy = out
    ms_b = _timed(lambda: dsa3d.dwconv3d_backward(x, w, dy, grid), steps, warmup)
    bf, bb = 3.0 * N * C * 2, 3.0 * N * C * 2
    res["dwconv3d_term"] = {
        "workload": f"DWConv3D term on {wl.name} (grid {wl.F}x{wl.Hp}x{wl.Wp}, N={N}, C={C} channels, bf16), "
                    "3x3x3 filter, added into the attention output",
        "fwd_ms": ms_f, "bwd_ms": ms_b, "ms_per_step": ms_f + ms_b,
        "roofline": {"bound": "hbm", "achieved": (bf + bb) / ((ms_f + ms_b) / 1e3) / 1e9, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": (bf + bb) / ((ms_f + ms_b) / 1e3) / 1e9 / PEAK_HBM_GBS,
                     "fwd_frac": bf / (ms_f / 1e3) / 1e9 / PEAK_HBM_GBS,
                     "note": "algorithmic bytes: forward reads x and the attention output and writes the sum "
                             "(3 N C s), backward reads x and dy and writes dx (3 N C s)"}}
    del x, out, dy, w, b
    torch.cuda.empty_cache()

    wl = configs.S_FREE
    grid, N, C, O = (wl.F, wl.Hp, wl.Wp), wl.N, wl.heads * wl.head_dim, wl.heads * wl.K * 3
    x = torch.randn((N, C), generator=gen, device="cuda").bfloat16()
    w1 = 0.1 * torch.randn((C, 3, 3, 3), generator=gen, device="cuda")
    b1 = torch.randn((C,), generator=gen, device="cuda")
    w2 = (0.05 * torch.randn((O, C), generator=gen, device="cuda")).bfloat16()
    b2 = torch.randn((O,), generator=gen, device="cuda")
    dy = torch.randn((N, O), generator=gen, device="cuda")
    box = {}

    def fwd():
        box["h"] = dsa3d.dwconv3d_forward(x, w1, b1, grid)
        box["y"] = dsa3d.linear_forward(box["h"], w2, b2)

    def bwd():
        dh, _, _ = dsa3d.linear_backward(box["h"], w2, dy)
        dsa3d.dwconv3d_backward(x, w1, dh, grid)

    fwd()
    ms_lf = _timed(lambda: dsa3d.linear_forward(box["h"], w2, b2), steps, warmup)
    ms_f = _timed(fwd, steps, warmup)
    ms_b = _timed(bwd, steps, warmup)
    gemm_fl = 2.0 * N * C * O
    res["offset_predictor"] = {
        "workload": f"offset predictor on {wl.name} (N={N}): 3x3x3 depthwise conv over {C} channels, then the "
                    f"pointwise layer {C} -> {O} ({wl.heads} heads x {wl.K} samples x 3), bf16",
        "fwd_ms": ms_f, "bwd_ms": ms_b, "ms_per_step": ms_f + ms_b, "linear_fwd_ms": ms_lf,
        "roofline": {"bound": "mfma", "achieved": gemm_fl / (ms_lf / 1e3) / 1e12, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": gemm_fl / (ms_lf / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
                     "note": "the pointwise layer's forward product (2 N C O flops) over its own time"}}
    del x, w1, b1, w2, b2, dy, box
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="C5", help="C1..C5 (default: the 256-frame workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (scales the HBM byte counters)")
    ap.add_argument("--no-extras", action="store_true",
                    help="main line only: no measured peaks, linear-in-N run or operator variants")
    ap.add_argument("--variants-only", action="store_true",
                    help="only the operator variants (for profiling their kernels)")
    ap.add_argument("--per-head-only", action="store_true",
                    help="only the per-head-offsets variant (for profiling its kernels)")
    ap.add_argument("--sampled-only", action="store_true",
                    help="only the sampled-window variants (for profiling their kernels)")
    ap.add_argument("--predictor-only", action="store_true",
                    help="only the DWConv3D term and offset predictor variants (for profiling their kernels)")
    ap.add_argument("--write-traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="write profiles/traffic.json from rocprofv3 counter CSVs (no GPU needed)")
    args = ap.parse_args()
    if args.write_traffic:
        from local_sparse_attention_amd import configs

        print(json.dumps(write_traffic(*args.write_traffic, configs.ALL[args.workload].name)), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the path shards by heads without "
              "communication, so an N-GPU figure would be N independent copies of this run.", file=sys.stderr)
        sys.exit(2)

    import torch

    from local_sparse_attention_amd import configs, dsa3d, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}), flush=True)
        return
    if args.predictor_only:
        print(json.dumps({"variants": run_predictor(dsa3d, 3, 1)}), flush=True)
        return
    if args.sampled_only:
        print(json.dumps({"variants": run_sampled(dsa3d, 3, 1)}), flush=True)
        return
    if args.variants_only or args.per_head_only:
        wl = configs.C5
        t = dev_inputs(wl)
        out = torch.empty_like(t["q"])
        lse = torch.empty((wl.heads, wl.N), dtype=torch.float32, device="cuda")
        g = [torch.empty_like(t["q"]) for _ in range(3)]
        ws = dsa3d.workspace((wl.F, wl.Hp, wl.Wp), wl.heads, (wl.kt, wl.ky, wl.kx), True)
        var = {"per_head_offsets": run_per_head(dsa3d, wl, t, out, lse, g, ws, 3, 1)}
        del t, out, lse, g, ws
        torch.cuda.empty_cache()
        if args.per_head_only:
            print(json.dumps({"variants": var}), flush=True)
            return
        var.update(run_sampled(dsa3d, 3, 1))
        var.update(run_predictor(dsa3d, 3, 1))
        print(json.dumps({"variants": var}), flush=True)
        return
    wl = configs.ALL[args.workload]
    grid, window = (wl.F, wl.Hp, wl.Wp), (wl.kt, wl.ky, wl.kx)
    lib = dsa3d.load()
    hip = Hip()
    log = lambda msg: print(f"[bench] {msg}", file=sys.stderr, flush=True)
    log(f"generating {wl.name} inputs")

    # inputs: generated on the host (seeded), copied once, resident in HBM
    shape = (wl.N, wl.heads, wl.head_dim)
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    dev = {}
    for name, stream_id in (("q", 0), ("k", 1), ("v", 2), ("dout", 3)):
        scale = wl.qkv_scale if name != "dout" else 1.0
        a = synth.normal(wl.seed, stream_id, shape, wl.dtype, scale)
        t = torch.from_numpy(a.view("int16") if wl.dtype == "bf16" else a)
        dev[name] = t.cuda().view(tdt) if wl.dtype == "bf16" else t.cuda()
        del a, t
    dev["offsets"] = torch.from_numpy(synth.make_offsets(wl)).cuda()
    out = torch.empty(shape, dtype=tdt, device="cuda")
    lse = torch.empty((wl.heads, wl.N), dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.empty(shape, dtype=tdt, device="cuda") for _ in range(3))
    ws = dsa3d.workspace(grid, wl.heads, window, True)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    dtc = 1 if wl.dtype == "bf16" else 0
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    fevs = [hip.events(3) for _ in range(args.steps)]
    bevs = [hip.events(4) for _ in range(args.steps)]

    def step(fev=None, bev=None):
        rc = lib.dsa3d_forward_ex(ptr(dev["q"]), ptr(dev["k"]), ptr(dev["v"]), ptr(dev["offsets"]), *grid,
                                  wl.heads, wl.head_dim, *window, wl.scale, dtc, ptr(out), ptr(lse), ptr(ws),
                                  ws.numel(), sp, 0, fev)
        assert rc == 0, dsa3d.status_string(rc)
        rc = lib.dsa3d_backward_ex(ptr(dev["q"]), ptr(dev["k"]), ptr(dev["v"]), ptr(dev["offsets"]), ptr(out),
                                   ptr(lse), ptr(dev["dout"]), *grid, wl.heads, wl.head_dim, *window, wl.scale,
                                   dtc, ptr(dq), ptr(dk), ptr(dv), ptr(ws), ws.numel(), sp, dsa3d.FLAG_REUSE_PREP,
                                   bev)
        assert rc == 0, dsa3d.status_string(rc)

    evp = ctypes.POINTER(ctypes.c_void_p)
    lib.dsa3d_forward_ex.argtypes = lib.dsa3d_forward.argtypes + [ctypes.c_uint, evp]
    lib.dsa3d_backward_ex.argtypes = lib.dsa3d_backward.argtypes + [ctypes.c_uint, evp]

    log("warm-up")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(fevs[i], bevs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    phases = {"fwd_prep": 0.0, "k_forward": 0.0, "bwd_prep": 0.0, "k_backward_dq": 0.0, "k_backward_dkdv": 0.0}
    for fev, bev in zip(fevs, bevs):
        phases["fwd_prep"] += hip.elapsed_ms(fev[0], fev[1])
        phases["k_forward"] += hip.elapsed_ms(fev[1], fev[2])
        phases["bwd_prep"] += hip.elapsed_ms(bev[0], bev[1])
        phases["k_backward_dq"] += hip.elapsed_ms(bev[1], bev[2])
        phases["k_backward_dkdv"] += hip.elapsed_ms(bev[2], bev[3])
    phases = {k: v / args.steps for k, v in phases.items()}
    ms_per_step = wall * 1000.0 / args.steps
    device_ms = sum(phases.values())

    NH = wl.N * wl.heads
    value = NH / (ms_per_step / 1000.0)
    flops = wl.flops()
    work = kernel_work(wl)
    dom = max(work, key=lambda k: phases[k])
    kf, kb = work[dom]
    t_dom = phases[dom] / 1000.0
    ai = kf / kb
    peak_flops = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_TFLOPS
    ridge = peak_flops * 1e12 / (PEAK_HBM_GBS * 1e9)
    if ai < ridge:
        roof = {"bound": "hbm", "achieved": kb / t_dom / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": kf / t_dom / 1e12, "peak": peak_flops, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(KERNEL_OF[dom], wl.name)
    roof["traffic_note"] = ("bytes between L2 and the memory fabric (FETCH_SIZE x fetch scale + WRITE_SIZE x write "
                            "scale, both scales from a device copy of known size; fabric reads that hit the "
                            "Infinity Cache count too), from profiles/traffic.json when it matches the sources")
    if roof["traffic"] is not None:
        # the same kernel time over the bytes it actually moved (counters), not the algorithmic ones
        roof["traffic_gbs"] = roof["traffic"] / t_dom / 1e9
        roof["traffic_frac"] = roof["traffic_gbs"] / PEAK_HBM_GBS
        roof["traffic_over_algorithmic"] = roof["traffic"] / kb
    roof["kernel"] = KERNEL_OF[dom] if wl.dtype == "bf16" else dom
    roof["kernel_ms"] = phases[dom]

    res = {
        "metric": METRIC,
        "value": value,
        "unit": "query-token-heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: grid {wl.F}x{wl.Hp}x{wl.Wp} (N={wl.N}), {wl.heads} heads x "
                               f"head_dim {wl.head_dim}, window {wl.kt}x{wl.ky}x{wl.kx}, {wl.dtype}, fwd+bwd",
                   "global_batch": 1, "seq_len": wl.N, "parallelism": "single-gpu"},
        "useful_tflops": flops / (ms_per_step / 1000.0) / 1e12,
        "mfma_frac": flops / (ms_per_step / 1000.0) / 1e12 / peak_flops,
        "alg_hbm_frac": wl.bytes() / (ms_per_step / 1000.0) / 1e9 / PEAK_HBM_GBS,
        "device_ms_per_step": device_ms,
        "phases_ms": phases,
        "roofline": roof,
        "cpu_baseline": None,
    }

    if not args.no_extras and wl.name == configs.C5.name:
        # time linear in N at a fixed window: the same step on the first 64 and 128 frames
        # (token order is frame-major, so those are prefixes of the same tensors)
        lin = []
        for F in (64, 128):
            wF = wl.with_frames(F)
            gF = (F, wl.Hp, wl.Wp)
            log(f"linear-in-N run, {F} frames")

            def stepF():
                rc = lib.dsa3d_forward_ex(ptr(dev["q"]), ptr(dev["k"]), ptr(dev["v"]), ptr(dev["offsets"]), *gF,
                                          wl.heads, wl.head_dim, *window, wl.scale, dtc, ptr(out), ptr(lse), ptr(ws),
                                          ws.numel(), sp, 0, None)
                assert rc == 0, dsa3d.status_string(rc)
                rc = lib.dsa3d_backward_ex(ptr(dev["q"]), ptr(dev["k"]), ptr(dev["v"]), ptr(dev["offsets"]),
                                           ptr(out), ptr(lse), ptr(dev["dout"]), *gF, wl.heads, wl.head_dim, *window,
                                           wl.scale, dtc, ptr(dq), ptr(dk), ptr(dv), ptr(ws), ws.numel(), sp,
                                           dsa3d.FLAG_REUSE_PREP, None)
                assert rc == 0, dsa3d.status_string(rc)

            stepF()
            torch.cuda.synchronize()
            a = time.perf_counter()
            for _ in range(3):
                stepF()
            torch.cuda.synchronize()
            msF = (time.perf_counter() - a) * 1e3 / 3
            lin.append({"frames": F, "N": wF.N, "ms_per_step": msF, "value": wF.N * wl.heads / (msF / 1e3)})
        lin.append({"frames": wl.F, "N": wl.N, "ms_per_step": ms_per_step, "value": value})
        res["linear_in_n"] = lin
        log("per-head offsets variant")
        res["variants"] = {"per_head_offsets": run_per_head(dsa3d, wl, dev, out, lse, [dq, dk, dv], ws, 3, 1)}

    del dev, out, lse, dq, dk, dv, ws
    torch.cuda.empty_cache()
    if not args.no_extras:
        log("measured peaks")
        peaks = measure_peaks(lib, hip, sp)
        res["peaks_measured"] = peaks
        if roof["unit"] == "GB/s":
            roof["measured_peak"] = peaks["read_gbs"]
        else:
            roof["measured_peak"] = peaks["mfma_bf16_tflops"]
        roof["frac_of_measured"] = roof["achieved"] / roof["measured_peak"]
        res["mfma_frac_of_measured"] = res["useful_tflops"] / peaks["mfma_bf16_tflops"]
        log("sampled-window variants")
        res.setdefault("variants", {}).update(run_sampled(dsa3d, 3, 1))
        log("DWConv3D term and offset predictor")
        res["variants"].update(run_predictor(dsa3d, 3, 1))
        log("bf16 forward workload, warm and cold caches")
        res["c2_forward_warm_cold"] = run_c2_warm_cold(dsa3d, 10)
    if not args.no_cpu_baseline:
        log("CPU oracle baseline")
        res["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
