"""Benchmark of the 3D-DSA hot path on one MI355X: forward + backward (window-start
bucketing, attention forward, dQ, dK/dV) on the 256-frame workload (grid 256 x 68 x 120,
N = 2,088,960 tokens, a 16-head slice of head_dim 128, window 5 x 9 x 9, bf16, smooth
drifting motion field), inputs resident in HBM.

One step = dsa3d_forward + dsa3d_backward over the whole grid.  Prints one JSON line.
  phases_ms  per step, from HIP events the library records on its stream: bucketing
             and work lists (+ Delta in the backward), then each attention kernel
  value      query-token-heads per second (N * heads / step time)
  roofline   the dominant kernel's algorithmic bytes per launch / its mean duration,
             timed with HIP events on the library's stream, against 8 TB/s HBM
  cpu_baseline  the CPU oracle (fp64, OpenMP) on the first 5 frames of the same workload
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


def source_hash():
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "local_sparse_attention_amd", "csrc", "*"))):
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


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


def cpu_baseline(wl_full, frames=5):
    """The oracle on the first `frames` frames of the workload (same heads, head size,
    window, generator words), fwd + bwd, wall time on this host's cores."""
    import oracle
    from local_sparse_attention_amd import synth

    wl = wl_full.with_frames(frames)
    inp = synth.make_inputs(wl)
    grid, window = (wl.F, wl.Hp, wl.Wp), (wl.kt, wl.ky, wl.kx)
    t0 = time.perf_counter()
    oracle.forward(inp["q"], inp["k"], inp["v"], inp["offsets"], grid, window, wl.scale)
    oracle.backward(inp["q"], inp["k"], inp["v"], inp["dout"], inp["offsets"], grid, window, wl.scale)
    dt = time.perf_counter() - t0
    cores = len(os.sched_getaffinity(0))
    threads = min(cores, int(os.environ.get("OMP_NUM_THREADS", cores)))
    return {"value": wl.N * wl.heads / dt, "unit": "query-token-heads/s", "cores": threads, "kind": "oracle",
            "sample": f"first {frames} of {wl_full.F} frames ({wl.N} tokens x {wl.heads} heads), fwd+bwd, "
                      f"{dt:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="C5", help="C1..C5 (default: the 256-frame workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (scales the HBM byte counters)")
    args = ap.parse_args()
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
    wl = configs.ALL[args.workload]
    grid, window = (wl.F, wl.Hp, wl.Wp), (wl.kt, wl.ky, wl.kx)
    lib = dsa3d.load()
    hip = Hip()

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
                                   dtc, ptr(dq), ptr(dk), ptr(dv), ptr(ws), ws.numel(), sp, 0, bev)
        assert rc == 0, dsa3d.status_string(rc)

    evp = ctypes.POINTER(ctypes.c_void_p)
    lib.dsa3d_forward_ex.argtypes = lib.dsa3d_forward.argtypes + [ctypes.c_uint, evp]
    lib.dsa3d_backward_ex.argtypes = lib.dsa3d_backward.argtypes + [ctypes.c_uint, evp]

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

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
    del dev, out, lse, dq, dk, dv, ws
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
