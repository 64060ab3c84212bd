#!/usr/bin/env python3
"""Benchmark of the attention forward (+lse) and backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = the whole hot path on one batch: sdpa_fwd_lse (forward kernel),
then sdpa_bwd, with inputs resident in device memory before the timed region
starts. The backward runs three passes: with a bounded (windowed) band at
D = 256, the Delta pass, the key-stationary dK/dV pass that also writes dS for
the band, and dQ = scale dS K from it; otherwise the query-stationary dQ pass
(recomputing S and dP, also forming Delta) and the dK/dV pass. Default workload: the causal +
sliding-window (1024) layer at L = 16384, D = 256, 32 query / 16 kv heads.
Prints one JSON line on stdout; diagnostics go to stderr.

Throughput is mask-aware useful FLOP: N = number of allowed (query, key)
pairs over all heads; forward 4*D*N (QK^T, PV), backward 10*D*N (QK^T,
dO V^T, dS K, dS^T Q, P^T dO). Masked edge-tile work, exp, and the side
passes cost time but add no FLOP.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd+bwd mask-aware TFLOP/s and % of bf16 MFMA peak; peak mem GB"
BF16_PEAK_TFLOPS = 2516.6   # MI355X dense bf16 MFMA, AMD public figure (no sparsity)
HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = "bf16_window1024_L16384_D256_h32kv16"


def dkdv_kernel(w):
    """Name of the dK/dV kernel the library picks for this (dense, 16-bit) workload: 16-key waves at
    D = 512, and at D = 256 unless the key blocks (128 keys per kv head) number fewer than 256, when
    32-key waves split each block's query tiles; 32-key waves below D = 256."""
    blocks = -(-w.Lkv // 128) * w.Hkv * w.B
    if w.D == 512 or (w.D == 256 and blocks >= 256):
        return f"kv16_kernel<{w.D}>"
    return f"kv_kernel<{w.D}>" + (" + share reduce" if blocks < 256 else "")


def uses_band(w, sdpa, dtype):
    """Whether the backward keeps dS for the band on this workload: the library does so for the
    16-key dK/dV kernel at D = 256 when its full workspace (the size the bench gives) exceeds the
    Delta rows (at D = 256 the 16-key kernel never splits)."""
    if not (w.D == 256 and dkdv_kernel(w).startswith("kv16")):
        return False
    full = sdpa.bwd_workspace_bytes(w.B, w.Hq, w.group, w.L, w.Lkv, w.D, dtype, w.mask, w.window)
    return full > sdpa.workspace_bytes(w.B, w.Hq, w.L, w.D, dtype)


def tile_config(w):
    """The kernels' tile shapes for this workload (as the library picks them)."""
    if w.dtype == "f32":
        return "fp32 VALU kernels (one query row per lane; one key per lane in dK/dV)"
    bk = 64 if w.D <= 256 else 32
    split = "" if w.D <= 256 else "; the dQ pass: 64 rows, head dim split over wave pairs"
    import torch
    import sdpa_backward_amd as sdpa
    fb = sdpa.fwd_workspace_bytes(w.B, w.Hq, w.group, w.L, w.Lkv, w.D, torch.bfloat16, w.mask, w.window)
    if fb:
        split += f"; each query tile's key range split over {fb // (w.B * w.Hq * w.L * (w.D + 2) * 4)} workgroups"
    kv = dkdv_kernel(w)
    if kv.startswith("kv16") and w.D == 256:
        # the launcher's choice: 8-wave workgroups when every key sees at least 2048 query rows (no band)
        from workloads import MASK_TWO_SIDED, MASK_WINDOW
        span = {MASK_WINDOW: w.window, MASK_TWO_SIDED: 2 * w.window - 1}.get(w.mask, w.L)
        eight = not uses_band(w, sdpa, torch.bfloat16) and min(span, w.L) >= 2048
        kv += f", {8 if eight else 4}-wave workgroups"
    return (f"forward and dQ: 128 query rows x {bk}-key tiles per workgroup (4 waves, 32x32x16 MFMA{split}); "
            f"dK/dV: {kv}")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def achievable_peak(torch, dev, ev, stream, n_wg=2048, iters=2048, reps=3):
    """bf16 MFMA TFLOP/s this GPU sustains at its running clock (libsdpa_probe.so:
    register-only MFMA chains, no memory traffic), median of `reps` launches."""
    from sdpa_backward_amd import build
    probe = ctypes.CDLL(build.PROBE_LIB)
    probe.sdpa_probe_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    probe.sdpa_probe_mfma_bf16_flop.argtypes = [ctypes.c_int32, ctypes.c_int32]
    probe.sdpa_probe_mfma_bf16_flop.restype = ctypes.c_double
    out = torch.empty(n_wg * 256, dtype=torch.float32, device=dev)
    flop = probe.sdpa_probe_mfma_bf16_flop(n_wg, iters)
    e = [ev.create() for _ in range(2 * reps)]
    assert probe.sdpa_probe_mfma_bf16(ctypes.c_void_p(out.data_ptr()), n_wg, iters, ctypes.c_void_p(stream)) == 0
    for r in range(reps):
        ev.record(e[2 * r], stream)
        assert probe.sdpa_probe_mfma_bf16(ctypes.c_void_p(out.data_ptr()), n_wg, iters, ctypes.c_void_p(stream)) == 0
        ev.record(e[2 * r + 1], stream)
    torch.cuda.synchronize()
    ms = statistics.median(ev.ms(e[2 * r], e[2 * r + 1]) for r in range(reps))
    return flop / (ms * 1e-3) / 1e12


def row_key_counts(w, rows):
    """Allowed keys of each query row in ``rows`` (the queries are the last L of Lk positions)."""
    import numpy as np

    Lq, Lk, W = w.L, w.Lkv, w.window
    pos = np.asarray(rows, dtype=np.int64) + (Lk - Lq)   # the row's diagonal key
    lo, hi = np.zeros_like(pos), np.full_like(pos, Lk - 1)
    if w.mask in ("causal", "causal_window", "window"):
        hi = np.minimum(hi, pos + (W - 1 if w.mask == "window" else 0))
    if w.mask in ("causal_window", "window"):
        lo = np.maximum(lo, pos - W + 1)
    return np.maximum(hi - lo + 1, 0)


def allowed_pairs(w) -> int:
    """Allowed (i, j) pairs over all heads."""
    import numpy as np

    return w.B * w.Hq * int(row_key_counts(w, np.arange(w.L)).sum())


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch already loaded (same process, same streams)."""

    def __init__(self):
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        self.hip = ctypes.CDLL(path or "libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def record(self, e, stream):
        assert self.hip.hipEventRecord(ctypes.c_void_p(e), ctypes.c_void_p(stream)) == 0

    def ms(self, a, b):
        out = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(out), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
        return out.value


def measured_traffic(w):
    """HBM bytes per dK/dV-kernel launch from the committed counter runs on this workload
    (profiles/traffic_<kernel>_<workload tag>.json), if they were taken on this source."""
    from sdpa_backward_amd.profsum import sources_sha256, tag
    kernel = dkdv_kernel(w).split("<")[0]
    try:
        with open(os.path.join(ROOT, "profiles", f"traffic_{kernel}_{tag(w)}.json")) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("sources_sha256") != sources_sha256(kernel) or t.get("workload") != w.name:
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(w, inp, seconds):
    """The fp64 oracle, as it stands, on a bounded sample: one q-head, blocks of 1024 query rows."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import head_rows

    h, g = 0, 0
    qh = inp["q"][0, h].double().numpy()
    kg = inp["k"][0, g].double().numpy()
    vg = inp["v"][0, g].double().numpy()
    doh = inp["do"][0, h].double().numpy()
    block = min(1024, w.L)
    start = min(max(0, w.L // 2 - block), w.L - block)
    r = start
    pairs = 0
    n = 0
    t0 = time.perf_counter()
    while True:
        rows = np.arange(r, min(w.L, r + block))
        head_rows(qh, kg, vg, doh, w.scale, w.mask, w.window, rows)
        pairs += int(row_key_counts(w, rows).sum())
        n += 1
        r += block
        if r + block > w.L:
            r = 0
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    threads = [p.get("num_threads", 1) for p in threadpool_info() if p.get("internal_api") == "openblas"]
    cores = max(threads) if threads else 1
    return {
        "value": 14 * w.D * pairs / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"q-head {h}: {n} blocks of {block} query rows x all {w.Lkv} keys (full-width fp64 rows), "
                  f"fwd+bwd, {pairs} allowed pairs, {dt:.1f} s wall; useful-FLOP rate",
        "host_cpus": os.cpu_count(),
        "affinity_cpus": len(os.sched_getaffinity(0)),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--cold", type=int, default=3,
                    help="steps timed after a 1 GiB device write (caches cold), before the timed steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after timing, run one 1 GiB device copy (reference kernel for HBM counter scaling)")
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import sdpa_backward_amd as sdpa
    from workloads import BY_NAME, make_inputs

    w = BY_NAME[a.workload]
    dev = torch.device("cuda:0")
    sdpa.load()
    log(f"device: {torch.cuda.get_device_name(dev)}  torch {torch.__version__}  workload {w.name}")
    t = time.perf_counter()
    cpu_inp = make_inputs(w)
    inp = {n: x.to(dev) for n, x in cpu_inp.items()}
    torch.cuda.synchronize()
    log(f"inputs ready ({time.perf_counter() - t:.1f} s)")
    q, k, v, do = inp["q"], inp["k"], inp["v"], inp["do"]
    in_bytes = sum(x.numel() * x.element_size() for x in inp.values())

    # peak device memory of one fwd+bwd, outputs and workspace allocated inside
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(dev)
    o, lse = sdpa.sdpa_fwd_lse(q, k, v, w.mask, w.window, w.scale)
    dq, dk, dv = sdpa.sdpa_bwd(q, k, v, o, do, lse, w.mask, w.window, w.scale)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated(dev)
    del o, lse, dq, dk, dv
    torch.cuda.empty_cache()

    o = torch.empty_like(q)
    lse = torch.empty(w.B, w.Hq, w.L, dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_bytes = sdpa.bwd_workspace_bytes(w.B, w.Hq, w.group, w.L, w.Lkv, w.D, q.dtype, w.mask, w.window)
    ws = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device=dev)
    # the forward's key-range split of small problems (empty: no split)
    fws = torch.empty(sdpa.fwd_workspace_bytes(w.B, w.Hq, w.group, w.L, w.Lkv, w.D, q.dtype, w.mask, w.window),
                      dtype=torch.uint8, device=dev)
    band = uses_band(w, sdpa, q.dtype)
    stream = torch.cuda.current_stream(dev).cuda_stream
    ev = HipEvents()
    # per step: [0] forward start, [1] forward end = backward start, [2] after the
    # backward's first pass, [3] after the dK/dV pass, [4] backward end
    evs = [[ev.create() for _ in range(5)] for _ in range(a.steps)]

    def step(e=None):
        if e:
            ev.record(e[0], stream)
        sdpa.sdpa_fwd_lse(q, k, v, w.mask, w.window, w.scale, out=o, lse=lse, workspace=fws)
        sdpa.sdpa_bwd(q, k, v, o, do, lse, w.mask, w.window, w.scale, workspace=ws, out=(dq, dk, dv),
                      events=e[1:] if e else None)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    # cold caches: a 1 GiB write (well above the L2s and the 256 MB MALL) before each
    # of these steps; they run before the timed steps, which stay the last calls
    cold = []
    if a.cold > 0:
        scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        for i in range(a.cold):
            scratch.fill_(float(i))
            e = [ev.create() for _ in range(5)]
            step(e)
            torch.cuda.synchronize()
            cold.append((ev.ms(e[0], e[1]), ev.ms(e[1], e[4])))
        del scratch
        torch.cuda.empty_cache()
    t0 = time.perf_counter()
    for i in range(a.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    log(f"timed {a.steps} steps in {t1 - t0:.3f} s")

    if a.copy_probe:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1.0)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()

    peak_meas = achievable_peak(torch, dev, ev, stream)

    fwd_ms = [ev.ms(e[0], e[1]) for e in evs]
    bwd_ms = [ev.ms(e[1], e[4]) for e in evs]
    p1_ms = [ev.ms(e[1], e[2]) for e in evs]
    main_ms = [ev.ms(e[2], e[3]) for e in evs]
    p3_ms = [ev.ms(e[3], e[4]) for e in evs]
    ms_per_step = (t1 - t0) * 1e3 / a.steps
    N = allowed_pairs(w)
    fwd_flop, bwd_flop = 4 * w.D * N, 10 * w.D * N
    value = (fwd_flop + bwd_flop) / (ms_per_step * 1e-3) / 1e12
    kv_flop = 8 * w.D * N  # the dK/dV kernel's own work: S, dP, dV, dK contractions
    achieved = kv_flop / (statistics.mean(main_ms) * 1e-3) / 1e12
    traffic = measured_traffic(w)
    med = statistics.median
    esz = 4 if w.dtype == "f32" else 2
    q_bytes = w.B * w.Hq * w.L * w.D * esz

    def mfma_entry(name, flop, what, ms_list):
        t = statistics.mean(ms_list)
        return {"kernel": name, "bound": "mfma", "algorithmic": what, "avg_launch_ms": round(t, 4),
                "achieved": round(flop / (t * 1e-3) / 1e12, 1), "unit": "TFLOP/s",
                "frac": round(flop / (t * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}

    def hbm_entry(name, nbytes, what, ms_list):
        t = statistics.mean(ms_list)
        return {"kernel": name, "bound": "hbm", "algorithmic": what, "avg_launch_ms": round(t, 4),
                "achieved": round(nbytes / (t * 1e-3) / 1e9, 1), "unit": "GB/s",
                "frac": round(nbytes / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}

    kernels = [mfma_entry(f"qs_kernel<{w.D}, forward>", fwd_flop, "4*D FLOP per allowed pair (S, PV)", fwd_ms)]
    if band:
        kernels.append(hbm_entry("delta_kernel", 2 * q_bytes, "O and dO read once", p1_ms))
        kernels.append(mfma_entry(dkdv_kernel(w) + " writing dS", kv_flop,
                                  "8*D FLOP per allowed pair (S, dP, dV, dK)", main_ms))
        kernels.append(mfma_entry(f"dsq_kernel<{w.D}>", 2 * w.D * N, "2*D FLOP per allowed pair (dS K)", p3_ms))
    else:
        kernels.append(mfma_entry(f"qs_kernel<{w.D}, dQ>", 6 * w.D * N,
                                  "6*D FLOP per allowed pair (S, dP recomputed; dS K)", p1_ms))
        kernels.append(mfma_entry(dkdv_kernel(w), kv_flop, "8*D FLOP per allowed pair (S, dP, dV, dK)", main_ms))
    bwd_useful = bwd_flop / (statistics.mean(bwd_ms) * 1e-3) / 1e12

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded i.i.d. N(0,1) Q, K, V, dO)",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "L": w.L, "Lk": w.Lkv, "D": w.D,
                   "mask": w.mask, "window": w.window, "scale": w.scale, "allowed_pairs": N},
        "pct_of_bf16_peak": round(100 * value / BF16_PEAK_TFLOPS, 2),
        "peak_mem_gb": round(peak / 1e9, 3),
        "peak_mem_above_inputs_gb": round((peak - in_bytes) / 1e9, 3),
        "phases": {
            "fwd": {"ms_median": round(med(fwd_ms), 4), "ms_min": round(min(fwd_ms), 4),
                    "tflops": round(fwd_flop / med(fwd_ms) / 1e9, 1)},
            "bwd": {"ms_median": round(med(bwd_ms), 4), "ms_min": round(min(bwd_ms), 4),
                    "tflops": round(bwd_flop / med(bwd_ms) / 1e9, 1),
                    "plan": "Delta pass, dK/dV pass writing dS for the band, dQ = scale dS K" if band else
                            "dQ pass (recomputes S and dP, forms Delta), dK/dV pass"},
            "bwd_pass1": {"what": "Delta" if band else "dQ (6*D*N)", "ms_median": round(med(p1_ms), 4)},
            "bwd_dkdv_kernel": {"ms_median": round(med(main_ms), 4), "ms_min": round(min(main_ms), 4),
                                "tflops_8DN": round(kv_flop / med(main_ms) / 1e9, 1)},
            "bwd_pass3": {"what": "dQ from dS (2*D*N)" if band else "none", "ms_median": round(med(p3_ms), 4)},
            "fwd_plus_bwd_wall": {"ms": round(ms_per_step, 4)},
        },
        "cold": None if not cold else {
            "steps": len(cold), "note": "each step after a 1 GiB device write",
            "fwd_ms_median": round(med([c[0] for c in cold]), 4),
            "bwd_ms_median": round(med([c[1] for c in cold]), 4)},
        "roofline": {
            "kernel": f"{dkdv_kernel(w)} (dK/dV pass)",
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
            "traffic": traffic,
            "achievable_peak": round(peak_meas, 1),
            "frac_of_achievable": round(achieved / peak_meas, 4),
            "achievable_peak_note": "bf16 MFMA chains on registers at the running clock (libsdpa_probe.so)",
            "algorithmic_flop_per_launch": kv_flop,
            "algorithmic_unit": "8*D FLOP per allowed (query, key) pair (S, dP, dV, dK)",
            "avg_launch_ms": round(statistics.mean(main_ms), 4),
            "kernels": kernels,
            "backward_useful": {"flop": bwd_flop, "algorithmic": "10*D FLOP per allowed pair",
                                "avg_ms": round(statistics.mean(bwd_ms), 4), "achieved": round(bwd_useful, 1),
                                "frac": round(bwd_useful / BF16_PEAK_TFLOPS, 4), "target_frac": 0.5},
        },
    }
    result["env"] = {"device": torch.cuda.get_device_name(dev), "torch": torch.__version__,
                     "hip": getattr(torch.version, "hip", None), "arch": "gfx950",
                     "abi": sdpa.load().sdpa_abi_version(),
                     "clock_ghz_from_mfma_probe": round(peak_meas / (BF16_PEAK_TFLOPS / 2.4), 3),
                     "tiles": tile_config(w)}
    if not a.no_cpu_baseline:
        log("timing the fp64 oracle on a bounded sample ...")
        result["cpu_baseline"] = cpu_baseline(w, cpu_inp, a.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
