"""Summaries of rocprofv3 output for the attention kernels (kernel time,
hardware counters, HBM traffic of the dK/dV kernel).

    python -m sdpa_backward_amd.profsum OUTDIR [--workload NAME] [--cmd-prefix TEXT]

OUTDIR is what collect_profiles.sh wrote: trace/ (kernel trace), p1..p4/
(counter passes), trace.log (the bench JSON line of the traced run). Writes
kernel_stats_<tag>.md, counters_<tag>.md and traffic_<dK/dV kernel>_<tag>.json into
OUTDIR; <tag> names the workload by its mask and sizes.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

# sources of each dK/dV kernel (and the build script, which holds the compiler
# flags), hashed into its traffic file: the counters hold only for the code
# they were taken on
KERNEL_SOURCES = {"kv16_kernel": ["sdpa_backward_amd/csrc/kv16_mfma.hip", "sdpa_backward_amd/csrc/common.h",
                                  "sdpa_backward_amd/build.py"],
                  "dsq_kernel": ["sdpa_backward_amd/csrc/dsq_mfma.hip", "sdpa_backward_amd/csrc/common.h",
                                 "sdpa_backward_amd/build.py"],
                  "kv_kernel": ["sdpa_backward_amd/csrc/kv_mfma.hip", "sdpa_backward_amd/csrc/common.h",
                                "sdpa_backward_amd/build.py"]}
COPY_KERNEL = "copyBuffer"   # the 1 GiB device copy bench.py --copy-probe runs
COPY_BYTES = 1 << 30


def sources_sha256(kernel: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def tag(w) -> str:
    mask = {"causal_window": f"window{w.window}", "window": f"twosided{w.window}"}.get(w.mask, w.mask)
    length = f"L{w.L}" if w.Lkv == w.L else f"Lq{w.L}_Lk{w.Lkv}"
    return f"{mask}_{length}_D{w.D}"


def short(name: str) -> str:
    """Kernel name without its signature and element type: sdpa::qs_kernel<256, 0>, sdpa::kv_kernel<256>."""
    m = re.match(r"_ZN4sdpa\d+(\w+?_kernel)I((?:Li\d+E)+)", name)  # names the tool left mangled
    if re.match(r"_ZN4sdpa\d+kv_reduce_kernel", name):
        return "sdpa::kv_reduce_kernel"
    if m:
        ints = re.findall(r"Li(\d+)E", m.group(2))
        keep = 2 if m.group(1) in ("qs_kernel", "qs_combine_kernel") else 1
        return f"sdpa::{m.group(1)}<{', '.join(ints[:keep])}>"
    name = name.replace("void ", "")
    name = re.sub(r"\(.*", "", name)
    name = re.sub(r"<(\d+), (\d+), [^<>]+>", r"<\1, \2>", name)  # the workloads here are bf16
    name = re.sub(r"^(sdpa::kv(?:16)?_kernel)<(\d+), [^<>]+>", r"\1<\2>", name)
    name = re.sub(r"^(sdpa::kv_reduce_kernel)<[^<>]+>", r"\1", name)
    name = re.sub(r"^(sdpa::(dsq|delta)_kernel)<(\d+), [^<>]+>", r"\1<\3>", name)
    return name


def band_geometry(w):
    """(row blocks, key tiles per block) of the dS band buffer for this workload (the library's
    rule: D = 256 with the 16-key dK/dV kernel, i.e. at least 256 blocks of 128 keys; 128-row
    blocks, 64-key tiles, a block's band at most 9 D keys wide), or None."""
    if w.D != 256 or w.dtype == "f32" or -(-w.Lkv // 128) * w.Hkv * w.B < 256:
        return None
    off = w.Lkv - w.L
    lo, hi = -(w.L - 1), w.Lkv - 1
    if w.mask == "causal":
        hi = off
    if w.mask == "causal_window":
        lo, hi = off - w.window + 1, off
    if w.mask == "window":
        lo, hi = off - w.window + 1, off + w.window - 1
    lo, hi = max(lo, -(w.L - 1)), min(hi, w.Lkv - 1)
    nkb = min((127 + hi) // 64 - lo // 64 + 1, -(-w.Lkv // 64))
    return (-(-w.L // 128), nkb) if nkb * 64 <= 9 * w.D else None


def key_range_shares(w):
    """Shares of the forward's (and, without the dS band buffer, the dQ pass's) key-range split
    on this workload (1: none), from the library's own workspace rule."""
    import torch
    from sdpa_backward_amd import fwd_workspace_bytes
    b = fwd_workspace_bytes(w.B, w.Hq, w.group, w.L, w.Lkv, w.D, torch.bfloat16, w.mask, w.window)
    return b // (w.B * w.Hq * w.L * (w.D + 2) * 4) if b else 1


def roles(w):
    """kernel-name prefix -> (role, useful FLOP per call, algorithmic bytes read, written)."""
    from bench import allowed_pairs
    N = allowed_pairs(w)
    e = 2  # bf16
    q = w.B * w.Hq * w.L * w.D * e
    kv = w.B * w.Hkv * w.Lkv * w.D * e
    row = w.B * w.Hq * w.L * 4
    D = w.D
    r = {
        f"sdpa::qs_kernel<{D}, 0>": ("forward (O, lse)", 4 * D * N, q + 2 * kv, q + row),
        f"sdpa::qs_kernel<{D}, 1>": ("dQ pass (+Delta)", 6 * D * N, 3 * q + 2 * kv + row, q + row),
        f"sdpa::kv_kernel<{D}>": ("dK/dV pass (32-key waves)", 8 * D * N, 2 * q + 2 * kv + 2 * row, 2 * kv),
        "sdpa::kv_reduce_kernel": ("dK/dV share reduce (split pass)", 0, 0, 2 * kv),
        f"sdpa::kv16_kernel<{D}>": ("dK/dV pass (16-key waves)", 8 * D * N, 2 * q + 2 * kv + 2 * row, 2 * kv),
    }
    bg = band_geometry(w)
    if bg:  # the backward that keeps dS for the band: the dK/dV pass also writes it
        band = w.B * w.Hq * bg[0] * bg[1] * 64 * 128 * e
        r[f"sdpa::delta_kernel<{D}>"] = ("Delta pass", 0, 2 * q, row)
        r[f"sdpa::kv16_kernel<{D}>"] = ("dK/dV pass writing dS (16-key waves)", 8 * D * N,
                                        2 * q + 2 * kv + 2 * row, 2 * kv + band)
        r[f"sdpa::dsq_kernel<{D}>"] = ("dQ = scale dS K pass", 2 * D * N, band + kv, q)
    ns = key_range_shares(w)
    if ns > 1:  # small grid: each query tile's key range split into ns shares, fp32 partials merged
        part = ns * w.B * w.Hq * w.L * 4
        r[f"sdpa::qs_kernel<{D}, 0>"] = (f"forward, key range split in {ns}", 4 * D * N, q + 2 * kv, part * (D + 2))
        r[f"sdpa::qs_combine_kernel<{D}, 0>"] = ("forward split merge (O, lse)", 0, part * (D + 2), q + row)
        if not bg:
            r[f"sdpa::qs_kernel<{D}, 1>"] = (f"dQ pass (+Delta), key range split in {ns}", 6 * D * N,
                                             3 * q + 2 * kv + row, part * D + row)
            r[f"sdpa::qs_combine_kernel<{D}, 1>"] = ("dQ split merge", 0, part * D, q)
    return r


def read_trace(d):
    f = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)[0]
    rows = sorted(csv.DictReader(open(f)), key=lambda r: int(r["Start_Timestamp"]))
    per = collections.defaultdict(list)
    for r in rows:
        per[short(r["Kernel_Name"])].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return per


def read_counters(d):
    f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)[0]
    agg = collections.defaultdict(float)
    names = {}
    for r in csv.DictReader(open(f)):
        k = (r["Dispatch_Id"], r["Counter_Name"])
        agg[k] += float(r["Counter_Value"])
        names[r["Dispatch_Id"]] = short(r["Kernel_Name"])
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    for (disp, counter), v in agg.items():
        per[names[disp]][counter].append(v)
    return per


def bench_line(path):
    if not os.path.exists(path):
        return None
    for line in open(path):
        line = line.strip()
        if line.startswith("{") and '"metric"' in line:
            return json.loads(line)
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("outdir")
    ap.add_argument("--workload", default="bf16_window1024_L16384_D256_h32kv16")
    ap.add_argument("--steps", type=int, default=10, help="timed steps of the traced bench run")
    a = ap.parse_args()
    from workloads import BY_NAME
    w = BY_NAME[a.workload]
    t = tag(w)
    R = roles(w)
    out = a.outdir
    script = "bash sdpa_backward_amd/collect_profiles.sh OUTDIR " + w.name
    wl = f"{w.name}: B={w.B}, Hq={w.Hq}, Hkv={w.Hkv}, L={w.L}, D={w.D}, mask={w.mask}" + \
         (f", Lk={w.Lkv}" if w.Lkv != w.L else "") + (f", window={w.window}" if w.window else "")

    # ---------------------------------------------------------------- kernel time
    tr = read_trace(os.path.join(out, "trace"))
    bl = bench_line(os.path.join(out, "trace.log"))
    lines = [f"# Kernel time: {wl}", "",
             "Collected on one MI355X by (repository root):", "", "```", script, "```", "",
             "whose trace step is:", "", "```",
             f"rocprofv3 --kernel-trace --stats --output-format csv -d OUTDIR/trace -o run -- "
             f"python -u bench.py --no-cpu-baseline --workload {w.name} --steps {a.steps} --warmup 2", "```", "",
             f"'timed avg' is the mean over the last {a.steps} calls (the timed steps of bench.py).", "",
             "| kernel | role | calls | all avg (us) | timed avg (us) | min (us) | useful FLOP per call | TFLOP/s at timed avg |",
             "|---|---|---|---|---|---|---|---|"]
    timed = {}
    for k, v in tr.items():
        if k not in R:
            continue
        role, flop, _, _ = R[k]
        ta = statistics.mean(v[-a.steps:])
        timed[k] = ta
        lines.append(f"| `{k}` | {role} | {len(v)} | {statistics.mean(v):.1f} | {ta:.1f} | {min(v):.1f} | "
                     f"{flop:.4e} | {flop / ta / 1e6:.1f} |")
    main_k = next((k for k in (f"sdpa::kv16_kernel<{w.D}>", f"sdpa::kv_kernel<{w.D}>") if k in timed), None)
    if bl and main_k in timed:
        ev = bl["roofline"]["avg_launch_ms"] * 1e3
        red = next((k for k in tr if "kv_reduce_kernel" in k), None)
        if red:  # split dK/dV pass: the events bracket the share reduce as well
            t_ref = timed[main_k] + statistics.mean(tr[red][-a.steps:])
            what = f"`{main_k}` + `sdpa::kv_reduce_kernel` (split pass; the events also span the gap between the two launches)"
        else:
            t_ref, what = timed[main_k], f"`{main_k}`"
        lines += ["", f"In-bench HIP events around {what} in the same run (mean over the timed steps): "
                  f"{ev:.1f} us; rocprofv3 timed average: {t_ref:.1f} us "
                  f"({abs(ev - t_ref) / t_ref * 100:.1f} % apart)."]
    lines += ["", "Useful FLOP per call: forward 4*D*N, dQ pass 6*D*N (S, dP, dQ), dK/dV pass 8*D*N "
              "(S, dP, dV, dK), dQ = scale dS K pass 2*D*N; N = allowed (query, key) pairs over all heads. The "
              "backward's useful work is 10*D*N: with the dS band buffer (Delta pass, dK/dV pass writing dS, "
              "dS K pass) it computes 10*D*N, with the dQ pass that recomputes S and dP 14*D*N."]
    open(os.path.join(out, f"kernel_stats_{t}.md"), "w").write("\n".join(lines) + "\n")

    # ---------------------------------------------------------------- counters
    p = {i: read_counters(os.path.join(out, f"p{i}")) for i in range(1, len(PASSES) + 1)}

    def mean_of(i, k, c):
        v = p[i].get(k, {}).get(c)
        return statistics.mean(v) if v else float("nan")

    copy_k = next((k for k in p[3] if COPY_KERNEL in k), None)
    fetch_scale = COPY_BYTES / 1024 / mean_of(3, copy_k, "FETCH_SIZE") if copy_k else float("nan")
    copy_k4 = next((k for k in p[4] if COPY_KERNEL in k), None)
    write_scale = COPY_BYTES / 1024 / mean_of(4, copy_k4, "WRITE_SIZE") if copy_k4 else float("nan")
    lines = [f"# Hardware counters: {wl}", "", "Collected on one MI355X by (repository root):", "", "```", script,
             "```", "", "whose counter passes are (one rocprofv3 run each):", "", "```"]
    for i, cs in enumerate(PASSES, 1):
        lines.append(f"timeout -s KILL 120 rocprofv3 --pmc {cs} --output-format csv -d OUTDIR/p{i} -o run -- "
                     f"python -u bench.py --no-cpu-baseline --workload {w.name} --steps 2 --warmup 1 --cold 0 --copy-probe")
    lines += ["```", "",
              f"HBM byte scaling from the 1 GiB device copy in the same runs: FETCH_SIZE KiB x {fetch_scale:.3f} "
              f"= bytes read / 1024, WRITE_SIZE KiB x {write_scale:.3f} = bytes written / 1024.", "",
              "| kernel | MFMA busy | VALU instr / MFMA instr | LDS bank-conflict cycles / LDS active cycles "
              "| L2 hit rate | HBM read | algorithmic read | HBM write | algorithmic write |",
              "|---|---|---|---|---|---|---|---|---|"]
    traffic = None
    for k in R:
        if k not in timed:
            continue
        role, flop, ar, aw = R[k]
        busy = mean_of(1, k, "SQ_VALU_MFMA_BUSY_CYCLES") / (1024 * timed[k] * 1e-6 * 2.4e9)
        mf = mean_of(1, k, "SQ_INSTS_MFMA")
        valu = mean_of(1, k, "SQ_INSTS_VALU") / mf if mf > 0 else float("nan")
        lds_act = mean_of(2, k, "SQ_ACTIVE_INST_LDS")
        bank = mean_of(2, k, "SQ_LDS_BANK_CONFLICT") / lds_act if lds_act > 0 else float("nan")
        rd = mean_of(3, k, "FETCH_SIZE") * 1024 * fetch_scale
        wr = mean_of(4, k, "WRITE_SIZE") * 1024 * write_scale
        hit, miss = mean_of(5, k, "TCC_HIT_sum"), mean_of(5, k, "TCC_MISS_sum")
        lines.append(f"| `{k}` | {100 * busy:.1f} % | {valu:.2f} | {bank:.3f} | {100 * hit / (hit + miss):.1f} % "
                     f"| {rd / 1e9:.3f} GB | {ar / 1e9:.3f} GB | {wr / 1e9:.3f} GB | {aw / 1e9:.3f} GB |")
        if k == main_k:
            traffic = {"kernel": f"{main_k[len('sdpa::'):]} (dK/dV pass)", "workload": w.name,
                       "sources_sha256": sources_sha256("kv16_kernel" if "kv16" in main_k else "kv_kernel"),
                       "fetch_kib_per_launch": mean_of(3, k, "FETCH_SIZE"),
                       "write_kib_per_launch": mean_of(4, k, "WRITE_SIZE"),
                       "fetch_scale": fetch_scale, "write_scale": write_scale,
                       "hbm_bytes_per_launch": int(rd + wr),
                       "source": f"profiles/counters_{t}.md"}
    lines += ["", "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x timed avg kernel time x 2.4 GHz). "
              "SQ_INSTS_VALU counts the MFMA instructions too. Algorithmic bytes: every input read once, every "
              "output written once (bf16 tensors, fp32 lse / Delta rows)."]
    open(os.path.join(out, f"counters_{t}.md"), "w").write("\n".join(lines) + "\n")
    if traffic:
        name = "kv16_kernel" if "kv16" in traffic["kernel"] else "kv_kernel"
        json.dump(traffic, open(os.path.join(out, f"traffic_{name}_{t}.json"), "w"), indent=1)
    print(f"wrote summaries for {t} into {out}")


PASSES = [
    "SQ_WAVES SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA SQ_INSTS_VALU SQ_INSTS_LDS SQ_INSTS_SALU",
    "SQ_LDS_BANK_CONFLICT SQ_ACTIVE_INST_LDS SQ_WAIT_INST_LDS SQ_LDS_ADDR_CONFLICT SQ_INSTS_VMEM_RD SQ_INSTS_VMEM_WR SQ_WAIT_INST_ANY SQ_LDS_IDX_ACTIVE",
    "FETCH_SIZE",
    "WRITE_SIZE",
    "TCC_HIT_sum TCC_MISS_sum TCC_EA0_RDREQ_sum",
]

if __name__ == "__main__":
    main()
