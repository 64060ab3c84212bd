"""Build libsdpa.so (gfx950) in-tree with hipcc.

    python -m sdpa_backward_amd.build          # compile every source, link
    python -m sdpa_backward_amd.build --asm    # also keep gfx950 assembly under _build/asm

Every HIP source is compiled with the packed-fp32 instructions disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops): the compiler would
otherwise form v_pk_* fp32 ops on its own. The machine scheduler runs its
ILP strategy (-amdgpu-sched-strategy=iterative-ilp). No kernel uses atomics.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsdpa.so")
SOURCES = ["sdpa_api.hip", "qs_mfma.hip", "kv_mfma.hip", "kv16_mfma.hip", "dsq_mfma.hip", "f32_valu.hip",
           "sinks.hip"]
# measurement helper, its own library (include/sdpa_probe.h)
PROBE_LIB = os.path.join(PKG, "libsdpa_probe.so")
PROBE_SOURCES = ["probe_mfma.hip"]
ARCH = "gfx950"
# per-source extra flags: the dK/dV kernels that fill all 512 registers (the
# 16-key one at D = 512, the 32-key one) keep MFMA results in VGPRs; their tile
# loops then move far fewer values between the register files (16-key D = 512:
# 23 instead of 148; 32-key D = 256: 69 instead of 256), and the passes run
# 5-7 % faster. The 16-key D = 256 code does not change.
SOURCE_FLAGS = {"kv16_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "kv_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def common_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # the ILP-oriented machine scheduler keeps more LDS reads in flight ahead of
        # their MFMAs in these one-wave-per-SIMD kernels (measured faster than default)
        "-mllvm", "-amdgpu-sched-strategy=iterative-ilp",
        "-Wno-unused-result",
        f"-I{os.path.join(ROOT, 'include')}",
    ]


def _compile(src, asm):
    odir = os.path.join(BUILD, "asm") if asm else BUILD
    os.makedirs(odir, exist_ok=True)
    obj = os.path.join(odir, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *common_flags(), *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if asm:
        cmd.append("-save-temps=obj")
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; that is harmless
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(msgs))
    return obj, msgs


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)


def build(asm: bool = False, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = dict(zip(srcs, ex.map(lambda s: _compile(s, asm), srcs)))
    if verbose:
        for _, msgs in results.values():
            for m in msgs:
                print(m)
    _link([results[s][0] for s in SOURCES], LIB)
    _link([results[s][0] for s in PROBE_SOURCES], PROBE_LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", action="store_true")
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args()
    print(build(asm=a.asm, verbose=a.verbose))
    sys.exit(0)
