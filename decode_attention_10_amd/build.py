"""Builds the HIP sources into in-tree shared libraries for gfx950.

    python decode_attention_10_amd/build.py        (or build_all() from Python)

libkvq.so       <- decode_attention_10_amd/csrc/*.hip   (the C ABI of include/kvq.h)
libkvq_debug.so <- the same sources with -DKVQ_DEBUG (device-side bounds checks)
libkvq_synth.so <- kvq_synth/synth.hip                 (seeded input generator)

Flags: contraction off (the quantizer's fp32 arithmetic must be one rounding per
operation), packed-fp32 instructions disabled, IEEE divide (hipcc's default), matrix
instructions writing ordinary VGPRs (no accumulator-register copies).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wno-unused-command-line-argument",
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def _build_lib(sources, out, includes, objdir, extra=()):
    os.makedirs(objdir, exist_ok=True)
    objs = []
    cmds = []
    for src in sources:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmds.append([HIPCC, *CFLAGS, *extra, *[f"-I{i}" for i in includes], "-c", src, "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
        list(ex.map(_run, cmds))
    tmp = out + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, out)
    return out


def build_kvq(debug: bool = False) -> str:
    """libkvq.so, or with debug=True libkvq_debug.so: the same library compiled with
    -DKVQ_DEBUG (device-side bounds checks that set flags instead of trapping; every entry
    point then waits for its launches and reports a failed check as KVQ_ERR_HIP).  Select
    it at run time with KVQ_LIBRARY=<path>."""
    csrc = os.path.join(PKG, "csrc")
    srcs = sorted(os.path.join(csrc, f) for f in os.listdir(csrc) if f.endswith(".hip"))
    name, sub = ("libkvq_debug.so", "kvq_debug") if debug else ("libkvq.so", "kvq")
    return _build_lib(srcs, os.path.join(PKG, name), [os.path.join(ROOT, "include"), csrc],
                      os.path.join(ROOT, "_build", sub), ["-DKVQ_DEBUG"] if debug else [])


def build_synth() -> str:
    d = os.path.join(ROOT, "kvq_synth")
    return _build_lib([os.path.join(d, "synth.hip")], os.path.join(d, "libkvq_synth.so"),
                      [d], os.path.join(ROOT, "_build", "synth"))


def build_all() -> list[str]:
    return [build_kvq(), build_kvq(debug=True), build_synth()]


if __name__ == "__main__":
    for p in build_all():
        print(p)
    sys.exit(0)
