"""Build libpkvfp8.so in-tree with hipcc for gfx950.

Usage: ``python -m paged_kv_fp8_amd.build`` (or ``build()`` from Python).
Always recompiles. The library lands next to this file, where
``paged_kv_fp8_amd.native`` loads it.
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpkvfp8.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["api.cpp", "plan.cpp", "decode_gqa.hip", "decode_mla.hip", "merge.hip", "producers.hip", "probe.hip"]

# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU ops
# (v_pk_*_f32); the host pass warns that it does not know the feature.
# -amdgpu-atomic-optimizer-strategy=None: a lane-0 atomic stays one atomic; the
# optimizer's wave-wide rewrite reads its result back at once, which waits
# for every load issued before it.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "-mllvm", "-amdgpu-atomic-optimizer-strategy=None", "-Wall", "-Wno-unused-function",
         "-Wno-unknown-pragmas"]


def build(verbose=False, extra_flags=(), jobs=None, out=LIB):
    """Compile every source (in parallel, one hipcc per source) and link the
    library at `out` (default: the in-tree library); returns its path."""
    from concurrent.futures import ThreadPoolExecutor

    build_dir = os.path.join(HERE, "_build" if out == LIB else "_build_" + os.path.splitext(os.path.basename(out))[0])
    os.makedirs(build_dir, exist_ok=True)
    cmds, objs = [], []
    for src in SOURCES:
        obj = os.path.join(build_dir, src + ".o")
        cmd = [HIPCC, *FLAGS, *extra_flags, "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        cmds.append(cmd)
        objs.append(obj)
    jobs = jobs or min(len(cmds), max(1, min(os.cpu_count() or 1, 8)))
    with ThreadPoolExecutor(jobs) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = out + ".tmp"
    _run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs], verbose)
    os.replace(tmp, out)
    return out


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(ln for ln in r.stderr.splitlines() if noise not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
