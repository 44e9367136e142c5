"""Build librpa.so in-tree with hipcc for gfx950.

    python -m ragged_paged_kv_append_amd.build        # or: python ragged_paged_kv_append_amd/build.py

Compiles every source under csrc/ to an object in _build/ (in parallel) and
links ragged_paged_kv_append_amd/librpa.so.  It always recompiles: this is the
"does it build" check as well as the build.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "librpa.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
          "-I" + os.path.join(PKG, "..", "include")]
# Packed fp32 instructions are kept out of the device code on purpose.
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


# Per-file device flags.  The prefill kernel runs with the IEEE mode bit off:
# its row maxima then need no NaN-quieting operand copies (no NaN reaches them:
# masked keys carry a large negative finite value and unused key slots are
# filled from a valid key).
FILE_FLAGS = {
    # the prefill step loop is unrolled over its 64 slots (two steps): a body
    # above the default pragma threshold would stay rolled, its register
    # arrays in scratch memory
    "prefill.hip": ["-mno-amdgpu-ieee", "-fno-honor-nans", "-mllvm", "-pragma-unroll-threshold=200000"],
    "mla.hip": ["-mno-amdgpu-ieee", "-fno-honor-nans"],
}


def sources():
    out = []
    for root, _, files in os.walk(CSRC):
        for f in sorted(files):
            if f.endswith((".hip", ".cpp")):
                out.append(os.path.join(root, f))
    return sorted(out)


def _compile(src: str) -> tuple[str, str, int, str]:
    rel = os.path.relpath(src, CSRC).replace(os.sep, "_")
    obj = os.path.join(BUILD, rel + ".o")
    if src.endswith(".hip"):
        extra = FILE_FLAGS.get(os.path.basename(src), [])
        cmd = [HIPCC, "-x", "hip", *DEVICE, *COMMON, *extra, "-c", src, "-o", obj]
    else:
        cmd = [HIPCC, *COMMON, "-D__HIP_PLATFORM_AMD__", "-c", src, "-o", obj]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    return obj, " ".join(cmd), proc.returncode, proc.stdout + proc.stderr


def build(verbose: bool = False) -> str:
    """Compile and link; returns the library path.  Raises on failure."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    objs = []
    errors = []
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 4)) as ex:
        for obj, cmd, rc, log in ex.map(_compile, srcs):
            objs.append(obj)
            if verbose or rc != 0:
                print(cmd)
                if log.strip():
                    print(log)
            if rc != 0:
                errors.append(obj)
    if errors:
        raise RuntimeError("compilation failed: " + ", ".join(errors))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "--offload-arch=" + ARCH, "-fPIC", *objs, "-o", tmp]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        print(" ".join(cmd))
        print(proc.stdout + proc.stderr)
        raise RuntimeError("link failed")
    shutil.move(tmp, LIB)
    return LIB


if __name__ == "__main__":
    try:
        path = build(verbose="-v" in sys.argv)
    except RuntimeError as e:
        print(f"build failed: {e}", file=sys.stderr)
        sys.exit(1)
    print(path)
