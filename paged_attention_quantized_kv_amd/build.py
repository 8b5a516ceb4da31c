"""Build libkvq.so (the HIP C-ABI library) in-tree with hipcc for gfx950.

Every source is compiled to an object of its own, in parallel (the attention
kernels are split by KV format over attn_f<FMT>.hip), then linked into one
shared library.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libkvq.so")
OBJ_DIR = os.path.join(HERE, "_build")
SOURCES = [os.path.join(HERE, "csrc", f) for f in
           ("kvq_api.hip", "append.hip", "attn.hip", "attn_f0.hip", "attn_f1.hip", "attn_f2.hip", "attn_f3.hip",
            "attn_f4.hip", "check.hip", "probe.hip", "shape.cpp")]
HEADERS = [os.path.join(HERE, "csrc", f) for f in ("internal.h", "shape.h", "quant_row.h", "attn_kernels.h")] + \
          [os.path.join(ROOT, "include", "kvq.h"), os.path.join(ROOT, "include", "kvq_probe.h")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # IEEE fp32 division: quantization codes are decided by x / scale
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # no packed-fp32 instructions in any kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]
NOISE = "is not a recognized feature for this target"


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if NOISE not in l)
    return r.returncode, err


def build(verbose: bool = False, jobs: int | None = None, out: str | None = None, src_dir: str | None = None,
          defines: tuple = ()) -> str:
    """Compile and link; `out`, `src_dir` and `defines` (-D flags) build a variant library
    (another tree's sources, or a compile-time option) beside the default one."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    lib = out or LIB
    obj_dir = OBJ_DIR if out is None else os.path.join(OBJ_DIR, os.path.basename(out)[:-3])
    os.makedirs(obj_dir, exist_ok=True)
    sources = SOURCES if src_dir is None else [os.path.join(src_dir, os.path.basename(s)) for s in SOURCES]
    objs = [os.path.join(obj_dir, os.path.splitext(os.path.basename(s))[0] + ".o") for s in sources]
    flags = HIPCC_FLAGS + [f"-D{d}" for d in defines]
    if src_dir is not None:
        flags += ["-I", os.path.join(src_dir, "..", "..", "include")]
    jobs = jobs or min(len(SOURCES), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        res = list(ex.map(lambda so: _run([hipcc] + flags + ["-c", so[0], "-o", so[1]]), zip(sources, objs)))
    for (rc, err), src in zip(res, sources):
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n" + err)
        if verbose and err.strip():
            print(err, file=sys.stderr)
    rc, err = _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", lib + ".tmp"])
    if rc != 0:
        raise RuntimeError("hipcc link failed:\n" + err)
    os.replace(lib + ".tmp", lib)
    return lib


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose=True))
