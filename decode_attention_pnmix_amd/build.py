"""Build libpnmix.so (gfx950 HIP kernels + the C ABI host code) in-tree with hipcc.

Each source compiles to its own object in parallel (decode.hip, with its many kernel
instantiations, dominates), then hipcc links the shared library.
"""
from __future__ import annotations

import os
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpnmix.so")
SOURCES = ["pnmix_api.hip", "score.hip", "quant.hip", "decode.hip", "decode_generic.hip",
           "prefill.hip", "cache_ops.hip"]

# -ffp-contract=off: no FMA contraction (bit-exact quantizer and score).
# packed-fp32-ops off: no v_pk_{add,mul,fma}_f32 generated from fp32 code.
# HIP's default correctly rounded fp32 division and square root stay on (no fast-math).
COMPILE = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
           "-fno-fast-math", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall",
           "-Wno-unused-function"]
LINK = ["--offload-arch=gfx950", "-shared", "-fPIC"]


def hipcc() -> str:
    for p in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if p and (os.path.sep not in p or os.path.exists(p)):
            return p
    return "hipcc"


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}\n{res.stdout}\n"
                           f"{res.stderr}")
    return res


def build(verbose: bool = False, jobs: int | None = None) -> str:
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    with tempfile.TemporaryDirectory(prefix="pnmix_build_") as tmp:
        cmds, objs = [], []
        for s in SOURCES:
            obj = os.path.join(tmp, s.replace(".hip", ".o"))
            objs.append(obj)
            cmds.append([hipcc()] + COMPILE + inc + ["-c", os.path.join(CSRC, s), "-o", obj])
        if verbose:
            for c in cmds:
                print(" ".join(c))
        n = jobs or min(len(cmds), max(1, (os.cpu_count() or 1)))
        with ThreadPoolExecutor(max_workers=n) as ex:
            list(ex.map(_run, cmds))
        out = LIB + ".tmp"
        link = [hipcc()] + LINK + ["-o", out] + objs
        if verbose:
            print(" ".join(link))
        _run(link)
        os.replace(out, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
