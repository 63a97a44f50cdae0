"""Builds libdrafthead.so from csrc/*.hip with hipcc for gfx950."""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libdrafthead.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no v_pk_*_f32: keep fp32 VALU work in unpacked instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # quantizer bit-exactness: every float op rounds on its own
    "-ffp-contract=off",
    # keep the quantizer's one-lane atomicMax as written (no wave-level
    # rewrite of it by the atomic optimizer); the device pass reads this
    # option, the host pass reports it unused
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wall", "-Wno-unused-result",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def _run(cmd: list[str]) -> str:
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    return err


def build(verbose: bool = False) -> str:
    """Compiles every source to an object in parallel, then links."""
    obj_dir = os.path.join(ROOT, "_build", "drafthead")
    os.makedirs(obj_dir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc")]
    compile_flags = [f for f in HIP_FLAGS if f != "-shared"]
    jobs = []
    for src in sources():
        obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
        jobs.append((obj, [HIPCC, *compile_flags, *inc, "-c", src, "-o", obj]))
    workers = min(len(jobs), os.cpu_count() or 1, 8)
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        errs = list(ex.map(lambda j: _run(j[1]), jobs))
    tmp = LIB + ".tmp"
    errs.append(_run([HIPCC, *HIP_FLAGS, *[o for o, _ in jobs], "-o", tmp]))
    if verbose:
        for e in errs:
            if e.strip():
                print(e)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
