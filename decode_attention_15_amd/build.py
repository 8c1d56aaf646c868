"""Compile libkvq.so (HIP kernels + C ABI) for gfx950, in-tree."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkvq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    # no packed fp32 (v_pk_*_f32) anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wno-unused-command-line-argument",
]

SOURCES = {
    # the write path must round exactly as the cache format states: no contraction
    "kvq_write.hip": ["-ffp-contract=off"],
    "kvq_decode.hip": [],
    # matrix-core results straight into VGPRs (no accumulator-register copies in the group loop)
    "kvq_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    # read-bandwidth probe of the decode's read pattern
    "kvq_probe.hip": [],
    "kvq_api.cpp": ["-x", "hip", "-ffp-contract=off"],
    "kvq_calib.cpp": ["-x", "hip", "-ffp-contract=off"],
}


def _compile(name: str, extra, csrc: str = CSRC, build_dir: str = BUILD) -> str:
    src = os.path.join(csrc, name)
    obj = os.path.join(build_dir, name + ".o")
    cmd = [HIPCC, *COMMON, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {name}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, csrc: str = CSRC, out: str = LIB, build_dir: str = BUILD) -> str:
    """Compile the sources in `csrc` into the shared library `out` (default: the in-tree libkvq.so)."""
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda kv: _compile(*kv, csrc=csrc, build_dir=build_dir), SOURCES.items()))
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
