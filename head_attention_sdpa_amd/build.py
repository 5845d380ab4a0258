"""Build libattn_sdpa.so (the C-ABI library) for gfx950 with hipcc, in-tree.

    python -m head_attention_sdpa_amd.build

Each source is compiled to an object in parallel, then linked.  All HIP code
is built with packed-fp32 instructions disabled (-packed-fp32-ops)."""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libattn_sdpa.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs (gfx950 allows it): no AGPR<->VGPR copies
    # around the softmax and the rescaling of the output accumulator
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _compile(src: str, cc: str, extra: list[str], build_dir: str = BUILD_DIR) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [cc, *COMMON, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(extra: list[str] | None = None, verbose: bool = False, out: str | None = None) -> str:
    """Compile every source and link the library (LIB_PATH unless `out` is
    given, e.g. for a tuning variant built with extra -D flags).  Always
    recompiles."""
    build_dir = BUILD_DIR if out is None else os.path.join(BUILD_DIR, os.path.basename(out))
    os.makedirs(build_dir, exist_ok=True)
    cc = hipcc()
    extra = list(extra or [])
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, cc, extra, build_dir), srcs))
    target = LIB_PATH if out is None else out
    tmp = target + f".tmp{os.getpid()}"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, target)
    if verbose:
        print(f"built {target} from {len(srcs)} sources")
    return target


DRIVER_SRC = os.path.join(ROOT, "tests", "c_abi", "sdpa_driver.cpp")
DRIVER_PATH = os.path.join(ROOT, "tests", "c_abi", "sdpa_driver")


def build_c_driver(verbose: bool = False) -> str:
    """Compile the test program that calls the library through its C ABI
    alone (tests/c_abi/sdpa_driver.cpp), linked against LIB_PATH with an
    $ORIGIN-relative run path.  Always recompiles."""
    cc = hipcc()
    tmp = DRIVER_PATH + f".tmp{os.getpid()}"
    rpath = "$ORIGIN/" + os.path.relpath(PKG, os.path.dirname(DRIVER_PATH))
    cmd = [cc, f"--offload-arch={ARCH}", "-O2", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), DRIVER_SRC, "-o", tmp,
           "-L", PKG, "-lattn_sdpa", f"-Wl,-rpath,{rpath}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"driver build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, DRIVER_PATH)
    if verbose:
        print(f"built {DRIVER_PATH}")
    return DRIVER_PATH


if __name__ == "__main__":
    build(extra=sys.argv[1:], verbose=True)
    build_c_driver(verbose=True)
