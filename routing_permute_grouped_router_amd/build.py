"""Build the gfx950 HIP library libmoe.so in-tree (hipcc, no JIT cache)."""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe.so")
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep the compiler from emitting packed fp32 ALU forms.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]


def sources() -> list:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


# The grouped GEMM kernels count their own memory operations (s_waitcnt
# vmcnt with fixed counts against inline-asm loads); scratch spills would add
# memory operations the counts do not know about, so they must have none.
_USAGE = re.compile(r"remark: Function Name: (\S+)|remark:\s+ScratchSize \[bytes/lane\]: (\d+)")


def _check_scratch(src: str, text: str) -> None:
    fn = None
    for m in _USAGE.finditer(text):
        if m.group(1):
            fn = m.group(1)
        elif fn and "grouped_gemm" in fn and int(m.group(2)) > 0:
            raise RuntimeError(f"{src}: kernel {fn} spills to scratch ({m.group(2)} bytes per lane)")


def _compile(src: str, verbose: bool, extra: list) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *extra, "-x", "hip", "-c", src, "-o", obj, "-Rpass-analysis=kernel-resource-usage"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    _check_scratch(src, r.stdout + r.stderr)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and "kernel-resource-usage" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if out.strip() and verbose:
        print(out)
    return obj


def build(verbose: bool = False, jobs: int | None = None, extra: tuple = ()) -> str:
    """extra: further hipcc flags for every compile and the link (host-only
    sanitizer builds pass -Xarch_host forms here)."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, list(extra)), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *extra, "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
