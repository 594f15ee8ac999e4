"""CPU sanitizer run of the oracle, the input generator and the host side of
libmoe (argument checks, workspace carving, the fused calls' sequencing).

The three libraries are rebuilt in a scratch copy of the repository with
clang's AddressSanitizer and UndefinedBehaviorSanitizer (UB is fatal), the
HIP library with the sanitizers on its host code only (-Xarch_host; the GPU
code is unchanged), and the CPU test suite (-m "not gpu") runs against those
builds with the sanitizer runtime preloaded into the interpreter.  The
working tree is not touched.  No GPU is needed or used.

    python tests/sanitize.py [extra pytest arguments]

Exit status: pytest's (a sanitizer report aborts the run and fails it).
Leak checking is off: the interpreter and torch keep allocations alive at
exit by design."""
import glob
import os
import shutil
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LLVM = "/opt/rocm/llvm"
CLANG = os.path.join(LLVM, "bin", "clang")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]
# hipcc: every sanitizer flag applies to the host compilation only
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-shared-libsan"]


def _runtime() -> str:
    libs = glob.glob(os.path.join(LLVM, "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so"))
    if not libs:
        raise SystemExit("clang's shared ASan runtime was not found under " + LLVM)
    return libs[0]


def _copy(dst: str) -> None:
    skip = shutil.ignore_patterns("*.so", "*.o", "_build", "__pycache__", "*.tmp")
    for name in ("include", "oracle", "routing_permute_grouped_router_amd", "tests"):
        shutil.copytree(os.path.join(ROOT, name), os.path.join(dst, name), ignore=skip)
    for name in ("pytest.ini", "__graft_entry__.py", "bench.py"):
        shutil.copy2(os.path.join(ROOT, name), dst)


def _cc(src: str, out: str) -> None:
    cmd = [CLANG, "-O1", "-fPIC", "-shared", "-shared-libsan", *SAN, "-Wall", "-o", out, src, "-lm"]
    print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def main() -> int:
    rt = _runtime()
    work = tempfile.mkdtemp(prefix="moe_sanitize_")
    try:
        _copy(work)
        _cc(os.path.join(work, "oracle", "moe_oracle.c"), os.path.join(work, "oracle", "liboracle.so"))
        wdir = os.path.join(work, "routing_permute_grouped_router_amd", "workload")
        _cc(os.path.join(wdir, "workload_gen.c"), os.path.join(wdir, "libworkload.so"))
        sys.path.insert(0, work)
        from routing_permute_grouped_router_amd import build as hipbuild

        print("libmoe.so with host sanitizers:", hipbuild.build(extra=tuple(HOST_SAN)), flush=True)
        env = dict(os.environ)
        env["LD_PRELOAD"] = rt  # the sanitizer runtime must be the interpreter's first library
        env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
        env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
        # The runtime is live and the libraries are the instrumented ones: an
        # oracle call told to write past the end of its output must be stopped.
        probe = ("import numpy as np; from oracle import oracle as orc; "
                 "src = np.zeros(8192); dst = np.zeros(4096, np.uint16); "
                 "orc._load().or_bf16_from_double_array(src.ctypes.data, dst.ctypes.data, 8192)")
        r = subprocess.run([sys.executable, "-c", probe], cwd=work, env=env, capture_output=True, text=True)
        if r.returncode == 0 or "AddressSanitizer" not in r.stderr:
            raise SystemExit("the sanitizer did not catch a planted overflow: the run would prove nothing")
        print("sanitizer live: a planted overflow in the oracle was reported", flush=True)
        lib = os.path.join(work, "routing_permute_grouped_router_amd", "libmoe.so")
        syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
        if "__asan_report" not in syms or "__ubsan_handle" not in syms:
            raise SystemExit("libmoe.so's host code is not instrumented")
        cmd = [sys.executable, "-m", "pytest", "tests", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
               *sys.argv[1:]]
        print(" ".join(cmd), flush=True)
        return subprocess.run(cmd, cwd=work, env=env).returncode
    finally:
        shutil.rmtree(work, ignore_errors=True)


if __name__ == "__main__":
    sys.exit(main())
