"""Build the HIP attention library in-tree for gfx950.

``python -m attention_fa_fwd_amd.build`` (or ``build_library()``) compiles every
``csrc/*.hip`` with hipcc (one process per file, in parallel) and links them into
``attention_fa_fwd_amd/libfa_fwd.so``.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libfa_fwd.so")

ARCH = "gfx950"
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # No packed-fp32 VALU instructions in the device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
]
# Extra flags of single translation units.  The backward kernels run about 2% faster
# without the post-register-allocation machine scheduler (interleaved timing of both
# backward workloads); the forward kernels are unaffected by it and keep the default.
PER_FILE_FLAGS = {
    "fa_bwd.hip": ["-mllvm", "-enable-post-misched=0"],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def build_library(verbose: bool = True, extra_flags=None, jobs=None) -> str:
    """Compile every ``csrc/*.hip`` to an object (in parallel) and link the shared
    library; returns its path.  Raises CalledProcessError on failure."""
    import concurrent.futures as cf
    import tempfile

    cc = hipcc()
    flags = [f for f in HIPCC_FLAGS if f != "-shared"] + list(extra_flags or [])
    with tempfile.TemporaryDirectory(prefix="fa_build_") as tmpdir:
        objs, cmds = [], []
        for src in sources():
            obj = os.path.join(tmpdir, os.path.basename(src)[:-4] + ".o")
            objs.append(obj)
            extra = PER_FILE_FLAGS.get(os.path.basename(src), [])
            cmds.append([cc, *flags, *extra, f"-I{INCLUDE}", f"-I{CSRC}", "-c", src, "-o", obj])
        n = jobs or min(len(cmds), max(1, min(16, os.cpu_count() or 1)))

        def run(cmd):
            if verbose:
                print("[build]", " ".join(cmd), flush=True)
            subprocess.run(cmd, check=True)

        with cf.ThreadPoolExecutor(max_workers=n) as ex:
            for fut in [ex.submit(run, c) for c in cmds]:
                fut.result()
        tmp = LIB_PATH + ".tmp"
        link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
        run(link)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


PROBE_SRC = os.path.join(PKG, "probe", "fa_peak_probe.hip")
PROBE_PATH = os.path.join(PKG, "libfa_probe.so")


def build_probe(verbose: bool = True) -> str:
    """Compile the benchmark's device and MFMA-peak probe (``probe/fa_peak_probe.hip``) into
    ``libfa_probe.so``, apart from the attention library; returns its path."""
    flags = [f for f in HIPCC_FLAGS]
    tmp = PROBE_PATH + ".tmp"
    cmd = [hipcc(), *flags, PROBE_SRC, "-o", tmp]
    if verbose:
        print("[build]", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, PROBE_PATH)
    return PROBE_PATH


C_CALLER_SRC = os.path.join(ROOT, "tests", "c", "fa_c_caller.c")
C_CALLER_BIN = os.path.join(ROOT, "tests", "c", "fa_c_caller")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_c_caller(verbose: bool = True) -> str:
    """Compile the plain-C test caller of the library (gcc, C99, HIP runtime API) against
    the built libfa_fwd.so; returns the binary's path."""
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler (gcc) found for the C-ABI test caller")
    cmd = [cc, "-std=c99", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROCM}/include", f"-I{INCLUDE}", C_CALLER_SRC, "-o", C_CALLER_BIN,
           f"-L{PKG}", "-lfa_fwd", f"-L{ROCM}/lib", "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../attention_fa_fwd_amd", f"-Wl,-rpath,{ROCM}/lib"]
    if verbose:
        print("[build]", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return C_CALLER_BIN


def main(argv=None) -> int:
    build_library(verbose=True, extra_flags=(argv if argv is not None else sys.argv[1:]))
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
