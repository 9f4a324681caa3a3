"""Build libgdn_decode.so for gfx950 with hipcc, in place next to this file.

libgdn_decode_checked.so is the same source compiled with GDN_DEVICE_CHECKS:
every entry point validates its index arrays on the host before launching.
"""
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libgdn_decode.so")
LIB_CHECKED = os.path.join(PKG, "libgdn_decode_checked.so")
SOURCES = [os.path.join(PKG, "csrc", "gdn_decode.hip")]
HEADERS = [os.path.join(PKG, "csrc", f) for f in ("decode_kernel.hpp", "prefill_kernel.hpp", "host_checks.hpp")] + \
    [os.path.join(ROOT, "include", "gdn_decode.h")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc():
    path = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; set HIPCC or install ROCm")
    return path


def _command(out, checked, extra_flags=()):
    return [hipcc(), *HIPCC_FLAGS, *(["-DGDN_DEVICE_CHECKS"] if checked else []), *extra_flags,
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"), *SOURCES, "-o", out]


def build(verbose=False, extra_flags=(), checked=False):
    """Compile one library (always), atomically replacing any previous build."""
    lib = LIB_CHECKED if checked else LIB
    tmp = lib + ".tmp"
    cmd = _command(tmp, checked, extra_flags)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib)
    return lib


def build_all(verbose=False):
    """Compile the release and the checked library side by side (two hipcc processes)."""
    jobs = []
    for lib, checked in ((LIB, False), (LIB_CHECKED, True)):
        cmd = _command(lib + ".tmp", checked)
        if verbose:
            print(" ".join(cmd), flush=True)
        jobs.append((lib, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    errors = []
    for lib, proc in jobs:
        out, err = proc.communicate()
        if proc.returncode != 0:
            errors.append(f"hipcc failed for {os.path.basename(lib)} ({proc.returncode}):\n{out}\n{err}")
    if errors:
        raise RuntimeError("\n".join(errors))
    for lib, _ in jobs:
        os.replace(lib + ".tmp", lib)
    return [lib for lib, _ in jobs]


if __name__ == "__main__":
    print(build_all(verbose=True))
