"""Build libhetlora.so in-tree for gfx950.

host.cpp and pool.cpp (no HIP) are compiled by g++, kernels.hip by hipcc;
hipcc links the shared library next to this file.  Every build compiles from
scratch.
"""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libhetlora.so")
ARCH = os.environ.get("HETLORA_ARCH", "gfx950")

# packed fp32 ops are disabled on purpose: plain fp32 VALU code only.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function", "-Wno-inline-asm", f"-I{INCLUDE}"]


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("build step failed: " + " ".join(cmd))
    return r


def build(verbose=False, out=LIB, defines=(), build_dir=None):
    """Compile and link the library to `out`.  `defines` are extra -D flags
    (tuning constants); the default build uses none."""
    out_dir = build_dir or os.path.join(HERE, "_build")
    os.makedirs(out_dir, exist_ok=True)
    host_o = [os.path.join(out_dir, f"{n}.o") for n in ("host", "pool")]
    kern_o = os.path.join(out_dir, "kernels.o")
    dflags = [f"-D{d}" for d in defines]
    for n, o in zip(("host", "pool"), host_o):
        _run(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", f"-I{INCLUDE}", *dflags, "-c",
              os.path.join(CSRC, f"{n}.cpp"), "-o", o])
    _run([_hipcc(), *HIP_FLAGS, *dflags, "-c", os.path.join(CSRC, "kernels.hip"), "-o", kern_o])
    tmp = out + ".tmp"
    _run([_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *host_o, kern_o, "-o", tmp])
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
