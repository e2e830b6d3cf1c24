"""Build the HIP library libmla_decode.so in-tree for gfx950 (MI355X).

Compiles csrc/mla_kernels.hip (device code + launchers) and csrc/mla_api.cpp
(the C ABI declared in include/mla.h) with hipcc and links them into
mla_decode_attention_02_amd/libmla_decode.so.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmla_decode.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# packed fp32 instructions are switched off for all device code
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"-I{os.path.join(ROOT, 'include')}"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = ("unknown target feature", "packed-fp32-ops", "warning generated", "warnings generated")
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if not any(n in l for n in noise))
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{msg}")
    if verbose and msg.strip():
        print(msg)


def build(verbose=False, extra=()):
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    k_obj = os.path.join(objdir, "mla_kernels.o")
    a_obj = os.path.join(objdir, "mla_api.o")
    _run([HIPCC, f"--offload-arch={ARCH}", *COMMON, *DEVICE_FLAGS, *extra, "-c",
          os.path.join(CSRC, "mla_kernels.hip"), "-o", k_obj], verbose)
    _run([HIPCC, *COMMON, *extra, "-c", os.path.join(CSRC, "mla_api.cpp"), "-o", a_obj], verbose)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", k_obj, a_obj, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
