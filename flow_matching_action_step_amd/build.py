"""Build libsmolexp.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Run as ``python flow_matching_action_step_amd/build.py`` (by path: importing the
package would load the library it is about to rebuild); no GPU is needed.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libsmolexp.so")
SOURCES = [os.path.join(PKG, "csrc", "kernels.hip"), os.path.join(PKG, "csrc", "train.hip"),
           os.path.join(PKG, "csrc", "smolexp_api.cpp")]


def hipcc():
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), "hipcc"):
        if os.path.sep not in c or os.path.exists(c):
            return c
    return "hipcc"


def build(verbose=False):
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-mcode-object-version=5", "-fPIC", "-shared",
           # no packed-fp32 instructions in device code
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           # MFMA accumulators in VGPRs: with AGPR accumulators the allocator shuffles
           # them between loop iterations (hundreds of v_accvgpr moves per k-slab)
           "-mllvm", "-amdgpu-mfma-vgpr-form=1",
           "-Wall", "-Wno-unused-function", "-Wl,--no-undefined",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
           "-o", tmp] + SOURCES
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l or "error" in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
