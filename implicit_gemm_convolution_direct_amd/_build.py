"""Build the HIP library libconvhip.so in-tree with hipcc for gfx950."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libconvhip.so")
SOURCES = [os.path.join(CSRC, "conv_kernels.hip"), os.path.join(CSRC, "unfused_kernels.hip"),
           os.path.join(CSRC, "valu_kernels.hip"), os.path.join(CSRC, "convhip_plan.cpp")]
HEADERS = [os.path.join(CSRC, "convhip_plan.h"),
           os.path.join(os.path.dirname(HERE), "include", "convhip.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # Keep the compiler from forming packed fp32 VALU instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def stale():
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(s) > t for s in SOURCES + HEADERS)


def build(force=True, verbose=False, extra_flags=()):
    cmd = [HIPCC, *FLAGS, *extra_flags, *SOURCES, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed:\n{out}")
    if verbose and out.strip():
        print(out)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
