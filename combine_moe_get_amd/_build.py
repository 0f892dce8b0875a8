"""Compile the HIP sources of the package into combine_moe_get_amd/libmoe_get.so (gfx950).

hipcc flags: -ffp-contract=off keeps every binary32 product of the
quantization rounded on its own (no fused multiply-add that the formula does
not state); fp32 division stays correctly rounded (hipcc's default); packed
fp32 instructions are disabled for all device code.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = ["api.hip", "layout.hip", "dispatch.hip", "combine.hip"]
LIB = os.path.join(HERE, "libmoe_get.so")
# write-pattern probes the benchmark times next to the dispatch (not part of libmoe_get)
PROBE_SOURCES = ["hbm_probe.hip"]
PROBE_LIB = os.path.join(HERE, "libmoe_hbm_probe.so")
ARCH = "gfx950"


def hipcc():
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), "hipcc"):
        if os.path.sep not in c or os.path.exists(c):
            return c
    return "hipcc"


def flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-ffp-contract=off", "-fno-fast-math",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        "-I", os.path.join(ROOT, "include"),
    ]


def _compile(sources, lib, verbose, extra):
    srcs = [os.path.join(HERE, "csrc", s) for s in sources]
    cmd = [hipcc()] + flags() + list(extra) + ["-o", lib + ".tmp"] + srcs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)


def build(verbose=False, extra=()):
    _compile(SOURCES, LIB, verbose, extra)
    _compile(PROBE_SOURCES, PROBE_LIB, verbose, extra)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
