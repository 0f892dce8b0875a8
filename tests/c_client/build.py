"""Compile the plain-C client of libmoe_get (tests/c_client/moe_client) with gcc."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
BIN = os.path.join(HERE, "moe_client")


def build(verbose=False, syntax_only=False):
    pkg = os.path.join(ROOT, "combine_moe_get_amd")
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Wno-unused-parameter",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           os.path.join(HERE, "moe_client.c")]
    if syntax_only:
        cmd += ["-fsyntax-only"]
    else:
        cmd += ["-o", BIN, "-L", pkg, "-lmoe_get", "-Wl,-rpath," + pkg,
                "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return BIN


if __name__ == "__main__":
    print(build(verbose=True))
