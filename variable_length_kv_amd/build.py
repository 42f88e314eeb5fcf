"""Build libvlkv_attn.so in-tree with hipcc for gfx950.

``python -m variable_length_kv_amd.build`` compiles every HIP source under
``csrc/`` into one shared library next to this file. All device code is built
without packed-FP32 instructions (``-packed-fp32-ops``).
"""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libvlkv_attn.so")
SOURCES = ["plan.hip", "decode.hip", "append.hip", "router.hip", "api.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(HERE, "..", "include")]


def build(verbose: bool = False, extra=()) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    cmd = [hipcc()] + flags() + list(extra) + ["-shared", "-o", LIB + ".tmp"] + srcs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + msgs)
    if verbose and msgs:
        print(msgs, file=sys.stderr)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def device_asm(out_dir: str) -> list:
    """Write the gfx950 assembly of each source (for inspection)."""
    os.makedirs(out_dir, exist_ok=True)
    outs = []
    for s in SOURCES:
        o = os.path.join(out_dir, s.replace(".hip", ".s"))
        cmd = [hipcc()] + flags() + ["-S", "--cuda-device-only", "-o", o, os.path.join(CSRC, s)]
        subprocess.run(cmd, check=True, capture_output=True)
        outs.append(o)
    return outs


if __name__ == "__main__":
    print(build(verbose=True))
