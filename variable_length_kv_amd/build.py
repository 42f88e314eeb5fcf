"""Build libvlkv_attn.so in-tree with hipcc for gfx950.

``python -m variable_length_kv_amd.build`` compiles every HIP source under
``csrc/`` into one shared library next to this file, and the same sources with
``VLKV_DEBUG_VISITS`` defined into libvlkv_attn_visits.so, the visit-counting
build that the work-list tests load (include/vlkv_attn_debug.h). All device
code is built without packed-FP32 instructions (``-packed-fp32-ops``).
"""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libvlkv_attn.so")
VISITS_LIB = os.path.join(HERE, "libvlkv_attn_visits.so")
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


def build(verbose: bool = False, extra=(), visits: bool = True) -> str:
    """Compile the library (and, with ``visits``, its visit-counting build,
    in a second hipcc process at the same time); returns the library's path."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    jobs = [(LIB, list(extra))]
    if visits:
        # -Bsymbolic: its own calls bind inside it when both libraries are loaded
        jobs.append((VISITS_LIB, list(extra) + ["-DVLKV_DEBUG_VISITS", "-Wl,-Bsymbolic"]))
    procs = []
    for out, ex in jobs:
        cmd = [hipcc()] + flags() + ex + ["-shared", "-o", out + ".tmp"] + srcs
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((out, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for out, p in procs:
        text, _ = p.communicate()
        msgs = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l and l.strip())
        if p.returncode != 0:
            failed.append(f"hipcc failed for {os.path.basename(out)}:\n{msgs}")
            continue
        if verbose and msgs:
            print(msgs, file=sys.stderr)
        os.replace(out + ".tmp", out)
    if failed:
        raise RuntimeError("\n".join(failed))
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
