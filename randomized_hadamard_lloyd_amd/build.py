"""Build libtq.so (HIP kernels for gfx950 + the C-ABI layer) in-tree with hipcc.

Flags: -ffp-contract=off keeps every fp32 operation separately rounded in the
order the kernels write it (explicit fmaf calls are the only fused operations);
packed fp32 instructions are disabled for the whole build.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libtq.so")
SOURCES = ["tq3.hip", "tq3_attn.hip", "orbit.hip", "orbit_linear.hip", "orbit_linear_lp.hip", "libtq.cpp"]
# Measurement probes timed by bench.py (the TQ3 kernels' memory traffic with
# no arithmetic); a library of their own, not part of the codec's ABI.
PROBE_LIB = os.path.join(HERE, "libtqprobe.so")
PROBE_SOURCES = ["stream_probe.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def sources():
    return [os.path.join(CSRC, s) for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)


def _finish(proc, what):
    out, _ = proc.communicate()
    # hipcc's host pass does not know the packed-fp32 feature name; drop that note
    out = "\n".join(l for l in out.splitlines()
                    if "packed-fp32-ops" not in l and "warning generated" not in l)
    if out.strip():
        print(out, file=sys.stderr)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed on {what} ({proc.returncode})")


def build(verbose: bool = False) -> str:
    """Compile every source to an object in parallel, then link libtq.so and
    the probe library."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs, pobjs, procs = [], [], []
    for src in sources() + [os.path.join(CSRC, s) for s in PROBE_SOURCES]:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        (pobjs if os.path.basename(src) in PROBE_SOURCES else objs).append(obj)
        procs.append((_run([HIPCC, *FLAGS, "-c", src, "-o", obj], verbose), src))
    for proc, src in procs:
        _finish(proc, os.path.basename(src))
    for out, o in ((LIB, objs), (PROBE_LIB, pobjs)):
        tmp = out + ".tmp"
        _finish(_run([HIPCC, *FLAGS, "-shared", *o, "-o", tmp], verbose), "link")
        os.replace(tmp, out)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
