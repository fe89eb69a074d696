"""Build ``libspecverify.so`` for gfx950 with hipcc, in-tree.

    python draft_verification_softmax_amd/build.py [-v]

Each source compiles to its own object (in parallel; every object carries its own device
code, no relocatable device code), then one hipcc line links the shared library.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libspecverify.so")
SOURCES = ["specverify.hip", "team_kernel.hip", "team_grad.hip", "team_sample.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-FP32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [l for l in (res.stderr or "").splitlines() if "packed-fp32-ops" not in l]
    return res.returncode, msgs


def build(verbose: bool = False) -> str:
    with tempfile.TemporaryDirectory(prefix="svbuild") as tmp:
        objs = [os.path.join(tmp, s.replace(".hip", ".o")) for s in SOURCES]
        cmds = [[HIPCC, *FLAGS, "-c", "-o", o, os.path.join(CSRC, s)] for s, o in zip(SOURCES, objs)]
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        jobs = max(1, min(len(cmds), os.cpu_count() or 1))
        with ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(_run, cmds))
        msgs = [m for _, ms in results for m in ms]
        if any(rc != 0 for rc, _ in results):
            raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
        link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", LIB + ".tmp", *objs]
        if verbose:
            print(" ".join(link), flush=True)
        rc, lmsgs = _run(link)
        if rc != 0:
            raise RuntimeError("hipcc link failed:\n" + "\n".join(lmsgs))
        msgs += lmsgs
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
