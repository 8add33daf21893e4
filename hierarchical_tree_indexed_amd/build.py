"""Compile the HIP library (gfx950) in-tree: libhti.so next to this file."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libhti.so")
SOURCES = ["hti_api.hip", "hti_build.hip", "hti_traverse.hip", "hti_decode.hip", "hti_prefill.hip",
           "hti_prefill_walk.hip", "hti_prefill_nodes.hip"]
# on-device floors for the measurement (latency, bandwidth, matrix-core peak):
# a library of its own, loaded only by the benchmark
PROBE_LIB = os.path.join(HERE, "libhti_probe.so")
PROBE_SOURCES = ["hti_probe.hip"]
# the same library with the split decode's phase timeline compiled in
# (HTI_DECODE_TIMELINE): used by `bench.py --timeline` only
TIMELINE_LIB = os.path.join(HERE, "libhti_timeline.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Wno-unused-function", "-Wno-unused-parameter",
         # keep the compiler from forming packed fp32 math
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str, defines=()) -> str:
    tag = "".join("_" + d.lower() for d in defines)
    obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + tag + ".o")
    cmd = [HIPCC, *FLAGS, *[f"-D{d}" for d in defines], "-I", os.path.join(HERE, "..", "include"), "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def _link(objs, lib):
    tmp = lib + f".tmp{os.getpid()}"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    jobs = [(s, ()) for s in SOURCES + PROBE_SOURCES] + [("hti_decode.hip", ("HTI_DECODE_TIMELINE",))]
    with cf.ThreadPoolExecutor(max_workers=min(7, len(jobs))) as ex:
        objs = dict(zip(jobs, ex.map(lambda j: _compile(*j), jobs)))
    _link([objs[(s, ())] for s in SOURCES], LIB)
    _link([objs[(s, ())] for s in PROBE_SOURCES], PROBE_LIB)
    _link([objs[(s, ("HTI_DECODE_TIMELINE",))] if s == "hti_decode.hip" else objs[(s, ())] for s in SOURCES],
          TIMELINE_LIB)
    if verbose:
        print("built", LIB, PROBE_LIB, "and", TIMELINE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
