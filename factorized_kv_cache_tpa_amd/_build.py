"""Build libtpa.so for gfx950 with hipcc (in-tree, no JIT cache).

Every HIP source is compiled with the packed-fp32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); the host pass warns
that it does not know that feature, which is harmless.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libtpa.so")
SOURCES = ["api.hip", "append.hip", "decode.hip", "prefill.hip"]
# measurement helper for the benchmark (a plain streaming read), built beside the library, not part of it
PROBE_SOURCE = "stream_probe.hip"
PROBE_OUT = os.path.join(HERE, "libtpa_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(os.path.dirname(HERE), "include")]


def _compile(src: str, obj_dir: str) -> str:
    obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    obj_dir = os.path.join(HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, obj_dir), SOURCES + [PROBE_SOURCE]))
    _link(objs[:-1], OUT)
    _link(objs[-1:], PROBE_OUT)
    if verbose:
        print(f"built {OUT} and {PROBE_OUT}", file=sys.stderr)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
