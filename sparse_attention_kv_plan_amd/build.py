"""Build libkvc.so (the HIP C-ABI library) for gfx950 with hipcc.

    python -m sparse_attention_kv_plan_amd.build

Each csrc/*.hip file is compiled to an object in _build/ (in parallel), then
linked into sparse_attention_kv_plan_amd/libkvc.so.  Only the symbols of
include/kvc.h are exported.

probe/stream_probe.hip (plain bandwidth streams that the benchmark times beside
the kernels; no part of libkvc.so) becomes probe/libstream_probe.so.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libkvc.so")
PROBE_SRC = os.path.join(PKG, "probe", "stream_probe.hip")
PROBE_LIB = os.path.join(PKG, "probe", "libstream_probe.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC] + FLAGS + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    out = r.stdout.decode(errors="replace")
    # the host pass does not know the packed-fp32 feature and says so; that is expected
    out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, out))
    return obj, out


def _link(objs, lib):
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout.decode(errors="replace"))
    os.replace(tmp, lib)


def build(verbose=False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs) + 1)) as ex:
        probe = ex.submit(_compile, PROBE_SRC)
        results = list(ex.map(_compile, srcs))
        probe_obj, probe_out = probe.result()
    if verbose:
        for _, out in results:
            if out.strip():
                print(out)
        if probe_out.strip():
            print(probe_out)
    _link([o for o, _ in results], LIB)
    _link([probe_obj], PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
