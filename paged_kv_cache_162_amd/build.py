"""Build libpagedkv.so in-tree with hipcc for gfx950.

The library is one shared object: the host block manager (plain C++) and the
HIP kernels with their C entry points. Each source is compiled to an object
of its own (in parallel; every device file carries its own code object), then
the objects are linked. Packed-FP32 instruction selection is turned off for
the device code.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpagedkv.so")
OBJDIR = os.path.join(HERE, "_build")
# (source, extra flags, object tag): decode_variants.hip is compiled once per
# block size and K/V load policy, so the decode kernels build in parallel
SOURCES = ([(os.path.join(CSRC, f), [], f) for f in
            ("host_pool.cpp", "plan.cpp", "cache.hip", "decode.hip", "prefill.hip",
             "shared_prefix.hip")] +
           [(os.path.join(CSRC, "decode_variants.hip"), [f"-DPAGEDKV_BS={bs}", f"-DPAGEDKV_NT={nt}"],
             f"decode_variants_b{bs}_nt{nt}") for bs in (8, 16, 32) for nt in (0, 1)])
ARCH = os.environ.get("PAGEDKV_ARCH", "gfx950")
# the host pass warns that it does not know the packed-fp32 feature
_NOISE = "is not a recognized feature for this target"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _flags() -> list:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include")]


def _run(cmd: list, verbose: bool) -> str:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if _NOISE not in l)
    if res.returncode != 0:
        sys.stderr.write(msgs + "\n")
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}: {' '.join(cmd[-4:])}")
    return msgs


def build(verbose: bool = False) -> str:
    """Compile every source and link paged_kv_cache_162_amd/libpagedkv.so."""
    os.makedirs(OBJDIR, exist_ok=True)
    tag = "%d" % os.getpid()
    objs = [os.path.join(OBJDIR, name + "." + tag + ".o") for _, _, name in SOURCES]
    cmds = [[hipcc()] + _flags() + extra + ["-c", "-o", o, src]
            for (src, extra, _), o in zip(SOURCES, objs)]
    jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    try:
        with ThreadPoolExecutor(jobs) as ex:
            outs = list(ex.map(lambda c: _run(c, verbose), cmds))
        tmp = LIB + ".tmp" + tag
        outs.append(_run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs,
                         verbose))
        os.replace(tmp, LIB)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    if verbose:
        text = "\n".join(m for m in outs if m)
        if text:
            print(text)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
