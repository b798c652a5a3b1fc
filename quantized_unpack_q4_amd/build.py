"""Build libgq.so (the HIP kernels and the C ABI) for gfx950 with hipcc, and
libgq_probe.so (the measurement probes the benchmark compares against).

Run ``python -m quantized_unpack_q4_amd.build``.  Objects go to ``_build/`` at
the repository root; the library lands next to this file so the Python
binding finds it in-tree.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgq.so")
PROBE_LIB = os.path.join(PKG, "libgq_probe.so")
PROBE_SOURCES = ["probes.hip"]
ARCH = os.environ.get("GQ_OFFLOAD_ARCH", "gfx950")

SOURCES = ["dequant.hip", "gemv.hip", "gemv_stream.hip", "gemv_mfma.hip", "gemm.hip", "gemm_big.hip", "moe.hip", "moe_skinny.hip", "moe_route.hip", "gemv_q8k.hip", "gemm_q8k.hip", "gemv_q8_0_mfma.hip", "gemv_q4k_f32.hip", "gq_api.cpp"]

FLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-I" + INCLUDE,
    "-I" + CSRC,
    # keep binary32 subnormals (no flush to zero) and IEEE semantics
    "-fno-gpu-flush-denormals-to-zero",
    "-fno-fast-math",
    # never emit packed binary32 arithmetic (v_pk_fma_f32 and friends)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libgq.so")


def _compile(src: str) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc(), *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    os.replace(tmp, lib)


BUILD_INFO = os.path.join(PKG, "build_info.json")


def _run_text(cmd) -> str:
    try:
        r = subprocess.run(cmd, capture_output=True, text=True, cwd=ROOT, timeout=30)
        return r.stdout.strip() if r.returncode == 0 else ""
    except (OSError, subprocess.SubprocessError):
        return ""


def write_build_info() -> dict:
    """What was built from what: the git revision (with a flag for uncommitted
    changes under the package, include/ and oracle/), the compiler version
    and a SHA-256 over the HIP/C++ sources; written next to the library so
    that benchmark receipts can quote it where no git checkout exists."""
    import hashlib
    import json
    h = hashlib.sha256()
    for d in (CSRC, INCLUDE):
        for f in sorted(os.listdir(d)):
            h.update(f.encode())
            with open(os.path.join(d, f), "rb") as fh:
                h.update(fh.read())
    info = {
        "git_rev": _run_text(["git", "rev-parse", "HEAD"]) or None,
        "git_dirty": bool(_run_text(["git", "status", "--porcelain", "--",
                                     "quantized_unpack_q4_amd", "include", "oracle"])),
        "hipcc": (_run_text([hipcc(), "--version"]).splitlines() or [""])[0] or None,
        "offload_arch": ARCH,
        "source_sha256": h.hexdigest(),
        "built_unix": int(time.time()),
    }
    with open(BUILD_INFO, "w") as fh:
        json.dump(info, fh, indent=1)
    return info


def build(jobs: int = 8, verbose: bool = False) -> str:
    srcs = SOURCES + PROBE_SOURCES
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB)
    write_build_info()
    if verbose:
        print("built", LIB, "and", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
