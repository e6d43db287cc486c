"""Builds libsa.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m sparse_causal_attention_amd.build

Each translation unit is compiled by hipcc into _build/, in parallel, then
linked into sparse_causal_attention_amd/libsa.so.  Always recompiles (the
caller asked for a build); pass --if-stale to skip when the library is
newer than every source.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-I" + os.path.join(ROOT, "include"),
]
# Device code: gfx950 only; no packed-fp32 instructions (hipcc warns that the
# host pass does not know the feature; harmless).
DEVICE = ["-x", "hip", "--offload-arch=" + ARCH, "-Xclang", "-target-feature",
          "-Xclang", "-packed-fp32-ops", "-munsafe-fp-atomics",
          # MFMA accumulators in ordinary VGPRs: the softmax works on them
          # directly instead of copying through AGPRs
          "-mllvm", "-amdgpu-mfma-vgpr-form=1"]


# Per-file additions.  The band kernels' MFMA chains keep more LDS operand
# reads in flight under the iterative ILP scheduler (measured 2.4 % faster
# backward, 1.3 % faster forward; neutral on the gather kernels).
PER_FILE = {
    "band.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
    "band_bwd.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
}


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def headers():
    return sorted(glob.glob(os.path.join(CSRC, "*.h")) + glob.glob(os.path.join(ROOT, "include", "*.h")))


def lib_headers():
    """The headers libsa.so is built from (its own and include/sa.h; not the
    probe library's header)."""
    return sorted(glob.glob(os.path.join(CSRC, "*.h")) + [os.path.join(ROOT, "include", "sa.h")])


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON + DEVICE + PER_FILE.get(os.path.basename(src), []) + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def source_digest() -> str:
    """sha256 over every source and build flag that goes into libsa.so (used to
    tell whether profiler counters were taken on the kernels as they are now)."""
    import hashlib

    h = hashlib.sha256()
    for f in sources() + lib_headers():
        h.update(os.path.relpath(f, ROOT).encode())
        h.update(open(f, "rb").read())
    # flags with the checkout location taken out, so the digest is the same
    # wherever the repository sits
    h.update(" ".join(COMMON + DEVICE).replace(ROOT, "<root>").encode())
    h.update(repr(sorted(PER_FILE.items())).encode())
    return h.hexdigest()


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(f) > t for f in sources() + headers())


PROBE_SRC = os.path.join(PKG, "probe", "probe.hip")
PROBE_LIB = os.path.join(PKG, "libsa_probe.so")


def build_probe() -> str:
    """libsa_probe.so: the benchmark's measurement probes (copy, MFMA loop,
    empty launch), a library of their own beside libsa.so."""
    obj = _compile(PROBE_SRC)
    tmp = PROBE_LIB + ".tmp%d" % os.getpid()
    r = subprocess.run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, obj],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("probe link failed:\n%s" % r.stderr)
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def build(jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs) + 1, max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        probe = ex.submit(build_probe)
        objs = list(ex.map(_compile, srcs))
        probe.result()
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    if "--if-stale" in sys.argv and not stale():
        print(LIB, "(up to date)")
    else:
        print(build())
