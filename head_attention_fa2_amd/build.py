"""Build the HIP libraries (kernels for gfx950 + the C ABI) in place, next to this file.

libmha.so         the library: pipelined kernels behind include/mha.h
libmha_serial.so  the same ABI built with MHA_SERIALIZE=1: the race-check form of every
                  LDS tile loop (one buffer, each tile copied, waited for and fenced by
                  barriers before it is read).  Only the tests load it, to compare its
                  results bit for bit with libmha.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libmha.so")
LIB_SERIAL = os.path.join(HERE, "libmha_serial.so")

SOURCES = ["mha_fwd_kernel.hip", "gemm_kernel.hip", "mha_api.cpp"]
KERNEL_SOURCES = ["mha_fwd_kernel.hip", "gemm_kernel.hip"]   # built twice (pipelined, serialized)

# -Xclang -target-feature -Xclang -packed-fp32-ops: never emit v_pk_{add,mul,fma}_f32.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    # the LDS copies set m0 in inline asm right before use; nothing else reads m0
    "-Wno-inline-asm",
    # NaN inputs are outside the contract (include/mha.h), so maxima and minima need no
    # NaN quieting (v_max3_f32 straight on MFMA results)
    "-fno-honor-nans",
]
_NOISE = ("packed-fp32-ops' is not a recognized feature",)


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if not any(n in ln for n in _NOISE)]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 into libmha.so and libmha_serial.so; returns
    the path of libmha.so."""
    cc = hipcc()
    inc = [f"-I{INCLUDE}", f"-I{CSRC}"]
    with tempfile.TemporaryDirectory(prefix="mha_build_") as tmp:
        jobs = []   # (source, object, extra flags)
        for src in SOURCES:
            jobs.append((src, os.path.join(tmp, src + ".o"), []))
        for src in KERNEL_SOURCES:
            jobs.append((src, os.path.join(tmp, src + ".serial.o"), ["-DMHA_SERIALIZE=1"]))
        workers = max(1, min(len(jobs), len(os.sched_getaffinity(0))))
        with cf.ThreadPoolExecutor(max_workers=workers) as ex:
            futs = [ex.submit(_run, [cc, *HIPCC_FLAGS, *extra, *inc, "-c", os.path.join(CSRC, src), "-o", obj],
                              verbose) for src, obj, extra in jobs]
            for f in futs:
                f.result()
        objs = {obj: (src, extra) for src, obj, extra in jobs}
        plain = [o for o, (s, e) in objs.items() if not e]
        serial = [o for o, (s, e) in objs.items() if e] + [os.path.join(tmp, "mha_api.cpp.o")]
        for out, parts in ((LIB, plain), (LIB_SERIAL, serial)):
            _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", *parts, "-o", out + ".tmp"], verbose)
            os.replace(out + ".tmp", out)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
