"""Compile the HIP sources into pool_stencil_amd/libpool_stencil.so (gfx950).

Every HIP source is compiled with packed-FP32 instructions disabled
(-target-feature -packed-fp32-ops): the fp32 math stays on single-issue VALU
ops and the matrix cores.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpool_stencil.so")
SOURCES = ["api.hip", "maxpool.hip", "conv_pool.hip", "conv_general.hip", "convt_softmax.hip",
           "convt_rows.hip", "convt_softmax_bf16.hip", "two_stage.hip"]
ARCH = os.environ.get("PS_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=fast", "-Wall", "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), "hipcc"):
        if os.path.sep not in c or os.path.exists(c):
            return c
    return "hipcc"


def build(verbose: bool = False) -> str:
    """Compile all sources (in parallel) and link the shared library.  Always rebuilds."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    hipcc = _hipcc()
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [hipcc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the device-only feature name; drop that note
        text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
        if text.strip() and (verbose or p.returncode):
            print(f"[{src}]\n{text}", file=sys.stderr)
        if p.returncode:
            failed.append(src)
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(failed))
    tmp = LIB + f".tmp{os.getpid()}"
    subprocess.check_call([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    # The host pass can leave a kernel's launch handle undefined without any diagnostic
    # (seen with a lambda call passed straight to the LDS-DMA load builtin); the library
    # then fails only when it is loaded.  Refuse such a library here.
    undefined = _undefined_own_symbols(tmp)
    if undefined:
        os.remove(tmp)
        raise RuntimeError("library leaves its own symbols undefined: " + ", ".join(undefined))
    os.replace(tmp, LIB)
    return LIB


def _undefined_own_symbols(lib: str) -> list:
    """Undefined dynamic symbols of the library that belong to its own namespace (ps::)."""
    try:
        out = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True,
                             text=True, check=True).stdout
    except (OSError, subprocess.CalledProcessError):
        return []  # no nm: the load-time check in the binding still catches it
    return [l.split()[-1] for l in out.splitlines() if l.split() and l.split()[-1].startswith("_ZN2ps")]


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
