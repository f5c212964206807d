"""Build libselscan.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libselscan.so")
SOURCES = ["csrc/sscan_api.hip", "csrc/sscan_fwd.hip", "csrc/sscan_fwd_zoh.hip", "csrc/sscan_fwd_euler.hip",
           "csrc/sscan_fwd_row_zoh.hip", "csrc/sscan_fwd_row_euler.hip", "csrc/sscan_fwd_row_conv.hip",
           "csrc/sscan_fwd_row_struct.hip", "csrc/sscan_fwd_row_ckagg.hip",
           "csrc/sscan_fwd_conv.hip",
           "csrc/sscan_step.hip", "csrc/sscan_bwd.hip"]

# Packed-FP32 instructions are disabled on purpose: the VALU code is written for
# plain fp32 issue.
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if "is not a recognized feature" not in ln
            and "packed-fp32-ops" not in ln and ln.strip()]
    return res.returncode, msgs


def _source_key(src: str) -> str:
    """Hash of one translation unit's inputs: its source, every header it can include
    (all of csrc/*.h and the public header) and the compiler flags."""
    import glob
    import hashlib
    h = hashlib.sha256(" ".join(HIPCC_FLAGS).encode())
    for f in [os.path.join(HERE, src)] + sorted(glob.glob(os.path.join(HERE, "csrc", "*.h"))) + \
            [os.path.join(ROOT, "include", "selscan.h")]:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def build(verbose: bool = False, incremental: bool = False) -> str:
    """Compile every source to an object (in parallel), then link libselscan.so.

    incremental: keep objects in _build/ keyed by a hash of their inputs and reuse
    those that are current (a development convenience; the default compiles all)."""
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    tag = "%d" % os.getpid()
    if incremental:
        objs = [os.path.join(objdir, os.path.basename(src).replace(".hip", ".%s.o" % _source_key(src)))
                for src in SOURCES]
    else:
        objs = [os.path.join(objdir, os.path.basename(src).replace(".hip", ".%s.o" % tag)) for src in SOURCES]
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    jobs = [(src, o, [hipcc()] + compile_flags + ["-I" + os.path.join(ROOT, "include"), "-c", "-o", o + ".tmp" + tag,
                                                  os.path.join(HERE, src)])
            for src, o in zip(SOURCES, objs) if not (incremental and os.path.exists(o))]

    def compile_one(job):
        src, o, cmd = job
        rc, msgs = _run(cmd, verbose)
        if rc == 0:
            os.replace(o + ".tmp" + tag, o)
        return rc, msgs, src

    try:
        with ThreadPoolExecutor(max(1, min(len(jobs) or 1, os.cpu_count() or 1))) as ex:
            results = list(ex.map(compile_one, jobs))
        for rc, msgs, src in results:
            if rc != 0:
                sys.stderr.write("\n".join(msgs) + "\n")
                raise RuntimeError("hipcc failed compiling %s" % src)
            if verbose and msgs:
                print("\n".join(msgs))
        tmp = LIB + ".tmp" + tag
        rc, msgs = _run([hipcc()] + HIPCC_FLAGS + ["-o", tmp] + objs, verbose)
        if rc != 0:
            sys.stderr.write("\n".join(msgs) + "\n")
            raise RuntimeError("hipcc failed linking libselscan.so")
        os.replace(tmp, LIB)
    finally:
        if not incremental:
            for o in objs:
                if os.path.exists(o):
                    os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, incremental="--incremental" in sys.argv))
