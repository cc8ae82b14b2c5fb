"""Build libattn.so (the HIP library) in-tree with hipcc for gfx950.

    python -m exact_attention_08_amd.build

Every source is compiled for gfx950 only.  Packed FP32 instructions are disabled on the
device side (-packed-fp32-ops); hipcc's host pass prints a harmless warning about it.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libattn.so")
# the benchmark's streaming-read kernel (HBM ceiling), a library of its own
PROBE_SRC = "hbm_probe.hip"
PROBE_LIB = os.path.join(HERE, "libhbmprobe.so")
SOURCES = ["attn_fwd.hip", "attn_fwd_d128.hip", "attn_decode.hip", "attn_noalloc.hip", "attn_abi.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]
# Per-source extra flags.  The decode kernel's atomics are all issued by a single lane and
# their results are needed only much later; the compiler's atomic optimizer would expand
# each into a wave-wide broadcast that reads the result at once (a wait on every load in
# flight), so it is off for that file.
EXTRA_FLAGS = {"attn_decode.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


def build(verbose: bool = False) -> str:
    with tempfile.TemporaryDirectory(prefix="attn_build_") as tmp:
        objs, procs = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            lang = ["-x", "hip"] if src.endswith(".hip") else []
            cmd = [HIPCC, *COMMON_FLAGS, *EXTRA_FLAGS.get(src, []), *lang, "-c",
                   os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                stderr=subprocess.STDOUT, text=True)))
            objs.append(obj)
        failed = []
        for src, p in procs:
            out, _ = p.communicate()
            msgs = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
            if p.returncode != 0:
                failed.append(src)
                sys.stderr.write("\n".join(msgs) + "\n")
            elif verbose and msgs:
                print("\n".join(msgs))
        if failed:
            raise RuntimeError(f"hipcc failed for {failed}")
        tmp_lib = LIB + ".tmp"
        subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib],
                       check=True)
        os.replace(tmp_lib, LIB)
        tmp_probe = PROBE_LIB + ".tmp"
        p = subprocess.run([HIPCC, *COMMON_FLAGS, "-shared", "-x", "hip",
                            os.path.join(CSRC, PROBE_SRC), "-o", tmp_probe],
                           stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if p.returncode != 0:
            sys.stderr.write(p.stdout)
            raise RuntimeError(f"hipcc failed for {PROBE_SRC}")
        os.replace(tmp_probe, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
