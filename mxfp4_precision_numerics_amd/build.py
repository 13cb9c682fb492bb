"""Build libmx355.so (the HIP library behind include/mx.h) for gfx950.

Run as ``python -m mxfp4_precision_numerics_amd.build``.  The library is
built in-tree, next to this file.  Flags:
  -ffp-contract=off                 no add fused into a multiply: the RHT's fp32
                                    rounding order is part of the contract
  -fno-gpu-flush-denormals-to-zero  fp32 subnormals are kept (they can set codes)
  -target-feature -packed-fp32-ops  no packed fp32 math
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmx355.so")
SOURCES = ["mx_quant.hip", "mx_gemm.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


PROBE = os.path.join(HERE, "hbm_probe")


def _hipcc(cmd, out, verbose):
    tmp = out + ".tmp%d" % os.getpid()
    res = subprocess.run([HIPCC] + cmd + ["-o", tmp], capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature name and says so
    err = "\n".join(l for l in res.stderr.splitlines() if "not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    _hipcc(FLAGS + [os.path.join(CSRC, s) for s in SOURCES], LIB, verbose)
    # the HBM-rate probe the quantizers' rooflines are read against (an
    # executable, not part of the library; bench.py --hbm-ceiling runs it)
    probe_flags = [f for f in FLAGS if f not in ("-fPIC", "-shared")]
    _hipcc(probe_flags + [os.path.join(CSRC, "hbm_probe.hip")], PROBE, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
