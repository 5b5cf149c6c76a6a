"""Build step of the HIP library: hipcc for gfx950 into libdiffattn.so,
in-tree beside this file."""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "csrc", "diffattn_fwd.hip"),
           os.path.join(HERE, "csrc", "diffattn_kv.hip"),
           os.path.join(HERE, "csrc", "diffattn_bwd.hip")]
LIBRARY = os.path.join(HERE, "libdiffattn.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Werror",
    # no packed-fp32 VALU instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the machine scheduler's iterative ILP strategy orders the prefill
    # loop's MFMAs and VALU work better: +2.3% on the 8 x 4096 prefill,
    # -1.6% time on the backward, the cache kernels unchanged (and fewer
    # spills in the fp32 d = 64 prefill)
    "-mllvm", "-amdgpu-sched-strategy=iterative-ilp",
    "-I", os.path.join(ROOT, "include"),
]
# per-source additions: the prefill kernel runs 0.5-1.4% faster without the
# post-RA scheduler (paired runs on the 8 x 4096 and varlen prefills), while
# the backward and cache kernels run about 1% slower without it
FILE_FLAGS = {
    "diffattn_fwd.hip": ["-mllvm", "-disable-post-ra"],
}


def _run(cmd, verbose):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                         text=True)
    msg = "\n".join(l for l in res.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msg}")
    if verbose and msg.strip():
        print(msg, file=sys.stderr)


def build(output: str = LIBRARY, extra=(), verbose: bool = False) -> str:
    """Compiles each source (its FILE_FLAGS added) in parallel, then links
    the shared library."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    common = [f for f in HIPCC_FLAGS if f != "-shared"]
    objs, procs = [], []
    for src in SOURCES:
        obj = output + "." + os.path.basename(src) + ".o"
        objs.append(obj)
        cmd = [hipcc, *common, *FILE_FLAGS.get(os.path.basename(src), []), *extra,
               "-c", src, "-o", obj]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                            stderr=subprocess.STDOUT, text=True)))
    for cmd, pr in procs:
        out, _ = pr.communicate()
        msg = "\n".join(l for l in out.splitlines()
                        if "packed-fp32-ops' is not a recognized feature" not in l)
        if pr.returncode != 0:
            raise RuntimeError(f"hipcc failed ({pr.returncode}): {' '.join(cmd)}\n{msg}")
        if verbose and msg.strip():
            print(msg, file=sys.stderr)
    try:
        _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", output + ".tmp"],
             verbose)
    finally:
        for obj in objs:
            if os.path.exists(obj):
                os.remove(obj)
    os.replace(output + ".tmp", output)
    return output


if __name__ == "__main__":
    print(build(verbose=True))
