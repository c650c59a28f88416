"""Build libattnbwd.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

    python -m sparse_attention_backward_amd.build [-v] [-j N]

Each source compiles to its own object (in parallel) under _build/, then one
shared library is linked next to this file.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libattnbwd.so")
SOURCES = ["api.hip", "preprocess.hip", "dense_fp32.hip", "dense_kv.hip", "dense_dq.hip", "attn_q.hip",
           "index.hip", "sel_kv.hip", "sel_reduce.hip", "sel_fwd_kv.hip", "indexer.hip"]
ARCH = os.environ.get("ATTN_BWD_ARCH", "gfx950")
# Compilation units: (object name, source, extra options).  sel_kv.hip is compiled twice,
# once per key-block width.  Both run one wave per SIMD; asking for MFMA results in VGPRs
# keeps their score, dS and dQ-product accumulators out of the AGPRs and saves the register
# moves between the two files (64 keys: 3% faster at S = 32K; 128 keys: 508 -> 415
# registers, 4% faster on the Zipf workload).  The machine scheduler's instruction-level-
# parallelism strategy suits the selected kernels (KV-major pass 2.5% faster at S = 128K and
# 4% on the Zipf workload, the forward and row-statistic passes 1-4%, the dQ reduction 2%)
# but not the dense or indexer kernels or the row statistics (slower by 3-50%).
ILP = ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]
# The dense KV-major kernel gains 1% from the AMDGPU-specific register-pressure trackers.
UNIT_FLAGS = {"sel_fwd_kv": ILP, "sel_reduce": ILP, "dense_kv": ["-mllvm", "-amdgpu-use-amdgpu-trackers"]}
UNITS = [(os.path.splitext(s)[0], s, UNIT_FLAGS.get(os.path.splitext(s)[0], []))
         for s in SOURCES if s != "sel_kv.hip"] + [
    ("sel_kv_b64", "sel_kv.hip", ["-DSEL_KV_KEYS=64", "-mllvm", "-amdgpu-mfma-vgpr-form=1", *ILP]),
    ("sel_kv_b128", "sel_kv.hip", ["-DSEL_KV_KEYS=128", "-mllvm", "-amdgpu-mfma-vgpr-form=1", *ILP]),
]
# Units whose kernels wait for their own global->LDS transfers with hand-counted vmcnt values
# (the transfers are inline asm, which the compiler's wait counting does not see).  The counts
# assume that the compiler issues no vector-memory operations of its own in the step loops; a
# register spill would add scratch loads and stores there and make a count too small, so the
# build refuses any kernel of these units that uses scratch.
NO_SCRATCH = {"sel_kv_b64", "sel_kv_b128", "dense_dq"}


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC)")


def flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            # packed fp32 VALU ops are kept out of every kernel
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def scratch_users(remarks: str) -> list:
    """Kernels with a nonzero scratch size in hipcc's kernel-resource-usage remarks."""
    users, name = [], None
    for line in remarks.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name is not None and int(m.group(1)) > 0:
            users.append(name)
    return users


def _compile(unit, verbose):
    name, src, extra = unit
    obj = os.path.join(BUILD, name + ".o")
    check = ["-Rpass-analysis=kernel-resource-usage"] if name in NO_SCRATCH else []
    cmd = [hipcc(), *flags(), *extra, *check, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = r.stdout + r.stderr
    msgs = "\n".join(line for line in out.splitlines()
                     if "packed-fp32-ops" not in line and "kernel-resource-usage" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    if check:
        spilled = scratch_users(out)
        if spilled:
            raise RuntimeError(f"{name}: kernels use scratch (register spills), which their hand-counted "
                               f"vmcnt waits do not allow: {', '.join(spilled)}")
    if verbose and msgs.strip():
        print(msgs)
    return obj


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda u: _compile(u, verbose), UNITS))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("-v", "--verbose", action="store_true")
    ap.add_argument("-j", "--jobs", type=int, default=8)
    args = ap.parse_args(argv)
    print(build(args.verbose, args.jobs))


if __name__ == "__main__":
    sys.exit(main())
