"""Build the HIP library libaq.so in-tree for gfx950.

    python -m mixed_precision_int_amd.build

Every source is compiled with hipcc for gfx950 (objects under _build/, in
parallel) and linked into mixed_precision_int_amd/libaq.so.  Packed FP32 VALU
instructions are disabled for all device code.
"""

from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libaq.so")
SOURCES = ["aq_api.cpp", "aq_plan.cpp", "aq_pack.hip", "aq_quant_act.hip", "aq_decode.hip", "aq_prefill.hip",
           "aq_expand.hip", "aq_prefill_dense.hip", "aq_prefill_big.hip", "aq_transform.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def compile_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
        "-I", os.path.join(ROOT, "include"),
        # packed FP32 VALU ops off for all device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    ]


# Kernels allowed to use scratch (private) memory.  Every other kernel must
# be spill-free: the long-prompt GEMM counts its outstanding vector-memory
# operations by hand at each column boundary, and a kernel that spills adds
# memory operations the count was not written for (and loses time to them).
# The debug tile-product variants store INT32 products inside the column
# loop and spill by design; they are never on the timed path.
SCRATCH_ALLOWED = [
    re.compile(r"prefill_dense_kernelILi\d+ELi\d+ELi\d+ELi\d+ELb1E"),   # debug products
    re.compile(r"prefill_kernelILi\d+ELi\d+ELi\d+ELb1E"),                # debug products
    re.compile(r"prefill_big_kernelILb1E"),                              # debug products
    # The persistent 256 x 256 GEMM spills 8 B/lane at 256 VGPRs (12 with the
    # output transform in its epilogue).  Its column boundary waits for all of
    # the wave's memory operations (vmcnt(0), lgkmcnt(0)), so no hand count
    # depends on the spill's loads and stores.
    re.compile(r"prefill_big_kernelILb0E"),
]


def scratch_report(stderr: str) -> list[tuple[str, int]]:
    """(kernel, scratch bytes per lane) from hipcc's kernel-resource-usage
    remarks."""
    names = re.findall(r"remark: Function Name: (\S+)", stderr)
    sizes = [int(x) for x in re.findall(r"remark: +ScratchSize \[bytes/lane\]: (\d+)", stderr)]
    if len(names) != len(sizes):
        raise RuntimeError("could not parse the kernel-resource-usage remarks")
    return list(zip(names, sizes))


def _compile(src: str) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *compile_flags(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
    if src.endswith(".hip"):
        bad = [(n, b) for n, b in scratch_report(res.stderr)
               if b > 0 and not any(p.search(n) for p in SCRATCH_ALLOWED)]
        if bad:
            raise RuntimeError(f"{src}: kernels that spill to scratch memory: " +
                               ", ".join(f"{n} ({b} B/lane)" for n, b in bad))
    return obj


PROBE_SRC = os.path.join(PKG, "probes", "issue_rates.hip")
PROBE_BIN = os.path.join(PKG, "probes", "issue_rates")


def build_probe() -> str:
    """The issue-rate probe (a standalone program, measurement only; not part
    of libaq.so).  Its MFMAs take their accumulators in VGPRs, as the GEMM's
    do, so that the rescale reads them without copies."""
    cmd = [hipcc(), *compile_flags(), "-mllvm", "-amdgpu-mfma-vgpr-form=1", PROBE_SRC, "-o", PROBE_BIN]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for the issue-rate probe:\n{res.stderr}")
    return PROBE_BIN


def build(verbose: bool = False) -> str:
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    build_probe()
    if verbose:
        print(f"built {LIB_PATH} and {PROBE_BIN}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
