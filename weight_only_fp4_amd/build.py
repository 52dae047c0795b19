"""Build the HIP library ``libnvfp4_w4a16.so`` in-tree for gfx950.

    python -m weight_only_fp4_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

if __package__:
    from . import isa_check
else:   # run as a script
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    from weight_only_fp4_amd import isa_check

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libnvfp4_w4a16.so")
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]
# (source, extra flags, object tag).  The kernel families are split into
# translation units per activation type (and scale format for the
# activation-resident and MFMA-bound kernels, pre-scale form for the latter)
# so that they compile in parallel.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form"]   # MFMA results in VGPRs (post-processed by VALU)
SOURCES = [
    ("nvfp4_w4a16.hip", VGPR_FORM, "abi"),
    ("nvfp4_mfma.hip", [], "mfma_plan"),
] + [
    (f"gemm_{fam}.hip", VGPR_FORM + [f"-DNVFP4_ACT_F16={f16}"], f"{fam}_{f16}")
    for fam in ("small", "tile") for f16 in (0, 1)
] + [
    # one unit per scale format too (NVFP4 / MXFP4)
    ("gemm_xres.hip", VGPR_FORM + [f"-DNVFP4_ACT_F16={f16}", f"-DNVFP4_MX={mx}"], f"xres_{f16}{mx}")
    for f16 in (0, 1) for mx in (0, 1)
] + [
    # the MFMA-bound kernel keeps its 256 accumulators in AGPRs
    ("gemm_mfma.hip", [f"-DNVFP4_ACT_F16={f16}", f"-DNVFP4_PRE={pre}", f"-DNVFP4_MX={mx}"], f"mfma_{f16}{pre}{mx}")
    for f16 in (0, 1) for pre in (0, 1) for mx in (0, 1)
]
NOISE = "not a recognized feature for this target"


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if NOISE not in l and l.strip())
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + msgs)
    return msgs


# Units whose kernels hold inline-asm MFMAs and copies: their assembly is
# checked for the wait states the compiler does not insert around those.
ASM_CHECKED = ("gemm_mfma.hip",)


def _check_asm(cmd, path):
    _run(cmd)
    with open(path) as f:
        found = isa_check.hazards(f.read())
    if found:
        raise RuntimeError("wait-state violations in the generated assembly of " + " ".join(cmd) + ":\n  "
                           + "\n  ".join(found[:20]))
    return ""


def build(verbose: bool = False) -> str:
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    with tempfile.TemporaryDirectory(prefix="nvfp4_build_") as tmpd:
        jobs, checks = [], []
        for src, extra, tag in SOURCES:
            obj = os.path.join(tmpd, tag + ".o")
            jobs.append((obj, [hipcc, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]))
            if src in ASM_CHECKED:
                asm = os.path.join(tmpd, tag + ".s")
                checks.append((asm, [hipcc, *COMMON, *extra, "--cuda-device-only", "-S",
                                     os.path.join(CSRC, src), "-o", asm]))
        with ThreadPoolExecutor(max(1, os.cpu_count() or 1)) as ex:
            futs = [ex.submit(lambda j: (j[1], _run(j[1])), j) for j in jobs]
            futs += [ex.submit(lambda c: (c[1], _check_asm(c[1], c[0])), c) for c in checks]
            outs = [f.result() for f in futs]
        for cmd, msgs in outs:
            if verbose:
                print(" ".join(cmd), flush=True)
                if msgs:
                    print(msgs, flush=True)
        tmp = LIB + ".tmp%d" % os.getpid()
        link = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *[o for o, _ in jobs], "-o", tmp]
        msgs = _run(link)
        if verbose:
            print(" ".join(link), flush=True)
            if msgs:
                print(msgs, flush=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
