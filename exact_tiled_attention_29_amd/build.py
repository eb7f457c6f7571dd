"""Build libfa.so in-tree with hipcc for gfx950.

Usage: python -m exact_tiled_attention_29_amd.build  (or call build()).
Each .hip source under csrc/ is compiled to an object in parallel, then the
objects are linked into exact_tiled_attention_29_amd/libfa.so.
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
OUT = os.path.join(PKG, "libfa.so")
BUILD_DIR = os.path.join(ROOT, "_build")

ARCH = "gfx950"
COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # Keep the compiler from forming packed fp32 VALU ops (v_pk_*_f32).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]

# Per-source additions. The backward's MFMA results feed VALU work (the
# softmax) right away: keep them in VGPRs (the default puts them in AGPRs
# and copies every element back before use).
FILE_FLAGS = {
    "fa_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return path


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


# Kernels whose registers must never spill to scratch (a spill in the hot
# loop puts memory waits between the MFMAs or FMAs): every attention and row
# kernel (the float32 ones spread a row over up to four lanes so that at
# most 32 columns of each row vector sit in a thread's registers).
NO_SPILL = ("fwd_bf16_kernel", "fwd_pp_kernel", "bwd_dkdv_kernel", "bwd_dq_kernel",
            "bwd_pre_kernel", "row_softmax_kernel", "fwd_merge_kernel", "split_reduce_kernel",
            "fwd_f32_kernel", "bwd_dkdv_f32_kernel", "bwd_dq_f32_kernel", "bwd_pre_f32_kernel")
_REMARK = re.compile(r"remark:\s+(Function Name|VGPRs Spill|ScratchSize \[bytes/lane\]|VGPRs|AGPRs|"
                     r"Occupancy \[waves/SIMD\]):\s+(\S+)")


def resource_usage(stderr: str):
    """Per kernel {VGPRs, AGPRs, VGPRs Spill, ScratchSize, Occupancy} from
    the compiler's kernel-resource-usage remarks."""
    out, cur = {}, None
    for m in _REMARK.finditer(stderr):
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None:
            cur[key.split(" [")[0]] = int(val)
    return out


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), *extra,
           "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    usage = resource_usage(r.stderr)
    with open(obj + ".resources.txt", "w") as fh:
        for name, u in sorted(usage.items()):
            fh.write(f"{name} {u}\n")
    spilled = [n for n, u in usage.items()
               if any(k in n for k in NO_SPILL) and (u.get("VGPRs Spill", 0) or u.get("ScratchSize", 0))]
    if spilled:
        raise RuntimeError(f"{src}: kernels spill registers to scratch: {spilled}")
    # hipcc's host pass warns about the gfx-only feature flag; keep real warnings.
    lines = [ln for ln in r.stderr.splitlines()
             if ln.strip() and "packed-fp32-ops" not in ln and "kernel-resource-usage" not in ln
             and not ln.lstrip().startswith(("|", "^")) and not re.match(r"^\s*\d+ \|", ln)]
    if lines:
        sys.stderr.write("\n".join(lines) + "\n")
    return obj


def build(verbose: bool = False, extra=()) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra)), srcs))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
