"""Build libautoround_hip.so (gfx950) in-tree with hipcc.

    python autoround_signsgd_rounding_amd/build.py

(run as a script, or through __graft_entry__.build(): importing the package
loads the library being built).
"""
import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libautoround_hip.so")
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["ar_api.hip", "ar_gemm.hip", "ar_gemm_small.hip", "ar_gram.hip", "ar_quant.hip",
           "ar_dequant.hip", "ar_block.hip", "ar_layers.cpp"]

# -ffp-contract=off: the quantizer's float32 steps must round exactly as
# written (no fused multiply-adds). Packed-fp32 instructions are disabled.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-fno-gpu-rdc", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


# Kernels whose speed depends on running without register spills: the MFMA
# contractions sit at the register file's limit. A spill (to scratch memory,
# behind a full vector-memory wait) is reported as a warning.
HOT = ("k_fwd_stream", "k_gemm", "k_gemm_small", "k_dq_mfma", "k_attention")
_FN = re.compile(r"Function Name: (\S+)")
_SPILL = re.compile(r"VGPRs Spill: (\d+)")


def _spills(remarks):
    out, fn = [], None
    for ln in remarks:
        m = _FN.search(ln)
        if m:
            fn = m.group(1)
            continue
        m = _SPILL.search(ln)
        if m and fn and int(m.group(1)) > 0 and any(h in fn for h in HOT):
            out.append((fn, int(m.group(1))))
    return out


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    lines = (r.stderr or "").splitlines()
    remarks = [ln for ln in lines if "kernel-resource-usage" in ln]
    msgs = [ln for ln in lines if noise not in ln and ("warning:" in ln or "error:" in ln)]
    if msgs:
        print("\n".join(msgs), file=sys.stderr)
    for fn, n in _spills(remarks):
        print(f"warning: {src}: {fn} spills {n} VGPRs (scratch traffic in a hot loop)",
              file=sys.stderr)
    return obj


def build(verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build()
