"""Build libdetattn.so (HIP, gfx950) in-tree with hipcc.

Each translation unit is compiled to an object in parallel, then linked into
``deterministic_attention_backward_fa_amd/libdetattn.so``. Run as
``python -m deterministic_attention_backward_fa_amd.build``.
"""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdetattn.so")
ARCH = "gfx950"

MAIN_SOURCES = ["bwd_d64.hip", "bwd_d128.hip", "bwd_d64_trace.hip", "bwd_d128_trace.hip"]
SOURCES = ["capi.cpp", "kernels_misc.hip", "noalloc.hip", "xcd_probe.hip"] + MAIN_SOURCES
# The main backward kernel keeps MFMA results the VALU reads in VGPRs (its
# AGPR-resident accumulations are written as explicit AGPR-form MFMAs).
PER_SOURCE = {src: ["-mllvm", "-amdgpu-mfma-vgpr-form"] for src in MAIN_SOURCES}

# -packed-fp32-ops: keep the compiler from forming packed fp32 instructions.
COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", "-I", INCLUDE, "-I", CSRC, "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), "-c", "-x", "hip", os.path.join(CSRC, src), "-o", obj] + COMMON + PER_SOURCE.get(src, []) + list(extra)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


_REMARK = re.compile(r"remark: +(Function Name|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]|"
                     r"SGPRs Spill|VGPRs Spill|LDS Size \[bytes/block\]): (\S+)")


def resource_usage(src: str = "bwd_d128.hip", extra=()):
    """Per-kernel register and spill counts of one translation unit, from the
    compiler's kernel-resource-usage remarks: {mangled name: {field: value}}."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    obj = os.path.join(BUILD_DIR, "resource_" + os.path.basename(src) + ".o")
    cmd = ([hipcc(), "-c", "-x", "hip", os.path.join(CSRC, src), "-o", obj] + COMMON + PER_SOURCE.get(src, []) +
           list(extra) + ["-Rpass-analysis=kernel-resource-usage"])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stderr}")
    out, cur = {}, None
    for m in _REMARK.finditer(r.stderr):
        key, val = m.group(1).split(" [")[0], m.group(2)
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None:
            cur[key] = int(val)
    return out


def build(extra_flags=(), verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra_flags), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    if sys.argv[1:2] == ["--resource-usage"]:
        # python -m deterministic_attention_backward_fa_amd.build --resource-usage [source.hip]
        for name, f in resource_usage(*(sys.argv[2:3] or ["bwd_d128.hip"])).items():
            print(name, " ".join(f"{k}={v}" for k, v in f.items()))
    else:
        build(extra_flags=sys.argv[1:], verbose=True)
