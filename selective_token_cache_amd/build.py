"""Build libdcu.so (gfx950) in-tree with hipcc.

    python -m selective_token_cache_amd.build [--jobs N]

Compiles every HIP source under csrc/ for gfx950 and links the shared library next to this file.
Object files go to <repo>/_build/ (not versioned). The device assembly of the kernels that drive the
LDS DMA from inline asm is listed and checked for compiler uses of M0 (check_m0) and for full
memory waits inside their staged loops (check_stage_waits).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdcu.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
CXX = os.environ.get("CXX", shutil.which("g++") or "g++")

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 are generated
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    if src.endswith(".hip"):
        cmd = [HIPCC, *HIP_FLAGS, "-c", src, "-o", obj]
    else:
        cmd = [CXX, "-O2", "-std=c++17", "-fPIC", "-I", INCLUDE, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


# Kernels that issue the LDS DMA through the inline-asm helper in gemm.h, which writes M0 (the DMA's
# LDS base) itself. M0 is reserved by the compiler, so it neither saves it nor knows that the asm
# changed it: these kernels are only correct if the compiler never relies on M0 in them. The build
# checks that in their gfx950 assembly.
DMA_SOURCES = ["layer.hip"]
# instructions that read M0 without naming it
_IMPLICIT_M0 = re.compile(r"^\s*(s_sendmsg|s_sendmsghalt|s_movrel|v_movrel|ds_gws|v_interp|"
                          r"ds_append|ds_consume|ds_ordered_count|buffer_load_\w+\s.*\blds\b|"
                          r"global_load_lds_(?!dwordx4))")


def _device_asm(src: str) -> str:
    out = os.path.join(BUILD, os.path.basename(src) + ".gfx950.s")
    cmd = [HIPCC, *HIP_FLAGS, "--cuda-device-only", "-S", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"assembly listing failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return out


def _functions(asm: str) -> list[tuple[str, list[str]]]:
    """(name, instructions) of every function in a gfx950 assembly listing."""
    funcs, cur, name = [], [], None
    for line in asm.splitlines():
        m = re.match(r"^(_Z\w+):", line)
        if m:
            if name:
                funcs.append((name, cur))
            name, cur = m.group(1), []
        elif name:
            code = line.split(";", 1)[0].strip()
            if code and not code.startswith(".") and not code.endswith(":"):
                cur.append(code)
    if name:
        funcs.append((name, cur))
    return funcs


def check_m0(asm: str) -> list[str]:
    """Problems with M0 in the functions of a gfx950 assembly listing that use the LDS DMA: every
    write of M0 must be the helper's own `s_mov_b32 m0, sN` directly followed by its
    global_load_lds_dwordx4, and no instruction may read M0 otherwise (explicitly or implicitly)."""
    bad = []
    for name, ins in _functions(asm):
        if not any(i.startswith("global_load_lds_dwordx4") for i in ins):
            continue
        for k, i in enumerate(ins):
            if re.search(r"\bm0\b", i):
                ok = (re.fullmatch(r"s_mov_b32 m0, s\d+", i) is not None and k + 1 < len(ins)
                      and ins[k + 1].startswith("global_load_lds_dwordx4"))
                if not ok:
                    bad.append(f"{name}: M0 used by the compiler: {i}")
            elif i.startswith("global_load_lds_dwordx4"):
                if k == 0 or not re.fullmatch(r"s_mov_b32 m0, s\d+", ins[k - 1]):
                    bad.append(f"{name}: LDS DMA without its M0 write: {i}")
            elif _IMPLICIT_M0.match(i):
                bad.append(f"{name}: instruction reading M0: {i}")
    return bad


def check_stage_waits(asm: str) -> list[str]:
    """Full memory waits that the compiler placed inside the staged loops of the LDS-DMA kernels.
    Their stages are synchronised by an explicit `s_waitcnt vmcnt(n)` before each `s_barrier`; the
    DMAs are asm that the compiler does not count, so a `s_waitcnt vmcnt(0)` it inserts right after
    such a barrier (for a load or store of its own still pending at the loop head) drains every DMA
    in flight and serialises the stages: correct, but it cost the K-looped projections 10-15%."""
    bad = []
    for name, ins in _functions(asm):
        if not any(i.startswith("global_load_lds_dwordx4") for i in ins):
            continue
        for k, i in enumerate(ins):
            if i == "s_barrier":
                for j in ins[k + 1:k + 4]:
                    if j.startswith("s_waitcnt") and "vmcnt(0)" in j:
                        bad.append(f"{name}: full wait after a stage barrier: {j}")
    return bad


def build(jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    jobs = jobs or min(8, os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        asm_jobs = [ex.submit(_device_asm, os.path.join(CSRC, f)) for f in DMA_SOURCES]
        objs = list(ex.map(_compile, srcs))
        listings = [j.result() for j in asm_jobs]
    for path in listings:
        asm = open(path).read()
        problems = check_m0(asm)
        if problems:
            raise RuntimeError("M0 check failed in " + path + ":\n  " + "\n  ".join(problems[:20]))
        problems = check_stage_waits(asm)
        if problems:
            raise RuntimeError("stage wait check failed in " + path + ":\n  " +
                               "\n  ".join(problems[:20]))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    a = ap.parse_args()
    build(a.jobs, verbose=True)
    sys.exit(0)
