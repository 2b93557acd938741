"""Build the HIP attention library (libfa_mi355x.so) in-tree for gfx950.

Usage: ``python -m tiled_online_softmax_flashattention_amd.build [--jobs N]``.
Each translation unit is compiled separately with hipcc, then linked into one
shared library next to this file.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libfa_mi355x.so")
BUILD = os.path.join(PKG, "_build")
ARCH = "gfx950"

SOURCES = ["fa_api.cpp", "fa_rtc.cpp", "fa_fwd16.hip", "fa_fwd32.hip", "fa_bwd16.hip", "fa_dq16.hip",
           "fa_bwd32.hip", "fa_decode.hip"]
# Options for one translation unit only (beside COMMON).  The dQ pass is
# scheduled by LLVM's iterative ILP strategy, which measured faster for it
# (key-padding backward at head_dim 128: 2.14 -> 2.07 ms, same box; the other
# 16-bit kernels measured slower under it, up to twice as slow).
FILE_FLAGS: dict = {"fa_dq16.hip": ["-mllvm", "--amdgpu-sched-strategy=iterative-ilp"]}
# headers compiled again at run time (caller-defined score_mods), embedded as strings
RTC_EMBED = (("kRtcCommon", "fa_common.hpp"), ("kRtcCustom", "fa_custom.hpp"), ("kRtcFwd32", "fa_fwd32.hip"),
             ("kRtcBwd32", "fa_bwd32.hip"))

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU instructions are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", BUILD,
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


# The race-check library: the same sources with FA_DEBUG_BARRIERS (every
# barrier and wait drains the wave's outstanding memory operations first); a
# GPU test requires its results to equal the normal library's bit for bit.
RACECHECK_OUT = os.path.join(PKG, "libfa_mi355x_racecheck.so")
RACECHECK_BUILD = os.path.join(PKG, "_build_racecheck")


def _compile(src: str, racecheck: bool = False) -> str:
    out_dir = RACECHECK_BUILD if racecheck else BUILD
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    extra = ["-DFA_DEBUG_BARRIERS"] if racecheck else []
    cmd = [hipcc(), *COMMON, *FILE_FLAGS.get(src, []), *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def write_rtc_sources() -> None:
    """fa_rtc_sources.inc: the headers the run-time compiler needs, as raw
    string literals."""
    delim = "FA_RTC_SRC"
    parts = []
    for name, fname in RTC_EMBED:
        text = open(os.path.join(CSRC, fname)).read()
        if f"){delim}" in text:
            raise RuntimeError(f"{fname} contains the raw-string delimiter")
        parts.append(f'static const char {name}[] = R"{delim}({text}){delim}";\n')
    path = os.path.join(BUILD, "fa_rtc_sources.inc")
    new = "".join(parts)
    if not os.path.exists(path) or open(path).read() != new:
        with open(path, "w") as fh:
            fh.write(new)


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp, "-lhiprtc"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(jobs: int = 0, verbose: bool = True, racecheck: bool = True) -> str:
    """Compile every source and link the shared library (and, with
    racecheck, the race-check library); returns the library's path."""
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(RACECHECK_BUILD, exist_ok=True)
    write_rtc_sources()
    t0 = time.time()
    variants = [False, True] if racecheck else [False]
    tasks = [(src, rc) for rc in variants for src in SOURCES]
    jobs = jobs or min(len(tasks), os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda t: _compile(*t), tasks))
    _link(objs[:len(SOURCES)], OUT)
    if racecheck:
        _link(objs[len(SOURCES):], RACECHECK_OUT)
    if verbose:
        print(f"built {OUT}" + (f" and {RACECHECK_OUT}" if racecheck else "") + f" in {time.time() - t0:.1f}s",
              file=sys.stderr)
    return OUT


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=0)
    build(ap.parse_args().jobs)
