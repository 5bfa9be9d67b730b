"""Build libhm.so (HIP, gfx950) in-tree with hipcc.

The translation units are compiled in parallel to objects under _build/ and
linked into selective_state_space_hm_amd/libhm.so, next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libhm.so")
SOURCES = ["hm_abi.hip", "k_fwd_bf16.hip", "k_fwd_bf16_decay.hip", "k_fwd_f32.hip", "k_step_feat.hip",
           "k_conv.hip", "k_bwd.hip", "k_fwd_rope_bf16.hip", "k_fwd_rope_bf16_decay.hip", "k_fwd_rope_f32.hip",
           "k_pc.hip", "k_fwd_c128.hip", "k_fwd_f32_d64.hip", "k_cp_bf16.hip", "k_cp_f32.hip", "k_step_bf16.hip", "k_step_f32.hip"]
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms stay disabled in every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libhm.so)")


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass reports the disabled packed-fp32 feature as unknown: harmless
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"command failed: {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs = [os.path.join(BUILD, s.replace(".hip", ".o")) for s in SOURCES]
    cmds = [[cc, *FLAGS, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    jobs = jobs or min(len(cmds), os.cpu_count() or 4, 8)
    with ThreadPoolExecutor(jobs) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out, file=sys.stderr)
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
