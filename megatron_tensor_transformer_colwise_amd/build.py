"""Builds the native libraries of the package, in-tree.

* ``libtpshard.so`` -- the HIP kernels for gfx950 and the C ABI declared in
  ``include/tpshard.h``.
* ``synth/_synth.so`` -- the seeded synthetic-input generator (plain C, OpenMP).

Every HIP translation unit is compiled with packed-fp32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); ``FILE_FLAGS`` adds
per-file code-generation options.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
REPO = PKG.parent
CSRC = PKG / "csrc"
OBJ = PKG / "_build"
HIP_LIB = PKG / "libtpshard.so"
SYNTH_SRC = PKG / "synth" / "synth.c"
SYNTH_LIB = PKG / "synth" / "_synth.so"

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{REPO / 'include'}",
    f"-I{CSRC}",
]


# Per-file additions.  The attention kernels post-process every score (and
# score-gradient) accumulator with vector ALU code; left to its default, the
# register allocator places those accumulators in AGPRs and moves each value
# to a VGPR and back (hundreds of moves per tile), so the backward's MFMAs are
# told to write VGPRs (the forward, at two workgroups per CU, gets VGPR-form
# MFMAs by default).  The forward's max trees assume no NaN scores (its inputs
# are finite), so each fmax is one v_max/v_max3 without a quieting copy of its
# operands.  In the GEMM file, the scheduler's high-register-pressure
# rescheduling pass otherwise splits the 16x16 kernel's 256 accumulator
# registers between AGPRs and VGPRs and copies them around the k loop (one
# move per MFMA); without it the loop is MFMAs, fragment reads and loads only
# (the other GEMM kernels compile to the same code either way).
FILE_FLAGS = {
    "gemm.hip": ["-mllvm", "-amdgpu-disable-unclustered-high-rp-reschedule=1"],
    "flash_attn.hip": ["-fno-honor-nans"],
    "flash_attn_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _run(cmd: list[str]) -> None:
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(
        ln for ln in proc.stdout.splitlines() if "packed-fp32-ops" not in ln and ln.strip()
    )
    if proc.returncode != 0:
        raise RuntimeError(f"command failed ({proc.returncode}): {' '.join(cmd)}\n{out}")
    if out:
        print(out, file=sys.stderr)


def build_synth() -> Path:
    tmp = SYNTH_LIB.with_suffix(".so.tmp")
    _run(["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-o", str(tmp), str(SYNTH_SRC), "-lm"])
    os.replace(tmp, SYNTH_LIB)
    return SYNTH_LIB


def hip_sources() -> list[Path]:
    return sorted(CSRC.glob("*.hip")) + sorted(CSRC.glob("*.cpp"))


def build_hip(jobs: int | None = None) -> Path:
    OBJ.mkdir(exist_ok=True)
    srcs = hip_sources()
    objs = [OBJ / (s.name + ".o") for s in srcs]

    def compile_one(pair):
        src, obj = pair
        lang = ["-x", "hip"] if src.suffix == ".hip" else []
        _run([HIPCC, *HIP_FLAGS, *FILE_FLAGS.get(src.name, []), *lang, "-c", str(src), "-o", str(obj)])

    jobs = jobs or min(len(srcs), os.cpu_count() or 4, 16)
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(compile_one, zip(srcs, objs)))
    tmp = HIP_LIB.with_suffix(".so.tmp")
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", str(tmp), *map(str, objs)])
    os.replace(tmp, HIP_LIB)
    return HIP_LIB


def build_all() -> None:
    build_synth()
    build_hip()


if __name__ == "__main__":
    build_all()
    print(f"built {HIP_LIB} and {SYNTH_LIB}")
