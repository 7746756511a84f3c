"""Build libssm_recurrent_decode.so for gfx950 in-tree with hipcc.

    python -m ssm_recurrent_decode_amd.build [--jobs N]

Each csrc/*.hip file is compiled to an object under _build/ (in parallel), then the
objects are linked into ssm_recurrent_decode_amd/libssm_recurrent_decode.so.  The
device assembly of every object is kept next to it and scanned for instructions
this library must never contain (see isa_check.py, when present).
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
LIB_NAME = "libssm_recurrent_decode.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep hipcc from forming packed fp32 arithmetic on its own
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the only atomics (error-flag ORs, taken on anomalies) stay plain per-lane
    # operations: no wave-level rewrite with its extra waits
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-I", INCLUDE, "-I", CSRC,
    "-Wall", "-Wno-unused-result",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build")


def _run(cmd, what):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{what} failed:\n{r.stdout}\n{r.stderr}")


def _jobs(src: str):
    """The object file and, separately, the device assembly of the same
    translation unit (for the instruction scan); the two run in parallel."""
    name = os.path.splitext(os.path.basename(src))[0]
    obj = os.path.join(BUILD, name + ".o")
    asm = os.path.join(BUILD, name + f"-{ARCH}.s")
    hipcc = _hipcc()
    return (obj, [hipcc, *HIPCC_FLAGS, "-c", src, "-o", obj]), \
           (asm, [hipcc, *HIPCC_FLAGS, "--cuda-device-only", "-S", src, "-o", asm])


def build(jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources found")
    work = [j for src in srcs for j in _jobs(src)]
    jobs = jobs or min(len(work), max(1, os.cpu_count() or 1))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda j: _run(j[1], f"hipcc ({os.path.basename(j[0])})"), work))
    objs = [out for out, _ in work if out.endswith(".o")]
    asms = [out for out, _ in work if out.endswith(".s")]
    try:
        from . import isa_check  # not shipped to every machine; building happens here
    except ImportError:
        isa_check = None
    if isa_check is not None:
        isa_check.check(asms)
    check_no_spills(asms)
    tmp = LIB_PATH + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    _build_c_example(verbose)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


_KERNEL_META = re.compile(r"^\s+\.name:\s+(\S+)\s*$|^\s+\.private_segment_fixed_size:\s+(\d+)\s*$",
                          re.MULTILINE)


def kernel_scratch(asm_text: str) -> dict:
    """Per-kernel scratch bytes per work-item (.private_segment_fixed_size of the
    code-object metadata) in one device assembly file.  Within a kernel's
    metadata entry the fields are listed alphabetically, so .name precedes
    .private_segment_fixed_size."""
    out, name = {}, None
    for m in _KERNEL_META.finditer(asm_text):
        if m.group(1) is not None:
            name = m.group(1)
        elif name is not None:
            out[name] = int(m.group(2))
            name = None
    return out


def check_no_spills(asm_files) -> None:
    """Every decode kernel streams HBM: registers spilled to scratch would add
    per-lane memory traffic, so a kernel with any private segment fails the build."""
    bad = []
    for path in asm_files:
        with open(path) as f:
            for name, nbytes in kernel_scratch(f.read()).items():
                if nbytes:
                    bad.append(f"{os.path.basename(path)}: {name} spills {nbytes} B per work-item")
    if bad:
        raise RuntimeError("kernels spill registers to scratch:\n" + "\n".join(bad))


C_EXAMPLE = os.path.join(ROOT, "tests", "c_abi", "abi_roundtrip.cpp")


def _build_c_example(verbose: bool) -> None:
    """The C++ program that drives the C ABI without Python (a GPU test runs it),
    linked against the in-tree library through an rpath relative to itself."""
    if not os.path.exists(C_EXAMPLE):
        return
    exe = os.path.splitext(C_EXAMPLE)[0]
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-O2", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", INCLUDE, C_EXAMPLE, "-o", exe + ".tmp", "-L", PKG, "-lssm_recurrent_decode",
           "-Wl,-rpath,$ORIGIN/../../ssm_recurrent_decode_amd"]
    _run(cmd, "hipcc (abi_roundtrip)")
    os.replace(exe + ".tmp", exe)
    if verbose:
        print(f"built {exe}")


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=None)
    a = ap.parse_args(argv)
    build(a.jobs, verbose=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
