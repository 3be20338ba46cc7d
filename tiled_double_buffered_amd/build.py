"""Build the gfx950 library libgemmf32.so in-tree with hipcc, and expose its device
assembly and per-kernel resource usage for the structural tests.

    python -m tiled_double_buffered_amd.build          # builds the library
"""
from __future__ import annotations

import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
SOURCES = [os.path.join(CSRC, "gemm_f32.hip")]
HEADERS = [os.path.join(CSRC, f) for f in ("gemm_common.h", "kernels_sb_db.h", "kernels_ms.h",
                                            "splitk_reduce.h", "dispatch_table.h",
                                            "mfma_peak.h")]
DEPS = SOURCES + HEADERS + [os.path.join(INCLUDE, "gemmf32.h")]
LIB = os.path.join(PKG, "libgemmf32.so")
BUILD_DIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed FP32 instructions are switched off: the matrix cores do the arithmetic and the
# compiler must not form v_pk_* FP32 operations from the scalar code around them.
DEVICE_FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-I", INCLUDE,
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-Wall", "-Wno-unused-command-line-argument"]


def _run(cmd, **kw):
    return subprocess.run(cmd, check=True, **kw)


def build_library() -> str:
    """Compile libgemmf32.so (always recompiles).  Returns its path."""
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, *DEVICE_FLAGS, "-fPIC", "-shared", *SOURCES, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


def library_is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in DEPS)


def device_asm() -> str:
    """gfx950 assembly of the library's device code (cached under _build/)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    out = os.path.join(BUILD_DIR, "gemm_f32-gfx950.s")
    if not os.path.exists(out) or os.path.getmtime(out) < max(os.path.getmtime(p) for p in DEPS):
        tmp = out + ".tmp%d" % os.getpid()
        _run([HIPCC, *DEVICE_FLAGS, "--cuda-device-only", "-S", *SOURCES, "-o", tmp])
        os.replace(tmp, out)
    with open(out) as f:
        return f.read()


def kernel_functions(asm: str) -> dict:
    """Map mangled kernel name -> its assembly body (from the label to .Lfunc_end)."""
    out = {}
    for m in re.finditer(r"^(_Z\S*gemm_f32_(?:tile|ms)_kernel\S*):[ \t]*(?:;.*)?$", asm, re.M):
        name = m.group(1)
        end = asm.find(f".Lfunc_end", m.end())
        out[name] = asm[m.end():end]
    return out


def kernel_metadata(asm: str) -> dict:
    """Per-kernel resource figures from the assembler directives / metadata."""
    meta = {}
    for m in re.finditer(r"\.amdhsa_kernel\s+(\S+)(.*?)\.end_amdhsa_kernel", asm, re.S):
        name, body = m.group(1), m.group(2)
        d = {}
        for key in ("next_free_vgpr", "next_free_sgpr", "accum_offset",
                    "private_segment_fixed_size", "group_segment_fixed_size"):
            mm = re.search(r"\.amdhsa_%s\s+(\d+)" % key, body)
            if mm:
                d[key] = int(mm.group(1))
        meta[name] = d
    return meta


def main(argv=None) -> int:
    path = build_library()
    print(path)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
