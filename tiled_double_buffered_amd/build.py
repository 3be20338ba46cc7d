"""Build the gfx950 library libgemmf32.so in-tree with hipcc, and expose its device
assembly and per-kernel resource usage for the structural tests.

    python -m tiled_double_buffered_amd.build              # builds the library and its
                                                           # LDS-poison debug variant
    python -m tiled_double_buffered_amd.build --resources  # per-kernel registers, LDS,
                                                           # scratch, barriers per loop

The debug variant libgemmf32_lds_poison.so is the same source built with
GEMMF32_LDS_POISON=1: every LDS slot is filled with NaN right after the barrier that frees
it, so a loop that read a slot after that barrier would put NaN into C.  Only the tests
load it.
"""
from __future__ import annotations

import concurrent.futures
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
MAIN_SOURCE = os.path.join(CSRC, "gemm_f32.hip")
CFG_SOURCE = os.path.join(CSRC, "cfg_kernels.hip")
NUM_CONFIGS = 20  # configs.h: kNumConfigs
SOURCES = [MAIN_SOURCE, CFG_SOURCE]
HEADERS = [os.path.join(CSRC, f) for f in ("configs.h", "gemm_common.h", "kernels_sb_db.h",
                                            "kernels_ms.h", "kernels_ks.h", "kernels_ks16.h", "splitk_reduce.h",
                                            "dispatch_table.h", "mfma_peak.h")]
DEPS = SOURCES + HEADERS + [os.path.join(INCLUDE, "gemmf32.h")]
LIB = os.path.join(PKG, "libgemmf32.so")
LIB_POISON = os.path.join(PKG, "libgemmf32_lds_poison.so")
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


def _units():
    """(name, source, extra flags) of every translation unit: the host code and reduction
    kernels, then one unit per tile configuration."""
    units = [("gemm_f32", MAIN_SOURCE, [])]
    units += [(f"cfg{i}", CFG_SOURCE, [f"-DGEMMF32_CFG_ID={i}"]) for i in range(NUM_CONFIGS)]
    return units


def _parallel(cmds):
    jobs = max(1, min(16, os.cpu_count() or 1))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        for f in [ex.submit(_run, c) for c in cmds]:
            f.result()


def _library_jobs(poison: bool):
    """(compile commands, objects, link command, temporary output, output) of one build."""
    obj_dir = os.path.join(BUILD_DIR, "obj_poison" if poison else "obj")
    os.makedirs(obj_dir, exist_ok=True)
    flags = ["-DGEMMF32_LDS_POISON=1"] if poison else []
    out = LIB_POISON if poison else LIB
    objs, cmds = [], []
    for name, src, extra in _units():
        obj = os.path.join(obj_dir, name + ".o")
        objs.append(obj)
        cmds.append([HIPCC, *DEVICE_FLAGS, *flags, *extra, "-fPIC", "-c", src, "-o", obj])
    tmp = out + ".tmp%d" % os.getpid()
    return cmds, [HIPCC, f"--offload-arch={ARCH}", "-shared", *objs, "-o", tmp], tmp, out


def build_library(poison: bool = False) -> str:
    """Compile libgemmf32.so, or with `poison` its LDS-poison debug variant (always
    recompiles; the translation units in parallel).  Returns its path."""
    cmds, link, tmp, out = _library_jobs(poison)
    _parallel(cmds)
    _run(link)
    os.replace(tmp, out)
    return out


def build_all() -> list:
    """Both libraries, every translation unit of both in one parallel pool."""
    jobs = [_library_jobs(False), _library_jobs(True)]
    _parallel([c for cmds, _, _, _ in jobs for c in cmds])
    outs = []
    for _, link, tmp, out in jobs:
        _run(link)
        os.replace(tmp, out)
        outs.append(out)
    return outs


def library_is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in DEPS)


def device_asm() -> str:
    """gfx950 assembly of the library's device code, all translation units (cached under
    _build/)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    newest = max(os.path.getmtime(p) for p in DEPS)
    outs, cmds = [], []
    for name, src, extra in _units():
        out = os.path.join(BUILD_DIR, f"{name}-gfx950.s")
        outs.append(out)
        if not os.path.exists(out) or os.path.getmtime(out) < newest:
            tmp = out + ".tmp%d" % os.getpid()
            cmds.append(([HIPCC, *DEVICE_FLAGS, *extra, "--cuda-device-only", "-S", src,
                          "-o", tmp], tmp, out))
    _parallel([c for c, _, _ in cmds])
    for _, tmp, out in cmds:
        os.replace(tmp, out)
    text = []
    for out in outs:
        with open(out) as f:
            text.append(f.read())
    return "\n".join(text)


def unit_asm(cfg_id: int, poison: bool = False) -> str:
    """gfx950 assembly of one configuration's translation unit, optionally the LDS-poison
    build (cached under _build/)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    out = os.path.join(BUILD_DIR, f"cfg{cfg_id}{'-poison' if poison else ''}-gfx950.s")
    if not os.path.exists(out) or os.path.getmtime(out) < max(os.path.getmtime(p) for p in DEPS):
        tmp = out + ".tmp%d" % os.getpid()
        flags = ["-DGEMMF32_LDS_POISON=1"] if poison else []
        _run([HIPCC, *DEVICE_FLAGS, *flags, f"-DGEMMF32_CFG_ID={cfg_id}", "--cuda-device-only",
              "-S", CFG_SOURCE, "-o", tmp])
        os.replace(tmp, out)
    with open(out) as f:
        return f.read()


def kernel_functions(asm: str) -> dict:
    """Map mangled kernel name -> its assembly body (from the label to .Lfunc_end)."""
    out = {}
    for m in re.finditer(r"^(_Z\S*gemm_f32_(?:tile|ms|ks|ks16)_kernel\S*):[ \t]*(?:;.*)?$", asm,
                         re.M):
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


def _loops(body: str) -> dict:
    """Loop header id -> instruction lines of the loop's blocks (from the compiler's own
    block annotations)."""
    loops, cur = {}, None
    for line in body.split("\n"):
        m = re.match(r"^\.LBB(\w+):(.*)", line)
        if m:
            hdr = m.group(1) if "Loop Header" in m.group(2) else None
            mm = re.search(r"Header=BB(\w+)", m.group(2))
            if mm:
                hdr = mm.group(1)
            cur = loops.setdefault(hdr, []) if hdr else None
            continue
        t = line.strip()
        if cur is not None and t and not t.startswith((";", ".")):
            cur.append(t)
    return loops


def resources_table(asm: str) -> str:
    """One line per kernel: tile, loop kind, registers, LDS, scratch, and the barriers and
    MFMAs of each barrier-carrying loop (barriers per MFMA-tile of that loop)."""
    meta = kernel_metadata(asm)
    rows = ["kernel                         vgpr agpr sgpr  lds_B scratch  loops: barriers/MFMAs"]
    for name, body in sorted(kernel_functions(asm).items()):
        m16 = re.search(r"Ks16CfgILi(\d+)ELi(\d+)ELb[01]ELi(\d+)E", name)
        if m16:  # the 16-row K-split kernel: 16 x 16 CB tile, 16-k blocks per group, W waves
            kind = "ks%s" % m16.group(1)
            tile = "16x%dx%d/%sx1" % (16 * int(m16.group(3)), 16 * int(m16.group(2)),
                                      m16.group(1))
        else:
            m = re.search(r"TileCfgILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)EEELi(\d+)E", name)
            kind = "ms%s" % m.group(6) if "_ms_kernel" in name else \
                "ks%s" % m.group(6) if "_ks_kernel" in name else \
                {"1": "sb", "2": "db", "4": "sb3"}[m.group(6)]
            tile = "%sx%sx%s/%sx%s" % m.groups()[:5]
        d = meta[name]
        # unified register file: architected VGPRs first, AGPRs from accum_offset on
        arch = min(d.get("accum_offset", d["next_free_vgpr"]), d["next_free_vgpr"])
        agpr = max(0, d["next_free_vgpr"] - d.get("accum_offset", d["next_free_vgpr"]))
        loops = []
        for ins in _loops(body).values():
            nb = sum(1 for t in ins if re.match(r"s_barrier\b", t))
            if nb:
                nm = sum(1 for t in ins if t.startswith("v_mfma"))
                loops.append(f"{nb}/{nm}")
        rows.append(f"{kind:>4} {tile:<24} {arch:>4} {agpr:>4} {d['next_free_sgpr']:>4} "
                    f"{d['group_segment_fixed_size']:>6} {d['private_segment_fixed_size']:>7}  "
                    + " ".join(loops))
    return "\n".join(rows)


def main(argv=None) -> int:
    argv = list(argv or [])
    if "--resources" in argv:
        print(resources_table(device_asm()))
        return 0
    for path in build_all():
        print(path)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
