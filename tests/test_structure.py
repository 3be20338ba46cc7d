"""Compile-time structure of the gfx950 kernels, read from this repository's own device
assembly (no GPU needed):

  * the double-buffered K-loop holds exactly one s_barrier and the single-buffered loop
    two ("Case Study: The Double-Buffered GEMM", second paragraph: one barrier per
    iteration instead of two; the code figure puts it at the top of the loop);
  * every kernel uses no scratch memory (no register spills), fits the 160 KiB LDS of a
    gfx950 compute unit, multiplies with the true FP32 matrix instruction and contains no
    packed FP32 instructions.
"""
import json
import os
import re

import pytest

from tiled_double_buffered_amd import build

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")


@pytest.fixture(scope="module")
def kernels():
    asm = build.device_asm()
    funcs = build.kernel_functions(asm)
    meta = build.kernel_metadata(asm)
    assert funcs and set(funcs) == set(meta)
    out = {}
    for name, body in funcs.items():
        m = re.search(r"TileCfgILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)EEELb([01])E", name)
        assert m, name
        bm, bn, bk, wm, wn, db = (int(x) for x in m.groups())
        out[name] = dict(cfg=(bm, bn, bk, wm, wn), db=bool(db), body=body, meta=meta[name])
    return out


def _loops(body: str):
    """(start, end) character spans of the loops: a label followed later by a branch back
    to it."""
    labels = {m.group(1): m.start() for m in re.finditer(r"^(\.LBB\w+):", body, re.M)}
    spans = []
    for m in re.finditer(r"^\s*s_(?:cbranch_\w+|branch)\s+(\.LBB\w+)", body, re.M):
        tgt = m.group(1)
        if tgt in labels and labels[tgt] < m.start():
            spans.append((labels[tgt], m.end()))
    return spans


def test_barriers_per_k_step(kernels):
    facts = json.load(open(GOLDEN))["barriers_per_k_step"]
    for name, k in kernels.items():
        body = k["body"]
        barriers = [m.start() for m in re.finditer(r"\bs_barrier\b", body)]
        expected = facts["double_buffered"] if k["db"] else facts["single_buffered"]
        assert len(barriers) == expected, (k["cfg"], k["db"], len(barriers))
        loops = _loops(body)
        assert loops, f"no K-loop found in {k['cfg']}"
        # every barrier sits inside one loop, and that loop holds all of them
        inside = [lp for lp in loops if all(lp[0] <= b <= lp[1] for b in barriers)]
        assert inside, (k["cfg"], k["db"], "barrier outside the K-loop")


def test_no_scratch_and_lds_fits(kernels):
    for name, k in kernels.items():
        meta = k["meta"]
        assert meta["private_segment_fixed_size"] == 0, k["cfg"]
        assert "scratch_" not in k["body"], k["cfg"]
        assert 0 < meta["group_segment_fixed_size"] <= 160 * 1024, k["cfg"]


def test_fp32_matrix_instruction_only(kernels):
    for name, k in kernels.items():
        body = k["body"]
        mfma = re.findall(r"\bv_mfma_\w+", body)
        assert mfma and set(mfma) == {"v_mfma_f32_32x32x2_f32"}, (k["cfg"], set(mfma))
        assert not re.search(r"\bv_pk_(fma|mul|add)_f32\b", body), k["cfg"]


def test_mfma_count_matches_tile(kernels):
    """Unrolled K tile: (BM/32) * (BN/32) * BK/2 MFMAs per workgroup = per wave
    FM * FN * BK / 2 (each MFMA consumes a k pair)."""
    for name, k in kernels.items():
        bm, bn, bk, wm, wn = k["cfg"]
        fm, fn = bm // wm // 32, bn // wn // 32
        n = len(re.findall(r"\bv_mfma_f32_32x32x2_f32\b", k["body"]))
        assert n == fm * fn * bk // 2, (k["cfg"], n)
