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
    assert funcs and set(funcs) <= set(meta)
    out = {}
    for name, body in funcs.items():
        m16 = re.search(r"Ks16CfgILi(\d+)ELi(\d+)ELb[01]ELi(\d+)E", name)
        if m16:  # the 16-row K-split kernel: a 16 x 16 CB tile, 16 k per block
            cb = int(m16.group(3))
            out[name] = dict(cfg=(16, 16 * cb, 16, int(m16.group(1)), 1), kind="ks16",
                             db=False, ms=False, stages=2, cb=cb, body=body, meta=meta[name])
            continue
        m = re.search(r"TileCfgILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)EEE(?:Lb([01])|Li(\d+))E",
                      name)
        assert m, name
        bm, bn, bk, wm, wn = (int(x) for x in m.groups()[:5])
        ms = "gemm_f32_ms_kernel" in name
        ks = "gemm_f32_ks_kernel" in name
        loop = int(m.group(7))
        kind = "ms" if ms else "ks" if ks else {1: "sb", 2: "db", 4: "sb3"}[loop]
        out[name] = dict(cfg=(bm, bn, bk, wm, wn), kind=kind, db=kind in ("db", "ms", "ks"),
                         ms=ms, stages=loop if ms else (2 if kind in ("db", "ks") else 1),
                         body=body, meta=meta[name])
    return out


def _loop_blocks(body: str):
    """Loops of a kernel, from the compiler's own block annotations: header id -> list of
    the instruction lines of every basic block in that loop (nested loops included)."""
    loops, cur = {}, None
    for line in body.split("\n"):
        m = re.match(r"^\.LBB(\w+):(.*)", line)
        if m:
            hdr = None
            if "Loop Header" in m.group(2):
                hdr = m.group(1)
            mm = re.search(r"Header=BB(\w+)", m.group(2))
            if mm:
                hdr = mm.group(1)
            cur = loops.setdefault(hdr, []) if hdr else None
            continue
        t = line.strip()
        if cur is not None and t and not t.startswith((";", ".")):
            cur.append(t)
    return loops


def _count_barriers(lines):
    return sum(1 for t in lines if re.match(r"s_barrier\b", t.strip()))


def _mfma_per_tile(cfg):
    bm, bn, bk, wm, wn = cfg
    return (bm // wm // 32) * (bn // wn // 32) * bk // 2


def test_barriers_per_k_step(kernels):
    """Barriers per K tile inside each K-loop: 1 (double-buffered and multi-stage), 2
    (single-buffered) or 3 (single-buffered with split copy barriers).  A loop body may
    hold several K tiles (the double-buffered loop is unrolled by two); the tiles per
    iteration are its MFMA count over one tile's.  Outside the loops the single-buffered
    kernels have exactly the barriers of one peeled last tile per loop (that tile's A
    columns past K are zeroed); the others have their prologue barriers and the barriers
    of the peeled step that copies the last tile."""
    facts = json.load(open(GOLDEN))["barriers_per_k_step"]
    for name, k in kernels.items():
        if k["kind"] == "ks16":
            # every wave's K groups pass through its own registers, with no LDS tile shared
            # between waves: no barrier in any loop, one for the hand-off of the sums
            assert not any(_count_barriers(ls) for ls in _loop_blocks(k["body"]).values())
            assert _count_barriers(k["body"].split("\n")) == 1, k["cfg"]
            continue
        if k["cfg"][3] * k["cfg"][4] == 1 and k["kind"] != "ks":
            # a one-wave workgroup: the compiler drops its barriers (the LDS operations of
            # one wave are performed in order), so the loop shape is all that remains
            assert _count_barriers(k["body"].split("\n")) == 0, (k["cfg"], k["kind"])
            continue
        expected = {"db": facts["double_buffered"], "ms": facts["double_buffered"],
                    "ks": facts["double_buffered"], "sb": facts["single_buffered"],
                    "sb3": facts["single_buffered_split_copies"]}[k["kind"]]
        per_tile = _mfma_per_tile(k["cfg"])
        loops = {h: ls for h, ls in _loop_blocks(k["body"]).items() if _count_barriers(ls)}
        if k["kind"] == "ks":
            # the K-split kernel's groups with fewer K tiles pass the missing tiles'
            # barriers in a loop of its own: one barrier, no MFMA
            pad = [h for h, ls in loops.items()
                   if not any(t.startswith("v_mfma") for t in ls)]
            assert len(pad) == 1 and _count_barriers(loops[pad[0]]) == 1, k["cfg"]
            del loops[pad[0]]
        assert loops, f"no K-loop with a barrier in {k['cfg']}"
        for h, ls in loops.items():
            mfma = sum(1 for t in ls if t.startswith("v_mfma"))
            assert mfma % per_tile == 0 and mfma > 0, (k["cfg"], k["kind"], h, mfma)
            tiles = mfma // per_tile
            assert _count_barriers(ls) == expected * tiles, (k["cfg"], k["kind"], h, tiles)
        outside = _count_barriers(k["body"].split("\n")) - sum(
            _count_barriers(ls) for ls in loops.values())
        if k["kind"] in ("sb", "sb3"):
            assert outside == expected * len(loops), (k["cfg"], k["kind"], outside)
        elif k["kind"] == "ks":  # plus the two of the hand-off
            assert 3 <= outside <= 3 * len(loops) + 2, (k["cfg"], k["kind"], outside)
        else:
            assert 1 <= outside <= 3 * len(loops), (k["cfg"], k["kind"], outside)


def test_bench_pair_keeps_two_and_one_barriers(kernels):
    """The single- against double-buffered pair that bench.py reports per workload shape
    runs on a configuration whose single-buffered loop holds two barriers per K tile and
    whose double-buffered loop holds one (one-wave workgroups, whose barriers the compiler
    drops, never form the pair)."""
    import bench
    import tdb_inputs as ti
    import tiled_double_buffered_amd as tdb
    for name, (M, N, K, _) in ti.WORKLOADS.items():
        sb = tdb.gemm_f32_select_cfg(M, N, K, tdb.VARIANT_SB)
        db = tdb.gemm_f32_select_cfg(M, N, K, tdb.VARIANT_DB)
        c = bench._pair_cfg(tdb, sb, db)
        _, i = tdb.gemm_f32_config_info(c)
        assert i["threads"] >= 128, (name, c)
        per_kind = {}
        for k in kernels.values():
            bm, bn, bk, wm, wn = k["cfg"]
            if (bm, bn, bk) == (i["BM"], i["BN"], i["BK"]) and wm * wn * 64 == i["threads"] \
                    and k["kind"] in ("sb", "db"):
                per_tile = _mfma_per_tile(k["cfg"])
                for ls in _loop_blocks(k["body"]).values():
                    bars = _count_barriers(ls)
                    mfma = sum(1 for t in ls if t.startswith("v_mfma"))
                    if bars:
                        per_kind.setdefault(k["kind"], set()).add(bars * per_tile // mfma)
        assert per_kind == {"sb": {2}, "db": {1}}, (name, c, per_kind)


def test_no_scratch_and_lds_fits(kernels):
    for name, k in kernels.items():
        meta = k["meta"]
        assert meta["private_segment_fixed_size"] == 0, k["cfg"]
        assert "scratch_" not in k["body"], k["cfg"]
        assert 0 < meta["group_segment_fixed_size"] <= 160 * 1024, k["cfg"]


def test_fp32_matrix_instruction_only(kernels):
    """True FP32 matrix instructions only: the 32 x 32 x 2 one, and the 16 x 16 x 4 one in
    the 16-row K-split kernel (whose 16-row tiles would leave half of a 32-row block idle);
    no packed FP32 arithmetic."""
    for name, k in kernels.items():
        body = k["body"]
        mfma = re.findall(r"\bv_mfma_\w+", body)
        want = "v_mfma_f32_16x16x4_f32" if k["kind"] == "ks16" else "v_mfma_f32_32x32x2_f32"
        assert mfma and set(mfma) == {want}, (k["cfg"], set(mfma))
        assert not re.search(r"\bv_pk_(fma|mul|add)_f32\b", body), k["cfg"]


def test_mfma_count_matches_tile(kernels):
    """One K tile is FM * FN * BK / 2 MFMAs per wave (each MFMA consumes a k pair); every
    kernel holds whole copies of that tile body (loops, unrolled steps, peeled tiles)."""
    for name, k in kernels.items():
        if k["kind"] == "ks16":  # 4 MFMAs of 16 x 16 x 4 per 16-deep block and column block
            n = len(re.findall(r"\bv_mfma_f32_16x16x4_f32\b", k["body"]))
            assert n > 0 and n % (4 * k["cb"]) == 0, (k["cfg"], n)
            continue
        per_tile = _mfma_per_tile(k["cfg"])
        n = len(re.findall(r"\bv_mfma_f32_32x32x2_f32\b", k["body"]))
        assert n > 0 and n % per_tile == 0, (k["cfg"], k["kind"], n, per_tile)


def test_multistage_copies_and_m0(kernels):
    """The multi-stage kernels copy with buffer_load_dwordx4 ... lds only, each copy one wait
    state after the s_mov_b32 that sets its LDS destination in M0, and nothing else touches M0.
    The per-tile copy count is (BM*BK + BK*BN) * 4 bytes / 1 KiB / waves, issued S-1 times
    in the prologue, S times in the unrolled steps and once in the remainder step, in the
    loop for interior tiles and in the one for edge tiles."""
    seen = 0
    for name, k in kernels.items():
        lines = [t.strip() for t in k["body"].split("\n")]
        m0_lines = [i for i, t in enumerate(lines) if re.search(r"\bm0\b", t)]
        dma = [t for t in lines if re.match(r"buffer_load_dwordx4\b.*\blds$", t)]
        if not k["ms"]:
            assert not dma and "global_load_lds" not in k["body"], k["cfg"]
            continue
        seen += 1
        for i in m0_lines:
            # the M0 write, one wait state (the hazard between a scalar M0 write and a
            # direct-to-LDS load), then the load
            assert lines[i].startswith("s_mov_b32 m0,"), (k["cfg"], lines[i])
            assert lines[i + 1] == "s_nop 0", (k["cfg"], lines[i + 1])
            assert re.match(r"buffer_load_dwordx4\b.*\blds$", lines[i + 2]), \
                (k["cfg"], lines[i + 2])
        bm, bn, bk, wm, wn = k["cfg"]
        per_wave = (bm * bk + bk * bn) * 4 // 1024 // (wm * wn)
        n = len(dma)
        # issue sites: S-1 in the prologue, S in the unrolled steps, 1 in the remainder step,
        # in each of the two copies of the loop (interior tiles, edge tiles)
        assert n == 2 * per_wave * 2 * k["stages"], (k["cfg"], n, per_wave, k["stages"])
        assert len(m0_lines) == n
    assert seen >= 1


def test_every_kernel_has_no_scratch():
    """All kernels of the library, the split-K reduction included."""
    meta = build.kernel_metadata(build.device_asm())
    assert any("splitk_reduce" in n for n in meta)
    for name, m in meta.items():
        assert m["private_segment_fixed_size"] == 0, name


def test_unguarded_copies_are_buffer_loads_without_vector_address_math(kernels):
    """The register-staged kernels' unguarded K-loop (the one with no element-wise
    guarded loads) copies with buffer loads from a scalar base plus fixed per-thread
    offsets: no 64-bit vector address additions are left in it."""
    seen = 0
    for name, k in kernels.items():
        if k["ms"]:
            continue
        # the K-loops are the loops with MFMAs; the unguarded ones have no element loads
        fast = [ins for ins in _loop_blocks(k["body"]).values()
                if any(t.startswith("v_mfma") for t in ins) and
                not any(re.match(r"global_load_dword\b", t) for t in ins)]
        assert fast, k["cfg"]
        for ins in fast:
            assert any(t.startswith("buffer_load_dwordx4") for t in ins), (k["cfg"], k["kind"])
            assert not any(t.startswith("global_load_dwordx4") for t in ins), k["cfg"]
            assert not any(t.startswith("v_lshl_add_u64") for t in ins), (k["cfg"], k["kind"])
        seen += 1
    assert seen >= 3


def test_lds_poison_build_fills_every_freed_slot():
    """The LDS-poison debug build (GEMMF32_LDS_POISON=1, the library's test variant) stores
    NaN into each slot right after the barrier that frees it: in every K-loop of the
    64 x 64 x 32 four-wave kernels, one extra 16-byte store per 16-byte copy store (the
    register-staged loops) or per direct-to-LDS copy of the wave (the multi-stage loop),
    per K tile; the production build has none of them."""
    cfg = 6  # 64 x 64 x 32, four waves: A and B copies of 2 + 2 groups per thread
    normal = build.kernel_functions(build.unit_asm(cfg))
    poison = build.kernel_functions(build.unit_asm(cfg, poison=True))
    assert set(normal) == set(poison)
    per_tile_mfma = 16          # one 32 x 32 block per wave, BK / 2 k pairs
    copies_per_tile = 4         # (64*32 + 32*64) floats: 4 x 16 bytes per thread / 1 KiB per wave
    seen = 0
    for name in normal:
        def loops(body):
            out = []
            for ins in _loop_blocks(body).values():
                if _count_barriers(ins):
                    mfma = sum(1 for t in ins if t.startswith("v_mfma"))
                    stores = sum(1 for t in ins if t.startswith("ds_write_b128"))
                    out.append((mfma // per_tile_mfma, stores))
            return sorted(out)
        ln, lp = loops(normal[name]), loops(poison[name])
        assert len(ln) == len(lp) and ln, name
        for (tiles, st_n), (tiles_p, st_p) in zip(ln, lp):
            assert tiles == tiles_p
            assert st_p - st_n == copies_per_tile * tiles, (name, tiles, st_n, st_p)
        assert "0x7fc00000" in poison[name] and "0x7fc00000" not in normal[name]
        seen += 1
    assert seen == 4  # single-, double-buffered, split-barrier and multi-stage
