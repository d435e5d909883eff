"""The gfx950 code of our own build holds the instructions the design rests
on (CPU only: hipcc compiles the library's device code to assembly).

- The headline segment merge (tiles stored from registers) moves HBM data
  as 16-byte vectors (global_load_dwordx4 / global_store_dwordx4), writes
  refills to LDS as 128-bit rows (ds_write_b128), swaps halves of lane pairs
  by DPP (quad_perm 1,0,3,2), and uses no scratch memory.
- Its staged variant (unaligned outputs) also reads the LDS stage as
  128-bit rows (ds_read_b128).
- No instantiation of the segment merge uses scratch memory.
- The block sort's in-wavefront rounds move lanes' keys with DPP row moves
  and ds_swizzle, keep one side of each exchange by v_med3_i32 (one per key
  per cross-lane stage), copy no key before a DPP move, and use no scratch
  memory.
"""
import re

import pytest

import isa_asm

MERGE = "_ZN6omerge21merge_segments_kernelILi256ELi8ELi0ELi0ELb0ELb1ELb0EE"
MERGE_STAGED = "_ZN6omerge21merge_segments_kernelILi256ELi8ELi0ELi0ELb0ELb0ELb0EE"
BLOCK_SORT = "_ZN6omerge17block_sort_kernelILi512ELi32ELi0ELi0EE"


@pytest.fixture(scope="module")
def asm():
    if not isa_asm.available():
        pytest.skip("hipcc is not installed")
    return isa_asm.assembly()


def body(asm, prefix):
    """The assembly of the first function whose symbol starts with prefix,
    and the scratch size the compiler reports for it."""
    m = re.search(r"^(%s\w*):" % re.escape(prefix), asm, re.M)
    assert m, "no function " + prefix
    end = asm.index("s_endpgm", m.end())
    meta = re.search(r"; ScratchSize: (\d+)", asm[end:])
    return asm[m.end():end], int(meta.group(1))


def test_segment_merge_vector_accesses(asm):
    code, scratch = body(asm, MERGE)
    for ins in ("global_load_dwordx4", "global_store_dwordx4", "ds_write_b128",
                "quad_perm:[1,0,3,2]"):
        assert ins in code, ins
    assert scratch == 0
    code, scratch = body(asm, MERGE_STAGED)
    for ins in ("global_load_dwordx4", "global_store_dwordx4", "ds_write_b128", "ds_read_b128"):
        assert ins in code, ins
    assert scratch == 0


def test_no_merge_kernel_spills(asm):
    """Every instantiation of the segment merge (each key order, payload
    width, mode and store path) runs without scratch: a spill of the
    register-stored outputs once made the 8-byte-key merge twice as slow."""
    names = sorted(set(re.findall(r"^(_ZN6omerge21merge_segments_kernel\w*):", asm, re.M)))
    assert len(names) >= 24, len(names)
    spilled = [n for n in names if body(asm, n)[1] != 0]
    assert not spilled, spilled


def test_multiway_kernels_without_scratch(asm):
    """The 4-way pass's plan and cell kernels, every key order, run without
    scratch.  Selects over a small array of words once compiled to a
    dynamically indexed private load (scratch memory) in every candidate
    read, and a select chain over an array of per-run offsets did the same;
    the cell kernel moves its windows and its output by 16-byte accesses."""
    names = sorted(set(re.findall(r"^(_ZN6omerge2\d(?:plan|merge)_multiway_kernel\w*):", asm,
                                  re.M)))
    assert len(names) >= 24, len(names)
    scratch = [n for n in names if body(asm, n)[1] != 0]
    assert not scratch, scratch
    code, _ = body(asm, "_ZN6omerge21merge_multiway_kernelILi256ELi32ELi4ELi0EE")
    for ins in ("global_load_dwordx4", "global_store_dwordx4", "ds_read_b128", "ds_write_b128"):
        assert ins in code, ins


def test_block_sort_lane_exchanges(asm):
    code, scratch = body(asm, BLOCK_SORT)
    assert "v_mov_b32_dpp" in code
    for pattern in ("quad_perm", "row_mirror", "row_half_mirror", "row_ror:8"):
        assert pattern in code, pattern
    assert "ds_swizzle_b32" in code
    assert scratch == 0
    # six rounds of in-wavefront merges hold 1 + 2 + ... + 6 = 21 cross-lane
    # stages, each one med3 per key (32 per lane)
    assert len(re.findall(r"\bv_med3_i32\b", code)) == 21 * 32
    # DPP moves write a fresh register: no v_mov_b32 copy of a key before one
    lines = [ln.split() for ln in code.splitlines() if ln.strip()]
    for prev, cur in zip(lines, lines[1:]):
        if cur[0] == "v_mov_b32_dpp" and prev[0] == "v_mov_b32_e32":
            assert prev[1].rstrip(",") != cur[1].rstrip(","), (prev, cur)


def test_block_sorts_without_scratch(asm):
    """Every block sort instantiation, (key, position) pairs and packed
    (image, position) keys included, runs without scratch."""
    names = sorted(set(re.findall(r"^(_ZN6omerge\d+block_sort(?:_packed)?_kernel\w*):", asm,
                                  re.M)))
    assert any("block_sort_packed_kernel" in n for n in names), names
    assert len(names) >= 12, len(names)
    scratch = [n for n in names if body(asm, n)[1] != 0]
    assert not scratch, scratch
