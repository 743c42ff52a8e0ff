"""LDS placements of the kernels: rows must not overlap and the operand reads
must be free of bank conflicts under the gfx950 LDS model (64 banks of 4
bytes; a 16-byte read is served 16 lanes at a time, an 8-byte transposing read
32 lanes at a time). The model matches the hardware's own counter:
SQ_LDS_BANK_CONFLICT reads 0 for these kernels. The constants are read from
the kernel sources, so a change to them is checked here on the CPU."""
import os
import re

import pytest

CSRC = os.path.join(os.path.dirname(__file__), "..", "exact_attention_31_amd", "csrc")


def _src(name):
    with open(os.path.join(CSRC, name)) as f:
        return f.read()


def _pair(src, pattern):
    m = re.search(pattern + r"\s*=\s*\(D == 128\) \? (\d+) : (\d+);", src)
    assert m, pattern
    return {128: int(m.group(1)), 64: int(m.group(2))}


def _conflict_free(accesses, banks=64):
    """accesses: (first dword, dwords) per lane of one LDS cycle."""
    used = set()
    for a, n in accesses:
        for k in range(n):
            b = (a + k) % banks
            if b in used:
                return False
            used.add(b)
    return True


def _grouped(D):
    src = _src("backward.hip")
    IN, GRP = _pair(src, r"static constexpr int IN"), _pair(src, r"static constexpr int GRP")
    return IN[D], GRP[D]


@pytest.mark.parametrize("D", [64, 128])
def test_backward_grouped_rows_do_not_overlap(D):
    IN, GRP = _grouped(D)
    row = lambda r: GRP * (r // 4) + IN * (r % 4)  # elements
    spans = sorted((row(r), row(r) + D) for r in range(64))
    assert all(a_end <= b for (_, a_end), (b, _) in zip(spans, spans[1:]))
    assert spans[-1][1] <= GRP * 16  # the tile's allocation (64 rows)
    assert (IN * 2) % 16 == 0 and (GRP * 2) % 16 == 0  # 16-byte aligned rows


@pytest.mark.parametrize("D", [64, 128])
def test_backward_grouped_reads_are_conflict_free(D):
    IN, GRP = _grouped(D)
    row = lambda r: (GRP * (r // 4) + IN * (r % 4)) // 2  # dwords
    # 16-byte row reads: 16 lanes take 16 consecutive rows at one column
    for r0 in range(0, 64, 16):
        for col in range(0, D // 2, 4):
            assert _conflict_free([(row(r0 + i) + col, 4) for i in range(16)])
    # transposing reads: 32 lanes take 4 consecutive rows x 16 dwords
    for r0 in range(0, 64, 4):
        for col in range(0, D // 2, 16):
            assert _conflict_free([(row(r0 + i) + col, 16) for i in range(4)])


def test_a_single_padded_stride_cannot_serve_both_reads():
    # why the grouped placement exists: no stride satisfies both patterns
    for stride in range(64, 64 + 128):
        rows = _conflict_free([(stride * i, 4) for i in range(16)])
        tr = _conflict_free([(stride * i, 16) for i in range(4)])
        assert not (rows and tr), stride


@pytest.mark.parametrize("D", [64, 128])
def test_prefill_tile_strides_are_conflict_free(D):
    src = _src("prefill.hip")
    m = re.search(r"static constexpr int kK = D \+ (\d+);", src)
    kK = D + int(m.group(1))
    kV = _pair(src, r"static constexpr int kV")[D]
    # K rows: 16-byte reads of 16 consecutive rows
    assert _conflict_free([(kK // 2 * i, 4) for i in range(16)])
    # V rows: transposing reads of 4 consecutive rows, two 16-lane groups
    # 8 dwords apart (4 rows x 16 dwords per 32 lanes)
    assert _conflict_free([(kV // 2 * i, 16) for i in range(4)])


# the ring form's XOR swizzle, as written in prefill.hip (RingLds)
_KSWZ = "return (r / RPB) & (CPR - 1);"
_VSWZ = "return 4 * ((r / RPB) & (RPB == 1 ? 3 : 1));"


@pytest.mark.parametrize("D", [64, 128])
def test_ring_swizzle_is_conflict_free(D):
    """Unpadded rows of D 16-bit elements, 16-byte chunk c of row r stored at
    chunk c ^ swz(r): K is read 16 consecutive rows at one logical chunk per
    LDS cycle, V by transposing reads of 4 consecutive rows x 4 chunks per 32
    lanes. Both must hit 64 distinct banks, for every row group of a 64-key
    tile and every chunk."""
    src = _src("prefill.hip")
    assert _KSWZ in src and _VSWZ in src
    RB = 2 * D
    CPR, RPB = D // 8, 256 // RB
    kswz = lambda r: (r // RPB) & (CPR - 1)
    vswz = lambda r: 4 * ((r // RPB) & (3 if RPB == 1 else 1))
    dword = lambda r, slot: (r * RB + 16 * slot) // 4
    for r0 in range(0, 64, 16):
        for c in range(CPR):
            assert _conflict_free([(dword(r, c ^ kswz(r)), 4) for r in range(r0, r0 + 16)]), (D, r0, c)
    for r0 in range(0, 64, 4):
        for c0 in range(0, CPR, 4):
            acc = [(dword(r, c ^ vswz(r)), 4) for r in range(r0, r0 + 4) for c in range(c0, c0 + 4)]
            assert _conflict_free(acc), (D, r0, c0)
