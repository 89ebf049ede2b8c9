"""Host-side check of the LDS tile layout rules the kernel uses (CPU only).

K and V tiles are stored as unpadded rows of d 16-bit elements with the 16-byte
chunks of row r XOR-permuted by swz(r). This test restates those rules and checks
that (a) every row's permutation is a bijection, (b) the K fragment reads (lanes
0-15 read 16 consecutive rows at one chunk) hit 16 distinct 16-byte bank slots of a
256-byte bank line, and (c) each half-wave of a transposing V read (ds_read_b64_tr_b16:
4 rows x 64 bytes) hits 32 distinct 8-byte slots. The same properties show up on
the GPU as SQ_LDS_BANK_CONFLICT = 0.
"""
import pytest


def swz(d, r):
    if d == 64:
        return (((r >> 1) & 1) << 2) | ((r >> 2) & 3)
    return ((r & 3) << 2) | ((r >> 2) & 3)


@pytest.mark.parametrize("d", [64, 128])
def test_swizzle_is_a_permutation(d):
    nch = d // 8
    for r in range(64):
        assert sorted(c ^ swz(d, r) for c in range(nch)) == list(range(nch))


@pytest.mark.parametrize("d", [64, 128])
def test_k_row_reads_are_conflict_free(d):
    row_bytes = 2 * d
    for kb in range(2):
        for c in range(d // 8):
            slots = {((kb * 32 + l) * row_bytes + 16 * (c ^ swz(d, kb * 32 + l))) % 256 // 16 for l in range(16)}
            assert len(slots) == 16


@pytest.mark.parametrize("d", [64, 128])
def test_v_transposing_reads_are_conflict_free(d):
    row_bytes = 2 * d
    for tt in range(4):                 # 16-key steps of a 64-key tile
        for sec in range(2):            # first / second read of a fragment
            for hi in range(2):         # half wave
                for db in range(d // 32):
                    slots = set()
                    for lane in range(32 * hi, 32 * hi + 32):
                        r = (tt >> 1) * 32 + 16 * (tt & 1) + 4 * hi + ((lane & 15) >> 2) + 8 * sec
                        ch = 4 * db + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)
                        addr = r * row_bytes + 16 * (ch ^ swz(d, r)) + 8 * (lane & 1)
                        slots.add(addr % 256 // 8)
                    assert len(slots) == 32


@pytest.mark.parametrize("d", [64, 128])
def test_direct_load_lanes_cover_each_tile_once(d):
    """Load i writes LDS bytes [1024 i, 1024 i + 1024); lane l fetches source chunk
    p ^ swz(row) for its destination (row, chunk position p). Over a tile every
    (row, source chunk) must be fetched exactly once."""
    rows_per_load = 1024 // (2 * d)
    for bn in (32, 64):
        seen = set()
        for i in range(bn * d * 2 // 1024):
            for lane in range(64):
                r = rows_per_load * i + (16 * lane) // (2 * d)
                p = ((16 * lane) % (2 * d)) // 16
                seen.add((r, p ^ swz(d, r)))
        assert seen == {(r, c) for r in range(bn) for c in range(d // 8)}
