"""CPU models of the skinny kernel's direct-to-LDS stage copies (no GPU).

The dword-copy path of skinny.hip reads rows through raw buffer resources.
The hardware range check on those loads covers the lane's voffset (plus the
instruction offset) against the resource's num_records; the scalar offset is
not part of the check.  These tests restate the kernel's address arithmetic
(DwordCopies and ChunkCopies, and the launcher's split of the block pairs)
and check, for every token count 1..64 (and, for token tiles in workgroups
of their own, counts up to 256), several ragged out_dims, every n_pairs % 4
case and every split the launcher can pick:
  * every copy that passes the range check reads inside the operand buffer;
  * every byte the kernel multiplies (a valid row, a pair below the split's
    end) passes the range check and lands at the LDS byte the operand reads
    expect (staged row, byte of the 144-byte row);
  * every step of every split is taken by exactly one wave per token tile.
"""
import numpy as np
import pytest

PAIR = 68            # bytes of a block pair
STEP_PAIRS = 2       # pairs of a row per step
SLICE = STEP_PAIRS * PAIR        # 136 bytes of a row per step
PITCH = 144          # LDS bytes per staged row: nine 16-byte slots
PITCH_DW = PITCH // 4            # 36 dwords
SLOTS = PITCH // 16  # 9
PERIOD = 9           # 9 dword copies of 64 = 16 staged rows
WAVES = 8
STEP_ROWS = 64       # a wave's step: 32 token rows, then 32 weight rows


def slot_byte(j):
    """Byte of the slice that 16-byte slot j holds: 0..127, then 120..135."""
    return 16 * j if j < SLOTS - 1 else SLICE - 16


def lds_dword_byte(d):
    """Byte of the slice that staged dword d (0..35) of a row holds."""
    return np.where(d < 32, 4 * d, SLICE - 16 + 4 * (d - 32))


def launcher_split(n_pairs, split):
    """Pairs per split and split count, as launch_skinny computes them."""
    pps = ((n_pairs + split - 1) // split + STEP_PAIRS - 1) // STEP_PAIRS * STEP_PAIRS
    return pps, (n_pairs + pps - 1) // pps


def wave_steps(mt, wave, p_begin, p_end):
    """Token tile of the wave and the first pair of each of its steps."""
    kq_count = WAVES // mt
    m, kq = divmod(wave, kq_count)
    nsteps = (p_end - p_begin + STEP_PAIRS - 1) // STEP_PAIRS
    return m, [p_begin + STEP_PAIRS * j for j in range(kq, nsteps, kq_count)]


def dword_groups(m, o_tile, n_tok, out_dim):
    """(operand, first row in the operand, valid rows) of the wave's four
    16-row groups, as DwordCopies' constructor sets them."""
    out = []
    for g in range(STEP_ROWS // 16):
        if g < 2:
            first = 32 * m + 16 * g
            out.append(("x", first, max(0, min(16, n_tok - first))))
        else:
            o0 = o_tile + 16 * (g - 2)
            out.append(("w", o0, max(0, min(16, out_dim - o0))))
    return out


def check_shape(n_tok, in_dim, out_dim, split, mt=None):
    if mt is None:
        mt = 2 if n_tok > 32 else 1
    nb = in_dim // 32
    row_bytes = nb * 34
    n_pairs = in_dim // 64
    pps, n_split = launcher_split(n_pairs, split)
    sizes = {"x": n_tok * row_bytes, "w": out_dim * row_bytes}
    lane = np.arange(64)
    k = np.arange(PERIOD)[:, None]
    f = 64 * k + lane[None, :]                       # staged dword of 16 rows
    r = f // PITCH_DW
    byte_in_slice = lds_dword_byte(f - r * PITCH_DW)
    off = r * row_bytes + byte_in_slice              # the kernel's off[k]
    pairs_seen = 0
    for by in range(n_split):
        p_begin = by * pps
        p_end = min(p_begin + pps, n_pairs)
        for bx in range((out_dim + 31) // 32):
            o_tile = 32 * bx
            covered = {}
            for wave in range(WAVES):
                m, firsts = wave_steps(mt, wave, p_begin, p_end)
                for pair0 in firsts:
                    covered[(m, pair0)] = covered.get((m, pair0), 0) + 1
                    start = pair0 * PAIR
                    for g, (operand, first_row, valid) in enumerate(
                            dword_groups(m, o_tile, n_tok, out_dim)):
                        base0 = first_row * row_bytes        # group base, bytes into the operand
                        num_records = max(valid * row_bytes - start, 0)
                        in_range = off < num_records
                        addr = base0 + start + off           # byte address in the operand
                        assert np.all(addr[in_range] >= 0)
                        assert np.all(addr[in_range] + 4 <= sizes[operand]), (
                            n_tok, in_dim, out_dim, split, by, bx, wave, pair0, g)
                        # Bytes the kernel uses: rows below `valid`, pairs below p_end.
                        pair = pair0 + byte_in_slice // PAIR
                        used = (r < valid) & (pair < p_end)
                        assert np.all(in_range[used]), (n_tok, in_dim, out_dim, split, pair0, wave)
                        want = (first_row + r) * row_bytes + start + byte_in_slice
                        assert np.array_equal(addr[used], want[used])
                        # LDS: copy k writes 256 bytes at 16 g * 144 + 256 k of the step.
                        lds = 16 * g * PITCH + 256 * k + 4 * lane[None, :] + 0 * f
                        assert np.array_equal(lds, (16 * g + r) * PITCH + 4 * (f - r * PITCH_DW))
            # Every step of the split is taken once for every token tile.
            want = {(m, p_begin + STEP_PAIRS * j): 1 for m in range(mt)
                    for j in range((p_end - p_begin + STEP_PAIRS - 1) // STEP_PAIRS)}
            assert covered == want, (n_tok, in_dim, out_dim, split, by)
            pairs_seen += p_end - p_begin
    assert pairs_seen == n_pairs * ((out_dim + 31) // 32)


def check_chunk_copies(mt, n_tok, out_dim, n_pairs, o_tile, pair0):
    """ChunkCopies: every 16-byte slot of a wave's step is written, each
    source in bounds and 8-byte aligned; the multiplied slots (valid rows)
    hold the right bytes of the right row."""
    row_bytes = n_pairs * 2 * 34
    sizes = {"x": n_tok * row_bytes, "w": out_dim * row_bytes}
    for m in range(mt):
        written = {}
        for kk in range(STEP_ROWS * SLOTS // 64):
            for l in range(64):
                c = 64 * kk + l
                row, slot = divmod(c, SLOTS)
                if row < 32:
                    operand, g = "x", min(32 * m + row, n_tok - 1)
                else:
                    operand, g = "w", min(o_tile + row - 32, out_dim - 1)
                src = g * row_bytes + slot_byte(slot) + pair0 * PAIR
                assert 0 <= src and src + 16 <= sizes[operand]
                assert src % 8 == 0, "16-byte copies read 8-byte-aligned bytes"
                dst = 1024 * kk + 16 * l
                assert dst not in written
                written[dst] = (operand, src)
                assert divmod(dst, PITCH) == (row, 16 * slot)
                valid = 32 * m + row < n_tok if row < 32 else o_tile + row - 32 < out_dim
                if valid:
                    op_row = 32 * m + row if row < 32 else o_tile + row - 32
                    assert src == op_row * row_bytes + pair0 * PAIR + slot_byte(slot)
        assert sorted(written) == [16 * c for c in range(STEP_ROWS * SLOTS)]


@pytest.mark.parametrize("mt", [1, 2])
def test_skinny_chunk_copies_cover_the_step(mt):
    for n_tok in ((1, 17, 32) if mt == 1 else (33, 50, 64)):
        for out_dim in (32, 67, 2048):
            for n_pairs in (4, 8, 12, 64):
                for pair0 in range(0, n_pairs, STEP_PAIRS):
                    for o_tile in sorted({0, 32 * ((out_dim - 1) // 32)}):
                        check_chunk_copies(mt, n_tok, out_dim, n_pairs, o_tile, pair0)


@pytest.mark.parametrize("n_pairs", [1, 2, 3, 5, 6, 7, 9, 13, 18])
def test_skinny_dword_copies_stay_in_bounds(n_pairs):
    in_dim = 64 * n_pairs
    for n_tok in range(1, 65):
        for out_dim in (32, 48, 67):
            for split in sorted({1, 2, 3, max(1, n_pairs // 4), 16}):
                check_shape(n_tok, in_dim, out_dim, split)


def test_skinny_token_tiles_in_separate_workgroups_stay_in_bounds():
    """From 33 tokens the launcher may give every 32-token tile workgroups of
    its own (grid z; always above 64 tokens, up to 256, then with one or two
    token tiles per workgroup): the workgroup at z reads the x rows from
    32 mt z on, n_tok - 32 mt z of them (possibly fewer than its mt tiles
    hold).  Its copies are those of an mt-tile call on that slice."""
    for n_pairs in (1, 3, 5, 13, 64):
        for n_tok in (33, 40, 63, 64, 65, 100, 128, 200, 255, 256):
            for out_dim in (32, 67):
                for mt in (1, 2):   # token tiles per workgroup
                    for z in range((n_tok + 32 * mt - 1) // (32 * mt)):
                        rest = n_tok - 32 * mt * z
                        if n_pairs <= 13:
                            check_shape(rest, 64 * n_pairs, out_dim, 1, mt=mt)
                        if n_pairs % 4 == 0:
                            for pair0 in (0, n_pairs - STEP_PAIRS):
                                check_chunk_copies(mt, rest, out_dim, n_pairs, 0, pair0)


def test_skinny_dword_copies_model_catches_an_unchecked_offset():
    """The model itself must see the hazard the scalar offset caused: with
    the stage offset outside the checked range (the old addressing), a ragged
    last row group reads past the operand."""
    row_bytes = 3 * 68
    n_tok = 17
    lane = np.arange(64)
    f = 64 * np.arange(PERIOD)[:, None] + lane[None, :]
    r = f // PITCH_DW
    off = r * row_bytes + lds_dword_byte(f - r * PITCH_DW)
    rows16 = 16 * row_bytes
    valid_bytes = n_tok * row_bytes      # all 17 valid token rows from row 0
    # Old form: num_records = valid_bytes from the first row, the upper
    # group's offset in the unchecked scalar offset.
    in_range = off < valid_bytes
    addr = rows16 + off
    assert np.any(addr[in_range] + 4 > n_tok * row_bytes)
