"""CPU models of the skinny kernel's direct-to-LDS stage copies (no GPU).

The dword-copy path of skinny.hip reads rows through raw buffer resources.
The hardware range check on those loads covers the lane's voffset (plus the
instruction offset) against the resource's num_records; the scalar offset is
not part of the check.  These tests restate the kernel's address arithmetic
(DwordCopies and the launcher's split of the block pairs) and check, for every
token count 1..64, several ragged out_dims, every n_pairs % 4 case and every
split the launcher can pick:
  * every copy that passes the range check reads inside the operand buffer;
  * every byte the kernel multiplies (a valid row, a pair below the split's
    end) passes the range check and lands at the LDS byte the operand reads
    expect (stage row r, byte 68 * (pair - stage start) + offset in pair).
"""
import numpy as np
import pytest

PAIR = 68            # bytes of a block pair
STAGE_PAIRS = 4      # pairs per stage
STAGE_ROW = STAGE_PAIRS * PAIR   # 272 bytes per staged row
STAGE_DW = STAGE_ROW // 4        # 68 dwords
PERIOD = 17          # 17 copies of 64 dwords = 16 rows


def launcher_split(n_pairs, split):
    """Pairs per split and split count, as launch_skinny computes them."""
    pps = ((n_pairs + split - 1) // split + STAGE_PAIRS - 1) // STAGE_PAIRS * STAGE_PAIRS
    return pps, (n_pairs + pps - 1) // pps


def wave_groups(mt, wave, o_tile, n_tok, out_dim, row_bytes):
    """(operand, first row in the operand, stage row, valid rows, group rows)
    of one wave, as DwordCopies' constructor sets them; None for an idle wave."""
    if wave < mt:
        first = 32 * wave
        return "x", first, first, max(0, min(32, n_tok - first)), 32
    if wave >= 2:
        o0 = o_tile + 16 * (wave - 2)
        return "w", o0, 32 * mt + 16 * (wave - 2), max(0, min(16, out_dim - o0)), 16
    return None


def check_shape(n_tok, in_dim, out_dim, split):
    mt = 2 if n_tok > 32 else 1
    nb = in_dim // 32
    row_bytes = nb * 34
    n_pairs = in_dim // 64
    pps, n_split = launcher_split(n_pairs, split)
    sizes = {"x": n_tok * row_bytes, "w": out_dim * row_bytes}
    lane = np.arange(64)
    k = np.arange(PERIOD)[:, None]
    f = 64 * k + lane[None, :]                       # flat dword of 16 rows
    r = f // STAGE_DW
    off = r * row_bytes + 4 * (f - r * STAGE_DW)     # the kernel's off[k]
    for by in range(n_split):
        p_begin = by * pps
        p_end = min(p_begin + pps, n_pairs)
        nstages = (p_end - p_begin + STAGE_PAIRS - 1) // STAGE_PAIRS
        for bx in range((out_dim + 31) // 32):
            o_tile = 32 * bx
            for wave in range(4):
                g = wave_groups(mt, wave, o_tile, n_tok, out_dim, row_bytes)
                if g is None:
                    continue
                operand, first_row, stage_row0, valid, grp_rows = g
                base0 = first_row * row_bytes            # gbase, bytes into the operand
                valid_bytes = valid * row_bytes
                for s in range(nstages):
                    sb = (p_begin + s * STAGE_PAIRS) * PAIR
                    for grp in range(grp_rows // 16):
                        start = sb + grp * 16 * row_bytes
                        num_records = max(valid_bytes - start, 0)
                        in_range = off < num_records
                        addr = base0 + start + off       # byte address in the operand
                        assert np.all(addr[in_range] >= 0)
                        assert np.all(addr[in_range] + 4 <= sizes[operand]), (
                            n_tok, in_dim, out_dim, split, by, bx, wave, s, grp)
                        # Bytes the kernel uses: rows below `valid`, pairs below p_end.
                        row_in_wave = 16 * grp + r
                        byte_in_stage = 4 * (f - r * STAGE_DW)
                        pair = p_begin + s * STAGE_PAIRS + byte_in_stage // PAIR
                        used = (row_in_wave < valid) & (pair < p_end)
                        assert np.all(in_range[used]), (n_tok, in_dim, out_dim, split, s, grp)
                        want = ((first_row + row_in_wave) * row_bytes + sb + byte_in_stage)
                        assert np.array_equal(addr[used], want[used])
                        # LDS destination: copy k of group grp writes 256 bytes at
                        # 256 * (k + 17 grp) past the wave's first stage row.
                        lds = (stage_row0 * STAGE_ROW + 256 * (k + PERIOD * grp)
                               + 4 * lane[None, :]) + 0 * f
                        lds_want = (stage_row0 + row_in_wave) * STAGE_ROW + byte_in_stage
                        assert np.array_equal(lds[used], lds_want[used])


@pytest.mark.parametrize("n_pairs", [1, 2, 3, 5, 6, 7, 9, 13, 18])
def test_skinny_dword_copies_stay_in_bounds(n_pairs):
    in_dim = 64 * n_pairs
    for n_tok in range(1, 65):
        for out_dim in (32, 48, 67):
            for split in sorted({1, 2, 3, max(1, n_pairs // 4), 16}):
                check_shape(n_tok, in_dim, out_dim, split)


def test_skinny_dword_copies_model_catches_an_unchecked_offset():
    """The model itself must see the hazard the scalar offset caused: with
    the stage offset outside the checked range (the old addressing), a ragged
    last row group reads past the operand."""
    row_bytes = 3 * 68
    n_tok, out_dim = 17, 32
    lane = np.arange(64)
    f = 64 * np.arange(PERIOD)[:, None] + lane[None, :]
    r = f // STAGE_DW
    off = r * row_bytes + 4 * (f - r * STAGE_DW)
    rows16 = 16 * row_bytes
    valid_bytes = n_tok * row_bytes      # wave 0's 17 valid token rows
    # Old form: num_records = valid_bytes from the wave's base, upper group
    # offset in the unchecked scalar offset.
    in_range = off < valid_bytes
    addr = rows16 + off
    assert np.any(addr[in_range] + 4 > n_tok * row_bytes)
    del out_dim
