"""Host checks of the LDS chunk swizzles of the 16x16x32 kernels.

Each kernel stages row-major tiles (rows of D 16-bit values, 16-byte chunks)
into LDS with an XOR swizzle of the chunk index by a function of the row, and
reads them back either row-wise (ds_read_b128: 16 lanes, one chunk each, per
LDS pass) or transposed (ds_read_b64_tr_b16: 32 lanes, 8 bytes each, per
pass). The swizzles are restated here from the kernels' comments, and each
read pattern the kernels issue is checked to touch every one of the 64 banks
(4 bytes each) at most once per pass, i.e. to be free of bank conflicts. The
backward swizzles must also ignore row bit 2, which the kernels' constant
offsets (second row block, second transpose read) rely on.
"""

from __future__ import annotations

import pytest


def banks_b128(addrs):
    """Bank groups (16 bytes) of one pass of 16-byte reads."""
    return [(a // 16) % 16 for a in addrs]


def banks_b64(addrs):
    """Banks of one pass of 8-byte reads (two banks each)."""
    out = []
    for a in addrs:
        b = (a // 4) % 64
        out += [b, b + 1]
    return out


# forward, D = 128 (fa_fwd_mfma16.hip): K tile read row-wise, V tile transposed
def k16_swz(key):
    return (key & 3) | (((key >> 3) & 3) << 2)


def v16_swz(key):
    return 2 * ((key & 3) | (((key >> 3) & 1) << 2))


def test_forward_k_rows_conflict_free():
    D = 128
    for kb in range(4):
        for kc in range(4):
            for g in range(4):
                addrs = []
                for n in range(16):
                    key = 32 * (kb >> 1) + 4 * (kb & 1) + 8 * (n >> 2) + (n & 3)
                    addrs.append(key * D * 2 + ((4 * kc + g) ^ k16_swz(key)) * 16)
                assert len(set(banks_b128(addrs))) == 16, (kb, kc, g)


def test_forward_v_transpose_conflict_free():
    D = 128
    for c in range(2):
        for db in range(8):
            for rd in range(2):
                for half in range(2):
                    addrs = []
                    for lane in range(32 * half, 32 * half + 32):
                        n, g = lane & 15, lane >> 4
                        key = 32 * c + 8 * g + 4 * rd + (n >> 2)
                        col = 16 * db + 4 * (n & 3)
                        addrs.append(key * D * 2 + (((col >> 3) ^ v16_swz(key)) * 8 + (col & 7)) * 2)
                    assert len(set(banks_b64(addrs))) == 64, (c, db, rd, half)


# backward (fa_bwd.hip): Q, dO, K, V tiles read both ways; the dK/dV kernel's V block row-wise
def tile_swz(D, row):
    if D == 128:
        return ((row & 3) << 1) | (((row >> 3) & 1) << 3) | ((row >> 4) & 1)
    return (((row >> 1) & 1) << 1) | (((row >> 3) & 1) << 2) | ((row >> 4) & 1)


def vblk_swz(D, row):
    return row & 15 if D == 128 else (row >> 1) & 7


@pytest.mark.parametrize("D", [64, 128])
def test_backward_tile_rows_conflict_free(D):
    for b in range(2):
        for kc in range(D // 32):
            for g in range(4):
                addrs = []
                for n in range(16):
                    row = 8 * (n >> 2) + 4 * b + (n & 3)
                    addrs.append(row * D * 2 + ((4 * kc + g) ^ tile_swz(D, row)) * 16)
                assert len(set(banks_b128(addrs))) == 16, (D, b, kc, g)


@pytest.mark.parametrize("D", [64, 128])
def test_backward_tile_transpose_conflict_free(D):
    for db in range(D // 16):
        for rd in range(2):
            for half in range(2):
                addrs = []
                for lane in range(32 * half, 32 * half + 32):
                    n, g = lane & 15, lane >> 4
                    q = 8 * g + 4 * rd + (n >> 2)
                    col = 16 * db + 4 * (n & 3)
                    addrs.append(q * D * 2 + (((col >> 3) ^ tile_swz(D, q)) * 8 + (col & 7)) * 2)
                assert len(set(banks_b64(addrs))) == 64, (D, db, rd, half)


@pytest.mark.parametrize("D", [64, 128])
def test_backward_v_block_rows_conflict_free(D):
    for base in range(0, 128, 16):
        for kc in range(D // 32):
            for g in range(4):
                addrs = [(base + n) * D * 2 + ((4 * kc + g) ^ vblk_swz(D, base + n)) * 16 for n in range(16)]
                assert len(set(banks_b128(addrs))) == 16, (D, base, kc, g)


@pytest.mark.parametrize("D", [64, 128])
def test_backward_swizzle_ignores_row_bit_2(D):
    assert all(tile_swz(D, r) == tile_swz(D, r ^ 4) for r in range(32))


@pytest.mark.parametrize("D", [64, 128])
def test_swizzles_permute_the_chunks_of_a_row(D):
    """Staging and reading use the same map, so it must be a bijection per row."""
    cpr = D // 8
    for row in range(128):
        assert sorted(c ^ tile_swz(D, row) for c in range(cpr)) == list(range(cpr))
        assert sorted(c ^ vblk_swz(D, row) for c in range(cpr)) == list(range(cpr))
