"""Host check of the address identity the attention kernels' LDS reads rely on
(aa_internal.h: SwzTile, tr_operand, tr_lane_offsets / tr_operand_x).

In a swizzled tile row the byte offset of chunk c is that of chunk
(c mod 2^k) XOR 16 (c - c mod 2^k): one per-lane register plus one XOR per
read gives the same address as the per-read swizzled offset.  Checked here
for every lane, every row/feature block the kernels use and both head
dimensions, with the swizzle written out as in the header."""
import pytest


def swz(D, row):
    return (((row & 3) << 2) | ((row >> 2) & 3)) if D == 128 else ((row >> 1) & 7)


def chunk_off(D, row, c):             # element offset, as SwzTile<D>::chunk_off
    return row * D + ((c ^ swz(D, row)) & (D // 8 - 1)) * 8


def off(D, row, f):                   # element offset of (row, feature f), f % 4 == 0
    return chunk_off(D, row, f >> 3) + (f & 7)


def tr_piece_rows(lane):
    g, t = lane >> 4, lane & 15
    return 4 * (g >> 1) + (t >> 2), 16 * (g & 1) + 4 * (t & 3)


@pytest.mark.parametrize("D", [64, 128])
def test_row_reads_by_xor(D):
    # S / dP operands: lane (col, h) reads chunk 2kk + h of row rb + col
    for rb in range(0, 64, 32):
        for lane in range(64):
            h, col = lane >> 5, lane & 31
            base = 2 * chunk_off(D, col, h)
            for kk in range(D // 16):
                want = 2 * chunk_off(D, rb + col, 2 * kk + h)
                got = (base ^ (32 * kk)) + 2 * rb * D
                assert got == want, (D, rb, lane, kk)


@pytest.mark.parametrize("D", [64, 128])
def test_transposing_reads_by_xor(D):
    # tr_operand(tile, r0, f0): two 8-byte pieces at rows row, row + 8
    for lane in range(64):
        row, f = tr_piece_rows(lane)
        o0, o8 = 2 * off(D, row, f), 2 * off(D, row + 8, f)
        for r0 in range(0, 64, 16):
            for f0 in range(0, D, 32):
                want0 = 2 * off(D, r0 + row, f0 + f)
                want8 = 2 * off(D, r0 + row + 8, f0 + f)
                assert (o0 ^ (2 * f0)) + 2 * r0 * D == want0, (D, lane, r0, f0)
                assert (o8 ^ (2 * f0)) + 2 * r0 * D == want8, (D, lane, r0, f0)


@pytest.mark.parametrize("D", [64, 128])
def test_buffer_base_leaves_the_xor_bits_alone(D):
    # a per-step buffer base added before the XOR (dK/dV: cur * 4 * 32 * D
    # bytes) must not reach the bits the XOR flips
    buf = 4 * 32 * D
    for lane in range(64):
        h, col = lane >> 5, lane & 31
        o = 2 * chunk_off(D, col, h)
        for cur in (0, 1):
            for kk in range(D // 16):
                assert ((cur * buf + o) ^ (32 * kk)) == cur * buf + (o ^ (32 * kk))
