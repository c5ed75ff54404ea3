"""Host check of the backward kernels' LDS offset identities.

The backward kernels keep two per-lane base offsets and derive every other
LDS offset by XOR with a constant.  This restates the swizzled row layout
(16-byte chunk c of row r stored at chunk c ^ fk(r), fk(r) = r for d = 128
and r >> 1 for d = 64, modulo the chunks per row) and checks, for every lane,
that the XOR forms equal the offsets computed directly from that layout.
"""
import pytest


def fk(d, r):
    cpr = d // 8
    return (r if cpr == 16 else r >> 1) & (cpr - 1)


@pytest.mark.parametrize("d", [64, 128])
def test_row_and_transposing_offsets(d):
    p = 2 * d
    thi = 0x880 if d == 128 else 0x440
    for lane in range(64):
        l32, hf = lane & 31, lane >> 5
        row0 = l32 * p + ((hf ^ fk(d, l32)) << 4)
        for s in range(d // 16):
            assert row0 ^ (s << 5) == l32 * p + (((2 * s + hf) ^ fk(d, l32)) << 4)
        g, e, q = lane >> 4, (lane >> 2) & 3, lane & 3
        r = 4 * (g >> 1) + e
        tr0 = r * p + (((2 * (g & 1) + (q >> 1)) ^ fk(d, r)) << 4) + 8 * (q & 1)
        for dt in range(d // 32):
            c = 4 * dt + 2 * (g & 1) + (q >> 1)
            assert tr0 ^ (dt << 6) == r * p + ((c ^ fk(d, r)) << 4) + 8 * (q & 1)
            assert tr0 ^ (dt << 6) ^ thi == (r + 8) * p + ((c ^ fk(d, r + 8)) << 4) + 8 * (q & 1)


@pytest.mark.parametrize("d", [64, 128])
def test_dma_piece_offsets(d):
    p = 2 * d
    ppw = 64 * p // 1024 // 4

    def goff(n, lane):
        o = 1024 * n + 16 * lane
        r, slot = o // p, (o % p) >> 4
        return r * p + ((slot ^ fk(d, r)) << 4)

    for wave in range(4):
        for lane in range(64):
            g0 = goff(wave * ppw, lane)
            for x in range(ppw):
                assert goff(wave * ppw + x, lane) == g0 ^ (x * 0x440)
