"""Host check of the backward kernels' LDS offset identities.

The backward kernels keep two per-lane base offsets and derive every other
LDS offset by XOR with a constant.  This restates the swizzled row layout
(16-byte chunk c of row r stored at chunk c ^ fb(r), fb(r) = 4 (r mod 4) +
(r / 4 mod 4) for d = 128 and 4 (r / 2 mod 2) + (r / 4 mod 4) for d = 64)
and checks, for every lane, that the XOR forms equal the offsets computed
directly from that layout, and that both read patterns are free of LDS bank
conflicts (64 banks of 4 bytes; 16 lanes per ds_read_b128 pass, 32 per
ds_read_b64_tr_b16 pass).
"""
import pytest


def fk(d, r):
    if d == 128:
        return 4 * (r & 3) + ((r >> 2) & 3)
    return 4 * ((r >> 1) & 1) + ((r >> 2) & 3)


def _max_way(addrs, nbytes, per_pass):
    worst = 0
    for p0 in range(0, len(addrs), per_pass):
        banks = {}
        for a in addrs[p0:p0 + per_pass]:
            for w in range(nbytes // 4):
                banks.setdefault((a // 4 + w) % 64, set()).add(a // 4 + w)
        worst = max(worst, max(len(v) for v in banks.values()))
    return worst


@pytest.mark.parametrize("d", [64, 128])
def test_row_and_transposing_offsets(d):
    p = 2 * d
    thi = 0x820 if d == 128 else 0x420
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
                assert goff(wave * ppw + x, lane) == g0 ^ (x * (0x410 if d == 128 else 0x420))


@pytest.mark.parametrize("d", [64, 128])
def test_reads_are_bank_conflict_free(d):
    p = 2 * d
    for s in range(d // 16):
        addrs = [(l & 31) * p + (((2 * s + (l >> 5)) ^ fk(d, l & 31)) << 4) for l in range(64)]
        assert _max_way(addrs, 16, 16) == 1
    for dt in range(d // 32):
        for hi in (0, 8):
            addrs = []
            for lane in range(64):
                g, e, q = lane >> 4, (lane >> 2) & 3, lane & 3
                r = 4 * (g >> 1) + e + hi
                c = 4 * dt + 2 * (g & 1) + (q >> 1)
                addrs.append(r * p + ((c ^ fk(d, r)) << 4) + 8 * (q & 1))
            assert _max_way(addrs, 8, 32) == 1
