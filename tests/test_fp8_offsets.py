"""Host checks of the FP8 forward kernel's K-tile layout arithmetic.

FP8 K tiles hold rows of d bytes in LDS, 16-byte chunk c of row r stored at
chunk c ^ fk(r) with fk(r) = (r / (256 / d)) mod (d / 16).  Checked here for
every lane: the closed form the kernel uses for its DMA pieces, and that one
16-lane pass of the 16-byte score-operand reads touches each of the 64 LDS
banks exactly once.
"""
import pytest

BC = 128          # keys per K tile
NW = 8            # waves per workgroup


def fk(d, r):
    return (r // (256 // d)) & (d // 16 - 1)


@pytest.mark.parametrize("d", [64, 128])
def test_dma_piece_offsets(d):
    pk = d
    lpwk = BC * pk // 1024 // NW

    def goff(n, lane):              # global chunk that LDS slot 1024n + 16 lane holds
        o = 1024 * n + 16 * lane
        r, slot = o // pk, (o % pk) >> 4
        return r * pk + ((slot ^ fk(d, r)) << 4)

    for wq in range(4):
        for lane in range(64):
            kd0 = goff(wq * lpwk, lane)
            for x in range(lpwk):
                for hi in range(2):
                    n = wq * lpwk + x + hi * 4 * lpwk
                    assert goff(n, lane) == (kd0 ^ (x * 0x440)) + hi * 4096 * lpwk


@pytest.mark.parametrize("d", [64, 128])
def test_score_operand_reads_are_conflict_free(d):
    for s in range(d // 32):                        # the lane's chunk index
        for hf in range(2):
            for base in (0, 16):                    # lanes 0-15 / 16-31 of each half
                banks = []
                for l32 in range(base, base + 16):
                    ch = 4 * (s >> 1) + 2 * hf + (s & 1)
                    off = l32 * d + ((ch ^ fk(d, l32)) << 4)
                    banks += [(off // 4 + w) % 64 for w in range(4)]
                assert sorted(banks) == list(range(64))
