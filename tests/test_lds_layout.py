"""Host checks of the attention kernel's LDS tile layout (latent tile of 64
keys x r fp16, r = 64, 128, 256).

The index formulas below restate those of csrc/attention.hip: the XOR mask
of a key row, the staging order of the 16-byte global pieces, the score
operand reads (16 bytes), the transposed PV reads (8 bytes) and the staging
writes (two 8-byte halves). Checked: every access stays inside its key row,
the staging covers the tile once, and no two lanes of one LDS cycle hit the
same bank at different addresses under the bank model measured on gfx950
(16-byte reads: four cycles of 16 lanes grouped by lane >> 5 and the parity
of lane bits 2..4, 64 banks; 8-byte reads: 32 consecutive lanes, 64 banks;
8-byte writes: 16 consecutive lanes, 32 banks).
"""
import pytest

BN = 64


def mask(R, key):
    return 2 * (key & 7) if R == 64 else 4 * (key & 7) + 2 * (key & 1)


def chunk_slot(q):
    return 2 * q if q < 4 else 2 * (q - 4) + 1


def parity(x):
    return bin(x).count("1") & 1


GROUPS_B128 = [[l for l in range(64) if (l >> 5) == h and parity((l >> 2) & 7) == p]
               for h in (0, 1) for p in (0, 1)]
GROUPS_R64 = [list(range(0, 32)), list(range(32, 64))]
GROUPS_W64 = [list(range(s, s + 16)) for s in range(0, 64, 16)]


def cycles(byte_addrs, groups, width, nbanks):
    total = 0
    for gr in groups:
        banks = {}
        for lane in gr:
            a = byte_addrs[lane]
            for w in range(width // 4):
                banks.setdefault((a // 4 + w) % nbanks, set()).add(a // 4 + w)
        total += max(len(s) for s in banks.values())
    return total


def staging(R, idx):
    w = idx % (R // 4)
    key = 2 * (idx // (R // 4)) + ((w >> 3) & 1)
    j = (w & 7) + 8 * (w >> 4)
    return key, j


@pytest.mark.parametrize("R,threads", [(64, 256), (128, 256), (256, 512)])
def test_score_reads_in_row_and_conflict_free(R, threads):
    nks = R // 32
    for i in range(4 * nks):
        ks = i // 4
        addrs = []
        for lane in range(64):
            g, l16 = lane >> 4, lane & 15
            col = ((8 * (ks % 4) + 2 * g) ^ mask(R, l16)) * 4 + (ks // 4) * 128
            assert 0 <= col and col + 8 <= R
            addrs.append(2 * ((i % 4) * 16 * R + l16 * R + col))
        assert cycles(addrs, GROUPS_B128, 16, 64) == 4


@pytest.mark.parametrize("R,threads", [(64, 256), (128, 256), (256, 512)])
def test_transposed_reads_in_row_and_conflict_free(R, threads):
    for kk in range(2):
        for add in (0, 16):
            for rb in range(R // 16):
                addrs = []
                for lane in range(64):
                    g, l16 = lane >> 4, lane & 15
                    tk = 4 * g + (l16 >> 2)
                    kt = mask(R, tk)
                    col = (4 * ((l16 & 3) ^ (kt & 3)) + (((rb % 8) * 16) ^ (16 * (kt >> 2)))
                           + (rb // 8) * 128)
                    assert 0 <= col and col + 4 <= R
                    addrs.append(2 * ((kk * 32 + add + tk) * R + col))
                assert cycles(addrs, GROUPS_R64, 8, 64) == 2


@pytest.mark.parametrize("R,threads", [(64, 256), (128, 256), (256, 512)])
def test_staging_covers_tile_and_writes_conflict_free(R, threads):
    pieces = BN * R // 8
    seen = {staging(R, idx) for idx in range(pieces)}
    assert seen == {(k, j) for k in range(BN) for j in range(R // 8)}
    for wave in range(threads // 64):
        for i in range(pieces // threads):
            for half in (0, 1):
                addrs = []
                for lane in range(64):
                    key, j = staging(R, wave * 64 + lane + i * threads)
                    col = ((8 * (j // 4) + chunk_slot(2 * (j % 4) + half)) ^ mask(R, key)) * 4
                    assert 0 <= col and col + 4 <= R
                    addrs.append(2 * (key * R + col))
                assert cycles(addrs, GROUPS_W64, 8, 32) == 4


def test_bank_model_flags_a_conflicting_layout():
    # the previous mask (4 (key & 7) + 2 (key >> 3)) puts keys k and k + 8
    # (one 16-byte read cycle) on the same 16-byte slot pair
    R = 128
    old = lambda key: 4 * (key & 7) + 2 * ((key & 15) >> 3)
    addrs = []
    for lane in range(64):
        g, l16 = lane >> 4, lane & 15
        addrs.append(2 * (l16 * R + ((2 * g) ^ old(l16)) * 4))
    assert cycles(addrs, GROUPS_B128, 16, 64) == 8
