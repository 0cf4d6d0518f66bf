"""Host check of the dropout kernels' lane arithmetic: an emulation of the
64 lanes of a wave running the shared mask generator (DropRow / DropCol in
exact_second_order_fa_amd/csrc/fa_kernels.hip) must hand every lane, for every
element it holds, the byte the oracle's element mask uses.

The emulated scheme: for a granule of NS 32 x 32 sub-tiles, lane r of a group
(4 lanes on the row side, 8 on the column side) runs one Philox4x64-10 block,
then a butterfly of lane exchanges (one stage per lane bit: keep the items
whose index matches the lane's bit, swap the rest with the partner, re-slot by
the partner's bit) leaves in slot s what lane s's block holds for this lane.
Accumulator element idx of a lane sits at streamed position
sig(8 (idx / 4) + 4 (lane / 32) + idx % 4) of its sub-tile (fa_tile.h)."""
import numpy as np
import pytest

from oracle.dropout import philox4x64_10

SEED, BH = 12345, 3


def sig(m):
    return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1)


def acc_pos(idx, hh):
    return sig(8 * (idx >> 2) + 4 * hh + (idx & 3))


def block(c0, c1):
    w = philox4x64_10(np.uint64(c0), np.uint64(c1), np.uint64(BH), np.uint64(0), SEED, 0)
    return [int(x) for x in w]


def oracle_byte(i, j):
    """Byte of element (i, j) as the oracle defines it: byte j % 8 of word
    i % 4 of the block for counter (i // 4, j // 8, bh, 0)."""
    return (block(i // 4, j // 8)[i % 4] >> (8 * (j % 8))) & 0xFF


def xor_transpose(A, M):
    """A[lane][slot][k] over 64 lanes; groups are the lanes with equal lane // M."""
    K = len(A[0][0])
    bit = 1
    while bit < M:
        new = [[list(v) for v in lane] for lane in A]
        for l in range(64):
            up = (l & (M - 1)) & bit
            p = l ^ bit
            pup = (p & (M - 1)) & bit
            for s in range(M):
                if s & bit:
                    continue
                for k in range(K):
                    recv = A[p][s][k] if pup else A[p][s | bit][k]
                    new[l][s][k] = recv if up else A[l][s][k]
                    new[l][s | bit][k] = A[l][s | bit][k] if up else recv
        A = new
        bit <<= 1
    return A


def row_side(NS, rowbase, s0):
    A = []
    for l in range(64):
        hh, r, i = l >> 5, l & 3, rowbase + (l & 31)
        sub = r >> 1 if NS == 2 else 0
        w = block(i >> 2, s0 // 8 + 4 * sub + 2 * (r & 1) + hh)
        A.append([[w[q] & 0xFFFFFFFF, w[q] >> 32] for q in range(4)])
    A = xor_transpose(A, 4)
    bad = 0
    for l in range(64):
        hh, i = l >> 5, rowbase + (l & 31)
        for sub in range(NS):
            for idx in range(16):
                b, e = idx >> 2, idx & 3
                d = A[l][(2 * sub if NS == 2 else 0) + (b >> 1)][b & 1]
                bad += ((d >> (8 * e)) & 0xFF) != oracle_byte(i, s0 + 32 * sub + acc_pos(idx, hh))
    return bad


def col_side(NS, colbase, s0):
    A = []
    for l in range(64):
        hh, r, j = l >> 5, l & 7, colbase + (l & 31)
        sub, b = (r >> 2 if NS == 2 else 0), r & 3
        w = block(s0 // 4 + 8 * sub + 4 * (b >> 1) + 2 * hh + (b & 1), j >> 3)
        A.append([[sum(((w[e] >> (8 * q)) & 0xFF) << (8 * e) for e in range(4))] for q in range(8)])
    A = xor_transpose(A, 8)
    bad = 0
    for l in range(64):
        hh, j = l >> 5, colbase + (l & 31)
        for sub in range(NS):
            for idx in range(16):
                d = A[l][(4 * sub if NS == 2 else 0) + (idx >> 2)][0]
                bad += ((d >> (8 * (idx & 3))) & 0xFF) != oracle_byte(s0 + 32 * sub + acc_pos(idx, hh), j)
    return bad


@pytest.mark.parametrize("NS", [1, 2])
@pytest.mark.parametrize("base,s0", [(0, 0), (160, 64), (4096 + 96, 8192)])
def test_lanes_receive_the_oracle_mask(NS, base, s0):
    assert row_side(NS, base, s0) == 0
    assert col_side(NS, base, s0) == 0


@pytest.mark.parametrize("M", [4, 8])
def test_butterfly_hands_each_lane_its_item_from_every_group_member(M):
    """The exchange on tagged items: lane l starts with items (l, q), q < M;
    afterwards slot s of lane l holds item (group base + s, l % M)."""
    A = [[[l * 100 + q] for q in range(M)] for l in range(64)]
    A = xor_transpose(A, M)
    for l in range(64):
        base = l - (l % M)
        assert [A[l][s][0] for s in range(M)] == [(base + s) * 100 + (l % M) for s in range(M)]
