"""Host model of the balanced split's arithmetic (no GPU).

The decode kernel lays the batch's 16-token tiles end to end per (sequence,
KV head) stream and cuts them into chunks by a guided schedule that depends
only on the tile count T, the grid size nW and a floor (two rounds of the
decode's tile ring, 8 to 20 tiles): nW chunks of C1 = max(1, 4A/5) tiles, nW
of C2 = max(A/7, F), then chunks of C3 = max(A/16, F), with A = T / nW and
F = max(floor, 4).  A cut that falls inside a stream moves to the nearer
end of that stream when it lies within an eighth of the smaller of the two
chunks the cut separates (a quarter for cuts after the first nW chunks).  Inside a chunk a piece of a stream is a segment: a whole
stream writes its output, any other segment is the first (slot 0) or last
(slot 1) of its chunk.  The decode records each stream's first chunk (and
whether its piece there is slot 1) and last chunk, and the reduce reads
them.  These tests replay the same integer formulas (written again here
from that description) and check what the two kernels rely on: chunks tile
[0, T) without gaps or empty chunks, the chunk count stays under the
workspace bound 5 nW + 8, at most two partial segments per chunk, in the
slots the reduce reads, and the pieces of every split stream cover it
exactly once."""
import numpy as np
import pytest


def sched(T, nW, floor):
    A = T // nW
    F = max(floor, 4)
    C1, C2, C3 = max(1, A * 4 // 5), max(F, A // 7), max(F, A // 16)
    e1 = min(nW * C1, T)
    e2 = min(nW * C1 + nW * C2, T)
    if T <= 0:
        chunks = 0
    elif nW * C1 >= T:
        chunks = -(-T // C1)
    elif nW * (C1 + C2) >= T:
        chunks = nW + -(-(T - nW * C1) // C2)
    else:
        chunks = 2 * nW + -(-(T - nW * (C1 + C2)) // C3)
    return dict(T=T, nW=nW, C1=C1, C2=C2, C3=C3, e1=e1, e2=e2, chunks=chunks)


def chunk_begin(q, c):
    nW, C1, C2, C3 = q["nW"], q["C1"], q["C2"], q["C3"]
    if c <= nW:
        b = c * C1
    elif c <= 2 * nW:
        b = nW * C1 + (c - nW) * C2
    else:
        b = nW * (C1 + C2) + (c - 2 * nW) * C3
    return min(b, q["T"])


def chunk_start(q, c, strm):
    """chunk_begin moved to the nearer end of the stream it falls in, when
    that end is within an eighth of the smaller neighbouring chunk (a
    quarter after the first nW chunks)."""
    b = chunk_begin(q, c)
    if c <= 0 or c >= q["chunks"]:
        return b
    d = min(b - chunk_begin(q, c - 1), chunk_begin(q, c + 1) - b) // (8 if c <= q["nW"] else 4)
    for g0, g1 in strm:
        if g0 <= b < g1:
            r = b - g0
            if r <= d:
                return g0
            if g1 - b <= d:
                return g1
            return b
    return b


def chunk_holding(starts, x):
    """The chunk c with starts[c] <= x < starts[c + 1]."""
    return int(np.searchsorted(starts, x, side="right")) - 1


def streams(lens, Hkv):
    out, g = [], 0
    for L in lens:
        n = -(-max(int(L), 0) // 16)
        for h in range(Hkv):
            out.append((g, g + n))
            g += n
    return out, g


FLOORS = [8, 10, 12, 16, 20]
CASES = [([3, 0, 17], 4, 2048, 12), ([1], 4, 2048, 20), ([0, 0, 700], 4, 64, 12),
         ([0, 0, 700], 4, 64, 20), ([5000], 1, 7, 12), ([5000], 1, 7, 20),
         ([16, 32, 48], 2, 5, 8), ([1, 1, 1, 0, 2], 4, 3, 10), ([0, 0, 0], 4, 64, 12)]


def random_case(seed):
    rng = np.random.default_rng(seed)
    S = int(rng.integers(1, 300))
    lens = rng.integers(0, 3000, size=S).tolist()
    return (lens, int(rng.integers(1, 9)), int(rng.integers(1, 2049)),
            FLOORS[int(rng.integers(0, len(FLOORS)))])


@pytest.mark.parametrize("lens,Hkv,nW,floor", CASES + [random_case(s) for s in range(40)])
def test_split_properties(lens, Hkv, nW, floor):
    strm, T = streams(lens, Hkv)
    q = sched(T, nW, floor)
    assert q["C2"] >= max(floor, 4) and q["C3"] >= max(floor, 4)
    assert q["chunks"] <= 5 * nW + 8
    if T == 0:
        assert q["chunks"] == 0
        return
    plain = [chunk_begin(q, c) for c in range(q["chunks"] + 1)]
    starts = [chunk_start(q, c, strm) for c in range(q["chunks"] + 1)]
    assert starts[0] == 0 and starts[-1] == T
    # none empty: each chunk keeps at least half its tiles
    for c in range(q["chunks"]):
        assert 2 * (starts[c + 1] - starts[c]) >= plain[c + 1] - plain[c] > 0
    # a moved cut lands on a stream end
    ends = {g for st in strm for g in st}
    for c in range(q["chunks"] + 1):
        assert starts[c] == plain[c] or starts[c] in ends
    # per chunk: middle segments are whole streams; partial ones are first/last
    slot_of = {}
    for c in range(q["chunks"]):
        b0, b1 = starts[c], starts[c + 1]
        segs = [(i, max(g0, b0), min(g1, b1)) for i, (g0, g1) in enumerate(strm)
                if max(g0, b0) < min(g1, b1)]
        for k, (i, lo, hi) in enumerate(segs):
            if not (lo == strm[i][0] and hi == strm[i][1]):
                assert k == 0 or k == len(segs) - 1
                slot_of[(i, c)] = 0 if k == 0 else 1
    # the reduce's view of every split stream matches the writers' slots
    for i, (g0, g1) in enumerate(strm):
        if g1 == g0:
            continue
        c0, c1 = chunk_holding(starts, g0), chunk_holding(starts, g1 - 1)
        if c0 == c1:
            assert (i, c0) not in slot_of          # finished by the decode
            continue
        for c in range(c0, c1 + 1):
            slot = (1 if starts[c0] < g0 else 0) if c == c0 else 0
            assert slot_of[(i, c)] == slot
        covered = sum(min(g1, starts[c + 1]) - max(g0, starts[c]) for c in range(c0, c1 + 1))
        assert covered == g1 - g0


@pytest.mark.parametrize("floor", [1, 4, 20, 64])
@pytest.mark.parametrize("nW", [1, 2, 3, 7, 64, 512, 2048])
def test_chunk_bound_over_all_sizes(nW, floor):
    """The workspace is sized for 5 nW + 8 chunks: check every T up to a few
    million (the phase sizes change with A = T / nW), for floors from below
    the raised minimum of 4 to the largest the reduce accepts."""
    for T in list(range(1, 40000)) + list(range(40000, 4_000_000, 1009)):
        assert sched(T, nW, floor)["chunks"] <= 5 * nW + 8, T
