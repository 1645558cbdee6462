"""Host-side check of the two-launch prefill's dispatch order (attn_kernel, chunked mode): the
chunk launch's per-pair item positions r = 0 .. S*Q + n_own0 - 1 map onto every (super-chunk j,
query tile) past item and every own-key item of query tiles [0, n_own0) exactly once, with every
index in range, and each super-chunk's fetchers come before the rest of its items; the finish
launch's positions r = 0 .. Q - 1 map onto every query tile once. The mapping below is the
kernel's, restated (a reader compares the two side by side)."""
import itertools

import pytest


def chunk_item(r, Q, S, F, Qa, ins):
    """('own', qt) or ('past', j, qt) for position r of the chunk launch."""
    F = min(F, Q)
    if F <= r < F + Qa:
        return ("own", Qa - 1 - (r - F))
    if r < F:
        j, idx = 0, r
    else:
        ins = min(ins, Q - F)
        o0 = r - F - Qa
        j = min(o0 // Q, S - 1)
        o = o0 - j * Q
        fj = F if j + 1 < S else 0
        if o < ins:
            idx = F + o
        elif o < ins + fj:
            idx = o - ins
            j += 1
        else:
            idx = F + o - fj
    return ("past", j, Q - 1 - idx)


def finish_item(r, Q, Qa):
    return ("own+merge", Q - 1 - r) if r < Q - Qa else ("merge", Q - 1 - r)


@pytest.mark.parametrize("Q,S,F,Qa,ins", [
    (128, 8, 8, 72, 40),      # the 8B-shaped prefill
    (2, 2, 8, 0, 0),          # fewer query tiles than fetchers
    (3, 5, 1, 3, 0),          # every own-key item in the chunk launch
    (5, 2, 0, 1, 99),         # no fetchers, insertion point past the end
    (17, 3, 4, 5, 13),        # insertion point at the end of the block
    (64, 11, 8, 20, 18),
])
def test_chunk_launch_covers_every_item_once(Q, S, F, Qa, ins):
    seen = [chunk_item(r, Q, S, F, Qa, ins) for r in range(S * Q + Qa)]
    want = [("past", j, qt) for j in range(S) for qt in range(Q)] + [("own", qt) for qt in range(Qa)]
    assert sorted(seen) == sorted(want)
    # a super-chunk's fetchers (its first min(F, Q) query tiles, highest first) come before its
    # other items, and chunk j+1's fetchers before the last of chunk j's items wherever some of
    # those come after the insertion point
    Fq = min(F, Q)
    for j in range(S):
        pos = [r for r, it in enumerate(seen) if it[0] == "past" and it[1] == j]
        fetch = [r for r in pos if seen[r][2] >= Q - Fq]
        rest = [r for r in pos if seen[r][2] < Q - Fq]
        if fetch and rest:
            assert max(fetch) < min(rest)
        if j + 1 < S and Fq and ins < Q - Fq:   # some of chunk j's items follow the insertion point
            nxt = [r for r, it in enumerate(seen) if it[0] == "past" and it[1] == j + 1 and it[2] >= Q - Fq]
            assert max(nxt) < max(pos)


def test_chunk_launch_exhaustive_small():
    for Q, S, F, Qa, ins in itertools.product(range(1, 6), range(2, 5), range(0, 4), range(0, 6), range(0, 7)):
        if Qa > Q:
            continue
        seen = [chunk_item(r, Q, S, F, Qa, ins) for r in range(S * Q + Qa)]
        want = [("past", j, qt) for j in range(S) for qt in range(Q)] + [("own", qt) for qt in range(Qa)]
        assert sorted(seen) == sorted(want), (Q, S, F, Qa, ins)


def test_finish_launch_covers_every_query_tile_once():
    for Q in range(1, 40):
        for Qa in range(0, Q + 1):
            seen = [finish_item(r, Q, Qa) for r in range(Q)]
            assert sorted(qt for _, qt in seen) == list(range(Q))
            assert all(kind == "merge" for kind, qt in seen if qt < Qa)
            assert all(kind == "own+merge" for kind, qt in seen if qt >= Qa)
