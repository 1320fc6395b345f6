"""CPU checks of the work split's arithmetic, restated from the decode kernel's
work walk and the merge kernel's segment lookup (both device code).

For many shapes (fixed and packed query lengths), grids, segment-start costs
and both split modes (unit by unit, and groups of U workgroups sharing each
request's cost range, chosen when every request holds the same U = 2, 4 or 8
units), the restated walk must
  * hand every (request, unit, tile) to exactly one segment,
  * give every segment a distinct workspace slot below grid + max units (the
    workspace the library sizes), and
  * agree with the merge's arithmetic: the slots the merge derives for a unit
    are its segments, in tile order, covering its tiles once.
"""

import numpy as np
import pytest

TILE, PAIRS = 32, 128


def cdiv(a, b):
    return (a + b - 1) // b


def walk(seq_lens, q_lens, H, G, S0, GU):
    """Segments {slot: (request, unit, t0, t1)} of the decode kernel's walk."""
    B = len(seq_lens)
    T = [cdiv(int(L), TILE) for L in seq_lens]
    U = [cdiv(int(q) * H, PAIRS) for q in q_lens]
    Uc = [min(u, 1) if GU > 1 else u for u in U]  # cost units per request
    tile_off = np.concatenate([[0], np.cumsum([uc * t for uc, t in zip(Uc, T)])]).astype(int)
    unit_off = np.concatenate([[0], np.cumsum(Uc)]).astype(int)
    TC = int(tile_off[B] + unit_off[B] * S0)
    C = max(1, cdiv(TC, G // GU))
    segs = {}
    for i in range(G):
        gw = ((i & 7) * (G >> 3) + (i >> 3)) if G % 8 == 0 else i
        g, q = gw // GU, gw % GU
        x, end = g * C, min(TC, g * C + C)
        b = rel = 0
        if x < end:
            b = int(np.searchsorted(tile_off + unit_off * S0, x, side="right")) - 1
            b = min(b, B - 1)
            rel = x - int(tile_off[b] + unit_off[b] * S0)
        u_base = int(unit_off[b])
        while x < end:
            Tb, span = T[b], S0 + T[b]
            if Tb == 0 or Uc[b] == 0:
                x += Uc[b] * S0 - rel
                rel, b, u_base = 0, b + 1, u_base + Uc[b]
                continue
            pb, r = divmod(rel, span)
            if r < S0:
                x, rel, r = x + S0 - r, rel + S0 - r, S0
                if x >= end:
                    break
            t0 = r - S0
            t1 = min(Tb, t0 + (end - x))
            slot = (g + u_base + pb) * GU + q
            assert slot not in segs, ("slot used twice", slot)
            segs[slot] = (b, q if GU > 1 else pb, t0, t1)
            x, rel = x + t1 - t0, rel + t1 - t0
            if rel >= Uc[b] * span:
                rel, b, u_base = 0, b + 1, u_base + Uc[b]
    return segs, T, U, tile_off, unit_off, C


def merge_slots(b, pb, T, tile_off, unit_off, C, S0, GU):
    """Slots the merge kernel reads for unit pb of request b, in order."""
    pbc = 0 if GU > 1 else pb
    q = pb - pbc
    u = int(unit_off[b]) + pbc
    U0 = int(tile_off[b]) + pbc * T[b] + (u + 1) * S0
    g0, g1 = U0 // C, (U0 + T[b] - 1) // C
    nseg = g1 - g0 + 1 if T[b] > 0 else 0
    return [(g0 + s + u) * GU + q for s in range(nseg)]


def check(seq_lens, q_lens, H, G, S0, GU):
    segs, T, U, tile_off, unit_off, C = walk(seq_lens, q_lens, H, G, S0, GU)
    seen = set()
    for b, pb, t0, t1 in segs.values():
        for t in range(t0, t1):
            assert (b, pb, t) not in seen
            seen.add((b, pb, t))
    assert seen == {(b, pb, t) for b in range(len(T)) for pb in range(U[b]) for t in range(T[b])}
    # the library's workspace slots: grid + batch x units of the longest query
    assert not segs or max(segs) < G + len(seq_lens) * cdiv(max(q_lens) * H, PAIRS)
    for b in range(len(T)):
        for pb in range(U[b]):
            got = [segs[s] for s in merge_slots(b, pb, T, tile_off, unit_off, C, S0, GU)]
            assert all(x[0] == b and x[1] == pb for x in got)
            assert [x[2] for x in got] == sorted(x[2] for x in got)
            assert sum(x[3] - x[2] for x in got) == T[b]


def group_size(q_lens, H, G):
    units = {cdiv(int(q) * H, PAIRS) for q in q_lens}
    U = units.pop() if len(units) == 1 else 0
    return U if U in (2, 4, 8) and G % (8 * U) == 0 else 1


@pytest.mark.parametrize("seed", range(6))
def test_walk_and_merge_agree(seed):
    rng = np.random.default_rng(seed)
    for _ in range(25):
        B = int(rng.integers(1, 24))
        H = int(rng.choice([16, 48, 64, 128]))
        q_lens = [int(rng.integers(1, 9))] * B
        if rng.random() < 0.4:  # packed: per-request lengths, sometimes with equal unit counts
            q_lens = list(rng.integers(1, int(rng.choice([2, 9, 17])), B))
        L = rng.integers(0, 2500, B)
        L[rng.random(B) < 0.1] = 0  # empty requests (outside the contract) still advance the walk
        for G in (8, 16, 48, 64, 256, 1000):
            for S0 in (0, 1, 8, 40):
                GU = group_size(q_lens, H, G)
                check(list(L), q_lens, H, G, S0, GU)
                if GU > 1:
                    check(list(L), q_lens, H, G, S0, 1)


@pytest.mark.parametrize("shape", [(32, 4, 128, (2048, 6144)), (8, 2, 128, (65536, 131072)),
                                   (64, 1, 128, (1024, 8192))])
def test_configured_shapes_at_one_workgroup_per_cu(shape):
    B, q_len, H, (lo, hi) = shape
    L = list(np.random.default_rng(B).integers(lo, hi + 1, B))
    for GU in {group_size([q_len] * B, H, 256), 1}:
        check(L, [q_len] * B, H, 256, 8, GU)
