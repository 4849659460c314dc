"""Pins for the reference planner: its items are checked against brute-force
enumeration of the valid set, and the deal against the zigzag rule.

Source: GDPA page ("Generalized Dot-Product Attention (GDPA): kernel optimisation
for real recommendation-system training loads"), "Section details", jagged-input
paragraph and zigzag tile-scheduling diagram.
"""
import itertools

import numpy as np
import pytest

from oracle import plan_ref as PR
from oracle.gdpa_ref import valid_mask

CASES = [
    ([5, 0, 70, 1, 33, 200], [64, 3, 0, 2, 129, 31], 0),
    ([70, 1, 33, 200, 0], [70, 1, 33, 200, 0], 9),
    ([300, 129, 64, 2], [300, 129, 64, 2], 128),
    ([32] * 6, [1, 1000, 31, 32, 33, 0], 0),
]


def _tiles_with_valid_pair(kind, lq, lk, H, window, t_stat, t_strm):
    """Brute force: every (b, h, t, s) whose tile pair holds a valid (i, j)."""
    out = set()
    for b in range(len(lq)):
        m = valid_mask(np.arange(lq[b]), np.arange(lk[b]), lq[b], lk[b], window)
        if kind == "dkdv":
            m = m.T
        for i, j in zip(*np.nonzero(m)):
            for h in range(H):
                out.add((b, h, i // t_stat, j // t_strm))
    return out


@pytest.mark.parametrize("lq,lk,window", CASES)
@pytest.mark.parametrize("kind", PR.LISTS)
@pytest.mark.parametrize("tiles", [(32, 32), (64, 32), (32, 64), (128, 64)])
def test_items_are_exactly_the_tiles_with_valid_pairs(lq, lk, window, kind, tiles):
    H = 2
    t_stat, t_strm = tiles
    items = PR.enumerate_items(kind, lq, lk, H, window, t_stat, t_strm)
    got = set()
    owned = set()
    for cost, b, h, t, s0, s1 in items:
        assert (b, h, t) not in owned          # each output tile has one owner
        owned.add((b, h, t))
        for s in range(s0, s1 + 1):
            got.add((b, h, t, s))
    assert got == _tiles_with_valid_pair(kind, lq, lk, H, window, t_stat, t_strm)
    # every stationary row of every (b, h) is owned, including rows with no partner
    ls = lk if kind == "dkdv" else lq
    want_owned = {(b, h, t) for b in range(len(ls)) for h in range(H)
                  for t in range(-(-ls[b] // t_stat))}
    assert owned == want_owned


@pytest.mark.parametrize("P", [1, 3, 8, 256])
def test_zigzag_deal(P):
    items = [(c, i, 0, 0, 0, 0) for i, c in enumerate([5, 9, 9, 1, 7, 3, 3, 8, 2, 2, 6] * 7)]
    bin_ptr, flat, cost = PR.deal(items, P)
    order = sorted(items, key=lambda it: (-it[0], it[1], it[2], it[3]))
    assert sorted(flat) == sorted(items)
    for r, it in enumerate(order):
        rnd, pos = divmod(r, P)
        p = pos if rnd % 2 == 0 else P - 1 - pos
        assert it in flat[bin_ptr[p]:bin_ptr[p + 1]]
    counts = np.diff(bin_ptr)
    assert counts.max() - counts.min() <= 1
    assert sum(cost) == sum(it[0] for it in items)


def test_zigzag_beats_round_robin_on_skewed_costs():
    items = [(c, i, 0, 0, 0, 0) for i, c in enumerate(range(1000, 0, -1))]
    _, _, zz = PR.deal(items, 16, zigzag=True)
    _, _, rr = PR.deal(items, 16, zigzag=False)
    assert PR.imbalance(zz) < PR.imbalance(rr)


def test_auto_layout_rules():
    # d = 128: two-wave forward teams from a mean query length of 48, one block per wave
    assert PR.auto_layout([32] * 8, [1000] * 8, 0, 128) == {"fwd": (1, 1), "dq": (1, 1), "dkdv": (1, 1)}
    assert PR.auto_layout([300] * 8, [32] * 8, 0, 128) == {"fwd": (2, 1), "dq": (1, 1), "dkdv": (1, 1)}
    assert PR.auto_layout([47, 49, 0], [5] * 3, 0, 128)["fwd"] == (2, 1)
    assert PR.auto_layout([47, 48, 0], [5] * 3, 0, 128)["fwd"] == (1, 1)
    # d <= 64: one-wave teams, two forward blocks from a mean query length of 64
    assert PR.auto_layout([63, 65, 0], [70] * 3, 0, 64) == {"fwd": (1, 2), "dq": (1, 1), "dkdv": (1, 1)}
    assert PR.auto_layout([63, 64, 0], [70] * 3, 0, 32) == {"fwd": (1, 1), "dq": (1, 1), "dkdv": (1, 1)}
    assert PR.auto_layout([0, 0], [5, 5], 0, 128) == {"fwd": (1, 1), "dq": (1, 1), "dkdv": (1, 1)}
    assert PR.tile_sizes("fwd", 2, 1) == (64, 32) and PR.tile_sizes("dkdv", 1, 1) == (32, 32)


def test_export_layout():
    pl = PR.plan_list("fwd", [70, 0, 5], [3, 9, 0], 2, 0, 4, 1, 2)
    ex = PR.export(pl)
    P, n = ex[0], ex[1]
    assert P == 4 and n == len(pl["items"])
    assert ex[2:6] == [64, 32, 1, 2]
    assert ex[6:6 + P + 1] == pl["bin_ptr"]
    assert len(ex) == 6 + P + 1 + 5 * n
