"""Pins for the reference planner: its items are checked against brute-force
enumeration of the valid set, and the deal against the zigzag rule.

Source: GDPA page ("Generalized Dot-Product Attention (GDPA): kernel optimisation
for real recommendation-system training loads"), "Section details", jagged-input
paragraph and zigzag tile-scheduling diagram.
"""
import itertools

import numpy as np
import pytest

from gdpa_workloads import WORKLOADS, workload_lengths
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
    bin_ptr, flat, cost = PR.deal(items, P, "zigzag")
    order = sorted(items, key=lambda it: (-it[0], it[1], it[2], it[3], it[4]))
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
    _, _, zz = PR.deal(items, 16, "zigzag")
    _, _, rr = PR.deal(items, 16, "round_robin")
    _, _, gr = PR.deal(items, 16, "greedy")
    assert PR.imbalance(gr) <= PR.imbalance(zz) < PR.imbalance(rr)


@pytest.mark.parametrize("P", [1, 3, 8, 64])
def test_greedy_deal_is_least_loaded_first(P):
    """Each item, in sorted order, goes to the bin of least cost so far (lowest
    index on ties): checked with a plain scan over the bins."""
    rng = np.random.default_rng(P)
    items = [(int(c), i, 0, 0, 0, 0) for i, c in enumerate(rng.integers(1, 500, 300))]
    bin_ptr, flat, cost = PR.deal(items, P, "greedy")
    order = sorted(items, key=lambda it: (-it[0], it[1], it[2], it[3], it[4]))
    load = [0] * P
    want = [[] for _ in range(P)]
    for it in order:
        p = min(range(P), key=lambda q: (load[q], q))
        want[p].append(it)
        load[p] += it[0]
    assert [flat[bin_ptr[p]:bin_ptr[p + 1]] for p in range(P)] == want
    assert cost == load
    # the classic bound of longest-first greedy: max load <= mean + largest item
    assert max(cost) <= sum(load) / P + max(it[0] for it in items)


def test_auto_layout_rules():
    # d = 128: two-wave forward teams from a mean query length of 48, one block per wave
    assert PR.auto_layout([32] * 8, [1000] * 8, 0, 128) == {"fwd": (1, 1), "dq": (1, 1), "dkdv": (1, 1)}
    assert PR.auto_layout([300] * 8, [32] * 8, 0, 128) == {"fwd": (2, 1), "dq": (1, 1), "dkdv": (1, 1)}
    assert PR.auto_layout([47, 49, 0], [5] * 3, 0, 128)["fwd"] == (2, 1)
    assert PR.auto_layout([47, 48, 0], [5] * 3, 0, 128)["fwd"] == (1, 1)
    # dQ: one block per wave at every d (d = 128: the stored-dS blocks are 32 rows)
    assert PR.auto_layout([63, 65, 0], [5] * 3, 0, 128)["dq"] == (1, 1)
    assert PR.auto_layout([300, 900], [5] * 2, 0, 128)["dq"] == (1, 1)
    assert PR.auto_layout([63, 65, 0], [5] * 3, 0, 64)["dq"] == (1, 1)
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
    assert len(ex) == 6 + P + 1 + 6 * n


SPLIT_CASES = [
    ([32] * 6, [1, 1000, 31, 32, 33, 0], 0, 2),
    ([32, 64, 5], [4096, 100, 3000], 0, 3),
    ([300, 129, 64, 2], [300, 129, 64, 2], 128, 2),
    ([70, 1, 33, 200, 0], [64, 3, 0, 2, 129], 0, 1),
]


@pytest.mark.parametrize("lq,lk,window,P", SPLIT_CASES)
@pytest.mark.parametrize("kind", PR.LISTS)
@pytest.mark.parametrize("layout", [(1, 1), (2, 1), (1, 2)])
def test_chunks_cover_each_tile_once(lq, lk, window, P, kind, layout):
    """Cutting items keeps the plan exact: every tile pair with a valid (i, j) is
    visited once, every output tile has one owner -- a whole item, or the chunks of
    one cut item with consecutive slots numbered in (b, h, t) order."""
    H = 2
    if kind == "dkdv" and layout != (1, 1):
        return
    pl = PR.plan_list(kind, lq, lk, H, window, P, *layout)
    t_stat, t_strm = pl["t_stat"], pl["t_strm"]
    seen, whole, chunks = set(), set(), {}
    for b, h, t, s0, s1, part in pl["items"]:
        for s in range(s0, s1 + 1):
            assert (b, h, t, s) not in seen
            seen.add((b, h, t, s))
        if part < 0:
            assert (b, h, t) not in whole and (b, h, t) not in chunks
            whole.add((b, h, t))
        else:
            assert (b, h, t) not in whole
            assert s1 >= s0
            chunks.setdefault((b, h, t), []).append((s0, s1, part))
    assert seen == _tiles_with_valid_pair(kind, lq, lk, H, window, t_stat, t_strm)
    slots = []
    for key in sorted(chunks):
        cs = sorted(chunks[key])
        assert len(cs) >= 2
        assert all(cs[i][1] + 1 == cs[i + 1][0] for i in range(len(cs) - 1))   # consecutive steps
        assert [c[2] for c in cs] == list(range(cs[0][2], cs[0][2] + len(cs)))  # consecutive slots
        slots += [c[2] for c in cs]
    assert slots == list(range(pl["n_parts"]))   # numbered in (b, h, t) order
    ls = lk if kind == "dkdv" else lq
    assert whole | set(chunks) == {(b, h, t) for b in range(len(ls)) for h in range(H)
                                   for t in range(-(-ls[b] // t_stat))}


def test_chunk_rule_on_a_long_item():
    """One sample of 32 queries and 4096 keys next to 63 one-step samples, 16 bins,
    no window: the long item (128 steps) costs 32 + 128 * 64 = 8224, each one-step
    item (one query row, one key row) 32 + (1 + 32) = 65 (the stationary side is
    charged as a whole 32-row tile), the total is 8224 + 63 * 65 = 12319, the mean bin
    cost m = ceil(12319 / 16) = 770, so the item is cut into
    k = ceil(8224 / ceil(770 / 4)) = ceil(8224 / 193) = 43 chunks of 2 or 3 steps; the
    one-step items stay whole."""
    lq, lk = [32] + [1] * 63, [4096] + [1] * 63
    pl = PR.plan_list("fwd", lq, lk, 1, 0, 16, 1, 1)
    parts = sorted((s0, s1, part) for b, h, t, s0, s1, part in pl["items"] if part >= 0)
    assert pl["n_parts"] == 43 and len(parts) == 43
    assert [s1 - s0 + 1 for s0, s1, _ in parts] == [(j + 1) * 128 // 43 - j * 128 // 43 for j in range(43)]
    assert all(part == -1 for b, h, t, s0, s1, part in pl["items"] if b > 0)
    # the chunked plan balances where the whole item could not
    whole = PR.plan_list("fwd", lq, lk, 1, 0, 16, 1, 1, split=False)
    assert max(whole["bin_cost"]) >= 8224
    for mode in PR.DEALS:
        cut = PR.plan_list("fwd", lq, lk, 1, 0, 16, 1, 1, mode=mode)
        assert max(cut["bin_cost"]) < 0.15 * max(whole["bin_cost"])
        assert sum(cut["bin_cost"]) == sum(whole["bin_cost"]) + 42 * 32   # each extra chunk reloads 32 rows
    g = PR.groups(pl, [0] + list(np.cumsum(lq)))
    assert g == [(0, 32, 0, 0, 43)]


def test_short_items_are_never_cut():
    # one step per item: nothing to cut
    lq, lk = [32] * 40, [20] * 40
    assert PR.plan_list("fwd", lq, lk, 2, 0, 4, 1, 1)["n_parts"] == 0
    assert PR.plan_list("dkdv", lk, lq, 2, 0, 4, 1, 1)["n_parts"] == 0


def test_kv_stationary_chunks_group_key_rows():
    """A 32-key sample with 4000 queries: its two dK/dV items (one per head) stream
    125 q tiles each and are cut; the groups name key rows (the sample's keys start
    after the 3 keys of sample 0)."""
    lq, lk = [5, 4000], [3, 32]
    pl = PR.plan_list("dkdv", lq, lk, 2, 0, 4, 1, 1)
    assert pl["n_parts"] > 0
    g = PR.groups(pl, [0, 3, 35])
    assert [(r0, rows, h) for r0, rows, h, _, _ in g] == [(3, 32, 0), (3, 32, 1)]
    assert sum(n for *_, n in g) == pl["n_parts"]


def test_few_items_are_cut_to_quarter_bins():
    """Fewer items than 2 P: 20 KV-stationary items over 16 bins, each 32 key rows
    streaming 1000 queries, cost 32 + 31 * (32 + 32) + (8 + 32) = 2056 (mean bin cost
    ceil(41120 / 16) = 2570).  Whole, two land in one bin; so every item above a
    quarter bin (643) is cut, into ceil(2056 / 643) = 4 chunks."""
    lq, lk = [1000], [300]
    pl = PR.plan_list("dkdv", lq, lk, 2, 0, 16, 1, 1)
    assert len(pl["items"]) == 80 and pl["n_parts"] == 80
    whole = PR.plan_list("dkdv", lq, lk, 2, 0, 16, 1, 1, split=False)
    assert max(whole["bin_cost"]) == 2 * 2056
    assert max(pl["bin_cost"]) <= 1.1 * sum(pl["bin_cost"]) / 16


def _tile_pairs_of_sample(kind, lq, lk, window, t_stat, t_strm):
    """Brute force for one sample, vectorised: the (t, s) tile pairs whose block of
    the dense validity mask holds a valid (i, j)."""
    m = valid_mask(np.arange(lq), np.arange(lk), lq, lk, window)
    if kind == "dkdv":
        m = m.T
    a, c = m.shape
    if a == 0 or c == 0:
        return set()
    nt, ns = -(-a // t_stat), -(-c // t_strm)
    pad = np.zeros((nt * t_stat, ns * t_strm), dtype=bool)
    pad[:a, :c] = m
    hit = pad.reshape(nt, t_stat, ns, t_strm).any(axis=(1, 3))
    return set(zip(*(x.tolist() for x in np.nonzero(hit))))


# the five workloads at seed 0; the windowed batch's check of the tiles runs on a
# subset of its samples (the shortest, the longest and six more), the rest in full
@pytest.mark.parametrize("cfg", sorted(WORKLOADS))
@pytest.mark.parametrize("kind", PR.LISTS)
def test_workload_plans_at_automatic_layouts_cover_each_tile_once(cfg, kind):
    """Each workload's plan at the layout auto_layout picks for it (a tuning rule: it
    changes tile shapes and the deal, never which pairs are computed), over 1024
    bins with items cut into chunks: every tile pair holding a valid (i, j) is
    visited exactly once, every stationary tile of every (sample, head) has one
    owner (a whole item or the chunks of one cut item, with consecutive steps and
    consecutive slots numbered in (b, h, t) order), and no bin is left idle while
    another holds more than one item."""
    w = WORKLOADS[cfg]
    lq, lk = workload_lengths(cfg, 0)
    H, window = w["H"], w["window"]
    team, nb = PR.auto_layout(lq, lk, window, w["d"])[kind]
    pl = PR.plan_list(kind, lq, lk, H, window, 1024, team, nb)
    t_stat, t_strm = pl["t_stat"], pl["t_strm"]
    ls = lk if kind == "dkdv" else lq
    B = len(lq)
    if cfg == 5:
        rng = np.random.default_rng(5)
        check = {int(np.argmin(ls)), int(np.argmax(ls))} | set(rng.choice(B, 6, replace=False).tolist())
    else:
        check = set(range(B))
    seen = {b: set() for b in check}
    whole, chunks = set(), {}
    for b, h, t, s0, s1, part in pl["items"]:
        if b in check:
            for s in range(s0, s1 + 1):
                assert (h, t, s) not in seen[b]
                seen[b].add((h, t, s))
        if part < 0:
            assert (b, h, t) not in whole and (b, h, t) not in chunks
            whole.add((b, h, t))
        else:
            assert (b, h, t) not in whole and s1 >= s0
            chunks.setdefault((b, h, t), []).append((s0, s1, part))
    for b in check:
        pairs = _tile_pairs_of_sample(kind, int(lq[b]), int(lk[b]), window, t_stat, t_strm)
        assert seen[b] == {(h, t, s) for h in range(H) for t, s in pairs}, b
    slots = []
    for key in sorted(chunks):
        cs = sorted(chunks[key])
        assert len(cs) >= 2
        assert all(cs[i][1] + 1 == cs[i + 1][0] for i in range(len(cs) - 1))
        assert [c[2] for c in cs] == list(range(cs[0][2], cs[0][2] + len(cs)))
        slots += [c[2] for c in cs]
    assert slots == list(range(pl["n_parts"]))
    assert whole | set(chunks) == {(b, h, t) for b in range(B) for h in range(H)
                                   for t in range(-(-int(ls[b]) // t_stat))}
    counts = np.diff(pl["bin_ptr"])
    assert not (counts.min() == 0 and counts.max() > 1)


def test_partial_tiles_sort_beside_their_neighbours():
    """The cost charges the stationary side as a whole tile, so the tiles of one (sample,
    head) that stream the same tiles cost the same whether or not the sample ends inside
    them: in the sorted order each (sample, head)'s items sit together, the last, partial
    tile among them (a whole-tile charge for every stationary tile, rows or not)."""
    lq = [100, 257, 33, 64, 1000, 95]          # every sample ends inside its last 64-row tile but one
    lk = [32] * len(lq)                        # one streaming tile: every item costs the same
    H = 3
    t_stat, t_strm = PR.tile_sizes("fwd", 2, 1)
    items = PR.enumerate_items("fwd", lq, lk, H, 0, t_stat, t_strm)
    assert len({it[0] for it in items}) == 1   # partial tiles cost what full ones do
    order = sorted(items, key=lambda it: (-it[0], it[1], it[2], it[4], it[3]))
    pos = {}
    for r, it in enumerate(order):
        pos.setdefault((it[1], it[2]), []).append(r)
    for key, rs in pos.items():
        assert rs == list(range(rs[0], rs[0] + len(rs))), key   # contiguous in the sorted order
        ts = [order[r][3] for r in rs]
        assert ts == sorted(ts)                                  # and in tile order
