"""Reference tile planner for jagged GDPA, in plain Python integers.

TEST INFRASTRUCTURE (see the header of gdpa_ref.py for who may import it).  The
C++ planner of the library must reproduce this plan bit for bit; it shares no
code with it.

Source: GDPA page (aitrends.kr/articles/26275, "Generalized Dot-Product Attention
(GDPA): kernel optimisation for real recommendation-system training loads"),
"Section details", paragraph and diagram on jagged inputs: the CPU enumerates the
valid tiles in advance, sorts them, and assigns them to processors in a zigzag
instead of round robin (max:min load 12:1 -> 5:4 in the diagram).

Readings (the page gives no cost model or tie-break):
  * a work item is (sample b, head h, stationary tile t) with a contiguous range
    [s0, s1] of streaming tiles that hold at least one valid pair; items whose
    other side is empty (Lk == 0 for Q-stationary lists, Lq == 0 for the
    KV-stationary list) have no steps (s0 = 0, s1 = -1) and only write zeros;
  * cost = (stationary tile rows) + sum over steps of (valid streaming rows + 32):
    rows moved through memory plus a fixed per-step charge, the stationary side
    charged as a whole tile even where the sample ends inside it (its products run
    on the whole tile, and a sample's last, partial tile then costs what its
    neighbours cost, so that it is sorted and dealt beside them);
  * chunks: with m = ceil(total cost / P), the mean bin cost, an item with n >= 2
    steps and cost > m (> ceil(m / 4) when the list has fewer than 2 P items, which
    no deal could balance) is cut into
    k = min(n, ceil(cost / ceil(m / 4))) chunks of consecutive steps (no bin could
    hold it at the mean), chunk j holding steps s0 + floor(j n / k) ..
    s0 + floor((j + 1) n / k) - 1 and costing its stationary tile plus its steps;
    chunk j of the g-th cut item (in (b, h, t) order) writes partial-output slot
    (chunks of earlier cut items) + j (O or dQ; dK and dV for the KV-stationary
    list), and the item's output is the sum of its slots.  The page deals tiles, not whole rows of tiles, so a long row of tiles
    need not sit in one bin; the chunks keep that freedom without atomics;
  * stable order: cost descending, then (b, h, s0, t) ascending: among equal
    costs, the items of one head that stream the same tiles (chunks of one step
    range over the stationary tiles, as in a KV-stationary pass over a long Q)
    follow each other, and the greedy deal puts them on neighbouring bins;
  * deal over P bins, by default greedy: each item, in sorted order, to the bin
    of least cost so far (lowest index on ties) -- the sorted assignment the page
    describes, taken to the least-loaded bin instead of a fixed snake; the page's
    zigzag (the r-th item to bin r mod P in even rounds and P - 1 - (r mod P) in
    odd rounds, round = r // P) and round robin are the alternatives;
  * per-bin CSR keeps each bin's items in deal order.

Three lists are planned: "fwd" and "dq" (Q-stationary: t is a q tile, steps are
kv tiles of 32 rows) and "dkdv" (KV-stationary: t is a kv tile, steps are q tiles
of 32 rows).  One team of waves processes one item; stationary tiles hold
32 * team * nb rows (team waves with nb 32-row blocks each), chosen from the head
dimension and the length statistics.
"""
from __future__ import annotations

import heapq

STEP_CHARGE = 32

LISTS = ("fwd", "dkdv", "dq")


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def auto_layout(lq, lk, window: int = 0, d: int = 128):
    """(team, nb) per list.  Forward: d = 128, two-wave teams with one block per
    wave when the mean non-empty query length is at least 48, else one wave and one
    block; d <= 64, one wave with nb = 2 when that mean is at least 64, else 1.
    dQ and dK/dV: one wave, one block.  (A tuning rule: it sets tile shapes, never
    which pairs are computed.)"""
    n = sum(1 for x in lq if x > 0)
    mean_at_least = lambda m: n > 0 and sum(lq) >= m * n
    fwd = ((2 if mean_at_least(48) else 1), 1) if d == 128 else (1, 2 if mean_at_least(64) else 1)
    return {"fwd": fwd, "dq": (1, 1), "dkdv": (1, 1)}


def tile_sizes(kind: str, team: int, nb: int):
    """(stationary tile rows, streaming tile rows) of a list."""
    if kind not in LISTS:
        raise ValueError(kind)
    return 32 * team * nb, 32


def enumerate_items(kind: str, lq, lk, H: int, window: int, t_stat: int, t_strm: int):
    """[(cost, b, h, t, s0, s1)] in (b, h, t) order."""
    items = []
    for b in range(len(lq)):
        if kind == "dkdv":
            ls, lo_other = int(lk[b]), int(lq[b])
        else:
            ls, lo_other = int(lq[b]), int(lk[b])
        for h in range(H):
            for t in range(_ceil_div(ls, t_stat)):
                a0 = t * t_stat
                a1 = min(ls, a0 + t_stat) - 1
                if lo_other == 0:
                    s0, s1 = 0, -1
                elif window == 0:
                    s0, s1 = 0, _ceil_div(lo_other, t_strm) - 1
                else:
                    lo = max(0, a0 - window + 1)
                    hi = min(lo_other - 1, a1 + window - 1)
                    s0, s1 = lo // t_strm, hi // t_strm
                cost = t_stat
                for s in range(s0, s1 + 1):
                    cost += min(lo_other, (s + 1) * t_strm) - s * t_strm + STEP_CHARGE
                items.append((cost, b, h, t, s0, s1))
    return items


def split_items(kind: str, items, lq, lk, P: int, t_stat: int, t_strm: int):
    """Cut the items longer than a mean bin into chunks.  Returns
    ([(cost, b, h, t, s0, s1, part)], number of slots); part = -1 for whole items."""
    out = []
    if P <= 0:
        return [it + (-1,) for it in items], 0
    ls, lo = (lk, lq) if kind == "dkdv" else (lq, lk)
    mean = max(1, _ceil_div(sum(it[0] for it in items), P))
    piece = max(1, _ceil_div(mean, 4))
    limit = piece if len(items) < 2 * P else mean
    slot = 0
    for cost, b, h, t, s0, s1 in items:
        n = s1 - s0 + 1
        if n < 2 or cost <= limit:
            out.append((cost, b, h, t, s0, s1, -1))
            continue
        k = min(n, _ceil_div(cost, piece))
        lo_other = int(lo[b])
        for j in range(k):
            f, l = s0 + j * n // k, s0 + (j + 1) * n // k - 1
            c = t_stat + sum(min(lo_other, (s + 1) * t_strm) - s * t_strm + STEP_CHARGE for s in range(f, l + 1))
            out.append((c, b, h, t, f, l, slot + j))
        slot += k
    return out, slot


DEALS = ("greedy", "zigzag", "round_robin")


def deal(items, P: int, mode: str = "greedy"):
    """Sort and deal items to P bins.  Returns (bin_ptr, ordered items, bin_cost)."""
    if mode not in DEALS:
        raise ValueError(mode)
    order = sorted(items, key=lambda it: (-it[0], it[1], it[2], it[4], it[3]))
    bins = [[] for _ in range(P)]
    cost = [0] * P
    least = [(0, p) for p in range(P)]   # (cost so far, bin), a heap: least cost, then lowest bin
    for r, it in enumerate(order):
        if mode == "greedy":
            _, p = heapq.heappop(least)
            heapq.heappush(least, (cost[p] + it[0], p))
        else:
            rnd, pos = divmod(r, P)
            p = pos if (mode == "round_robin" or rnd % 2 == 0) else P - 1 - pos
        bins[p].append(it)
        cost[p] += it[0]
    bin_ptr = [0]
    flat = []
    for p in range(P):
        flat.extend(bins[p])
        bin_ptr.append(len(flat))
    return bin_ptr, flat, cost


def plan_list(kind: str, lq, lk, H: int, window: int, P: int, team: int, nb: int, mode: str = "greedy",
              split: bool = True):
    t_stat, t_strm = tile_sizes(kind, team, nb)
    items = enumerate_items(kind, lq, lk, H, window, t_stat, t_strm)
    if split:
        items, n_parts = split_items(kind, items, lq, lk, P, t_stat, t_strm)
    else:
        items, n_parts = [it + (-1,) for it in items], 0
    bin_ptr, flat, cost = deal(items, P, mode)
    return dict(kind=kind, P=P, t_stat=t_stat, t_strm=t_strm, team=team, nb=nb,
                bin_ptr=bin_ptr, items=[it[1:] for it in flat], bin_cost=cost, n_parts=n_parts)


def export(pl) -> list:
    """The int32 serialisation the library's plan export produces:
    [P, n_items, t_stat, t_strm, team, nb, bin_ptr[0..P], then (b, h, t, s0, s1, part) per item]."""
    out = [pl["P"], len(pl["items"]), pl["t_stat"], pl["t_strm"], pl["team"], pl["nb"]]
    out += list(pl["bin_ptr"])
    for it in pl["items"]:
        out += list(it)
    return out


def plan(lq, lk, H: int, window: int, P: int, d: int = 128, layout=None, mode: str = "greedy",
         split: bool = True):
    """All three lists with the automatic (or given) layouts."""
    layout = layout or auto_layout(lq, lk, window, d)
    return {kind: plan_list(kind, lq, lk, H, window, P, *layout[kind], mode=mode, split=split) for kind in LISTS}


def groups(pl, off):
    """Cut items of a list in slot order: [(row0, rows, h, slot0, n)] where output
    rows row0 .. row0 + rows - 1 (absolute; off = query offsets, or key offsets for
    the dK/dV list) of head h are the sum of n slots."""
    by_slot = {}
    for b, h, t, s0, s1, part in pl["items"]:
        if part >= 0:
            by_slot[part] = (b, h, t)
    out = []
    for s in range(pl["n_parts"]):
        b, h, t = by_slot[s]
        if out and by_slot[s - 1] == (b, h, t):
            out[-1][4] += 1
            continue
        ln = off[b + 1] - off[b]
        ts = pl["t_stat"]
        out.append([off[b] + t * ts, min(ts, ln - t * ts), h, s, 1])
    return [tuple(g) for g in out]


def imbalance(cost) -> float:
    """max / min per-bin cost over bins with work (inf if some bin is idle)."""
    lo, hi = min(cost), max(cost)
    return float("inf") if lo == 0 else hi / lo
