// Host tile planner (see plan.hpp for the rules and the source they follow).
#include "plan.hpp"

#include <algorithm>
#include <functional>
#include <numeric>
#include <queue>

namespace gdpa {

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

Layout auto_layout(const std::vector<int64_t>& lq, const std::vector<int64_t>&, int d) {
    int64_t nq = 0, sq = 0;
    for (size_t b = 0; b < lq.size(); ++b) {
        nq += lq[b] > 0;
        sq += lq[b];
    }
    // mean non-empty length >= m  <=>  total >= m * count
    auto mean_at_least = [](int64_t total, int64_t count, int64_t m) { return count > 0 && total >= m * count; };
    Layout L;
    if (d == 128) {
        // two-wave forward teams once the queries are long enough to fill them;
        // 32-row dQ and dK/dV items (the backward's stored-dS blocks)
        L.team[LIST_FWD] = mean_at_least(sq, nq, 48) ? 2 : 1;
        L.nb[LIST_FWD] = 1;
        L.team[LIST_DQ] = L.team[LIST_DKDV] = 1;
        L.nb[LIST_DQ] = L.nb[LIST_DKDV] = 1;
    } else {
        L.team[LIST_FWD] = L.team[LIST_DQ] = L.team[LIST_DKDV] = 1;
        L.nb[LIST_FWD] = mean_at_least(sq, nq, 64) ? 2 : 1;
        L.nb[LIST_DQ] = L.nb[LIST_DKDV] = 1;
    }
    return L;
}

void tile_sizes(int, int team, int nb, int* t_stat, int* t_strm) {
    *t_stat = 32 * team * nb;
    *t_strm = 32;
}

namespace {
struct Cand {
    int64_t cost;
    Item it;
};
}  // namespace

WorkList plan_list(int kind, const std::vector<int64_t>& lq, const std::vector<int64_t>& lk,
                   int H, int window, int P, int team, int nb, int deal, bool split,
                   const std::vector<double>& bin_time) {
    WorkList wl;
    wl.kind = kind;
    wl.P = P;
    wl.team = team;
    wl.nb = nb;
    tile_sizes(kind, team, nb, &wl.t_stat, &wl.t_strm);
    const int64_t TS = wl.t_stat, TR = wl.t_strm;

    // whole items in (b, h, t) order
    std::vector<Cand> whole;
    for (size_t b = 0; b < lq.size(); ++b) {
        const int64_t ls = (kind == LIST_DKDV) ? lk[b] : lq[b];
        const int64_t lo = (kind == LIST_DKDV) ? lq[b] : lk[b];
        const int64_t ntiles = ceil_div(ls, TS);
        for (int h = 0; h < H; ++h) {
            for (int64_t t = 0; t < ntiles; ++t) {
                const int64_t a0 = t * TS;
                const int64_t a1 = std::min(ls, a0 + TS) - 1;
                int64_t s0, s1;
                if (lo == 0) {
                    s0 = 0;
                    s1 = -1;
                } else if (window == 0) {
                    s0 = 0;
                    s1 = ceil_div(lo, TR) - 1;
                } else {
                    const int64_t lo_row = std::max<int64_t>(0, a0 - window + 1);
                    const int64_t hi_row = std::min<int64_t>(lo - 1, a1 + window - 1);
                    s0 = lo_row / TR;
                    s1 = hi_row / TR;
                }
                // the stationary side as a whole tile: its products run on the whole tile, and a
                // sample's last, partial tile then costs what its neighbours cost, so that it is
                // sorted and dealt beside them (and, streaming the same tiles, meets them in L2)
                int64_t cost = TS;
                for (int64_t s = s0; s <= s1; ++s) cost += std::min(lo, (s + 1) * TR) - s * TR + kStepCharge;
                Cand c;
                c.cost = cost;
                c.it = Item{(int32_t)b, h, (int32_t)t, (int32_t)s0, (int32_t)s1, -1, 0, 0};
                whole.push_back(c);
            }
        }
    }

    // chunks of the items longer than a mean bin
    std::vector<Cand> cands;
    if (split && P > 0) {
        int64_t total = 0;
        for (const Cand& c : whole) total += c.cost;
        const int64_t mean = std::max<int64_t>(1, ceil_div(total, (int64_t)P));
        const int64_t piece = std::max<int64_t>(1, ceil_div(mean, 4));
        // fewer than two items per bin: no deal can balance them, so cut at a quarter bin
        const int64_t limit = (int64_t)whole.size() < 2 * (int64_t)P ? piece : mean;
        int32_t slot = 0;
        for (size_t i = 0; i < whole.size(); ++i) {
            const Cand& c = whole[i];
            const int64_t n = (int64_t)c.it.s1 - c.it.s0 + 1;
            if (n < 2 || c.cost <= limit) {
                cands.push_back(c);
                continue;
            }
            const int64_t k = std::min(n, ceil_div(c.cost, piece));
            const int64_t lo = (kind == LIST_DKDV) ? lq[c.it.b] : lk[c.it.b];
            for (int64_t j = 0; j < k; ++j) {
                const int64_t f = c.it.s0 + j * n / k, l = c.it.s0 + (j + 1) * n / k - 1;
                Cand p = c;
                p.cost = TS;
                for (int64_t s = f; s <= l; ++s) p.cost += std::min(lo, (s + 1) * TR) - s * TR + kStepCharge;
                p.it.s0 = (int32_t)f;
                p.it.s1 = (int32_t)l;
                p.it.part = slot + (int32_t)j;
                cands.push_back(p);
            }
            slot += (int32_t)k;
        }
        wl.n_parts = slot;
    } else {
        cands = std::move(whole);
    }
    std::sort(cands.begin(), cands.end(), [](const Cand& x, const Cand& y) {
        if (x.cost != y.cost) return x.cost > y.cost;
        if (x.it.b != y.it.b) return x.it.b < y.it.b;
        if (x.it.h != y.it.h) return x.it.h < y.it.h;
        if (x.it.s0 != y.it.s0) return x.it.s0 < y.it.s0;
        return x.it.t < y.it.t;
    });

    // deal, then a bin-major CSR keeping deal order
    std::vector<int32_t> bin_of(cands.size());
    std::vector<int32_t> count(P, 0);
    wl.bin_cost.assign(P, 0);
    // (cost so far times the bin's time factor, bin): least, then lowest bin.  Without
    // factors the keys are the integer costs, exact in a double
    typedef std::pair<double, int> Load;
    std::priority_queue<Load, std::vector<Load>, std::greater<Load>> least;
    const bool weighted = deal == DEAL_GREEDY && (int)bin_time.size() == P;
    wl.weighted = weighted;
    if (deal == DEAL_GREEDY)
        for (int p = 0; p < P; ++p) least.push(Load(0.0, p));
    for (size_t r = 0; r < cands.size(); ++r) {
        int p;
        if (deal == DEAL_GREEDY) {
            p = least.top().second;
            least.pop();
            const int64_t c = wl.bin_cost[p] + cands[r].cost;
            least.push(Load(weighted ? (double)c * bin_time[p] : (double)c, p));
        } else {
            const int64_t rnd = (int64_t)r / P, pos = (int64_t)r % P;
            p = (int)((deal == DEAL_ROUND_ROBIN || rnd % 2 == 0) ? pos : P - 1 - pos);
        }
        bin_of[r] = p;
        count[p]++;
        wl.bin_cost[p] += cands[r].cost;
    }
    wl.bin_ptr.assign(P + 1, 0);
    for (int p = 0; p < P; ++p) wl.bin_ptr[p + 1] = wl.bin_ptr[p] + count[p];
    std::vector<int32_t> fill(wl.bin_ptr.begin(), wl.bin_ptr.end() - 1);
    wl.items.resize(cands.size());
    wl.order.resize(cands.size());
    for (size_t r = 0; r < cands.size(); ++r) {
        wl.order[r] = fill[bin_of[r]];
        wl.items[fill[bin_of[r]]++] = cands[r].it;
        const Item& it = cands[r].it;
        if (it.s1 >= it.s0) wl.n_steps += it.s1 - it.s0 + 1;
    }
    return wl;
}

std::vector<int32_t> export_list(const WorkList& wl) {
    std::vector<int32_t> out = {wl.P, (int32_t)wl.items.size(), wl.t_stat, wl.t_strm, wl.team, wl.nb};
    out.insert(out.end(), wl.bin_ptr.begin(), wl.bin_ptr.end());
    for (const Item& it : wl.items) {
        out.push_back(it.b);
        out.push_back(it.h);
        out.push_back(it.t);
        out.push_back(it.s0);
        out.push_back(it.s1);
        out.push_back(it.part);
    }
    return out;
}

std::vector<DevRec> device_records(const WorkList& wl, const std::vector<int32_t>& q_off,
                                   const std::vector<int32_t>& kv_off) {
    std::vector<DevRec> out(wl.items.size());
    for (size_t i = 0; i < wl.items.size(); ++i) {
        const Item& it = wl.items[i];
        DevRec& d = out[i];
        d.qs = q_off[it.b];
        d.lq = q_off[it.b + 1] - q_off[it.b];
        d.ks = kv_off[it.b];
        d.lk = kv_off[it.b + 1] - kv_off[it.b];
        d.h = it.h;
        d.t = it.t;
        d.s0 = it.s0;
        d.s1 = it.s1;
        d.part = it.part;
        d.pad0 = d.pad1 = d.pad2 = 0;
    }
    return out;
}

// first kv tile with a pair for 32-row q tile i (the band rule plan_list applies)
static int64_t ds_js0(int64_t i, int window) {
    return window == 0 ? 0 : std::max<int64_t>(0, 32 * i - window + 1) / 32;
}

DsLayout ds_layout(const std::vector<int64_t>& lq, const std::vector<int64_t>& lk, int window) {
    DsLayout L;
    L.base.assign(lq.size(), 0);
    L.nj.assign(lq.size(), 0);
    int64_t total = 0;
    for (size_t b = 0; b < lq.size(); ++b) {
        const int64_t ntq = ceil_div(lq[b], 32);
        int64_t nj = 0;
        if (lk[b] > 0) {
            for (int64_t i = 0; i < ntq; ++i) {
                const int64_t a1 = std::min(lq[b], 32 * i + 32) - 1;
                const int64_t js1 = window == 0 ? ceil_div(lk[b], 32) - 1
                                                : std::min<int64_t>(lk[b] - 1, a1 + window - 1) / 32;
                nj = std::max(nj, js1 - ds_js0(i, window) + 1);
            }
        }
        L.base[b] = total;
        L.nj[b] = (int32_t)nj;
        total += ntq * nj;
    }
    L.nb_total = total;
    return L;
}

std::vector<DevRec> device_records(const WorkList& wl, const std::vector<int32_t>& q_off,
                                   const std::vector<int32_t>& kv_off, const DsLayout& ds, int window) {
    std::vector<DevRec> out = device_records(wl, q_off, kv_off);
    for (size_t i = 0; i < wl.items.size(); ++i) {
        const Item& it = wl.items[i];
        DevRec& d = out[i];
        const int64_t head = it.h * ds.nb_total + ds.base[it.b];
        if (wl.kind == LIST_DKDV) {
            d.pad0 = (int32_t)head;
            d.pad1 = ds.nj[it.b];
        } else if (wl.kind == LIST_DQ && wl.team == 2) {   // each wave finds its own q tile's blocks
            d.pad0 = (int32_t)head;
            d.pad1 = ds.nj[it.b];
        } else if (wl.kind == LIST_DQ && it.s1 >= it.s0) {
            d.pad0 = (int32_t)(head + (int64_t)it.t * ds.nj[it.b] + (it.s0 - ds_js0(it.t, window)));
        }
    }
    return out;
}

std::vector<DevGroup> device_groups(const WorkList& wl, const std::vector<int32_t>& q_off,
                                    const std::vector<int32_t>& kv_off) {
    // chunk j of a cut item holds slot slot0 + j; slots of one item are consecutive
    std::vector<const Item*> by_slot(wl.n_parts, nullptr);
    for (const Item& it : wl.items)
        if (it.part >= 0) by_slot[it.part] = &it;
    std::vector<DevGroup> out;
    for (int s = 0; s < wl.n_parts; ++s) {
        const Item* it = by_slot[s];
        const bool same = !out.empty() && s > 0 && by_slot[s - 1]->b == it->b && by_slot[s - 1]->h == it->h &&
                          by_slot[s - 1]->t == it->t;
        if (same) {
            out.back().n++;
            continue;
        }
        // output rows: queries of a Q-stationary list, keys of the KV-stationary one
        const std::vector<int32_t>& off = wl.kind == LIST_DKDV ? kv_off : q_off;
        const int32_t len = off[it->b + 1] - off[it->b];
        DevGroup g;
        g.row0 = off[it->b] + it->t * wl.t_stat;
        g.rows = std::min(wl.t_stat, len - it->t * wl.t_stat);
        g.h = it->h;
        g.slot0 = s;
        g.n = 1;
        g.pad0 = g.pad1 = g.pad2 = 0;
        out.push_back(g);
    }
    return out;
}

}  // namespace gdpa
