// Host tile planner for jagged GDPA.
//
// GDPA page (aitrends.kr/articles/26275, "Generalized Dot-Product Attention
// (GDPA): kernel optimisation for real recommendation-system training loads"),
// "Section details", jagged-input paragraph and zigzag scheduling diagram: the
// host enumerates only the tiles that hold valid (query, key) pairs, sorts them
// and deals them to the compute units in a zigzag so the per-unit load is even.
//
// A work item is (sample b, head h, stationary tile t) plus the contiguous range
// [s0, s1] of streaming tiles it visits; one team of waves processes one item.
// Stationary tiles have 32 * team * nb rows (team waves with nb 32-row blocks
// each), streaming tiles 32 rows: q tiles / kv steps for the Q-stationary lists
// ("fwd", "dq"), kv tiles / q steps for the KV-stationary list ("dkdv").  Items
// whose other side is empty get no steps and write zeros.
//
// Cost of an item: stationary tile rows (a whole tile, also where the sample ends
// inside it) + sum over steps of (valid streaming rows + 32).  Chunks: an item with at least two steps whose cost exceeds the
// mean bin cost m = ceil(total / P) (a quarter of it, ceil(m / 4), when the list
// has fewer than 2 P items) is cut into k = min(steps, ceil(cost / ceil(m / 4)))
// chunks of consecutive steps (chunk i: steps s0 + floor(i n / k) ..
// s0 + floor((i + 1) n / k) - 1); each chunk writes its partial output block(s)
// (O or dQ; dK and dV for the KV-stationary list) to its own slot (numbered in
// (b, h, t) order) and a reduction adds the slots of one item in chunk order.  Order: cost descending,
// then (b, h, s0, t) (equal-cost items of a head that stream the same tiles end up
// side by side, on neighbouring bins of one XCD).  Deal: greedy (default: each item, in order, to the bin of
// least cost so far, the lowest index on ties), zigzag (the r-th item goes to bin
// r mod P in even rounds and P-1 - (r mod P) in odd rounds) or round robin.
#pragma once

#include <cstdint>
#include <vector>

namespace gdpa {

enum ListKind { LIST_FWD = 0, LIST_DKDV = 1, LIST_DQ = 2 };

// One work item as the kernels read it (32 bytes, one scalar load).
// part: partial-output slot of a chunk, -1 for an item that stores its outputs.
struct Item {
    int32_t b, h, t, s0, s1, part, pad0, pad1;
};
static_assert(sizeof(Item) == 32, "Item must be 32 bytes");

// The record a kernel reads per work item: the sample's row ranges are
// resolved on the host, so a kernel needs one load per item and no dependent
// loads of the offset arrays.
struct DevRec {
    int32_t qs, lq, ks, lk, h, t, s0, s1, part, pad0, pad1, pad2;
};
static_assert(sizeof(DevRec) == 48, "DevRec must be 48 bytes");

// One item cut into chunks, for the reduction: output rows row0 .. row0 + rows - 1
// of head h (absolute query rows, or key rows for dK/dV) are the sum of slots
// slot0 .. slot0 + n - 1.
struct DevGroup {
    int32_t row0, rows, h, slot0, n, pad0, pad1, pad2;
};
static_assert(sizeof(DevGroup) == 32, "DevGroup must be 32 bytes");

enum Deal { DEAL_GREEDY = 0, DEAL_ZIGZAG = 1, DEAL_ROUND_ROBIN = 2 };

struct WorkList {
    int kind = 0, P = 0, t_stat = 0, t_strm = 0, team = 0, nb = 0;
    std::vector<int32_t> bin_ptr;   // P + 1
    std::vector<Item> items;        // bin-major, deal order inside a bin
    std::vector<int32_t> order;     // the items in planner order (cost descending, then the
                                    // tie-break): order[r] = index in `items` of the r-th
    std::vector<int64_t> bin_cost;  // P (unweighted)
    bool weighted = false;          // the greedy deal took per-bin time factors
    int64_t n_steps = 0;
    int n_parts = 0;                // partial-output slots (chunks of cut items)
};

// waves per team and 32-row stationary blocks per wave, per list
struct Layout {
    int team[3];
    int nb[3];
};

constexpr int kStepCharge = 32;

Layout auto_layout(const std::vector<int64_t>& lq, const std::vector<int64_t>& lk, int d);
void tile_sizes(int kind, int team, int nb, int* t_stat, int* t_strm);
// bin_time: per-bin factors on the greedy deal's costs (its key is a bin's cost times
// the factor: a bin expected to run slower gets less work); empty = all 1
WorkList plan_list(int kind, const std::vector<int64_t>& lq, const std::vector<int64_t>& lk,
                   int H, int window, int P, int team, int nb, int deal, bool split,
                   const std::vector<double>& bin_time = std::vector<double>());
std::vector<int32_t> export_list(const WorkList& wl);
// dS blocks of the two-kernel backward with stored scores' gradients: one 32 x 32
// bf16 block (2 KiB, kv row major) per (head, 32-row q tile, 32-row kv tile) that
// holds a valid pair.  Per head, samples follow each other; a sample gives each of
// its q tiles nj[b] consecutive blocks (nj[b] = the most kv tiles any of its q tiles
// pairs with), q tile i's blocks holding its kv tiles js0(i), js0(i) + 1, .. in order:
//   block(h, b, i, j) = h nb_total + base[b] + i nj[b] + (j - js0(i)),
//   js0(i) = max(0, 32 i - window + 1) / 32 for a window, else 0,
// so both kernels find a block by arithmetic on their record (no table).
struct DsLayout {
    int64_t nb_total = 0;             // blocks per head
    std::vector<int64_t> base;        // B: first block of each sample
    std::vector<int32_t> nj;          // B: blocks per q tile of each sample
};
DsLayout ds_layout(const std::vector<int64_t>& lq, const std::vector<int64_t>& lk, int window);

std::vector<DevRec> device_records(const WorkList& wl, const std::vector<int32_t>& q_off,
                                   const std::vector<int32_t>& kv_off);
// with a dS layout: the dK/dV list's records carry (pad0, pad1) = (h nb_total + base[b], nj[b]),
// and so do a dQ list's of 64-row items (two-wave teams); the dQ list's 32-row q items carry
// pad0 = the block of the item's first step (its steps' blocks follow it)
std::vector<DevRec> device_records(const WorkList& wl, const std::vector<int32_t>& q_off,
                                   const std::vector<int32_t>& kv_off, const DsLayout& ds, int window);
// the cut items of a list, in slot order (output rows: queries, or keys for dK/dV)
std::vector<DevGroup> device_groups(const WorkList& wl, const std::vector<int32_t>& q_off,
                                    const std::vector<int32_t>& kv_off);

}  // namespace gdpa
