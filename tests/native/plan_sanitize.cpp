// Host build of the tile planner for the address and undefined-behaviour
// sanitizers (g++ -fsanitize=address,undefined); test infrastructure only.
//
// Reads one planning problem from stdin:
//     B H window d P deal split team0 team1 team2 blocks0 blocks1 blocks2
//     lq[0] .. lq[B-1]
//     lk[0] .. lk[B-1]
// (team / blocks 0 = the automatic layout), plans the three work lists, resolves
// their device records and chunk groups, and prints each list's export, one list
// per line, so that the caller can compare it with the library's.  Exits non-zero
// on malformed input; a sanitizer finding aborts the run.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "plan.hpp"

using namespace gdpa;

int main() {
    int B, H, window, d, P, deal, split, team[3], blocks[3];
    if (std::scanf("%d %d %d %d %d %d %d", &B, &H, &window, &d, &P, &deal, &split) != 7) return 2;
    for (int l = 0; l < 3; ++l)
        if (std::scanf("%d", &team[l]) != 1) return 2;
    for (int l = 0; l < 3; ++l)
        if (std::scanf("%d", &blocks[l]) != 1) return 2;
    if (B < 0 || H < 1 || P < 1) return 2;
    std::vector<int64_t> lq(B), lk(B);
    std::vector<int32_t> q_off(B + 1, 0), kv_off(B + 1, 0);
    for (int b = 0; b < B; ++b) {
        long long x;
        if (std::scanf("%lld", &x) != 1 || x < 0) return 2;
        lq[b] = x;
        q_off[b + 1] = q_off[b] + (int32_t)x;
    }
    for (int b = 0; b < B; ++b) {
        long long x;
        if (std::scanf("%lld", &x) != 1 || x < 0) return 2;
        lk[b] = x;
        kv_off[b + 1] = kv_off[b] + (int32_t)x;
    }
    Layout L = auto_layout(lq, lk, d);
    for (int l = 0; l < 3; ++l) {
        if (team[l]) L.team[l] = team[l];
        if (blocks[l]) L.nb[l] = blocks[l];
    }
    for (int l = 0; l < 3; ++l) {
        const WorkList wl = plan_list(l, lq, lk, H, window, P, L.team[l], L.nb[l], deal, split != 0);
        // the device-side views the library uploads: every record and group is built
        const std::vector<DevRec> recs = device_records(wl, q_off, kv_off);
        const std::vector<DevGroup> groups = device_groups(wl, q_off, kv_off);
        if (recs.size() != wl.items.size()) return 3;
        long long rows = 0;
        for (const DevGroup& g : groups) rows += g.rows;
        const std::vector<int32_t> ex = export_list(wl);
        std::printf("%zu %lld", groups.size(), rows);
        for (int32_t v : ex) std::printf(" %d", v);
        std::printf("\n");
    }
    return 0;
}
