// C ABI of the GDPA library: argument validation, planning, upload and kernel
// dispatch.  See include/gdpa.h for the contract of every entry point.
#include "gdpa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "gelu_poly.h"
#include "kernels.hpp"
#include "plan.hpp"

using namespace gdpa;

namespace {

thread_local std::string g_err;

gdpa_status fail(gdpa_status s, const std::string& msg) {
    g_err = msg;
    return s;
}

gdpa_status fail_hip(hipError_t e, const char* what) {
    g_err = std::string(what) + ": " + hipGetErrorString(e);
    return GDPA_ERR_HIP;
}

bool debug_enabled() {
    const char* v = std::getenv("GDPA_DEBUG");
    return v && *v && std::strcmp(v, "0") != 0;
}

const void* fwd_kernel_ptr(int d, int team, int nb, int act) {
    switch (d) {
        case 32: return fwd_bf16_kernel_ptr_d32(team, nb, act);
        case 64: return fwd_bf16_kernel_ptr_d64(team, nb, act);
        case 128: return fwd_bf16_kernel_ptr_d128(team, nb, act);
    }
    return nullptr;
}
const void* dq_kernel_ptr(int d, int team, int nb, int act) {
    switch (d) {
        case 32: return dq_bf16_kernel_ptr_d32(team, nb, act);
        case 64: return dq_bf16_kernel_ptr_d64(team, nb, act);
        case 128: return dq_bf16_kernel_ptr_d128(team, nb, act);
    }
    return nullptr;
}
const void* dkdv_kernel_ptr(int d, int team, int nb, int act) {
    switch (d) {
        case 32: return dkdv_bf16_kernel_ptr_d32(team, nb, act);
        case 64: return dkdv_bf16_kernel_ptr_d64(team, nb, act);
        case 128: return dkdv_bf16_kernel_ptr_d128(team, nb, act);
    }
    return nullptr;
}

// work lists of a plan: GDPA_LIST_FWD, _DKDV, _DQ and the two-wave dQ-from-dS list
constexpr int kLists = 4;
constexpr int LIST_DQ_TEAM = 3;

// Time factors per dispatch round for the greedy deal.  A persistent launch of k
// workgroups per CU reaches each CU in k rounds (an XCD's first workgroups go one per
// CU, then the next round, ...), and on the kernels below, workgroups of the early
// rounds finished the same planned cost measurably sooner than those placed after
// them (busy times measured per workgroup with the clock-probe build; the cause, most
// likely how the CU's arbitration favours older waves, is not established).  A factor
// is a round's busy time over the mean of all rounds with every bin dealt equal cost
// (d = 128: windowed self-attention, 567,626 rows, H = 4, window 128; d = 64: the
// cross-attention batch, whose 8-round split was then tuned on its own timing); the
// deal gives a bin work in inverse proportion to its factor.
struct SlotTimes {
    int list, d, team, nb, per_cu;   // the list and its kernel's layout, workgroups per CU
    double f[8];                     // factor of each dispatch round (per_cu of them)
};
constexpr SlotTimes kSlotTimes[] = {
    // forward, two-wave teams
    {LIST_FWD, 128, 2, 1, 4, {0.92, 1.0, 1.01, 1.07}},
    // dK/dV, 16-row waves, two per 32-row team
    {LIST_DKDV, 128, 1, 1, 4, {0.88, 1.025, 1.025, 1.07}},
    // forward, one wave of two 32-row blocks
    {LIST_FWD, 64, 1, 2, 8, {0.93, 0.93, 0.93, 0.93, 1.07, 1.07, 1.07, 1.07}},
    // dQ from stored dS, two-wave teams over 64-row items (three teams per CU)
    {LIST_DQ_TEAM, 128, 2, 1, 3, {0.90, 1.045, 1.055}},
};

// Per-bin factors of list `list` (its kernel's layout d, team, nb) over P automatic bins,
// or none where the table has no entry: bin q runs on the workgroup the XCD remap gives
// it, position q % (P / 8) in its XCD's dispatch order, so in dispatch round
// position / (CUs per XCD).
std::vector<double> round_time_factors(int list, int d, int team, int nb, int P, int cus) {
    std::vector<double> bin_time;
    if (cus % 8 != 0) return bin_time;
    for (const SlotTimes& t : kSlotTimes)
        if (t.list == list && t.d == d && t.team == team && t.nb == nb && P == t.per_cu * cus) {
            bin_time.resize(P);
            for (int q = 0; q < P; ++q) bin_time[q] = t.f[(q % (P / 8)) / (cus / 8)];
        }
    return bin_time;
}

int64_t pairs_of(int64_t lq, int64_t lk, int64_t w) {
    if (w == 0) return lq * lk;
    int64_t n = 0;
    for (int64_t i = 0; i < lq; ++i) n += std::min(lk, i + w) - std::max<int64_t>(0, i - w + 1);
    return n;
}

}  // namespace

struct gdpa_plan_s;
static gdpa_status upload(gdpa_plan_s* p, hipStream_t s);
static gdpa_status plan_create(const int32_t* q_off_host, const int32_t* kv_off_host, int B, int H, int d,
                               int window, gdpa_dtype dtype, const gdpa_plan_opts* opts, hipStream_t stream,
                               bool pffn, gdpa_plan_s** out);

struct gdpa_plan_s {
    int B = 0, H = 0, d = 0, window = 0;
    gdpa_dtype dtype = GDPA_BF16;
    bool host_only = true;
    std::vector<int32_t> q_off, kv_off;
    std::vector<int64_t> lq, lk;
    int64_t Tq = 0, Tk = 0, valid_pairs = 0;
    int fused = 0;   // gdpa_bwd: 0 two kernels, 1 one KV-stationary pass, 2 one Q-stationary pass
    // the three lists of gdpa_list, and with stored dS (dq_team) a fourth: the dQ list
    // dealt again as 64-row items for the two-wave dQ-from-dS kernel (the dQ list
    // itself stays, for the kernels that recompute dS: JFA, the norm prologue)
    WorkList lists[kLists];
    bool dq_team = false;
    DevRec* d_items[kLists] = {};
    int32_t* d_bin_ptr[kLists] = {};
    // lists whose items the workgroups claim at run time: the claim order and the
    // (claims, finished workgroups) counters
    bool claimed[kLists] = {};
    int32_t* d_order[kLists] = {};
    int* d_claim[kLists] = {};
    // cut items of the Q-stationary lists: groups for the reduction, fp32 slots
    int n_groups[kLists] = {};
    DevGroup* d_groups[kLists] = {};
    float* d_part[kLists] = {};
    // pFFN plans: device copies of the offsets {0, Tq} and {0, M}
    int32_t* d_off = nullptr;
    // stored dS of the d = 128 two-kernel backward (see DsLayout)
    bool use_ds = false;
    DsLayout ds;
    __bf16* d_ds = nullptr;
    // the device records and chunk groups of each list, resolved on the host at
    // creation (bf16 plans; the upload and gdpa_fwd_noalloc copy them from here)
    std::vector<DevRec> h_recs[kLists];
    std::vector<DevGroup> h_groups[kLists];
    // pinned host copy of everything uploaded at creation (records, bin pointers,
    // chunk groups, pFFN offsets): the copies are enqueued on the creation stream
    // and read from here, so it lives as long as the plan
    char* h_stage = nullptr;
#ifdef GDPA_BIN_CLOCK
    unsigned long long* d_clock = nullptr;   // [max P][2], shared by every launch of the plan
    size_t n_clock = 0;
#endif
    bool pffn = false;

    ~gdpa_plan_s() {
        for (int l = 0; l < kLists; ++l) {
            if (d_items[l]) (void)hipFree(d_items[l]);
            if (d_bin_ptr[l]) (void)hipFree(d_bin_ptr[l]);
            if (d_order[l]) (void)hipFree(d_order[l]);
            if (d_claim[l]) (void)hipFree(d_claim[l]);
            if (d_groups[l]) (void)hipFree(d_groups[l]);
            if (d_part[l]) (void)hipFree(d_part[l]);
        }
        if (d_off) (void)hipFree(d_off);
        if (d_ds) (void)hipFree(d_ds);
        if (h_stage) (void)hipHostFree(h_stage);
#ifdef GDPA_BIN_CLOCK
        if (d_clock) (void)hipFree(d_clock);
#endif
    }
};

// Device work lists of a plan: allocate them (and the chunk slot buffers), stage
// the records, bin pointers and chunk groups in one pinned host buffer owned by
// the plan, and enqueue the copies on `s` (no synchronisation).
static gdpa_status upload(gdpa_plan_s* p, hipStream_t s) {
    const std::vector<DevRec>* recs = p->h_recs;
    const std::vector<DevGroup>* groups = p->h_groups;
    size_t bytes = 0;
    auto align = [](size_t n) { return (n + 255) & ~(size_t)255; };
    const int n_lists = p->dq_team ? kLists : 3;
    for (int l = 0; l < n_lists; ++l) {
        bytes += align(recs[l].size() * sizeof(DevRec)) + align(p->lists[l].bin_ptr.size() * sizeof(int32_t)) +
                 align(groups[l].size() * sizeof(DevGroup));
        if (p->claimed[l]) bytes += align(p->lists[l].order.size() * sizeof(int32_t)) + align(2 * sizeof(int));
    }
    const int32_t off[4] = {0, (int32_t)p->Tq, 0, (int32_t)p->Tk};
    if (p->pffn) bytes += align(sizeof(off));
    hipError_t e = hipHostMalloc((void**)&p->h_stage, std::max<size_t>(bytes, 256), hipHostMallocDefault);
    if (e != hipSuccess) {
        p->h_stage = nullptr;
        return e == hipErrorOutOfMemory ? fail(GDPA_ERR_NOMEM, "pinned staging buffer")
                                        : fail_hip(e, "pinned staging buffer");
    }
    char* h = p->h_stage;
    // copy n bytes of src into the staging buffer and enqueue them to *dst (allocated here)
    auto put = [&](void** dst, const void* src, size_t n) -> hipError_t {
        hipError_t r = hipMalloc(dst, std::max<size_t>(n, 1));
        if (r != hipSuccess || n == 0) return r;
        std::memcpy(h, src, n);
        r = hipMemcpyAsync(*dst, h, n, hipMemcpyHostToDevice, s);
        h += align(n);
        return r;
    };
    for (int l = 0; l < n_lists && e == hipSuccess; ++l) {
        const WorkList& wl = p->lists[l];
        e = put((void**)&p->d_items[l], recs[l].data(), recs[l].size() * sizeof(DevRec));
        if (e == hipSuccess) e = put((void**)&p->d_bin_ptr[l], wl.bin_ptr.data(), wl.bin_ptr.size() * sizeof(int32_t));
        if (e == hipSuccess && p->claimed[l]) {   // the claim order, and the counters at zero
            const int zero[2] = {0, 0};
            e = put((void**)&p->d_order[l], wl.order.data(), wl.order.size() * sizeof(int32_t));
            if (e == hipSuccess) e = put((void**)&p->d_claim[l], zero, sizeof(zero));
        }
        if (e == hipSuccess && wl.n_parts > 0) {
            p->n_groups[l] = (int)groups[l].size();
            e = put((void**)&p->d_groups[l], groups[l].data(), groups[l].size() * sizeof(DevGroup));
            // dK and dV blocks; the forward list also keeps two floats per slot row
            // (softmax chunks' row max and sum) after its blocks
            const size_t per_row = l == LIST_DKDV ? 2 * (size_t)p->d : l == LIST_FWD ? (size_t)p->d + 2 : (size_t)p->d;
            if (e == hipSuccess) e = hipMalloc((void**)&p->d_part[l], per_row * wl.n_parts * wl.t_stat * sizeof(float));
        }
    }
    if (e == hipSuccess && p->pffn) e = put((void**)&p->d_off, off, sizeof(off));
    if (e == hipSuccess && p->use_ds) {
        e = hipMalloc((void**)&p->d_ds, (size_t)p->ds.nb_total * p->H * 2048);
    }
    if (e != hipSuccess)
        return e == hipErrorOutOfMemory ? fail(GDPA_ERR_NOMEM, "work list upload") : fail_hip(e, "work list upload");
    return GDPA_OK;
}

extern "C" {

const char* gdpa_status_string(gdpa_status s) {
    switch (s) {
        case GDPA_OK: return "GDPA_OK";
        case GDPA_ERR_INVALID_ARG: return "GDPA_ERR_INVALID_ARG";
        case GDPA_ERR_BAD_OFFSETS: return "GDPA_ERR_BAD_OFFSETS";
        case GDPA_ERR_UNSUPPORTED: return "GDPA_ERR_UNSUPPORTED";
        case GDPA_ERR_PLAN_MISMATCH: return "GDPA_ERR_PLAN_MISMATCH";
        case GDPA_ERR_HIP: return "GDPA_ERR_HIP";
        case GDPA_ERR_NOMEM: return "GDPA_ERR_NOMEM";
    }
    return "GDPA_ERR_UNKNOWN";
}

const char* gdpa_last_error(void) { return g_err.c_str(); }

double gdpa_gelu_poly_bound(void) { return GDPA_GELU_POLY_BOUND; }
double gdpa_gelu_poly_grad_bound(void) { return GDPA_GELU_POLY_GRAD_BOUND; }

gdpa_status gdpa_plan_create(const int32_t* q_off_host, const int32_t* kv_off_host, int B, int H,
                             int d, int window, gdpa_dtype dtype, const gdpa_plan_opts* opts, void* stream,
                             gdpa_plan* out) {
    g_err.clear();
    return plan_create(q_off_host, kv_off_host, B, H, d, window, dtype, opts, (hipStream_t)stream, false, out);
}

}  // extern "C"

// gdpa_plan_create, and for pFFN plans (pffn) also device copies {0, Tq, 0, M} of the offsets
static gdpa_status plan_create(const int32_t* q_off_host, const int32_t* kv_off_host, int B, int H, int d,
                               int window, gdpa_dtype dtype, const gdpa_plan_opts* opts, hipStream_t stream,
                               bool pffn, gdpa_plan* out) {
    if (!out) return fail(GDPA_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (!q_off_host || !kv_off_host) return fail(GDPA_ERR_INVALID_ARG, "offsets are NULL");
    if (B < 0) return fail(GDPA_ERR_INVALID_ARG, "B < 0");
    if (H < 1 || H > 65535) return fail(GDPA_ERR_INVALID_ARG, "H out of range [1, 65535]");
    if (window < 0) return fail(GDPA_ERR_INVALID_ARG, "window < 0");
    if (dtype != GDPA_F32 && dtype != GDPA_BF16 && dtype != GDPA_BF16_F32OUT)
        return fail(GDPA_ERR_INVALID_ARG, "unknown dtype");
    if (d != 32 && d != 64 && d != 128) return fail(GDPA_ERR_UNSUPPORTED, "d must be 32, 64 or 128");
    gdpa_plan_opts o{};
    if (opts) o = *opts;
    for (int l = 0; l < 3; ++l) {
        if (o.bins[l] < 0) return fail(GDPA_ERR_INVALID_ARG, "bins < 0");
        if (o.blocks[l] < 0 || o.blocks[l] > 2) return fail(GDPA_ERR_INVALID_ARG, "blocks must be 0, 1 or 2");
        if (o.team[l] < 0 || o.team[l] > 2) return fail(GDPA_ERR_INVALID_ARG, "team must be 0, 1 or 2");
    }
    if (o.deal < 0 || o.deal > 2) return fail(GDPA_ERR_INVALID_ARG, "deal must be 0, 1 or 2");
    if (o.claim < 0 || o.claim > 2) return fail(GDPA_ERR_INVALID_ARG, "claim must be 0, 1 or 2");
    if (o.slot_time < 0 || o.slot_time > 1) return fail(GDPA_ERR_INVALID_ARG, "slot_time must be 0 or 1");
    if (o.dq_team < 0 || o.dq_team > 1) return fail(GDPA_ERR_INVALID_ARG, "dq_team must be 0 or 1");

    if (q_off_host[0] != 0 || kv_off_host[0] != 0)
        return fail(GDPA_ERR_BAD_OFFSETS, "offsets must start at 0");
    std::vector<int64_t> lq(B), lk(B);
    const int64_t elem_out = (dtype == GDPA_BF16) ? 2 : 4;
    for (int b = 0; b < B; ++b) {
        lq[b] = (int64_t)q_off_host[b + 1] - q_off_host[b];
        lk[b] = (int64_t)kv_off_host[b + 1] - kv_off_host[b];
        if (lq[b] < 0 || lk[b] < 0)
            return fail(GDPA_ERR_BAD_OFFSETS, "offsets decrease at sample " + std::to_string(b));
        if (window > 0 && lq[b] != lk[b])
            return fail(GDPA_ERR_BAD_OFFSETS, "a window needs Lq == Lk; sample " + std::to_string(b) + " differs");
        // every (sample, head) slice is addressed with 32-bit byte offsets
        if (std::max(lq[b], lk[b]) * (int64_t)H * d * elem_out >= (int64_t)1 << 31)
            return fail(GDPA_ERR_UNSUPPORTED, "sample " + std::to_string(b) + " exceeds 2 GiB per head slice");
    }

    gdpa_plan_s* p = new (std::nothrow) gdpa_plan_s;
    if (!p) return fail(GDPA_ERR_NOMEM, "plan allocation");
    p->B = B;
    p->H = H;
    p->d = d;
    p->window = window;
    p->dtype = dtype;
    p->host_only = o.host_only != 0;
    p->pffn = pffn;
    p->q_off.assign(q_off_host, q_off_host + B + 1);
    p->kv_off.assign(kv_off_host, kv_off_host + B + 1);
    p->lq = lq;
    p->lk = lk;
    p->Tq = q_off_host[B];
    p->Tk = kv_off_host[B];
    for (int b = 0; b < B; ++b) p->valid_pairs += pairs_of(lq[b], lk[b], window);

    Layout L = auto_layout(lq, lk, d);
    for (int l = 0; l < 3; ++l) {
        if (o.team[l]) L.team[l] = o.team[l];
        if (o.blocks[l]) L.nb[l] = o.blocks[l];
        // layouts with a kernel: teams of two only for d = 128 and with one block per
        // wave; dK/dV one block per wave
        const bool ok = (L.team[l] == 1 || (d == 128 && L.nb[l] == 1)) && (l != LIST_DKDV || L.nb[l] == 1);
        if (!ok) {
            delete p;
            return fail(GDPA_ERR_INVALID_ARG, "no kernel for team " + std::to_string(L.team[l]) + " x blocks " +
                                                  std::to_string(L.nb[l]) + " in list " + std::to_string(l) +
                                                  " at d = " + std::to_string(d));
        }
    }

    int cus = 256;
    if (!p->host_only) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) {
            delete p;
            return fail_hip(e, "device query");
        }
    }
    // one-pass backward: one side of every sample fits one 32-row tile, and no
    // sample has rows on that side only (their outputs would have no item)
    if (dtype != GDPA_F32 && o.unfused == 0) {
        bool kv_ok = L.team[LIST_DKDV] == 1 && L.nb[LIST_DKDV] == 1;
        bool q_ok = L.team[LIST_DQ] == 1 && L.nb[LIST_DQ] == 1;
        for (int b = 0; b < B; ++b) {
            kv_ok = kv_ok && lk[b] <= 32 && (lk[b] > 0 || lq[b] == 0);
            q_ok = q_ok && lq[b] <= 32 && (lq[b] > 0 || lk[b] == 0);
        }
        p->fused = kv_ok ? 1 : q_ok ? 2 : 0;
    }

    // stored dS: the two-kernel backward at d = 128 with 32- or 64-row dK/dV items and 32-row
    // dQ items
    if (dtype != GDPA_F32 && d == 128 && p->fused == 0 && o.no_ds == 0 && L.nb[LIST_DKDV] == 1 &&
        L.team[LIST_DQ] == 1 && L.nb[LIST_DQ] == 1) {
        p->ds = ds_layout(lq, lk, window);
        p->use_ds = p->ds.nb_total > 0 && p->ds.nb_total * (int64_t)H < ((int64_t)1 << 31);
    }

    for (int l = 0; l < 3; ++l) {
        // one bin per persistent workgroup (a team of waves): as many as the device
        // holds resident (host_only: 4 per CU)
        int P = o.bins[l];
        const bool auto_bins = P == 0;
        if (P == 0) {
            P = 4 * cus;
            if (!p->host_only && dtype != GDPA_F32) {
                const void* f = l == LIST_FWD ? fwd_kernel_ptr(d, L.team[l], L.nb[l], GDPA_ACT_GELU)
                              : l == LIST_DQ  ? (p->use_ds ? dq_from_ds_kernel_ptr()
                                                           : dq_kernel_ptr(d, L.team[l], L.nb[l], GDPA_ACT_GELU))
                                              : dkdv_kernel_ptr(d, L.team[l], L.nb[l], GDPA_ACT_GELU);
                // the d = 128 dK/dV list's 16-row kernel runs two waves per 32 team rows
                const bool k16 = l == LIST_DKDV && d == 128 && f && f == dkdv16_kernel_ptr(32 * L.team[l], GDPA_ACT_GELU);
                int per_cu = 0;
                if (f && hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, f, (k16 ? 128 : 64) * L.team[l], 0) == hipSuccess &&
                    per_cu > 0)
                    P = cus * per_cu;
            }
        }
        // the fp32 path runs no work lists; its plan keeps items whole
        const bool split = o.no_split == 0 && dtype != GDPA_F32;
        // dispatch-round factors: automatic bins only (the one-pass backward's kernels are not
        // in the table, so a fused backward's list takes none)
        const bool list_kernel = l == LIST_FWD || p->fused == 0;
        std::vector<double> bin_time;
        if (o.slot_time == 0 && auto_bins && dtype != GDPA_F32 && list_kernel)
            bin_time = round_time_factors(l, d, L.team[l], L.nb[l], P, cus);
        p->lists[l] = plan_list(l, lq, lk, H, window, P, L.team[l], L.nb[l], o.deal, split, bin_time);
    }

    // dQ from stored dS in two-wave teams (option dq_team, automatic): the dQ list dealt
    // again as 64-row items, one 32-row q tile per wave; the dQ list's bins when given,
    // else as many teams as the device holds resident (host_only: 4 per CU)
    if (p->use_ds && o.dq_team == 0) {
        int P = o.bins[LIST_DQ];
        const bool auto_bins = P == 0;
        if (P == 0) {
            P = 4 * cus;
            int per_cu = 0;
            if (!p->host_only &&
                hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, dq_from_ds_team_kernel_ptr(), 128, 0) ==
                    hipSuccess &&
                per_cu > 0)
                P = cus * per_cu;
        }
        const std::vector<double> bin_time =
            o.slot_time == 0 && auto_bins ? round_time_factors(LIST_DQ_TEAM, d, 2, 1, P, cus) : std::vector<double>();
        p->lists[LIST_DQ_TEAM] = plan_list(LIST_DQ, lq, lk, H, window, P, 2, 1, o.deal, o.no_split == 0, bin_time);
        p->dq_team = true;
    }

    // lists whose items are claimed at run time: those whose kernel walks them in one-wave
    // teams (not the d = 128 16-row dK/dV kernel, nor dQ from stored dS) and, by default,
    // whose items average 64 steps or more: a claim waits for every tile in flight, about
    // one memory latency at full load (several microseconds), which measured more than
    // the balance it buys on items of 10 to 30 steps
    for (int l = 0; l < 3 && dtype != GDPA_F32; ++l) {
        const WorkList& wl = p->lists[l];
        bool one_wave = L.team[l] == 1;
        if (l == LIST_DKDV && p->fused != 1 && d == 128) one_wave = false;
        if (l == LIST_DQ && p->fused != 2 && p->use_ds) one_wave = false;
        int64_t with_steps = 0;
        for (const Item& it : wl.items) with_steps += it.s1 >= it.s0;
        const bool long_items = with_steps > 0 && wl.n_steps >= 64 * with_steps;
        p->claimed[l] = o.claim != 1 && one_wave && !wl.items.empty() && (o.claim == 2 || long_items);
    }

    if (dtype != GDPA_F32) {
        for (int l = 0; l < (p->dq_team ? kLists : 3); ++l) {
            p->h_recs[l] = p->use_ds ? device_records(p->lists[l], p->q_off, p->kv_off, p->ds, window)
                                     : device_records(p->lists[l], p->q_off, p->kv_off);
            if (p->lists[l].n_parts > 0) p->h_groups[l] = device_groups(p->lists[l], p->q_off, p->kv_off);
        }
    }

    if (!p->host_only) {
        const gdpa_status st = upload(p, stream);
        if (st != GDPA_OK) {
            delete p;
            return st;
        }
#ifdef GDPA_BIN_CLOCK
        p->n_clock = 2 * (size_t)std::max(std::max(p->lists[0].P, p->lists[3].P), std::max(p->lists[1].P, p->lists[2].P));
        hipError_t e = hipMalloc((void**)&p->d_clock, p->n_clock * sizeof(unsigned long long));
        if (e == hipSuccess) e = hipMemset(p->d_clock, 0, p->n_clock * sizeof(unsigned long long));
        if (e != hipSuccess) {
            delete p;
            return fail_hip(e, "clock buffer");
        }
#endif
    }
    *out = p;
    return GDPA_OK;
}

extern "C" {

#ifdef GDPA_BIN_CLOCK
// Clock-probe builds only: copy the (start, end) stamps the last launch on this plan
// wrote per bin ([P][2], 100 MHz; 0 for bins without items) to `host` (n entries at
// most; *n is set to the buffer's size), then clear them.  The caller synchronises the
// stream first.
extern "C" gdpa_status gdpa_debug_bin_clock(gdpa_plan plan, unsigned long long* host, size_t* n) {
    g_err.clear();
    if (!plan || !host || !n) return fail(GDPA_ERR_INVALID_ARG, "plan, host or n is NULL");
    if (!plan->d_clock) return fail(GDPA_ERR_PLAN_MISMATCH, "host-only plan");
    const size_t m = std::min(*n, plan->n_clock);
    hipError_t e = hipMemcpy(host, plan->d_clock, m * sizeof(unsigned long long), hipMemcpyDeviceToHost);
    if (e == hipSuccess) e = hipMemset(plan->d_clock, 0, plan->n_clock * sizeof(unsigned long long));
    *n = plan->n_clock;
    return e == hipSuccess ? GDPA_OK : fail_hip(e, "clock readout");
}
#endif

void gdpa_plan_destroy(gdpa_plan plan) { delete plan; }

gdpa_status gdpa_plan_export(gdpa_plan plan, int list, int32_t* buf, size_t* n) {
    g_err.clear();
    if (!plan || !n) return fail(GDPA_ERR_INVALID_ARG, "plan or n is NULL");
    if (list < 0 || list > 3) return fail(GDPA_ERR_INVALID_ARG, "list must be 0, 1, 2 or 3");
    if (list == LIST_DQ_TEAM && !plan->dq_team)
        return fail(GDPA_ERR_INVALID_ARG, "list 3 (dQ from stored dS in two-wave teams) is not in this plan");
    const std::vector<int32_t> v = export_list(plan->lists[list]);
    if (!buf) {
        *n = v.size();
        return GDPA_OK;
    }
    if (*n < v.size()) {
        *n = v.size();
        return fail(GDPA_ERR_INVALID_ARG, "buffer too small");
    }
    std::memcpy(buf, v.data(), v.size() * sizeof(int32_t));
    *n = v.size();
    return GDPA_OK;
}

gdpa_status gdpa_plan_stats(gdpa_plan plan, gdpa_plan_stats_t* out) {
    g_err.clear();
    if (!plan || !out) return fail(GDPA_ERR_INVALID_ARG, "plan or out is NULL");
    std::memset(out, 0, sizeof(*out));
    out->Tq = plan->Tq;
    out->Tk = plan->Tk;
    out->valid_pairs = plan->valid_pairs;
    for (int l = 0; l < 3; ++l) {
        const WorkList& wl = plan->lists[l];
        out->n_items[l] = (int32_t)wl.items.size();
        out->n_steps[l] = (int32_t)wl.n_steps;
        out->bins[l] = wl.P;
        out->tile_stat[l] = wl.t_stat;
        out->tile_strm[l] = wl.t_strm;
        if (!wl.bin_cost.empty()) {
            out->bin_cost_max[l] = *std::max_element(wl.bin_cost.begin(), wl.bin_cost.end());
            out->bin_cost_min[l] = *std::min_element(wl.bin_cost.begin(), wl.bin_cost.end());
        }
    }
    out->bwd_fused = plan->fused;
    out->ds_bytes = plan->use_ds ? plan->ds.nb_total * plan->H * 2048 : 0;
    for (int l = 0; l < 3; ++l) {
        out->n_parts[l] = plan->lists[l].n_parts;
        out->claimed[l] = plan->claimed[l] ? 1 : 0;
        out->slot_weighted[l] = plan->lists[l].weighted ? 1 : 0;
    }
    out->dq_team = plan->use_ds ? (plan->dq_team ? 2 : 1) : 0;
    if (plan->dq_team) {
        const WorkList& wl = plan->lists[LIST_DQ_TEAM];
        out->dq_team_items = (int32_t)wl.items.size();
        out->dq_team_bins = wl.P;
        out->dq_team_parts = wl.n_parts;
        out->dq_team_slot_weighted = wl.weighted ? 1 : 0;
    }
    return GDPA_OK;
}

// RMSNorm prologue: eps under the root
constexpr float kRmsEps = 1e-6f;

// GDPA_DEBUG: the device offsets must equal the plan's (copied to the host and compared)
static gdpa_status check_offsets(gdpa_plan plan, const int32_t* q_off_dev, const int32_t* kv_off_dev) {
    const int B = plan->B;
    std::vector<int32_t> hq(B + 1), hk(B + 1);
    hipError_t e = hipMemcpy(hq.data(), q_off_dev, (B + 1) * sizeof(int32_t), hipMemcpyDeviceToHost);
    if (e == hipSuccess) e = hipMemcpy(hk.data(), kv_off_dev, (B + 1) * sizeof(int32_t), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return fail_hip(e, "GDPA_DEBUG offset check");
    if (hq != plan->q_off || hk != plan->kv_off)
        return fail(GDPA_ERR_PLAN_MISMATCH, "device offsets differ from the plan's");
    return GDPA_OK;
}

static gdpa_status check_call(gdpa_plan plan, const int32_t* q_off_dev, const int32_t* kv_off_dev, int B,
                              int H, int d, gdpa_act act, int window) {
    if (!plan) return fail(GDPA_ERR_INVALID_ARG, "plan is NULL");
    if (plan->host_only) return fail(GDPA_ERR_PLAN_MISMATCH, "host-only plan cannot run kernels");
    if (B != plan->B || H != plan->H || d != plan->d || window != plan->window)
        return fail(GDPA_ERR_PLAN_MISMATCH, "B, H, d or window differ from the plan");
    if ((int)act < 0 || (int)act > GDPA_ACT_ONE) return fail(GDPA_ERR_INVALID_ARG, "unknown activation");
    if (!q_off_dev || !kv_off_dev) return fail(GDPA_ERR_INVALID_ARG, "device offsets are NULL");
    if (debug_enabled()) return check_offsets(plan, q_off_dev, kv_off_dev);
    return GDPA_OK;
}

static KernelArgs base_args(gdpa_plan plan, const int32_t* q_off_dev, const int32_t* kv_off_dev) {
    KernelArgs a{};
    a.q_off = q_off_dev;
    a.kv_off = kv_off_dev;
    a.B = plan->B;
    a.H = plan->H;
    a.window = plan->window;
    a.scale = 1.0f / std::sqrt((float)plan->d);
    a.out_f32 = plan->dtype != GDPA_BF16;
#ifdef GDPA_BIN_CLOCK
    a.bin_clock = plan->d_clock;
#endif
    return a;
}

// claims of list l for a kernel launched over it (none where the plan does not claim
// that list's items)
static void set_claims(KernelArgs& b, gdpa_plan plan, int l) {
    const bool c = plan->claimed[l];
    b.order = c ? plan->d_order[l] : nullptr;
    b.claim = c ? plan->d_claim[l] : nullptr;
    b.n_items = c ? (int)plan->lists[l].items.size() : 0;
}

// outputs of the cut items of list l: the sum of their chunks' slots, times mul
// (the dK/dV list keeps two blocks per slot: block 0 dK, block 1 dV)
static hipError_t reduce_parts(gdpa_plan plan, int l, float mul, void* out, hipStream_t s, int block = 0) {
    if (plan->n_groups[l] == 0) return hipSuccess;
    return launch_partial_sum(plan->d_groups[l], plan->n_groups[l], plan->d_part[l], plan->lists[l].t_stat,
                              l == LIST_DKDV ? 2 : 1, block, plan->d, plan->H, mul, out,
                              plan->dtype != GDPA_BF16, s);
}

gdpa_status gdpa_fwd(gdpa_plan plan, const void* q, const void* k, const void* v,
                     const int32_t* q_off_dev, const int32_t* kv_off_dev, int B, int H, int d,
                     gdpa_act act, int window, void* o, void* stream) {
    g_err.clear();
    gdpa_status st = check_call(plan, q_off_dev, kv_off_dev, B, H, d, act, window);
    if (st != GDPA_OK) return st;
    if (plan->Tq > 0 && (!q || !o)) return fail(GDPA_ERR_INVALID_ARG, "q or o is NULL");
    if (plan->Tk > 0 && (!k || !v)) return fail(GDPA_ERR_INVALID_ARG, "k or v is NULL");
    if (plan->Tq == 0) return GDPA_OK;
    hipStream_t s = (hipStream_t)stream;
    KernelArgs a = base_args(plan, q_off_dev, kv_off_dev);
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    hipError_t e;
    if (plan->dtype == GDPA_F32) {
        e = launch_fwd_f32(a, (int)plan->Tq, d, act, s);
    } else {
        const WorkList& wl = plan->lists[LIST_FWD];
        a.items = plan->d_items[LIST_FWD];
        a.bin_ptr = plan->d_bin_ptr[LIST_FWD];
        set_claims(a, plan, LIST_FWD);
        a.P = wl.P;
        a.part = plan->d_part[LIST_FWD];
        switch (d) {
            case 32: e = launch_fwd_bf16_d32(a, wl.team, wl.nb, act, s); break;
            case 64: e = launch_fwd_bf16_d64(a, wl.team, wl.nb, act, s); break;
            default: e = launch_fwd_bf16_d128(a, wl.team, wl.nb, act, s); break;
        }
        if (e == hipSuccess) e = reduce_parts(plan, LIST_FWD, 1.0f, o, s);
    }
    if (e == hipErrorInvalidValue) return fail(GDPA_ERR_UNSUPPORTED, "no forward kernel for this configuration");
    if (e != hipSuccess) return fail_hip(e, "forward launch");
    return GDPA_OK;
}

gdpa_status gdpa_fwd_noalloc(gdpa_plan plan, const void* q, const void* k, const void* v,
                             const int32_t* q_off_dev, const int32_t* kv_off_dev, int B, int H, int d,
                             gdpa_act act, int window, void* o, void* stream) {
    g_err.clear();
    if (!plan) return fail(GDPA_ERR_INVALID_ARG, "plan is NULL");
    if (B != plan->B || H != plan->H || d != plan->d || window != plan->window)
        return fail(GDPA_ERR_PLAN_MISMATCH, "B, H, d or window differ from the plan");
    if ((int)act < 0 || (int)act > GDPA_ACT_ONE) return fail(GDPA_ERR_INVALID_ARG, "unknown activation");
    if (plan->dtype == GDPA_F32) return fail(GDPA_ERR_UNSUPPORTED, "the no-allocation forward runs bf16 plans");
    if (!q_off_dev || !kv_off_dev) return fail(GDPA_ERR_INVALID_ARG, "device offsets are NULL");
    if (plan->Tq > 0 && (!q || !o)) return fail(GDPA_ERR_INVALID_ARG, "q or o is NULL");
    if (plan->Tk > 0 && (!k || !v)) return fail(GDPA_ERR_INVALID_ARG, "k or v is NULL");
    if (plan->Tq == 0) return GDPA_OK;
    // the scratch layout: records, bin pointers, chunk groups, chunk slots (fp32
    // t_stat x (d + 2) per slot, as the plan's own slot buffer), each 256-byte aligned
    const WorkList& wl = plan->lists[LIST_FWD];
    const std::vector<DevRec>& recs = plan->h_recs[LIST_FWD];
    const std::vector<DevGroup>& groups = plan->h_groups[LIST_FWD];
    auto align = [](size_t n) { return (n + 255) & ~(size_t)255; };
    const size_t b_recs = recs.size() * sizeof(DevRec), b_ptr = wl.bin_ptr.size() * sizeof(int32_t);
    const size_t b_groups = groups.size() * sizeof(DevGroup);
    const size_t b_slots = (size_t)wl.n_parts * wl.t_stat * ((size_t)d + 2) * sizeof(float);
    const size_t o_ptr = align(b_recs), o_groups = o_ptr + align(b_ptr), o_slots = o_groups + align(b_groups);
    const size_t need = o_slots + b_slots;
    if (need > kNoallocScratchBytes)
        return fail(GDPA_ERR_INVALID_ARG, "the plan's forward work list needs " + std::to_string(need) +
                                              " bytes of scratch; the no-allocation forward has " +
                                              std::to_string(kNoallocScratchBytes));
    if (debug_enabled()) {
        const gdpa_status st = check_offsets(plan, q_off_dev, kv_off_dev);
        if (st != GDPA_OK) return st;
    }
    void* base = nullptr;
    hipError_t e = noalloc_scratch(&base);
    if (e != hipSuccess) return fail_hip(e, "scratch address");
    char* sc = (char*)base;
    hipStream_t s = (hipStream_t)stream;
    // the work list comes from the plan's host memory, which lives until the plan is destroyed
    if (b_recs) e = hipMemcpyAsync(sc, recs.data(), b_recs, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipMemcpyAsync(sc + o_ptr, wl.bin_ptr.data(), b_ptr, hipMemcpyHostToDevice, s);
    if (e == hipSuccess && b_groups) e = hipMemcpyAsync(sc + o_groups, groups.data(), b_groups, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return fail_hip(e, "work list copy into scratch");
    KernelArgs a = base_args(plan, q_off_dev, kv_off_dev);
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.items = sc;
    a.bin_ptr = (const int32_t*)(sc + o_ptr);
    a.P = wl.P;
    a.part = wl.n_parts > 0 ? (float*)(sc + o_slots) : nullptr;
    switch (d) {
        case 32: e = launch_fwd_bf16_d32(a, wl.team, wl.nb, act, s); break;
        case 64: e = launch_fwd_bf16_d64(a, wl.team, wl.nb, act, s); break;
        default: e = launch_fwd_bf16_d128(a, wl.team, wl.nb, act, s); break;
    }
    if (e == hipSuccess && !groups.empty())
        e = launch_partial_sum((const DevGroup*)(sc + o_groups), (int)groups.size(), a.part, wl.t_stat, 1, 0, d, H,
                               1.0f, o, plan->dtype != GDPA_BF16, s);
    if (e == hipErrorInvalidValue) return fail(GDPA_ERR_UNSUPPORTED, "no forward kernel for this configuration");
    if (e != hipSuccess) return fail_hip(e, "forward launch");
    return GDPA_OK;
}

// per-tensor factors of the fp8 backward's inputs (value = e4m3 byte's value * factor)
struct F8Factors {
    float q, k, dout;
};

static gdpa_status bwd_parts(gdpa_plan plan, const void* q, const void* k, const void* v, const void* dout,
                             const int32_t* q_off_dev, const int32_t* kv_off_dev, int B, int H, int d,
                             gdpa_act act, int window, void* dq, void* dk, void* dv, void* stream,
                             bool want_dkdv, bool want_dq, const F8Factors* f8 = nullptr) {
    g_err.clear();
    gdpa_status st = check_call(plan, q_off_dev, kv_off_dev, B, H, d, act, window);
    if (st != GDPA_OK) return st;
    if (act == GDPA_ACT_ONE) return fail(GDPA_ERR_UNSUPPORTED, "GDPA_ACT_ONE has no backward");
    if (f8) {
        if (plan->dtype == GDPA_F32) return fail(GDPA_ERR_UNSUPPORTED, "fp8 inputs run on bf16 plans");
        for (float x : {f8->q, f8->k, f8->dout})
            if (!(x > 0.0f) || !std::isfinite(x))
                return fail(GDPA_ERR_INVALID_ARG, "q_scale, k_scale and do_scale must be finite and > 0");
        if (!plan->fused && !plan->use_ds)
            return fail(GDPA_ERR_UNSUPPORTED,
                        "the fp8 backward runs on plans whose backward is one pass (every Lk <= 32 or every "
                        "Lq <= 32) or the d = 128 stored-dS kernels (gdpa_plan_stats: bwd_fused, ds_bytes)");
    }
    const bool any_q = plan->Tq > 0, any_k = plan->Tk > 0;
    if (any_q && (!q || !dout)) return fail(GDPA_ERR_INVALID_ARG, "q or dout is NULL");
    if (any_k && (!k || !v)) return fail(GDPA_ERR_INVALID_ARG, "k or v is NULL");
    if (want_dq && any_q && !dq) return fail(GDPA_ERR_INVALID_ARG, "dq is NULL");
    if (want_dkdv && any_k && (!dk || !dv)) return fail(GDPA_ERR_INVALID_ARG, "dk or dv is NULL");
    hipStream_t s = (hipStream_t)stream;
    KernelArgs a = base_args(plan, q_off_dev, kv_off_dev);
    a.q = q;
    a.k = k;
    a.v = v;
    a.dout = dout;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    // output factors of dQ, dK, dV (the fp8 inputs' factors folded in)
    float mq = a.scale, mk = a.scale, mv = 1.0f;
    int code = (int)act;
    if (f8) {
        mq = a.scale * f8->k;          // dQ = (dS k8) s_k / sqrt(d)
        mk = a.scale * f8->q;          // dK = (dS^T q8) s_q / sqrt(d)
        mv = f8->dout;                 // dV = (P^T do8) s_do
        a.f8_dp = f8->dout;            // dP = (do8 v^T) s_do
        a.f8_dq = mq;
        a.f8_dk = mk;
        a.f8_dv = mv;
        a.scale *= f8->q * f8->k;      // S = (q8 k8^T) s_q s_k / sqrt(d)
        code |= kActF8Bwd;
    }
    hipError_t e = hipSuccess;
    if (plan->dtype == GDPA_F32) {
        e = launch_bwd_f32(a, want_dq ? (int)plan->Tq : 0, want_dkdv ? (int)plan->Tk : 0, d, act, s);
    } else if (plan->fused && want_dkdv && want_dq) {
        const int l = plan->fused == 1 ? LIST_DKDV : LIST_DQ;
        KernelArgs b = a;
        b.items = plan->d_items[l];
        b.bin_ptr = plan->d_bin_ptr[l];
        set_claims(b, plan, l);
        b.P = plan->lists[l].P;
        const int kv = plan->fused == 1;
        b.part = plan->d_part[l];
        switch (d) {
            case 32: e = launch_bwd_fused_d32(b, kv, code, s); break;
            case 64: e = launch_bwd_fused_d64(b, kv, code, s); break;
            default: e = launch_bwd_fused_d128(b, kv, code, s); break;
        }
        if (e == hipSuccess && !kv) e = reduce_parts(plan, LIST_DQ, mq, dq, s);
        if (e == hipSuccess && kv) e = reduce_parts(plan, LIST_DKDV, mk, dk, s, 0);
        if (e == hipSuccess && kv) e = reduce_parts(plan, LIST_DKDV, mv, dv, s, 1);
    } else if (plan->use_ds) {
        // dK/dV storing dS, then dQ = dS K / sqrt(d) from the stored blocks (the two
        // halves separately: gdpa_bwd_dq reads what gdpa_bwd_dkdv stored)
        if (want_dkdv && any_k) {
            const WorkList& wl = plan->lists[LIST_DKDV];
            KernelArgs b = a;
            b.items = plan->d_items[LIST_DKDV];
            b.bin_ptr = plan->d_bin_ptr[LIST_DKDV];
            set_claims(b, plan, LIST_DKDV);
            b.P = wl.P;
            b.part = plan->d_part[LIST_DKDV];
            b.ds = plan->d_ds;
            e = launch_dkdv_bf16_d128(b, wl.team, wl.nb, code, s);
            if (e == hipSuccess) e = reduce_parts(plan, LIST_DKDV, mk, dk, s, 0);
            if (e == hipSuccess) e = reduce_parts(plan, LIST_DKDV, mv, dv, s, 1);
        }
        if (e == hipSuccess && want_dq && any_q) {
            const int l = plan->dq_team ? LIST_DQ_TEAM : LIST_DQ;
            KernelArgs b = a;
            b.items = plan->d_items[l];
            b.bin_ptr = plan->d_bin_ptr[l];
            set_claims(b, plan, l);
            b.P = plan->lists[l].P;
            b.part = plan->d_part[l];
            b.ds = plan->d_ds;
            e = plan->dq_team ? launch_dq_from_ds_team(b, f8 != nullptr, s) : launch_dq_from_ds(b, f8 != nullptr, s);
            if (e == hipSuccess) e = reduce_parts(plan, l, mq, dq, s);
        }
    } else {
        if (want_dkdv && any_k) {
            const WorkList& wl = plan->lists[LIST_DKDV];
            KernelArgs b = a;
            b.items = plan->d_items[LIST_DKDV];
            b.bin_ptr = plan->d_bin_ptr[LIST_DKDV];
            set_claims(b, plan, LIST_DKDV);
            b.P = wl.P;
            b.part = plan->d_part[LIST_DKDV];
            switch (d) {
                case 32: e = launch_dkdv_bf16_d32(b, wl.team, wl.nb, act, s); break;
                case 64: e = launch_dkdv_bf16_d64(b, wl.team, wl.nb, act, s); break;
                default: e = launch_dkdv_bf16_d128(b, wl.team, wl.nb, act, s); break;
            }
            if (e == hipSuccess) e = reduce_parts(plan, LIST_DKDV, a.scale, dk, s, 0);
            if (e == hipSuccess) e = reduce_parts(plan, LIST_DKDV, 1.0f, dv, s, 1);
        }
        if (e == hipSuccess && want_dq && any_q) {
            const WorkList& wl = plan->lists[LIST_DQ];
            KernelArgs b = a;
            b.items = plan->d_items[LIST_DQ];
            b.bin_ptr = plan->d_bin_ptr[LIST_DQ];
            set_claims(b, plan, LIST_DQ);
            b.P = wl.P;
            b.part = plan->d_part[LIST_DQ];
            switch (d) {
                case 32: e = launch_dq_bf16_d32(b, wl.team, wl.nb, act, s); break;
                case 64: e = launch_dq_bf16_d64(b, wl.team, wl.nb, act, s); break;
                default: e = launch_dq_bf16_d128(b, wl.team, wl.nb, act, s); break;
            }
            if (e == hipSuccess) e = reduce_parts(plan, LIST_DQ, a.scale, dq, s);
        }
    }
    if (e == hipErrorInvalidValue) return fail(GDPA_ERR_UNSUPPORTED, "no backward kernel for this configuration");
    if (e != hipSuccess) return fail_hip(e, "backward launch");
    return GDPA_OK;
}

gdpa_status gdpa_bwd(gdpa_plan plan, const void* q, const void* k, const void* v, const void* dout,
                     const int32_t* q_off_dev, const int32_t* kv_off_dev, int B, int H, int d,
                     gdpa_act act, int window, void* dq, void* dk, void* dv, void* stream) {
    return bwd_parts(plan, q, k, v, dout, q_off_dev, kv_off_dev, B, H, d, act, window, dq, dk, dv, stream,
                     true, true);
}

gdpa_status gdpa_fp8_bwd(gdpa_plan plan, const void* q8, const void* k8, const void* v, const void* do8,
                         const int32_t* q_off_dev, const int32_t* kv_off_dev, int B, int H, int d, gdpa_act act,
                         int window, float q_scale, float k_scale, float do_scale, void* dq, void* dk, void* dv,
                         void* stream) {
    const F8Factors f8{q_scale, k_scale, do_scale};
    return bwd_parts(plan, q8, k8, v, do8, q_off_dev, kv_off_dev, B, H, d, act, window, dq, dk, dv, stream, true,
                     true, &f8);
}

gdpa_status gdpa_bwd_dkdv(gdpa_plan plan, const void* q, const void* k, const void* v, const void* dout,
                          const int32_t* q_off_dev, const int32_t* kv_off_dev, int B, int H, int d,
                          gdpa_act act, int window, void* dk, void* dv, void* stream) {
    return bwd_parts(plan, q, k, v, dout, q_off_dev, kv_off_dev, B, H, d, act, window, nullptr, dk, dv, stream,
                     true, false);
}

gdpa_status gdpa_bwd_dq(gdpa_plan plan, const void* q, const void* k, const void* v, const void* dout,
                        const int32_t* q_off_dev, const int32_t* kv_off_dev, int B, int H, int d,
                        gdpa_act act, int window, void* dq, void* stream) {
    return bwd_parts(plan, q, k, v, dout, q_off_dev, kv_off_dev, B, H, d, act, window, dq, nullptr, nullptr,
                     stream, false, true);
}

gdpa_status gdpa_jfa_fwd(gdpa_plan plan, const void* q, const void* k, const void* v, const int32_t* q_off_dev,
                         const int32_t* kv_off_dev, int B, int H, int d, int window, void* o, float* lse,
                         void* stream) {
    g_err.clear();
    gdpa_status st = check_call(plan, q_off_dev, kv_off_dev, B, H, d, GDPA_ACT_GELU, window);
    if (st != GDPA_OK) return st;
    if (plan->dtype == GDPA_F32) return fail(GDPA_ERR_UNSUPPORTED, "JFA runs on bf16 plans");
    if (plan->Tq > 0 && (!q || !o || !lse)) return fail(GDPA_ERR_INVALID_ARG, "q, o or lse is NULL");
    if (plan->Tk > 0 && (!k || !v)) return fail(GDPA_ERR_INVALID_ARG, "k or v is NULL");
    if (plan->Tq == 0) return GDPA_OK;
    hipStream_t s = (hipStream_t)stream;
    KernelArgs a = base_args(plan, q_off_dev, kv_off_dev);
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.Tq = (int)plan->Tq;
    const WorkList& wl = plan->lists[LIST_FWD];
    a.items = plan->d_items[LIST_FWD];
    a.bin_ptr = plan->d_bin_ptr[LIST_FWD];
    set_claims(a, plan, LIST_FWD);
    a.P = wl.P;
    a.part = plan->d_part[LIST_FWD];
    a.part_stat = a.part ? a.part + (size_t)wl.n_parts * wl.t_stat * d : nullptr;
    hipError_t e;
    switch (d) {
        case 32: e = launch_fwd_bf16_d32(a, wl.team, wl.nb, kActSoftmax, s); break;
        case 64: e = launch_fwd_bf16_d64(a, wl.team, wl.nb, kActSoftmax, s); break;
        default: e = launch_fwd_bf16_d128(a, wl.team, wl.nb, kActSoftmax, s); break;
    }
    if (e == hipSuccess && plan->n_groups[LIST_FWD] > 0)
        e = launch_jfa_combine(plan->d_groups[LIST_FWD], plan->n_groups[LIST_FWD], a.part, a.part_stat, wl.t_stat,
                               d, H, (int)plan->Tq, o, plan->dtype != GDPA_BF16, lse, s);
    if (e == hipErrorInvalidValue) return fail(GDPA_ERR_UNSUPPORTED, "no forward kernel for this configuration");
    if (e != hipSuccess) return fail_hip(e, "JFA forward launch");
    return GDPA_OK;
}

// the JFA backward's row statistics: stat[h, i] = (LSE log2 e, sum dO * O)
static gdpa_status jfa_stat(gdpa_plan plan, const void* o, const float* lse, const void* dout, float* stat,
                            hipStream_t s) {
    if (plan->Tq == 0) return GDPA_OK;
    if (!o || !lse || !dout || !stat) return fail(GDPA_ERR_INVALID_ARG, "o, lse, dout or stat is NULL");
    const hipError_t e = launch_jfa_stat(o, dout, lse, (int)plan->Tq, plan->H, plan->d, stat, s);
    if (e != hipSuccess) return fail_hip(e, "JFA row-statistics launch");
    return GDPA_OK;
}

static gdpa_status jfa_check(gdpa_plan plan) {
    // the backward reads the forward's O as bf16: a BF16_F32OUT plan's forward writes fp32
    if (plan->dtype != GDPA_BF16) return fail(GDPA_ERR_UNSUPPORTED, "the JFA backward runs on GDPA_BF16 plans");
    if (plan->lists[LIST_DQ].team != 1 || plan->lists[LIST_DKDV].team != 1)
        return fail(GDPA_ERR_UNSUPPORTED, "the JFA backward runs one-wave dQ and dK/dV teams");
    return GDPA_OK;
}

// the JFA backward's gradient kernels: the dQ kernel (reads o and lse, writes stat),
// then the dK/dV kernel (reads stat); or, for both where every Lk <= 32, the one
// KV-stationary pass (reads lse)
static gdpa_status jfa_grads(gdpa_plan plan, const void* q, const void* k, const void* v, const void* o,
                             const float* lse, const void* dout, const int32_t* q_off_dev, const int32_t* kv_off_dev,
                             float* stat, void* dq, void* dk, void* dv, hipStream_t s, bool want_dkdv, bool want_dq) {
    const bool any_q = plan->Tq > 0, any_k = plan->Tk > 0;
    // both gradients where every Lk <= 32: one KV-stationary pass (reads neither o nor stat)
    const bool one_pass = want_dq && want_dkdv && plan->fused == 1;
    if (any_q && (!q || !dout || (!stat && !one_pass))) return fail(GDPA_ERR_INVALID_ARG, "q, dout or stat is NULL");
    if (any_k && (!k || !v)) return fail(GDPA_ERR_INVALID_ARG, "k or v is NULL");
    if (want_dq && any_q && (!dq || !lse || (!o && !one_pass)))
        return fail(GDPA_ERR_INVALID_ARG, "dq, o or lse is NULL");
    if (want_dkdv && any_k && (!dk || !dv)) return fail(GDPA_ERR_INVALID_ARG, "dk or dv is NULL");
    KernelArgs a = base_args(plan, q_off_dev, kv_off_dev);
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = const_cast<void*>(o);   // read only: the forward's output
    a.lse = const_cast<float*>(lse);
    a.dout = dout;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.stat = stat;
    a.Tq = (int)plan->Tq;
    const int d = plan->d;
    hipError_t e = hipSuccess;
    if (one_pass) {
        // every Lk <= 32: one KV-stationary pass, which forms D from P and dP itself
        // (stat is not written).  (A Q-stationary pass for every Lq <= 32 would need D
        // before its first step, from O as a third stationary tile; on the PMA batch it
        // measured slower than the two kernels, 958 against 708 us.)
        const WorkList& wl = plan->lists[LIST_DKDV];
        KernelArgs b = a;
        b.items = plan->d_items[LIST_DKDV];
        b.bin_ptr = plan->d_bin_ptr[LIST_DKDV];
        set_claims(b, plan, LIST_DKDV);
        b.P = wl.P;
        b.part = plan->d_part[LIST_DKDV];
        switch (d) {
            case 32: e = launch_bwd_fused_d32(b, 1, kActSoftmax, s); break;
            case 64: e = launch_bwd_fused_d64(b, 1, kActSoftmax, s); break;
            default: e = launch_bwd_fused_d128(b, 1, kActSoftmax, s); break;
        }
        if (e == hipSuccess) e = reduce_parts(plan, LIST_DKDV, a.scale, dk, s, 0);
        if (e == hipSuccess) e = reduce_parts(plan, LIST_DKDV, 1.0f, dv, s, 1);
        if (e == hipErrorInvalidValue) return fail(GDPA_ERR_UNSUPPORTED, "no JFA backward kernel for this configuration");
        if (e != hipSuccess) return fail_hip(e, "JFA backward launch");
        return GDPA_OK;
    }
    if (want_dq && any_q) {
        const WorkList& wl = plan->lists[LIST_DQ];
        KernelArgs b = a;
        b.items = plan->d_items[LIST_DQ];
        b.bin_ptr = plan->d_bin_ptr[LIST_DQ];
        set_claims(b, plan, LIST_DQ);
        b.P = wl.P;
        b.part = plan->d_part[LIST_DQ];
        switch (d) {
            case 32: e = launch_dq_bf16_d32(b, wl.team, wl.nb, kActSoftmax, s); break;
            case 64: e = launch_dq_bf16_d64(b, wl.team, wl.nb, kActSoftmax, s); break;
            default: e = launch_dq_bf16_d128(b, wl.team, wl.nb, kActSoftmax, s); break;
        }
        if (e == hipSuccess) e = reduce_parts(plan, LIST_DQ, a.scale, dq, s);
    }
    if (e == hipSuccess && want_dkdv && any_k) {
        const WorkList& wl = plan->lists[LIST_DKDV];
        KernelArgs b = a;
        b.items = plan->d_items[LIST_DKDV];
        b.bin_ptr = plan->d_bin_ptr[LIST_DKDV];
        set_claims(b, plan, LIST_DKDV);
        b.P = wl.P;
        b.part = plan->d_part[LIST_DKDV];
        switch (d) {
            case 32: e = launch_dkdv_bf16_d32(b, wl.team, wl.nb, kActSoftmax, s); break;
            case 64: e = launch_dkdv_bf16_d64(b, wl.team, wl.nb, kActSoftmax, s); break;
            default: e = launch_dkdv_bf16_d128(b, wl.team, wl.nb, kActSoftmax, s); break;
        }
        if (e == hipSuccess) e = reduce_parts(plan, LIST_DKDV, a.scale, dk, s, 0);
        if (e == hipSuccess) e = reduce_parts(plan, LIST_DKDV, 1.0f, dv, s, 1);
    }
    if (e == hipErrorInvalidValue) return fail(GDPA_ERR_UNSUPPORTED, "no JFA backward kernel for this configuration");
    if (e != hipSuccess) return fail_hip(e, "JFA backward launch");
    return GDPA_OK;
}

gdpa_status gdpa_jfa_bwd(gdpa_plan plan, const void* q, const void* k, const void* v, const void* o,
                         const float* lse, const void* dout, const int32_t* q_off_dev, const int32_t* kv_off_dev,
                         int B, int H, int d, int window, float* stat, void* dq, void* dk, void* dv, void* stream) {
    g_err.clear();
    gdpa_status st = check_call(plan, q_off_dev, kv_off_dev, B, H, d, GDPA_ACT_GELU, window);
    if (st == GDPA_OK) st = jfa_check(plan);
    if (st != GDPA_OK) return st;
    return jfa_grads(plan, q, k, v, o, lse, dout, q_off_dev, kv_off_dev, stat, dq, dk, dv, (hipStream_t)stream, true,
                     true);
}

gdpa_status gdpa_jfa_bwd_stat(gdpa_plan plan, const void* o, const float* lse, const void* dout, int H, int d,
                              float* stat, void* stream) {
    g_err.clear();
    if (!plan) return fail(GDPA_ERR_INVALID_ARG, "plan is NULL");
    if (plan->host_only) return fail(GDPA_ERR_PLAN_MISMATCH, "host-only plan cannot run kernels");
    if (H != plan->H || d != plan->d) return fail(GDPA_ERR_PLAN_MISMATCH, "H or d differ from the plan");
    const gdpa_status st = jfa_check(plan);
    if (st != GDPA_OK) return st;
    return jfa_stat(plan, o, lse, dout, stat, (hipStream_t)stream);
}

gdpa_status gdpa_jfa_bwd_dkdv(gdpa_plan plan, const void* q, const void* k, const void* v, const void* dout,
                              const int32_t* q_off_dev, const int32_t* kv_off_dev, int B, int H, int d, int window,
                              const float* stat, void* dk, void* dv, void* stream) {
    g_err.clear();
    gdpa_status st = check_call(plan, q_off_dev, kv_off_dev, B, H, d, GDPA_ACT_GELU, window);
    if (st == GDPA_OK) st = jfa_check(plan);
    if (st != GDPA_OK) return st;
    return jfa_grads(plan, q, k, v, nullptr, nullptr, dout, q_off_dev, kv_off_dev, const_cast<float*>(stat), nullptr,
                     dk, dv, (hipStream_t)stream, true, false);
}

gdpa_status gdpa_jfa_bwd_dq(gdpa_plan plan, const void* q, const void* k, const void* v, const void* o,
                            const float* lse, const void* dout, const int32_t* q_off_dev, const int32_t* kv_off_dev,
                            int B, int H, int d, int window, float* stat, void* dq, void* stream) {
    g_err.clear();
    gdpa_status st = check_call(plan, q_off_dev, kv_off_dev, B, H, d, GDPA_ACT_GELU, window);
    if (st == GDPA_OK) st = jfa_check(plan);
    if (st != GDPA_OK) return st;
    return jfa_grads(plan, q, k, v, o, lse, dout, q_off_dev, kv_off_dev, stat, dq, nullptr, nullptr,
                     (hipStream_t)stream, false, true);
}

// the RMSNorm prologue's checks and its factor arrays inside `rstd`
static gdpa_status norm_check(gdpa_plan plan, gdpa_act act, int norm, const float* rstd) {
    if (plan->dtype == GDPA_F32) return fail(GDPA_ERR_UNSUPPORTED, "the RMSNorm prologue runs on bf16 plans");
    if (act == GDPA_ACT_ONE) return fail(GDPA_ERR_UNSUPPORTED, "GDPA_ACT_ONE has no RMSNorm-prologue kernels");
    if (norm < 0 || norm > 7) return fail(GDPA_ERR_INVALID_ARG, "norm must be a combination of 1 (Q), 2 (K), 4 (V)");
    if ((plan->Tq > 0 || plan->Tk > 0) && !rstd) return fail(GDPA_ERR_INVALID_ARG, "rstd is NULL");
    return GDPA_OK;
}

static void norm_args(gdpa_plan plan, int norm, const float* rstd, KernelArgs& a) {
    a.rq = rstd;
    a.rkv = rstd ? rstd + (size_t)plan->H * plan->Tq : nullptr;
    a.Tq = (int)plan->Tq;
    a.Tk = (int)plan->Tk;
    a.norm = norm;
}

gdpa_status gdpa_norm_rstd(gdpa_plan plan, const void* q, const void* k, const void* v, int H, int d, int norm,
                           float* rstd, void* stream) {
    g_err.clear();
    if (!plan) return fail(GDPA_ERR_INVALID_ARG, "plan is NULL");
    if (plan->host_only) return fail(GDPA_ERR_PLAN_MISMATCH, "host-only plan cannot run kernels");
    if (H != plan->H || d != plan->d) return fail(GDPA_ERR_PLAN_MISMATCH, "H or d differ from the plan");
    gdpa_status st = norm_check(plan, GDPA_ACT_GELU, norm, rstd);
    if (st != GDPA_OK) return st;
    if ((plan->Tq > 0 && !q) || (plan->Tk > 0 && (!k || !v))) return fail(GDPA_ERR_INVALID_ARG, "q, k or v is NULL");
    const hipError_t e = launch_norm_rstd(q, k, v, (int)plan->Tq, (int)plan->Tk, H, d, norm, kRmsEps, rstd,
                                          rstd + (size_t)H * plan->Tq, (hipStream_t)stream);
    if (e != hipSuccess) return fail_hip(e, "RMSNorm pre-pass launch");
    return GDPA_OK;
}

gdpa_status gdpa_norm_fwd(gdpa_plan plan, const void* q, const void* k, const void* v, const int32_t* q_off_dev,
                          const int32_t* kv_off_dev, int B, int H, int d, gdpa_act act, int window, int norm,
                          const float* rstd, void* o, void* stream) {
    g_err.clear();
    gdpa_status st = check_call(plan, q_off_dev, kv_off_dev, B, H, d, act, window);
    if (st == GDPA_OK) st = norm_check(plan, act, norm, rstd);
    if (st != GDPA_OK) return st;
    if (plan->Tq > 0 && (!q || !o)) return fail(GDPA_ERR_INVALID_ARG, "q or o is NULL");
    if (plan->Tk > 0 && (!k || !v)) return fail(GDPA_ERR_INVALID_ARG, "k or v is NULL");
    if (plan->Tq == 0) return GDPA_OK;
    hipStream_t s = (hipStream_t)stream;
    KernelArgs a = base_args(plan, q_off_dev, kv_off_dev);
    norm_args(plan, norm, rstd, a);
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    const WorkList& wl = plan->lists[LIST_FWD];
    a.items = plan->d_items[LIST_FWD];
    a.bin_ptr = plan->d_bin_ptr[LIST_FWD];
    set_claims(a, plan, LIST_FWD);
    a.P = wl.P;
    a.part = plan->d_part[LIST_FWD];
    const int code = (int)act | kActNorm;
    hipError_t e;
    switch (d) {
        case 32: e = launch_fwd_bf16_d32(a, wl.team, wl.nb, code, s); break;
        case 64: e = launch_fwd_bf16_d64(a, wl.team, wl.nb, code, s); break;
        default: e = launch_fwd_bf16_d128(a, wl.team, wl.nb, code, s); break;
    }
    if (e == hipSuccess) e = reduce_parts(plan, LIST_FWD, 1.0f, o, s);
    if (e == hipErrorInvalidValue) return fail(GDPA_ERR_UNSUPPORTED, "no RMSNorm-prologue forward kernel here");
    if (e != hipSuccess) return fail_hip(e, "forward launch");
    return GDPA_OK;
}

static gdpa_status norm_bwd_parts(gdpa_plan plan, const void* q, const void* k, const void* v, const void* dout,
                                  const int32_t* q_off_dev, const int32_t* kv_off_dev, int B, int H, int d,
                                  gdpa_act act, int window, int norm, const float* rstd, void* dq, void* dk, void* dv,
                                  void* stream, bool want_dkdv, bool want_dq) {
    g_err.clear();
    gdpa_status st = check_call(plan, q_off_dev, kv_off_dev, B, H, d, act, window);
    if (st == GDPA_OK) st = norm_check(plan, act, norm, rstd);
    if (st != GDPA_OK) return st;
    const bool any_q = plan->Tq > 0, any_k = plan->Tk > 0;
    if (any_q && (!q || !dout)) return fail(GDPA_ERR_INVALID_ARG, "q or dout is NULL");
    if (any_k && (!k || !v)) return fail(GDPA_ERR_INVALID_ARG, "k or v is NULL");
    if (want_dq && any_q && !dq) return fail(GDPA_ERR_INVALID_ARG, "dq is NULL");
    if (want_dkdv && any_k && (!dk || !dv)) return fail(GDPA_ERR_INVALID_ARG, "dk or dv is NULL");
    hipStream_t s = (hipStream_t)stream;
    KernelArgs a = base_args(plan, q_off_dev, kv_off_dev);
    norm_args(plan, norm, rstd, a);
    a.q = q;
    a.k = k;
    a.v = v;
    a.dout = dout;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    const int code = (int)act | kActNorm;
    hipError_t e = hipSuccess;
    if (want_dkdv && any_k) {
        const WorkList& wl = plan->lists[LIST_DKDV];
        KernelArgs b = a;
        b.items = plan->d_items[LIST_DKDV];
        b.bin_ptr = plan->d_bin_ptr[LIST_DKDV];
        set_claims(b, plan, LIST_DKDV);
        b.P = wl.P;
        b.part = plan->d_part[LIST_DKDV];
        switch (d) {
            case 32: e = launch_dkdv_bf16_d32(b, wl.team, wl.nb, code, s); break;
            case 64: e = launch_dkdv_bf16_d64(b, wl.team, wl.nb, code, s); break;
            default: e = launch_dkdv_bf16_d128(b, wl.team, wl.nb, code, s); break;
        }
        if (e == hipSuccess) e = reduce_parts(plan, LIST_DKDV, a.scale, dk, s, 0);
        if (e == hipSuccess) e = reduce_parts(plan, LIST_DKDV, 1.0f, dv, s, 1);
    }
    if (e == hipSuccess && want_dq && any_q) {
        const WorkList& wl = plan->lists[LIST_DQ];
        KernelArgs b = a;
        b.items = plan->d_items[LIST_DQ];
        b.bin_ptr = plan->d_bin_ptr[LIST_DQ];
        set_claims(b, plan, LIST_DQ);
        b.P = wl.P;
        b.part = plan->d_part[LIST_DQ];
        switch (d) {
            case 32: e = launch_dq_bf16_d32(b, wl.team, wl.nb, code, s); break;
            case 64: e = launch_dq_bf16_d64(b, wl.team, wl.nb, code, s); break;
            default: e = launch_dq_bf16_d128(b, wl.team, wl.nb, code, s); break;
        }
        if (e == hipSuccess) e = reduce_parts(plan, LIST_DQ, a.scale, dq, s);
    }
    if (e == hipErrorInvalidValue) return fail(GDPA_ERR_UNSUPPORTED, "no RMSNorm-prologue backward kernel here");
    if (e != hipSuccess) return fail_hip(e, "backward launch");
    return GDPA_OK;
}

gdpa_status gdpa_norm_bwd(gdpa_plan plan, const void* q, const void* k, const void* v, const void* dout,
                          const int32_t* q_off_dev, const int32_t* kv_off_dev, int B, int H, int d, gdpa_act act,
                          int window, int norm, const float* rstd, void* dq, void* dk, void* dv, void* stream) {
    return norm_bwd_parts(plan, q, k, v, dout, q_off_dev, kv_off_dev, B, H, d, act, window, norm, rstd, dq, dk, dv,
                          stream, true, true);
}

gdpa_status gdpa_norm_bwd_dkdv(gdpa_plan plan, const void* q, const void* k, const void* v, const void* dout,
                               const int32_t* q_off_dev, const int32_t* kv_off_dev, int B, int H, int d,
                               gdpa_act act, int window, int norm, const float* rstd, void* dk, void* dv,
                               void* stream) {
    return norm_bwd_parts(plan, q, k, v, dout, q_off_dev, kv_off_dev, B, H, d, act, window, norm, rstd, nullptr,
                          dk, dv, stream, true, false);
}

gdpa_status gdpa_norm_bwd_dq(gdpa_plan plan, const void* q, const void* k, const void* v, const void* dout,
                             const int32_t* q_off_dev, const int32_t* kv_off_dev, int B, int H, int d, gdpa_act act,
                             int window, int norm, const float* rstd, void* dq, void* stream) {
    return norm_bwd_parts(plan, q, k, v, dout, q_off_dev, kv_off_dev, B, H, d, act, window, norm, rstd, dq, nullptr,
                          nullptr, stream, false, true);
}

gdpa_status gdpa_fp8_fwd(gdpa_plan plan, const void* q8, const void* k8, const void* v, const int32_t* q_off_dev,
                         const int32_t* kv_off_dev, int B, int H, int d, gdpa_act act, int window, float q_scale,
                         float k_scale, void* o, void* stream) {
    g_err.clear();
    gdpa_status st = check_call(plan, q_off_dev, kv_off_dev, B, H, d, act, window);
    if (st != GDPA_OK) return st;
    if (plan->dtype == GDPA_F32) return fail(GDPA_ERR_UNSUPPORTED, "fp8 Q and K run on bf16 plans");
    if (act == GDPA_ACT_ONE) return fail(GDPA_ERR_UNSUPPORTED, "GDPA_ACT_ONE has no fp8 kernels");
    if (!(q_scale > 0.0f) || !(k_scale > 0.0f) || !std::isfinite(q_scale) || !std::isfinite(k_scale))
        return fail(GDPA_ERR_INVALID_ARG, "q_scale and k_scale must be finite and > 0");
    if (plan->Tq > 0 && (!q8 || !o)) return fail(GDPA_ERR_INVALID_ARG, "q8 or o is NULL");
    if (plan->Tk > 0 && (!k8 || !v)) return fail(GDPA_ERR_INVALID_ARG, "k8 or v is NULL");
    if (plan->Tq == 0) return GDPA_OK;
    hipStream_t s = (hipStream_t)stream;
    KernelArgs a = base_args(plan, q_off_dev, kv_off_dev);
    a.scale *= q_scale * k_scale;   // S = (q8 . k8) q_scale k_scale / sqrt(d)
    a.q = q8;
    a.k = k8;
    a.v = v;
    a.o = o;
    const WorkList& wl = plan->lists[LIST_FWD];
    a.items = plan->d_items[LIST_FWD];
    a.bin_ptr = plan->d_bin_ptr[LIST_FWD];
    set_claims(a, plan, LIST_FWD);
    a.P = wl.P;
    a.part = plan->d_part[LIST_FWD];
    const int code = (int)act | kActF8;
    hipError_t e;
    switch (d) {
        case 32: e = launch_fwd_bf16_d32(a, wl.team, wl.nb, code, s); break;
        case 64: e = launch_fwd_bf16_d64(a, wl.team, wl.nb, code, s); break;
        default: e = launch_fwd_bf16_d128(a, wl.team, wl.nb, code, s); break;
    }
    if (e == hipSuccess) e = reduce_parts(plan, LIST_FWD, 1.0f, o, s);
    if (e == hipErrorInvalidValue) return fail(GDPA_ERR_UNSUPPORTED, "no fp8 forward kernel here");
    if (e != hipSuccess) return fail_hip(e, "fp8 forward launch");
    return GDPA_OK;
}

gdpa_status gdpa_mx_fwd(gdpa_plan plan, const void* q8, const void* q_scale, const void* k8, const void* k_scale,
                        const void* v, const int32_t* q_off_dev, const int32_t* kv_off_dev, int B, int H, int d,
                        gdpa_act act, int window, void* o, void* stream) {
    g_err.clear();
    gdpa_status st = check_call(plan, q_off_dev, kv_off_dev, B, H, d, act, window);
    if (st != GDPA_OK) return st;
    if (plan->dtype == GDPA_F32) return fail(GDPA_ERR_UNSUPPORTED, "block-scaled fp8 Q and K run on bf16 plans");
    if (d < 64) return fail(GDPA_ERR_UNSUPPORTED, "block-scaled fp8 Q and K need d = 64 or 128 (64-wide k blocks)");
    if (act == GDPA_ACT_ONE) return fail(GDPA_ERR_UNSUPPORTED, "GDPA_ACT_ONE has no fp8 kernels");
    if (plan->Tq > 0 && (!q8 || !q_scale || !o)) return fail(GDPA_ERR_INVALID_ARG, "q8, q_scale or o is NULL");
    if (plan->Tk > 0 && (!k8 || !k_scale || !v)) return fail(GDPA_ERR_INVALID_ARG, "k8, k_scale or v is NULL");
    if (plan->Tq == 0) return GDPA_OK;
    hipStream_t s = (hipStream_t)stream;
    KernelArgs a = base_args(plan, q_off_dev, kv_off_dev);
    a.q = q8;
    a.k = k8;
    a.v = v;
    a.o = o;
    a.q_mx = (const uint8_t*)q_scale;
    a.k_mx = (const uint8_t*)k_scale;
    a.Tq = (int)plan->Tq;
    a.Tk = (int)plan->Tk;
    const WorkList& wl = plan->lists[LIST_FWD];
    a.items = plan->d_items[LIST_FWD];
    a.bin_ptr = plan->d_bin_ptr[LIST_FWD];
    set_claims(a, plan, LIST_FWD);
    a.P = wl.P;
    a.part = plan->d_part[LIST_FWD];
    const int code = (int)act | kActMX;
    hipError_t e = d == 64 ? launch_fwd_bf16_d64(a, wl.team, wl.nb, code, s)
                           : launch_fwd_bf16_d128(a, wl.team, wl.nb, code, s);
    if (e == hipSuccess) e = reduce_parts(plan, LIST_FWD, 1.0f, o, s);
    if (e == hipErrorInvalidValue) return fail(GDPA_ERR_UNSUPPORTED, "no block-scaled fp8 forward kernel here");
    if (e != hipSuccess) return fail_hip(e, "block-scaled fp8 forward launch");
    return GDPA_OK;
}

gdpa_status gdpa_pffn_plan_create(int Tq, int M, int H, int d, gdpa_dtype dtype, const gdpa_plan_opts* opts,
                                  void* stream, gdpa_plan* out) {
    g_err.clear();
    if (!out) return fail(GDPA_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (Tq < 0 || M < 0) return fail(GDPA_ERR_INVALID_ARG, "Tq and M must be >= 0");
    const int32_t q_off[2] = {0, Tq}, kv_off[2] = {0, M};
    return plan_create(q_off, kv_off, 1, H, d, 0, dtype, opts, (hipStream_t)stream, true, out);
}

static gdpa_status check_pffn(gdpa_plan plan) {
    if (!plan) return fail(GDPA_ERR_INVALID_ARG, "plan is NULL");
    if (!plan->pffn) return fail(GDPA_ERR_PLAN_MISMATCH, "not a pFFN plan (use gdpa_pffn_plan_create)");
    if (plan->host_only) return fail(GDPA_ERR_PLAN_MISMATCH, "host-only plan cannot run kernels");
    return GDPA_OK;
}

gdpa_status gdpa_pffn_fwd(gdpa_plan plan, const void* q, const void* wk, const void* wv, gdpa_act act, void* o,
                          void* stream) {
    g_err.clear();
    gdpa_status st = check_pffn(plan);
    if (st != GDPA_OK) return st;
    return gdpa_fwd(plan, q, wk, wv, plan->d_off, plan->d_off + 2, 1, plan->H, plan->d, act, 0, o, stream);
}

gdpa_status gdpa_pffn_bwd(gdpa_plan plan, const void* q, const void* wk, const void* wv, const void* dout,
                          gdpa_act act, void* dq, void* dwk, void* dwv, void* stream) {
    g_err.clear();
    gdpa_status st = check_pffn(plan);
    if (st != GDPA_OK) return st;
    return gdpa_bwd(plan, q, wk, wv, dout, plan->d_off, plan->d_off + 2, 1, plan->H, plan->d, act, 0, dq, dwk,
                    dwv, stream);
}

}  // extern "C"
