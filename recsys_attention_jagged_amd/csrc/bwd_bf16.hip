// GDPA backward, bf16 inputs, fp32 MFMA accumulation, for one head dimension
// (compiled once per D with -DGDPA_D=32|64|128).
//
// Gradients of sum(O * dO) for O = act(S) V, S = Q K^T / sqrt(d) on the valid
// pairs.  With no softmax there is no row statistic to keep (GDPA page,
// aitrends.kr/articles/26275, "Section details": the softmax correction step
// is removed), so each kernel recomputes S and
//     dP = dO V^T,   dS = dP * act'(S),
//     dV = P^T dO,   dK = dS^T Q / sqrt(d),   dQ = dS K / sqrt(d).
//
// Two persistent kernels, no atomics (every output row has one owner):
//   * dq   - Q-stationary: an item is a q tile, steps stream K/V tiles.
//            S^T = K Q^T and dP^T = V dO^T (Q, dO in registers), then
//            dQ^T += K^T dS^T with the dS^T accumulator lanes as B operand and
//            K^T read from the row-major K tile with transposing LDS reads.
//   * dkdv - KV-stationary: an item is a kv tile, steps stream Q/dO tiles.
//            S = Q K^T and dP = dO V^T (K, V in registers), then
//            dV^T += dO^T P and dK^T += Q^T dS, with dO^T and Q^T read from
//            the row-major tiles with transposing LDS reads.
// Both run on the multi-stage DMA pipeline shared with the forward kernel.
#include "kernels.hpp"
#include "pipe.hpp"

#ifndef GDPA_D
#error "compile with -DGDPA_D=<32|64|128>"
#endif

namespace gdpa {
namespace {

// Sum the per-wave partial accumulators of NG waves that share an output block
// (group member `mem` of group `grp`; member 0 keeps the sum), through LDS.
template <int NDB, int NG, int NGRP>
__device__ __forceinline__ void reduce_groups(f32x16 (&acc)[NDB], char* lds, int grp, int mem, int lane) {
    f32x4* part = (f32x4*)lds;
    if (mem > 0) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4)
                part[((((mem - 1) * NGRP + grp) * NDB + db) * 4 + c4) * 64 + lane] =
                    f32x4{acc[db][4 * c4], acc[db][4 * c4 + 1], acc[db][4 * c4 + 2], acc[db][4 * c4 + 3]};
    }
    lds_barrier();
    if (mem == 0) {
#pragma unroll
        for (int m2 = 1; m2 < NG; ++m2)
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int c4 = 0; c4 < 4; ++c4) {
                    const f32x4 v = part[((((m2 - 1) * NGRP + grp) * NDB + db) * 4 + c4) * 64 + lane];
                    for (int i = 0; i < 4; ++i) acc[db][4 * c4 + i] += v[i];
                }
    }
    lds_barrier();
}

// Store an accumulator tile whose lanes hold column `rowbase + r` (an output
// row) and rows d = 32 db + 8 j + 4 hh + i: staged through LDS as bf16 rows,
// then written with coalesced 16-byte stores; rows beyond the slice are dropped.
template <int D, int NDB>
__device__ __forceinline__ void stage_rows(const f32x16 (&acc)[NDB], float mul, __bf16* sO, int row, int hh) {
    constexpr int SOST = D + 8;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            u32x2 w;
            w[0] = pack_bf16x2(acc[db][4 * j] * mul, acc[db][4 * j + 1] * mul);
            w[1] = pack_bf16x2(acc[db][4 * j + 2] * mul, acc[db][4 * j + 3] * mul);
            *(u32x2*)(sO + row * SOST + db * 32 + 8 * j + 4 * hh) = w;
        }
}

template <int D, int ROWS>
__device__ __forceinline__ void store_rows(const __bf16* sO, rsrc_t ro, int row0, uint32_t rso, int tid) {
    constexpr int SOST = D + 8, CPR = D / 8;
    for (int ci = tid; ci < ROWS * CPR; ci += 256) {
        const int row = ci / CPR, c = ci % CPR;
        buf_store16(ro, (uint32_t)(row0 + row) * rso + c * 16, *(const u32x4*)(sO + row * SOST + 8 * c));
    }
}

template <int NDB>
__device__ __forceinline__ void store_f32(const f32x16 (&acc)[NDB], float mul, rsrc_t ro, int row, uint32_t rso, int hh) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            u32x4 v;
            for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(acc[db][4 * j + i] * mul);
            buf_store16(ro, (uint32_t)row * rso + (db * 32 + 8 * j + 4 * hh) * 4, v);
        }
}

struct Lanes {
    int tid, lane, wave, r, hh;
    __device__ Lanes() {
        tid = threadIdx.x;
        lane = tid & 63;
        wave = tid >> 6;
        r = lane & 31;
        hh = lane >> 5;
    }
};

// =========================================================================
// dQ (Q-stationary)
// =========================================================================
template <int D, int WQ, int ACT>
struct DqPol : Lanes {
    static constexpr int WK = 4 / WQ, BM = 32 * WQ, BN = 32 * WK;
    static constexpr int NDB = D / 32, NKS = D / 16;
    using TQ = AsyncTile<BM, D>;
    using TK = AsyncTile<BN, D>;
    static constexpr int OFF_O = TQ::BYTES, OFF_K = 2 * TQ::BYTES, OFF_V = 2 * TQ::BYTES + TK::BYTES;
    static constexpr int STAGE_BYTES = 2 * TQ::BYTES + 2 * TK::BYTES;
    static constexpr int NS = Stages<STAGE_BYTES>::N;
    static_assert((WK - 1) * WQ * NDB * 4096 <= STAGE_BYTES && BM * (D + 8) * 2 <= STAGE_BYTES, "epilogue");

    const KernelArgs a;   // by value: kept in SGPRs, not re-read from the argument segment
    int wq, wk, H, win;
    uint32_t rs, rso;
    float scale;
    rsrc_t empty, rq, ro, rk, rv;
    TQ tq;
    TK tk;
    bf16x8 qf[NKS], of[NKS];
    f32x16 acc[NDB];

    __device__ DqPol(const KernelArgs& args) : a(args) {
        wq = wave / WK;
        wk = wave % WK;
        H = a.H;
        win = a.window > 0 ? a.window : (1 << 30);
        rs = (uint32_t)H * D * 2;
        rso = (uint32_t)H * D * (a.out_f32 ? 4 : 2);
        scale = a.scale;
        empty = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.q), 0, 0, 0x00020000);
        rq = ro = rk = rv = empty;
        tq.init(rs, wave, lane);
        tk.init(rs, wave, lane);
    }

    __device__ __forceinline__ void new_item(const Step& st) {
        const size_t kvb = ((size_t)st.r.ks * H + st.r.h) * D;
        rk = slice_rsrc((const __bf16*)a.k + kvb, st.r.lk, rs, D * 2);
        rv = slice_rsrc((const __bf16*)a.v + kvb, st.r.lk, rs, D * 2);
        const size_t qb = ((size_t)st.r.qs * H + st.r.h) * D;
        rq = slice_rsrc((const __bf16*)a.q + qb, st.r.lq, rs, D * 2);
        ro = slice_rsrc((const __bf16*)a.dout + qb, st.r.lq, rs, D * 2);
    }

    __device__ __forceinline__ int issue(const Step& st, uint32_t stage) {
        if (!st.valid || !st.has_steps()) return 0;
        int n = 0;
        if (st.first()) {
            const uint32_t sq = (uint32_t)(st.r.t * BM) * rs;
            n += tq.issue(rq, sq, stage, wave);
            n += tq.issue(ro, sq, stage + OFF_O, wave);
        }
        const uint32_t sk = (uint32_t)(st.s * BN) * rs;
        n += tk.issue(rk, sk, stage + OFF_K, wave);
        n += tk.issue(rv, sk, stage + OFF_V, wave);
        return n;
    }

    __device__ __forceinline__ void item_start(const Step& st, const char* stage) {
        if (st.has_steps()) {
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                qf[ks] = lds_row8<D>(stage, wq * 32 + r, 2 * ks + hh);
                of[ks] = lds_row8<D>(stage + OFF_O, wq * 32 + r, 2 * ks + hh);
            }
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
    }

    __device__ __forceinline__ void compute(const Step& st, const char* stage) {
        const int q0 = st.r.t * BM + wq * 32;
        const int jl = wk * 32;
        const int j0 = st.s * BN + jl;
        const int lq = st.r.lq, lk = st.r.lk;
        if (!st.has_steps() || !block_any(q0, j0, lq, lk, win)) return;
        const char* kt = stage + OFF_K;
        const char* vt = stage + OFF_V;
        f32x16 s = {}, dp = {};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            s = mfma32(lds_row8<D>(kt, jl + r, 2 * ks + hh), qf[ks], s);
            dp = mfma32(lds_row8<D>(vt, jl + r, 2 * ks + hh), of[ks], dp);
        }
        f32x16 ds;
        const bool full = block_all(q0, j0, lq, lk, win);
        const int qi = q0 + r;
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            float f, g;
            act_fwd_grad<ACT>(s[c] * scale, f, g);
            const int kj = j0 + 8 * (c >> 2) + 4 * hh + (c & 3);
            const int dd = qi - kj;
            const bool ok = full || (kj < lk && qi < lq && dd < win && -dd < win);
            ds[c] = ok ? dp[c] * g : 0.0f;
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const bf16x8 db8 = acc_to_bf16x8(ds, m);
#pragma unroll
            for (int db = 0; db < NDB; ++db) acc[db] = mfma32(lds_col8<D>(kt, jl + 16 * m, db * 32, lane), db8, acc[db]);
        }
    }

    __device__ __forceinline__ void epilogue(const Step& st, char* stage) {
        if constexpr (WK > 1) reduce_groups<NDB, WK, WQ>(acc, stage, wq, wk, lane);
        const size_t ob = ((size_t)st.r.qs * H + st.r.h) * D;
        if (a.out_f32) {
            if (wk == 0)
                store_f32<NDB>(acc, scale, slice_rsrc((const float*)a.dq + ob, st.r.lq, rso, D * 4),
                               st.r.t * BM + wq * 32 + r, rso, hh);
            return;
        }
        __bf16* sO = (__bf16*)stage;
        if (wk == 0) stage_rows<D, NDB>(acc, scale, sO, wq * 32 + r, hh);
        lds_barrier();
        store_rows<D, BM>(sO, slice_rsrc((const __bf16*)a.dq + ob, st.r.lq, rso, D * 2), st.r.t * BM, rso, tid);
    }
};

// =========================================================================
// dK / dV (KV-stationary)
// =========================================================================
template <int D, int WK, int ACT>
struct DkdvPol : Lanes {
    static constexpr int WQ = 4 / WK, BK = 32 * WK, BQ = 32 * WQ;
    static constexpr int NDB = D / 32, NKS = D / 16;
    using TK = AsyncTile<BK, D>;
    using TQ = AsyncTile<BQ, D>;
    static constexpr int OFF_V = TK::BYTES, OFF_Q = 2 * TK::BYTES, OFF_O = 2 * TK::BYTES + TQ::BYTES;
    static constexpr int STAGE_BYTES = 2 * TK::BYTES + 2 * TQ::BYTES;
    static constexpr int NS = Stages<STAGE_BYTES>::N;
    static_assert((WQ - 1) * WK * NDB * 4096 <= STAGE_BYTES && 2 * BK * (D + 8) * 2 <= STAGE_BYTES, "epilogue");

    const KernelArgs a;   // by value: kept in SGPRs, not re-read from the argument segment
    int wq, wk, H, win;
    uint32_t rs, rso;
    float scale;
    rsrc_t empty, rk, rv, rq, ro;
    TK tk;
    TQ tq;
    bf16x8 kf[NKS], vf[NKS];
    f32x16 accK[NDB], accV[NDB];

    __device__ DkdvPol(const KernelArgs& args) : a(args) {
        wk = wave / WQ;
        wq = wave % WQ;
        H = a.H;
        win = a.window > 0 ? a.window : (1 << 30);
        rs = (uint32_t)H * D * 2;
        rso = (uint32_t)H * D * (a.out_f32 ? 4 : 2);
        scale = a.scale;
        empty = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.k), 0, 0, 0x00020000);
        rk = rv = rq = ro = empty;
        tk.init(rs, wave, lane);
        tq.init(rs, wave, lane);
    }

    __device__ __forceinline__ void new_item(const Step& st) {
        const size_t kvb = ((size_t)st.r.ks * H + st.r.h) * D;
        rk = slice_rsrc((const __bf16*)a.k + kvb, st.r.lk, rs, D * 2);
        rv = slice_rsrc((const __bf16*)a.v + kvb, st.r.lk, rs, D * 2);
        const size_t qb = ((size_t)st.r.qs * H + st.r.h) * D;
        rq = slice_rsrc((const __bf16*)a.q + qb, st.r.lq, rs, D * 2);
        ro = slice_rsrc((const __bf16*)a.dout + qb, st.r.lq, rs, D * 2);
    }

    __device__ __forceinline__ int issue(const Step& st, uint32_t stage) {
        if (!st.valid || !st.has_steps()) return 0;
        int n = 0;
        if (st.first()) {
            const uint32_t sk = (uint32_t)(st.r.t * BK) * rs;
            n += tk.issue(rk, sk, stage, wave);
            n += tk.issue(rv, sk, stage + OFF_V, wave);
        }
        const uint32_t sq = (uint32_t)(st.s * BQ) * rs;
        n += tq.issue(rq, sq, stage + OFF_Q, wave);
        n += tq.issue(ro, sq, stage + OFF_O, wave);
        return n;
    }

    __device__ __forceinline__ void item_start(const Step& st, const char* stage) {
        if (st.has_steps()) {
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                kf[ks] = lds_row8<D>(stage, wk * 32 + r, 2 * ks + hh);
                vf[ks] = lds_row8<D>(stage + OFF_V, wk * 32 + r, 2 * ks + hh);
            }
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db) accK[db] = accV[db] = f32x16{};
    }

    __device__ __forceinline__ void compute(const Step& st, const char* stage) {
        const int il = wq * 32;
        const int i0 = st.s * BQ + il;          // q rows of this wave
        const int j0 = st.r.t * BK + wk * 32;   // kv rows of this wave
        const int lq = st.r.lq, lk = st.r.lk;
        if (!st.has_steps() || !block_any(i0, j0, lq, lk, win)) return;
        const char* qt = stage + OFF_Q;
        const char* ot = stage + OFF_O;
        f32x16 s = {}, dp = {};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            s = mfma32(lds_row8<D>(qt, il + r, 2 * ks + hh), kf[ks], s);
            dp = mfma32(lds_row8<D>(ot, il + r, 2 * ks + hh), vf[ks], dp);
        }
        // accumulator lane: column = kv row j0 + r, rows = q rows i0 + 8 j + 4 hh + i
        f32x16 p, ds;
        const bool full = block_all(i0, j0, lq, lk, win);
        const int kj = j0 + r;
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            float f, g;
            act_fwd_grad<ACT>(s[c] * scale, f, g);
            const int qi = i0 + 8 * (c >> 2) + 4 * hh + (c & 3);
            const int dd = qi - kj;
            const bool ok = full || (kj < lk && qi < lq && dd < win && -dd < win);
            p[c] = ok ? f : 0.0f;
            ds[c] = ok ? dp[c] * g : 0.0f;
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const bf16x8 pm = acc_to_bf16x8(p, m), dm = acc_to_bf16x8(ds, m);
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                accV[db] = mfma32(lds_col8<D>(ot, il + 16 * m, db * 32, lane), pm, accV[db]);
                accK[db] = mfma32(lds_col8<D>(qt, il + 16 * m, db * 32, lane), dm, accK[db]);
            }
        }
    }

    __device__ __forceinline__ void epilogue(const Step& st, char* stage) {
        if constexpr (WQ > 1) {
            reduce_groups<NDB, WQ, WK>(accK, stage, wk, wq, lane);
            reduce_groups<NDB, WQ, WK>(accV, stage, wk, wq, lane);
        }
        const size_t ob = ((size_t)st.r.ks * H + st.r.h) * D;
        const int row = st.r.t * BK + wk * 32 + r;
        if (a.out_f32) {
            if (wq == 0) {
                store_f32<NDB>(accK, scale, slice_rsrc((const float*)a.dk + ob, st.r.lk, rso, D * 4), row, rso, hh);
                store_f32<NDB>(accV, 1.0f, slice_rsrc((const float*)a.dv + ob, st.r.lk, rso, D * 4), row, rso, hh);
            }
            return;
        }
        __bf16* sK = (__bf16*)stage;
        __bf16* sV = sK + BK * (D + 8);
        if (wq == 0) {
            stage_rows<D, NDB>(accK, scale, sK, wk * 32 + r, hh);
            stage_rows<D, NDB>(accV, 1.0f, sV, wk * 32 + r, hh);
        }
        lds_barrier();
        store_rows<D, BK>(sK, slice_rsrc((const __bf16*)a.dk + ob, st.r.lk, rso, D * 2), st.r.t * BK, rso, tid);
        store_rows<D, BK>(sV, slice_rsrc((const __bf16*)a.dv + ob, st.r.lk, rso, D * 2), st.r.t * BK, rso, tid);
    }
};

template <int D, int WQ, int ACT>
__global__ __launch_bounds__(256, 1) void dq_bf16_kernel(const KernelArgs a, const Rec* __restrict__ recs,
                                                         const int32_t* __restrict__ bin_ptr) {
    using Pol = DqPol<D, WQ, ACT>;
    __shared__ __attribute__((aligned(1024))) char smem[Pol::NS * Pol::STAGE_BYTES];
    Pol pol(a);
    run_pipeline(pol, a.P, recs, bin_ptr, smem);
}

template <int D, int WK, int ACT>
__global__ __launch_bounds__(256, 1) void dkdv_bf16_kernel(const KernelArgs a, const Rec* __restrict__ recs,
                                                           const int32_t* __restrict__ bin_ptr) {
    using Pol = DkdvPol<D, WK, ACT>;
    __shared__ __attribute__((aligned(1024))) char smem[Pol::NS * Pol::STAGE_BYTES];
    Pol pol(a);
    run_pipeline(pol, a.P, recs, bin_ptr, smem);
}

template <int WQ, int ACT>
const void* dq_ptr() {
    return (const void*)&dq_bf16_kernel<GDPA_D, WQ, ACT>;
}
template <int WK, int ACT>
const void* dkdv_ptr() {
    return (const void*)&dkdv_bf16_kernel<GDPA_D, WK, ACT>;
}

#define GDPA_ACT_SWITCH(F, W)                                         \
    switch (act) {                                                    \
        case ACT_GELU: return F<W, ACT_GELU>();                       \
        case ACT_SILU: return F<W, ACT_SILU>();                       \
        case ACT_GELU_POLY: return F<W, ACT_GELU_POLY>();             \
        case ACT_GELU_TAYLOR6: return F<W, ACT_GELU_TAYLOR6>();       \
        case ACT_IDENTITY: return F<W, ACT_IDENTITY>();               \
    }                                                                 \
    return nullptr;

template <int W>
const void* dq_act(int act) { GDPA_ACT_SWITCH(dq_ptr, W) }
template <int W>
const void* dkdv_act(int act) { GDPA_ACT_SWITCH(dkdv_ptr, W) }

}  // namespace

#define GDPA_CAT2(a, b) a##b
#define GDPA_CAT(a, b) GDPA_CAT2(a, b)

const void* GDPA_CAT(dq_bf16_kernel_ptr_d, GDPA_D)(int waves, int act) {
    switch (waves) {
        case 1: return dq_act<1>(act);
        case 2: return dq_act<2>(act);
        case 4: return dq_act<4>(act);
    }
    return nullptr;
}

const void* GDPA_CAT(dkdv_bf16_kernel_ptr_d, GDPA_D)(int waves, int act) {
    switch (waves) {
        case 1: return dkdv_act<1>(act);
        case 2: return dkdv_act<2>(act);
        case 4: return dkdv_act<4>(act);
    }
    return nullptr;
}

static hipError_t launch(const void* f, const KernelArgs& a, hipStream_t s) {
    if (!f) return hipErrorInvalidValue;
    if (a.P <= 0) return hipSuccess;
    KernelArgs args = a;
    const void* recs = a.items;
    const int32_t* bin_ptr = a.bin_ptr;
    void* params[] = {&args, &recs, &bin_ptr};
    return hipLaunchKernel(f, dim3(a.P), dim3(256), params, 0, s);
}

hipError_t GDPA_CAT(launch_dq_bf16_d, GDPA_D)(const KernelArgs& a, int waves, int act, hipStream_t s) {
    return launch(GDPA_CAT(dq_bf16_kernel_ptr_d, GDPA_D)(waves, act), a, s);
}

hipError_t GDPA_CAT(launch_dkdv_bf16_d, GDPA_D)(const KernelArgs& a, int waves, int act, hipStream_t s) {
    return launch(GDPA_CAT(dkdv_bf16_kernel_ptr_d, GDPA_D)(waves, act), a, s);
}

}  // namespace gdpa
