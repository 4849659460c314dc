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
//   * dq_kernel   - Q-stationary: an item is a q tile, steps stream K/V tiles.
//                   S^T = K Q^T and dP^T = V dO^T (Q, dO in registers), then
//                   dQ^T += K^T dS^T with the dS^T accumulator lanes as the
//                   B operand (K^T from a transposed LDS copy).
//   * dkdv_kernel - KV-stationary: an item is a kv tile, steps stream Q/dO
//                   tiles.  S = Q K^T and dP = dO V^T (K, V in registers), then
//                   dV^T += dO^T P and dK^T += Q^T dS with P, dS accumulator
//                   lanes as B operands (Q^T, dO^T from transposed LDS copies).
// Both walk their bin's (item, step) pairs as one flattened, prefetched loop,
// as the forward kernel does.
#include "device.hpp"
#include "kernels.hpp"

#ifndef GDPA_D
#error "compile with -DGDPA_D=<32|64|128>"
#endif

namespace gdpa {
namespace {

// =========================================================================
// dQ kernel (Q-stationary)
// =========================================================================
template <int D, int WQ>
struct DqCfg {
    static constexpr int WK = 4 / WQ, BNW = 32, BM = 32 * WQ, BN = WK * BNW;
    static constexpr int NDB = D / 32, NKS = D / 16;
    static constexpr int KST = D + 8, VST = BN + 8;
    static constexpr int SZ_K = BN * KST, SZ_KT = D * VST, SZ_V = BN * KST, SZ_Q = BM * KST;
    static constexpr int STEP_BYTES = (SZ_K + SZ_KT + SZ_V) * 2;
    static constexpr int NBUF = (2 * STEP_BYTES + 2 * SZ_Q * 2) <= 160 * 1024 ? 2 : 1;
    static constexpr int MAIN = NBUF * STEP_BYTES + 2 * SZ_Q * 2;
    static constexpr int PART_BYTES = (WK - 1) * WQ * NDB * 64 * 16 * 4;
    static constexpr int EPI_BYTES = PART_BYTES + BM * KST * 2;
    static constexpr int LDS = MAIN > EPI_BYTES ? MAIN : EPI_BYTES;
    static_assert(LDS <= 160 * 1024, "LDS budget exceeded");
};

template <int D, int WQ, int ACT>
__global__ __launch_bounds__(256, 1) void dq_bf16_kernel(const KernelArgs a) {
    using C = DqCfg<D, WQ>;
    constexpr int WK = C::WK, BNW = C::BNW, BM = C::BM, BN = C::BN, NDB = C::NDB, NKS = C::NKS;
    constexpr int KST = C::KST, VST = C::VST;
    __shared__ __attribute__((aligned(16))) char smem[C::LDS];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wq = wave / WK, wk = wave % WK;
    const int r = lane & 31, hh = lane >> 5;

    const int bin = logical_bin(a.P);
    const ItemRec* items = reinterpret_cast<const ItemRec*>(a.items);
    StepIt cur;
    cur.end = a.bin_ptr[bin + 1];
    const int first_item = a.bin_ptr[bin];
    if (first_item >= cur.end) return;
    cur.load(items, a.q_off, a.kv_off, first_item);

    const int H = a.H;
    const uint32_t rs = (uint32_t)H * D * 2;
    const uint32_t rso = (uint32_t)H * D * (a.out_f32 ? 4 : 2);
    const int win = a.window > 0 ? a.window : (1 << 30);
    const float scale = a.scale;
    const __bf16* gq = (const __bf16*)a.q;
    const __bf16* gk = (const __bf16*)a.k;
    const __bf16* gv = (const __bf16*)a.v;
    const __bf16* gdo = (const __bf16*)a.dout;

    __bf16* sQ = (__bf16*)(smem + C::NBUF * C::STEP_BYTES);
    __bf16* sdO = sQ + C::SZ_Q;
    auto sK = [&](int buf) { return (__bf16*)(smem + buf * C::STEP_BYTES); };
    auto sKT = [&](int buf) { return (__bf16*)(smem + buf * C::STEP_BYTES) + C::SZ_K; };
    auto sV = [&](int buf) { return (__bf16*)(smem + buf * C::STEP_BYTES) + C::SZ_K + C::SZ_KT; };

    TileStage<BN, D> stK, stV;
    TileStage<BM, D> stQ, stO;

    auto issue_loads = [&](const StepIt& st, bool with_q) {
        if (st.has_steps()) {
            const size_t kvb = ((size_t)st.ks * H + st.h) * D;
            stK.load(slice_rsrc(gk + kvb, st.lk, rs, D * 2), st.s * BN, rs, tid);
            stV.load(slice_rsrc(gv + kvb, st.lk, rs, D * 2), st.s * BN, rs, tid);
        }
        if (with_q) {
            const size_t qb = ((size_t)st.qs * H + st.h) * D;
            stQ.load(slice_rsrc(gq + qb, st.lq, rs, D * 2), st.t * BM, rs, tid);
            stO.load(slice_rsrc(gdo + qb, st.lq, rs, D * 2), st.t * BM, rs, tid);
        }
    };
    auto commit = [&](const StepIt& st, int buf, bool with_q) {
        if (st.has_steps()) {
            stK.template store_rows<KST>(sK(buf), tid);
            stK.template store_cols<VST>(sKT(buf), tid);
            stV.template store_rows<KST>(sV(buf), tid);
        }
        if (with_q) {
            stQ.template store_rows<KST>(sQ, tid);
            stO.template store_rows<KST>(sdO, tid);
        }
    };

    issue_loads(cur, true);
    commit(cur, 0, true);
    __syncthreads();

    f32x16 acc[NDB];
    bf16x8 qf[NKS], of[NKS];
    int buf = 0;
    for (;;) {
        const bool first = cur.first(), last = cur.last();
        if (first) {
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                qf[ks] = *(const bf16x8*)(sQ + (wq * 32 + r) * KST + 16 * ks + 8 * hh);
                of[ks] = *(const bf16x8*)(sdO + (wq * 32 + r) * KST + 16 * ks + 8 * hh);
            }
#pragma unroll
            for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
        }

        StepIt nx = cur;
        const bool has_next = nx.advance(items, a.q_off, a.kv_off);
        const bool nx_first = has_next && nx.first();
        if (has_next) issue_loads(nx, nx_first);

        const int q0 = cur.t * BM + wq * 32;
        const int j0 = cur.s * BN + wk * BNW;
        if (cur.has_steps() && block_any(q0, j0, cur.lq, cur.lk, win)) {
            const __bf16* k_t = sK(buf);
            const __bf16* kt_t = sKT(buf);
            const __bf16* v_t = sV(buf);
            f32x16 st = {}, dpt = {};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const bf16x8 ka = *(const bf16x8*)(k_t + (wk * BNW + r) * KST + 16 * ks + 8 * hh);
                const bf16x8 va = *(const bf16x8*)(v_t + (wk * BNW + r) * KST + 16 * ks + 8 * hh);
                st = mfma32(ka, qf[ks], st);
                dpt = mfma32(va, of[ks], dpt);
            }
            f32x16 ds;
            const bool full = block_all(q0, j0, cur.lq, cur.lk, win);
            const int qi = q0 + r;
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                float f, g;
                act_fwd_grad<ACT>(st[c] * scale, f, g);
                const int kj = j0 + 8 * (c >> 2) + 4 * hh + (c & 3);
                const int dd = qi - kj;
                const bool ok = full || (kj < cur.lk && qi < cur.lq && dd < win && -dd < win);
                ds[c] = ok ? dpt[c] * g : 0.0f;
            }
            const bf16x8 d0 = acc_to_bf16x8(ds, 0), d1 = acc_to_bf16x8(ds, 1);
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const bf16x8 a0 = *(const bf16x8*)(kt_t + (db * 32 + r) * VST + wk * BNW + 8 * hh);
                acc[db] = mfma32(a0, d0, acc[db]);
            }
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const bf16x8 a1 = *(const bf16x8*)(kt_t + (db * 32 + r) * VST + wk * BNW + 16 + 8 * hh);
                acc[db] = mfma32(a1, d1, acc[db]);
            }
        }

        if (last) {
            __syncthreads();
            if constexpr (WK > 1) {
                float* part = (float*)smem;
                if (wk > 0) {
#pragma unroll
                    for (int db = 0; db < NDB; ++db) {
                        float* dst = part + ((((wk - 1) * WQ + wq) * NDB + db) * 64 + lane) * 16;
#pragma unroll
                        for (int c4 = 0; c4 < 4; ++c4)
                            *(f32x4*)(dst + 4 * c4) = f32x4{acc[db][4 * c4], acc[db][4 * c4 + 1], acc[db][4 * c4 + 2], acc[db][4 * c4 + 3]};
                    }
                }
                __syncthreads();
                if (wk == 0) {
#pragma unroll
                    for (int w2 = 1; w2 < WK; ++w2)
#pragma unroll
                        for (int db = 0; db < NDB; ++db) {
                            const float* src = part + ((((w2 - 1) * WQ + wq) * NDB + db) * 64 + lane) * 16;
#pragma unroll
                            for (int c = 0; c < 16; ++c) acc[db][c] += src[c];
                        }
                }
            }
            const size_t ob = ((size_t)cur.qs * H + cur.h) * D;
            if (a.out_f32) {
                const rsrc_t ro = slice_rsrc((const float*)a.dq + ob, cur.lq, rso, D * 4);
                if (wk == 0) {
                    const int row = cur.t * BM + wq * 32 + r;
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            u32x4 v;
                            for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(acc[db][4 * j + i] * scale);
                            buf_store16(ro, (uint32_t)row * rso + (db * 32 + 8 * j + 4 * hh) * 4, v);
                        }
                }
            } else {
                __bf16* sO = (__bf16*)(smem + C::PART_BYTES);
                if (wk == 0) {
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            u32x2 w;
                            w[0] = pack_bf16x2(acc[db][4 * j] * scale, acc[db][4 * j + 1] * scale);
                            w[1] = pack_bf16x2(acc[db][4 * j + 2] * scale, acc[db][4 * j + 3] * scale);
                            *(u32x2*)(sO + (wq * 32 + r) * KST + db * 32 + 8 * j + 4 * hh) = w;
                        }
                }
                __syncthreads();
                const rsrc_t ro = slice_rsrc((const __bf16*)a.dq + ob, cur.lq, rso, D * 2);
                constexpr int CPR = D / 8;
                for (int ci = tid; ci < BM * CPR; ci += 256) {
                    const int row = ci / CPR, c = ci % CPR;
                    buf_store16(ro, (uint32_t)(cur.t * BM + row) * rso + c * 16, *(const u32x4*)(sO + row * KST + 8 * c));
                }
            }
        }

        if (!has_next) break;
        if constexpr (C::NBUF == 1) {
            __syncthreads();
            commit(nx, 0, nx_first);
        } else {
            if (last) __syncthreads();
            commit(nx, buf ^ 1, nx_first);
            buf ^= 1;
        }
        __syncthreads();
        cur = nx;
    }
}

// =========================================================================
// dK/dV kernel (KV-stationary)
// =========================================================================
template <int D, int WK>
struct DkdvCfg {
    static constexpr int WQ = 4 / WK, BK = 32 * WK, BQ = 32 * WQ;
    static constexpr int NDB = D / 32, NKS = D / 16;
    static constexpr int KST = D + 8, QTST = BQ + 8;
    static constexpr int SZ_Q = BQ * KST, SZ_QT = D * QTST, SZ_K = BK * KST;
    static constexpr int STEP_BYTES = 2 * (SZ_Q + SZ_QT) * 2;   // Q, Q^T, dO, dO^T
    static constexpr int NBUF = (2 * STEP_BYTES + 2 * SZ_K * 2) <= 160 * 1024 ? 2 : 1;
    static constexpr int MAIN = NBUF * STEP_BYTES + 2 * SZ_K * 2;
    static constexpr int PART_BYTES = (WQ - 1) * WK * NDB * 2 * 64 * 16 * 4;
    static constexpr int EPI_BYTES = PART_BYTES + 2 * BK * KST * 2;
    static constexpr int LDS = MAIN > EPI_BYTES ? MAIN : EPI_BYTES;
    static_assert(LDS <= 160 * 1024, "LDS budget exceeded");
};

template <int D, int WK, int ACT>
__global__ __launch_bounds__(256, 1) void dkdv_bf16_kernel(const KernelArgs a) {
    using C = DkdvCfg<D, WK>;
    constexpr int WQ = C::WQ, BK = C::BK, BQ = C::BQ, NDB = C::NDB, NKS = C::NKS;
    constexpr int KST = C::KST, QTST = C::QTST;
    __shared__ __attribute__((aligned(16))) char smem[C::LDS];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wk = wave / WQ, wq = wave % WQ;
    const int r = lane & 31, hh = lane >> 5;

    const int bin = logical_bin(a.P);
    const ItemRec* items = reinterpret_cast<const ItemRec*>(a.items);
    StepIt cur;
    cur.end = a.bin_ptr[bin + 1];
    const int first_item = a.bin_ptr[bin];
    if (first_item >= cur.end) return;
    cur.load(items, a.q_off, a.kv_off, first_item);

    const int H = a.H;
    const uint32_t rs = (uint32_t)H * D * 2;
    const uint32_t rso = (uint32_t)H * D * (a.out_f32 ? 4 : 2);
    const int win = a.window > 0 ? a.window : (1 << 30);
    const float scale = a.scale;
    const __bf16* gq = (const __bf16*)a.q;
    const __bf16* gk = (const __bf16*)a.k;
    const __bf16* gv = (const __bf16*)a.v;
    const __bf16* gdo = (const __bf16*)a.dout;

    __bf16* sKs = (__bf16*)(smem + C::NBUF * C::STEP_BYTES);
    __bf16* sVs = sKs + C::SZ_K;
    auto sQ = [&](int buf) { return (__bf16*)(smem + buf * C::STEP_BYTES); };
    auto sQT = [&](int buf) { return sQ(buf) + C::SZ_Q; };
    auto sO = [&](int buf) { return sQ(buf) + C::SZ_Q + C::SZ_QT; };
    auto sOT = [&](int buf) { return sQ(buf) + 2 * C::SZ_Q + C::SZ_QT; };

    TileStage<BQ, D> stQ, stO;
    TileStage<BK, D> stK, stV;

    auto issue_loads = [&](const StepIt& st, bool with_kv) {
        if (st.has_steps()) {
            const size_t qb = ((size_t)st.qs * H + st.h) * D;
            stQ.load(slice_rsrc(gq + qb, st.lq, rs, D * 2), st.s * BQ, rs, tid);
            stO.load(slice_rsrc(gdo + qb, st.lq, rs, D * 2), st.s * BQ, rs, tid);
        }
        if (with_kv) {
            const size_t kvb = ((size_t)st.ks * H + st.h) * D;
            stK.load(slice_rsrc(gk + kvb, st.lk, rs, D * 2), st.t * BK, rs, tid);
            stV.load(slice_rsrc(gv + kvb, st.lk, rs, D * 2), st.t * BK, rs, tid);
        }
    };
    auto commit = [&](const StepIt& st, int buf, bool with_kv) {
        if (st.has_steps()) {
            stQ.template store_rows<KST>(sQ(buf), tid);
            stQ.template store_cols<QTST>(sQT(buf), tid);
            stO.template store_rows<KST>(sO(buf), tid);
            stO.template store_cols<QTST>(sOT(buf), tid);
        }
        if (with_kv) {
            stK.template store_rows<KST>(sKs, tid);
            stV.template store_rows<KST>(sVs, tid);
        }
    };

    issue_loads(cur, true);
    commit(cur, 0, true);
    __syncthreads();

    f32x16 accK[NDB], accV[NDB];
    bf16x8 kf[NKS], vf[NKS];
    int buf = 0;
    for (;;) {
        const bool first = cur.first(), last = cur.last();
        if (first) {
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                kf[ks] = *(const bf16x8*)(sKs + (wk * 32 + r) * KST + 16 * ks + 8 * hh);
                vf[ks] = *(const bf16x8*)(sVs + (wk * 32 + r) * KST + 16 * ks + 8 * hh);
            }
#pragma unroll
            for (int db = 0; db < NDB; ++db) accK[db] = accV[db] = f32x16{};
        }

        StepIt nx = cur;
        const bool has_next = nx.advance(items, a.q_off, a.kv_off);
        const bool nx_first = has_next && nx.first();
        if (has_next) issue_loads(nx, nx_first);

        const int i0 = cur.s * BQ + wq * 32;   // q rows of this wave
        const int j0 = cur.t * BK + wk * 32;   // kv rows of this wave
        if (cur.has_steps() && block_any(i0, j0, cur.lq, cur.lk, win)) {
            const __bf16* q_t = sQ(buf);
            const __bf16* qt_t = sQT(buf);
            const __bf16* o_t = sO(buf);
            const __bf16* ot_t = sOT(buf);
            f32x16 s = {}, dp = {};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const bf16x8 qa = *(const bf16x8*)(q_t + (wq * 32 + r) * KST + 16 * ks + 8 * hh);
                const bf16x8 oa = *(const bf16x8*)(o_t + (wq * 32 + r) * KST + 16 * ks + 8 * hh);
                s = mfma32(qa, kf[ks], s);
                dp = mfma32(oa, vf[ks], dp);
            }
            // accumulator lane: column = kv row j0 + r, rows = q rows i0 + 8 j + 4 hh + i
            f32x16 p, ds;
            const bool full = block_all(i0, j0, cur.lq, cur.lk, win);
            const int kj = j0 + r;
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                float f, g;
                act_fwd_grad<ACT>(s[c] * scale, f, g);
                const int qi = i0 + 8 * (c >> 2) + 4 * hh + (c & 3);
                const int dd = qi - kj;
                const bool ok = full || (kj < cur.lk && qi < cur.lq && dd < win && -dd < win);
                p[c] = ok ? f : 0.0f;
                ds[c] = ok ? dp[c] * g : 0.0f;
            }
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const bf16x8 pm = acc_to_bf16x8(p, m), dm = acc_to_bf16x8(ds, m);
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const bf16x8 oa = *(const bf16x8*)(ot_t + (db * 32 + r) * QTST + wq * 32 + 16 * m + 8 * hh);
                    accV[db] = mfma32(oa, pm, accV[db]);
                    const bf16x8 qa = *(const bf16x8*)(qt_t + (db * 32 + r) * QTST + wq * 32 + 16 * m + 8 * hh);
                    accK[db] = mfma32(qa, dm, accK[db]);
                }
            }
        }

        if (last) {
            __syncthreads();
            if constexpr (WQ > 1) {
                float* part = (float*)smem;
                if (wq > 0) {
#pragma unroll
                    for (int db = 0; db < NDB; ++db) {
                        float* dk_dst = part + (((((wq - 1) * WK + wk) * NDB + db) * 2 + 0) * 64 + lane) * 16;
                        float* dv_dst = part + (((((wq - 1) * WK + wk) * NDB + db) * 2 + 1) * 64 + lane) * 16;
#pragma unroll
                        for (int c4 = 0; c4 < 4; ++c4) {
                            *(f32x4*)(dk_dst + 4 * c4) = f32x4{accK[db][4 * c4], accK[db][4 * c4 + 1], accK[db][4 * c4 + 2], accK[db][4 * c4 + 3]};
                            *(f32x4*)(dv_dst + 4 * c4) = f32x4{accV[db][4 * c4], accV[db][4 * c4 + 1], accV[db][4 * c4 + 2], accV[db][4 * c4 + 3]};
                        }
                    }
                }
                __syncthreads();
                if (wq == 0) {
#pragma unroll
                    for (int w2 = 1; w2 < WQ; ++w2)
#pragma unroll
                        for (int db = 0; db < NDB; ++db) {
                            const float* ks_ = part + (((((w2 - 1) * WK + wk) * NDB + db) * 2 + 0) * 64 + lane) * 16;
                            const float* vs_ = part + (((((w2 - 1) * WK + wk) * NDB + db) * 2 + 1) * 64 + lane) * 16;
#pragma unroll
                            for (int c = 0; c < 16; ++c) {
                                accK[db][c] += ks_[c];
                                accV[db][c] += vs_[c];
                            }
                        }
                }
            }
            const size_t ob = ((size_t)cur.ks * H + cur.h) * D;
            if (a.out_f32) {
                const rsrc_t rk = slice_rsrc((const float*)a.dk + ob, cur.lk, rso, D * 4);
                const rsrc_t rv = slice_rsrc((const float*)a.dv + ob, cur.lk, rso, D * 4);
                if (wq == 0) {
                    const int row = cur.t * BK + wk * 32 + r;
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            u32x4 vk, vv;
                            for (int i = 0; i < 4; ++i) {
                                vk[i] = __float_as_uint(accK[db][4 * j + i] * scale);
                                vv[i] = __float_as_uint(accV[db][4 * j + i]);
                            }
                            const uint32_t off = (uint32_t)row * rso + (db * 32 + 8 * j + 4 * hh) * 4;
                            buf_store16(rk, off, vk);
                            buf_store16(rv, off, vv);
                        }
                }
            } else {
                __bf16* oK = (__bf16*)(smem + C::PART_BYTES);
                __bf16* oV = oK + BK * KST;
                if (wq == 0) {
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            u32x2 wkk, wvv;
                            wkk[0] = pack_bf16x2(accK[db][4 * j] * scale, accK[db][4 * j + 1] * scale);
                            wkk[1] = pack_bf16x2(accK[db][4 * j + 2] * scale, accK[db][4 * j + 3] * scale);
                            wvv[0] = pack_bf16x2(accV[db][4 * j], accV[db][4 * j + 1]);
                            wvv[1] = pack_bf16x2(accV[db][4 * j + 2], accV[db][4 * j + 3]);
                            const int off = (wk * 32 + r) * KST + db * 32 + 8 * j + 4 * hh;
                            *(u32x2*)(oK + off) = wkk;
                            *(u32x2*)(oV + off) = wvv;
                        }
                }
                __syncthreads();
                const rsrc_t rk = slice_rsrc((const __bf16*)a.dk + ob, cur.lk, rso, D * 2);
                const rsrc_t rv = slice_rsrc((const __bf16*)a.dv + ob, cur.lk, rso, D * 2);
                constexpr int CPR = D / 8;
                for (int ci = tid; ci < BK * CPR; ci += 256) {
                    const int row = ci / CPR, c = ci % CPR;
                    const uint32_t off = (uint32_t)(cur.t * BK + row) * rso + c * 16;
                    buf_store16(rk, off, *(const u32x4*)(oK + row * KST + 8 * c));
                    buf_store16(rv, off, *(const u32x4*)(oV + row * KST + 8 * c));
                }
            }
        }

        if (!has_next) break;
        if constexpr (C::NBUF == 1) {
            __syncthreads();
            commit(nx, 0, nx_first);
        } else {
            if (last) __syncthreads();
            commit(nx, buf ^ 1, nx_first);
            buf ^= 1;
        }
        __syncthreads();
        cur = nx;
    }
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
    void* params[] = {&args};
    return hipLaunchKernel(f, dim3(a.P), dim3(256), params, 0, s);
}

hipError_t GDPA_CAT(launch_dq_bf16_d, GDPA_D)(const KernelArgs& a, int waves, int act, hipStream_t s) {
    return launch(GDPA_CAT(dq_bf16_kernel_ptr_d, GDPA_D)(waves, act), a, s);
}

hipError_t GDPA_CAT(launch_dkdv_bf16_d, GDPA_D)(const KernelArgs& a, int waves, int act, hipStream_t s) {
    return launch(GDPA_CAT(dkdv_bf16_kernel_ptr_d, GDPA_D)(waves, act), a, s);
}

}  // namespace gdpa
