// GDPA forward, bf16 inputs, fp32 MFMA accumulation, for one head dimension
// (compiled once per D with -DGDPA_D=32|64|128).
//
// O = act(Q K^T / sqrt(d)) V over the valid pairs of each sample, with no
// softmax and no row normalisation (GDPA page, aitrends.kr/articles/26275,
// "Key summary" and "Section details": two matrix products with a general
// activation between them; the softmax correction step is gone, so partial
// products over kv tiles simply add).
//
// Work decomposition.  A persistent workgroup (256 threads = 4 waves) walks the
// items of its bin (host planner, zigzag deal) as one flattened sequence of
// (item, kv step) pairs, prefetching the next step's K/V (and the next item's Q)
// into registers while the current step computes, so short-KV items do not
// drain the pipeline (GDPA page, "Section details": software pipelining moved
// from the inner kv loop to the outer loop; loop flattening).
//
// Waves are WQ x WK: each wave owns 32 query rows of the item's q tile
// (BM = 32 WQ rows) and BNW kv rows of each step (BN = WK BNW).  Per 32-row kv
// block a wave computes S^T = K Q^T with MFMA (K from LDS, Q held in registers),
// masks, applies the activation in registers, and feeds the accumulator lanes
// straight back as the B operand of O^T += V^T P^T (V^T from LDS).  When WK > 1
// the waves' partial O are summed through LDS at the item's end.
#include "device.hpp"
#include "kernels.hpp"

#ifndef GDPA_D
#error "compile with -DGDPA_D=<32|64|128>"
#endif

namespace gdpa {
namespace {

template <int D, int WQ, int BNW>
struct FwdCfg {
    static constexpr int WK = 4 / WQ, BM = 32 * WQ, BN = WK * BNW;
    static constexpr int NKB = BNW / 32, NDB = D / 32, NKS = D / 16;
    static constexpr int KST = D + 8;         // row-major tile stride (elements)
    static constexpr int VST = BN + 8;        // transposed V tile stride
    static constexpr int SZ_K = BN * KST, SZ_VT = D * VST, SZ_Q = BM * KST;
    static constexpr int STEP_BYTES = (SZ_K + SZ_VT) * 2;
    static constexpr int PART_BYTES = (WK - 1) * WQ * NDB * 64 * 16 * 4;
    static constexpr int SO_BYTES = BM * KST * 2;
    static constexpr int EPI_BYTES = PART_BYTES + SO_BYTES;
    // double-buffer the step tiles when it fits
    static constexpr int NBUF = (2 * STEP_BYTES + SZ_Q * 2) <= 160 * 1024 ? 2 : 1;
    // At an item's end every region is free (Q is in registers, the next step's
    // tiles are still in staging registers), so the epilogue reuses LDS from 0.
    static constexpr int MAIN = NBUF * STEP_BYTES + SZ_Q * 2;
    static constexpr int LDS = MAIN > EPI_BYTES ? MAIN : EPI_BYTES;
    static_assert(LDS <= 160 * 1024, "LDS budget exceeded");
};

template <int D, int WQ, int BNW, int ACT>
__global__ __launch_bounds__(256, 1) void fwd_bf16_kernel(const KernelArgs a) {
    using C = FwdCfg<D, WQ, BNW>;
    constexpr int WK = C::WK, BM = C::BM, BN = C::BN, NKB = C::NKB, NDB = C::NDB, NKS = C::NKS;
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
    const uint32_t rs = (uint32_t)H * D * 2;                       // bf16 row stride
    const uint32_t rso = (uint32_t)H * D * (a.out_f32 ? 4 : 2);    // output row stride
    const int win = a.window > 0 ? a.window : (1 << 30);
    const float scale = a.scale;
    const __bf16* gq = (const __bf16*)a.q;
    const __bf16* gk = (const __bf16*)a.k;
    const __bf16* gv = (const __bf16*)a.v;

    __bf16* sQ = (__bf16*)(smem + C::NBUF * C::STEP_BYTES);
    auto sK = [&](int buf) { return (__bf16*)(smem + buf * C::STEP_BYTES); };
    auto sVT = [&](int buf) { return (__bf16*)(smem + buf * C::STEP_BYTES) + C::SZ_K; };

    TileStage<BN, D> stK, stV;
    TileStage<BM, D> stQ;

    auto issue_loads = [&](const StepIt& st, bool with_q) {
        if (st.has_steps()) {
            const size_t kvb = ((size_t)st.ks * H + st.h) * D;
            const rsrc_t rk = slice_rsrc(gk + kvb, st.lk, rs, D * 2);
            const rsrc_t rv = slice_rsrc(gv + kvb, st.lk, rs, D * 2);
            stK.load(rk, st.s * BN, rs, tid);
            stV.load(rv, st.s * BN, rs, tid);
        }
        if (with_q) {
            const rsrc_t rq = slice_rsrc(gq + ((size_t)st.qs * H + st.h) * D, st.lq, rs, D * 2);
            stQ.load(rq, st.t * BM, rs, tid);
        }
    };
    auto commit = [&](const StepIt& st, int buf, bool with_q) {
        if (st.has_steps()) {
            stK.template store_rows<KST>(sK(buf), tid);
            stV.template store_cols<VST>(sVT(buf), tid);
        }
        if (with_q) stQ.template store_rows<KST>(sQ, tid);
    };

    // prologue: the first step's tiles
    issue_loads(cur, true);
    commit(cur, 0, true);
    __syncthreads();

    f32x16 acc[NDB];
    bf16x8 qf[NKS];
    int buf = 0;
    for (;;) {
        const bool first = cur.first(), last = cur.last();
        if (first) {
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                qf[ks] = *(const bf16x8*)(sQ + (wq * 32 + r) * KST + 16 * ks + 8 * hh);
#pragma unroll
            for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
        }

        StepIt nx = cur;
        const bool has_next = nx.advance(items, a.q_off, a.kv_off);
        const bool nx_first = has_next && nx.first();
        if (has_next) issue_loads(nx, nx_first);

        // ---- compute this step ----
        const int q0 = cur.t * BM + wq * 32;
        if (cur.has_steps() && q0 < cur.lq) {
            const __bf16* k_t = sK(buf);
            const __bf16* vt_t = sVT(buf);
            bf16x8 pf[NKB][2];
            bool act_blk[NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const int j0 = cur.s * BN + wk * BNW + kb * 32;
                act_blk[kb] = block_any(q0, j0, cur.lq, cur.lk, win);
                if (!act_blk[kb]) continue;
                f32x16 s = {};
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const bf16x8 ka = *(const bf16x8*)(k_t + (wk * BNW + kb * 32 + r) * KST + 16 * ks + 8 * hh);
                    s = mfma32(ka, qf[ks], s);
                }
                f32x16 p;
                if (block_all(q0, j0, cur.lq, cur.lk, win)) {
#pragma unroll
                    for (int c = 0; c < 16; ++c) p[c] = act_fwd<ACT>(s[c] * scale);
                } else {
                    const int qi = q0 + r;
#pragma unroll
                    for (int c = 0; c < 16; ++c) {
                        const int kj = j0 + 8 * (c >> 2) + 4 * hh + (c & 3);
                        const int dd = qi - kj;
                        const bool ok = kj < cur.lk && qi < cur.lq && dd < win && -dd < win;
                        p[c] = ok ? act_fwd<ACT>(s[c] * scale) : 0.0f;
                    }
                }
                pf[kb][0] = acc_to_bf16x8(p, 0);
                pf[kb][1] = acc_to_bf16x8(p, 1);
            }
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                if (!act_blk[kb]) continue;
#pragma unroll
                for (int m = 0; m < 2; ++m) {
#pragma unroll
                    for (int db = 0; db < NDB; ++db) {
                        const bf16x8 va = *(const bf16x8*)(vt_t + (db * 32 + r) * VST + wk * BNW + kb * 32 + 16 * m + 8 * hh);
                        acc[db] = mfma32(va, pf[kb][m], acc[db]);
                    }
                }
            }
        }

        // ---- epilogue: the item's output tile ----
        if (last) {
            __syncthreads();   // every wave is done with this step's tiles
            char* epi = smem;
            if constexpr (WK > 1) {
                float* part = (float*)epi;
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
                    for (int w2 = 1; w2 < WK; ++w2) {
#pragma unroll
                        for (int db = 0; db < NDB; ++db) {
                            const float* src = part + ((((w2 - 1) * WQ + wq) * NDB + db) * 64 + lane) * 16;
#pragma unroll
                            for (int c = 0; c < 16; ++c) acc[db][c] += src[c];
                        }
                    }
                }
            }
            const size_t ob = ((size_t)cur.qs * H + cur.h) * D;
            if (a.out_f32) {
                const rsrc_t ro = slice_rsrc((const float*)a.o + ob, cur.lq, rso, D * 4);
                if (wk == 0) {
                    const int row = cur.t * BM + wq * 32 + r;
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int col = db * 32 + 8 * j + 4 * hh;
                            u32x4 v;
                            for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(acc[db][4 * j + i]);
                            buf_store16(ro, (uint32_t)row * rso + col * 4, v);
                        }
                }
            } else {
                __bf16* sO = (__bf16*)(epi + C::PART_BYTES);
                if (wk == 0) {
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            u32x2 w;
                            w[0] = pack_bf16x2(acc[db][4 * j], acc[db][4 * j + 1]);
                            w[1] = pack_bf16x2(acc[db][4 * j + 2], acc[db][4 * j + 3]);
                            *(u32x2*)(sO + (wq * 32 + r) * KST + db * 32 + 8 * j + 4 * hh) = w;
                        }
                }
                __syncthreads();
                const rsrc_t ro = slice_rsrc((const __bf16*)a.o + ob, cur.lq, rso, D * 2);
                constexpr int CPR = D / 8;
                for (int ci = tid; ci < BM * CPR; ci += 256) {
                    const int row = ci / CPR, c = ci % CPR;
                    const u32x4 v = *(const u32x4*)(sO + row * KST + 8 * c);
                    buf_store16(ro, (uint32_t)(cur.t * BM + row) * rso + c * 16, v);
                }
            }
        }

        if (!has_next) break;
        if constexpr (C::NBUF == 1) {
            __syncthreads();   // single buffer: all waves done before it is overwritten
            commit(nx, 0, nx_first);
        } else {
            if (last) __syncthreads();   // the epilogue's LDS reads are done
            commit(nx, buf ^ 1, nx_first);
            buf ^= 1;
        }
        __syncthreads();
        cur = nx;
    }
}

template <int WQ, int BNW, int ACT>
const void* kptr() {
    return (const void*)&fwd_bf16_kernel<GDPA_D, WQ, BNW, ACT>;
}

template <int WQ, int BNW>
const void* kptr_act(int act) {
    switch (act) {
        case ACT_GELU: return kptr<WQ, BNW, ACT_GELU>();
        case ACT_SILU: return kptr<WQ, BNW, ACT_SILU>();
        case ACT_GELU_POLY: return kptr<WQ, BNW, ACT_GELU_POLY>();
        case ACT_GELU_TAYLOR6: return kptr<WQ, BNW, ACT_GELU_TAYLOR6>();
        case ACT_IDENTITY: return kptr<WQ, BNW, ACT_IDENTITY>();
        case ACT_ONE: return kptr<WQ, BNW, ACT_ONE>();
    }
    return nullptr;
}

}  // namespace

#define GDPA_CAT2(a, b) a##b
#define GDPA_CAT(a, b) GDPA_CAT2(a, b)

const void* GDPA_CAT(fwd_bf16_kernel_ptr_d, GDPA_D)(int waves, int bnw, int act) {
    if (waves == 4 && bnw == 64) return kptr_act<4, 64>(act);
    if (waves == 4 && bnw == 32) return kptr_act<4, 32>(act);
    if (waves == 2 && bnw == 32) return kptr_act<2, 32>(act);
    if (waves == 1 && bnw == 32) return kptr_act<1, 32>(act);
    return nullptr;
}

hipError_t GDPA_CAT(launch_fwd_bf16_d, GDPA_D)(const KernelArgs& a, int waves, int bnw, int act, hipStream_t s) {
    const void* f = GDPA_CAT(fwd_bf16_kernel_ptr_d, GDPA_D)(waves, bnw, act);
    if (!f) return hipErrorInvalidValue;
    if (a.P <= 0) return hipSuccess;
    KernelArgs args = a;
    void* params[] = {&args};
    return hipLaunchKernel(f, dim3(a.P), dim3(256), params, 0, s);
}

}  // namespace gdpa
