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
// (item, kv step) pairs.  Each step's tiles (K, V, and Q when the step starts an
// item) are copied global -> LDS by DMA several steps ahead, so short-KV items do
// not drain the pipeline (GDPA page, "Section details": software pipelining moved
// from the inner kv loop to the outer loop; loop flattening).
//
// Waves are WQ x WK: each wave owns 32 query rows of the item's q tile
// (BM = 32 WQ rows) and BNW kv rows of each step (BN = WK BNW).  Per 32-row kv
// block a wave computes S^T = K Q^T with MFMA (K from LDS, Q held in registers),
// masks, applies the activation in registers, and feeds the accumulator lanes
// straight back as the B operand of O^T += V^T P^T (V^T read from the row-major
// V tile with transposing LDS reads).  When WK > 1 the waves' partial O are
// summed through LDS at the item's end.
#include "kernels.hpp"
#include "pipe.hpp"

#ifndef GDPA_D
#error "compile with -DGDPA_D=<32|64|128>"
#endif

namespace gdpa {
namespace {

template <int D, int WQ, int BNW, int ACT>
struct FwdPol {
    static constexpr int WK = 4 / WQ, BM = 32 * WQ, BN = WK * BNW;
    static constexpr int NKB = BNW / 32, NDB = D / 32, NKS = D / 16;
    using TQ = AsyncTile<BM, D>;
    using TK = AsyncTile<BN, D>;
    static constexpr int OFF_K = TQ::BYTES, OFF_V = TQ::BYTES + TK::BYTES;
    static constexpr int STAGE_BYTES = TQ::BYTES + 2 * TK::BYTES;
    static constexpr int NS = Stages<STAGE_BYTES>::N;
    static constexpr int SOST = D + 8;   // output staging row stride (bf16)
    static constexpr int PART_BYTES = (WK - 1) * WQ * NDB * 64 * 16 * 4;
    static constexpr int SO_BYTES = BM * SOST * 2;
    static_assert(PART_BYTES <= STAGE_BYTES && SO_BYTES <= STAGE_BYTES, "epilogue must fit in a stage");

    const KernelArgs a;   // by value: kept in SGPRs, not re-read from the argument segment
    int tid, lane, wave, wq, wk, r, hh, H, win;
    uint32_t rs, rso;
    float scale;
    rsrc_t empty, rq, rk, rv;   // issuing side: descriptors of the current item's slices
    TQ tq;
    TK tk;
    bf16x8 qf[NKS];
    f32x16 acc[NDB];

    __device__ FwdPol(const KernelArgs& args) : a(args) {
        tid = threadIdx.x;
        lane = tid & 63;
        wave = tid >> 6;
        wq = wave / WK;
        wk = wave % WK;
        r = lane & 31;
        hh = lane >> 5;
        H = a.H;
        win = a.window > 0 ? a.window : (1 << 30);
        rs = (uint32_t)H * D * 2;
        rso = (uint32_t)H * D * (a.out_f32 ? 4 : 2);
        scale = a.scale;
        empty = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.q), 0, 0, 0x00020000);
        rq = rk = rv = empty;
        tq.init(rs, wave, lane);
        tk.init(rs, wave, lane);
    }

    __device__ __forceinline__ void new_item(const Step& st) {
        const size_t kvb = ((size_t)st.r.ks * H + st.r.h) * D;
        rk = slice_rsrc((const __bf16*)a.k + kvb, st.r.lk, rs, D * 2);
        rv = slice_rsrc((const __bf16*)a.v + kvb, st.r.lk, rs, D * 2);
        rq = slice_rsrc((const __bf16*)a.q + ((size_t)st.r.qs * H + st.r.h) * D, st.r.lq, rs, D * 2);
    }

    __device__ __forceinline__ int issue(const Step& st, uint32_t stage) {
        if (!st.valid || !st.has_steps()) return 0;
        int n = 0;
        if (st.first()) n += tq.issue(rq, (uint32_t)(st.r.t * BM) * rs, stage, wave);
        const uint32_t so = (uint32_t)(st.s * BN) * rs;
        n += tk.issue(rk, so, stage + OFF_K, wave);
        n += tk.issue(rv, so, stage + OFF_V, wave);
        return n;
    }

    __device__ __forceinline__ void item_start(const Step& st, const char* stage) {
        if (st.has_steps()) {
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) qf[ks] = lds_row8<D>(stage, wq * 32 + r, 2 * ks + hh);
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
    }

    __device__ __forceinline__ void compute(const Step& st, const char* stage) {
        const int q0 = st.r.t * BM + wq * 32;
        const int lq = st.r.lq, lk = st.r.lk;
        if (!st.has_steps() || q0 >= lq) return;
        const char* kt = stage + OFF_K;
        const char* vt = stage + OFF_V;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            const int jl = wk * BNW + kb * 32;   // kv row inside the step tile
            const int j0 = st.s * BN + jl;
            if (!block_any(q0, j0, lq, lk, win)) continue;
            f32x16 s = {};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) s = mfma32(lds_row8<D>(kt, jl + r, 2 * ks + hh), qf[ks], s);
            f32x16 p;
            if (block_all(q0, j0, lq, lk, win)) {
#pragma unroll
                for (int c = 0; c < 16; ++c) p[c] = act_fwd<ACT>(s[c] * scale);
            } else {
                const int qi = q0 + r;
#pragma unroll
                for (int c = 0; c < 16; ++c) {
                    const int kj = j0 + 8 * (c >> 2) + 4 * hh + (c & 3);
                    const int dd = qi - kj;
                    const bool ok = kj < lk && qi < lq && dd < win && -dd < win;
                    p[c] = ok ? act_fwd<ACT>(s[c] * scale) : 0.0f;
                }
            }
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const bf16x8 pb = acc_to_bf16x8(p, m);
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    acc[db] = mfma32(lds_col8<D>(vt, jl + 16 * m, db * 32, lane), pb, acc[db]);
            }
        }
    }

    __device__ __forceinline__ void epilogue(const Step& st, char* stage) {
        if constexpr (WK > 1) {
            f32x4* part = (f32x4*)stage;
            if (wk > 0) {
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int c4 = 0; c4 < 4; ++c4)
                        part[((((wk - 1) * WQ + wq) * NDB + db) * 4 + c4) * 64 + lane] =
                            f32x4{acc[db][4 * c4], acc[db][4 * c4 + 1], acc[db][4 * c4 + 2], acc[db][4 * c4 + 3]};
            }
            lds_barrier();
            if (wk == 0) {
#pragma unroll
                for (int w2 = 1; w2 < WK; ++w2)
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
#pragma unroll
                        for (int c4 = 0; c4 < 4; ++c4) {
                            const f32x4 v = part[((((w2 - 1) * WQ + wq) * NDB + db) * 4 + c4) * 64 + lane];
                            for (int i = 0; i < 4; ++i) acc[db][4 * c4 + i] += v[i];
                        }
            }
            lds_barrier();
        }
        const size_t ob = ((size_t)st.r.qs * H + st.r.h) * D;
        if (a.out_f32) {
            const rsrc_t ro = slice_rsrc((const float*)a.o + ob, st.r.lq, rso, D * 4);
            if (wk == 0) {
                const int row = st.r.t * BM + wq * 32 + r;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        u32x4 v;
                        for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(acc[db][4 * j + i]);
                        buf_store16(ro, (uint32_t)row * rso + (db * 32 + 8 * j + 4 * hh) * 4, v);
                    }
            }
            return;
        }
        __bf16* sO = (__bf16*)stage;
        if (wk == 0) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    u32x2 w;
                    w[0] = pack_bf16x2(acc[db][4 * j], acc[db][4 * j + 1]);
                    w[1] = pack_bf16x2(acc[db][4 * j + 2], acc[db][4 * j + 3]);
                    *(u32x2*)(sO + (wq * 32 + r) * SOST + db * 32 + 8 * j + 4 * hh) = w;
                }
        }
        lds_barrier();
        const rsrc_t ro = slice_rsrc((const __bf16*)a.o + ob, st.r.lq, rso, D * 2);
        constexpr int CPR = D / 8;
        for (int ci = tid; ci < BM * CPR; ci += 256) {
            const int row = ci / CPR, c = ci % CPR;
            buf_store16(ro, (uint32_t)(st.r.t * BM + row) * rso + c * 16, *(const u32x4*)(sO + row * SOST + 8 * c));
        }
    }
};

template <int D, int WQ, int BNW, int ACT>
__global__ __launch_bounds__(256, 1) void fwd_bf16_kernel(const KernelArgs a, const Rec* __restrict__ recs,
                                                          const int32_t* __restrict__ bin_ptr) {
    using Pol = FwdPol<D, WQ, BNW, ACT>;
    __shared__ __attribute__((aligned(1024))) char smem[Pol::NS * Pol::STAGE_BYTES];
    Pol pol(a);
    run_pipeline(pol, a.P, recs, bin_ptr, smem);
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
    const void* recs = a.items;
    const int32_t* bin_ptr = a.bin_ptr;
    void* params[] = {&args, &recs, &bin_ptr};
    return hipLaunchKernel(f, dim3(a.P), dim3(256), params, 0, s);
}

}  // namespace gdpa
