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
// Two persistent kernels, no atomics (every output row has one owner); a team of
// T waves works on one item at a time (see ring.hpp):
//   * dq   - Q-stationary: an item is T x NB 32-row q blocks of one (sample, head),
//            NB per wave; steps stream 32-row K and V tiles.  S^T = K Q^T and
//            dP^T = V dO^T (Q, dO in registers), then dQ^T += K^T dS^T with the
//            dS^T accumulator lanes as B operand and K^T read from the row-major K
//            tile with transposing LDS reads.
//   * dkdv - KV-stationary: an item is T 32-row kv blocks, one per wave; steps
//            stream 32-row Q and dO tiles.  S = Q K^T and dP = dO V^T (K, V in
//            registers), then dV^T += dO^T P and dK^T += Q^T dS, with dO^T and Q^T
//            read from the row-major tiles with transposing LDS reads.
// Rows beyond a sample's lengths are zero tiles (their P, dS and products
// vanish), so only the local window needs a mask.
//
// With act = softmax the same kernels run the backward of jagged softmax attention
// (JFA): P = exp(S / sqrt(d) - LSE_i) from the forward's row log-sum-exp, and
// dS = P * (dP - D_i) with D_i = sum_c dO_ic O_ic (the softmax Jacobian applied to
// dP); dQ, dK and dV are then the products above.  The two row statistics of the
// 32 q rows of a tile travel with it: one more load instruction per job brings
// them into a side buffer of the tile's ring slot (ring.hpp), and jobs without
// statistics load a zero-range side so that every job counts the same.  Keys past
// a sample's length are masked in dQ: exp(0 - LSE) is not 0 there.  The dQ kernel
// runs first: it also loads each q tile's rows of the forward's O as a third
// stationary tile, forms D from them and the dO rows it holds, and stores the
// (LSE log2 e, D) pairs that the dK/dV kernel's side loads then read.
//
// With the RMSNorm prologue (NORM) the inputs are raw and each row's 1/rms r (from a
// pre-pass, carried in the side buffers like the JFA statistics) scales the
// products: S_ij = r_q,i r_k,j (q_i . k_j) / sqrt(d), dP_ij = r_v,j (dO_i . v_j), and
// the gradients of the normalised rows are dQ^_i = sum_j (dS_ij r_k,j) k_j / sqrt(d),
// dK^_j = sum_i (dS_ij r_q,i) q_i / sqrt(d), dV^_j = sum_i P_ij dO_i.  The item's end
// takes each normalised tensor's gradient through the norm,
// dx = r (dx^ - x^ mean_c(dx^_c x^_c)) with x^ = r x, reading the stationary rows
// once more from their tile in the accumulator's column layout.
#include "bwd_common.hpp"
#include "kernels.hpp"
#include "ring.hpp"

#ifndef GDPA_D
#error "compile with -DGDPA_D=<32|64|128>"
#endif
// GDPA_BWD_PART selects what one object holds: 0 both kernels, 1 the dQ kernel,
// 2 the dK/dV kernel, so that the two can be built with different code
// generation options (the build keeps the dK/dV kernel's MFMA accumulators in
// AGPRs at d = 128, the dQ kernel's in VGPRs)
#ifndef GDPA_BWD_PART
#define GDPA_BWD_PART 0
#endif

namespace gdpa {
namespace {

// =========================================================================
// dQ (Q-stationary)
// =========================================================================
// gradient through the RMSNorm of one 32-row block: lane (r, hh) holds row r's
// columns 32 db + 8 j + 4 hh + i of the normalised input's gradient in element
// 4 j + i of acc[db] and the raw input's same columns in x[db][j]; rr = 1/rms.
template <int NDB>
__device__ __forceinline__ void norm_grad(f32x16 (&acc)[NDB], const bf16x4 (&x)[NDB][4], float rr) {
    float dot = 0.0f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) dot = __builtin_fmaf(acc[db][4 * j + i], (float)x[db][j][i], dot);
    dot += __shfl_xor(dot, 32);
    const float m = dot * rr * rr * (1.0f / (32 * NDB));   // mean(dx^ x^) with x^ = rr x
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[db][4 * j + i] = rr * __builtin_fmaf(-(float)x[db][j][i], m, acc[db][4 * j + i]);
}

// a 32-row tile's row r in the accumulator's column layout (see norm_grad)
template <int D>
__device__ __forceinline__ void lds_acc_row(const char* tile, int r, int hh, bf16x4 (&x)[D / 32][4]) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) x[db][j] = *(const bf16x4*)(tile + tile_off<D>(r, 4 * db + j) + 8 * hh);
}

template <int D, int T, int NB, int ACT, int NORM>
struct DqPol : Common {
    static constexpr bool SM = ACT == ACT_SOFTMAX;
    // stationary tiles, wave-major: (Q, dO) of block 0, (Q, dO) of block 1, ...; softmax:
    // (Q, dO, O) per block, O for the row's D = sum dO * O
    static constexpr int K3 = SM ? 3 : 2;
    static constexpr int NSTAT = K3 * T * NB, NSTRM = 2;
    static constexpr int NDB = D / 32, NKS = D / 16;
    static constexpr int ROWS = 32 * T * NB;   // q rows per item
    static constexpr bool HOIST = TeamShape<D, T, 2>::HOIST;
    Slice wq, wo, wk, wv;   // issuing side
    Slice wst, wnull;       // softmax: LSE of the item's q rows; a zero-range side
    Slice wfo;              // softmax: the forward's O rows
    bf16x8 qf[NB][NKS], of[NB][NKS];
    f32x16 acc[NB][NDB];
    float l2q[NB], dq_[NB];  // softmax: this lane's q row's LSE log2(e) and D
    Slice wrq, wrkv;        // NORM: 1/rms of the item's q rows, (k, v) row pairs
    float rqv[NB];           // NORM: 1/rms of this lane's q row
    bf16x4 qa[NORM ? NB : 1][D / 32][4];   // NORM: this lane's q row in the accumulator's layout

    __device__ DqPol(const KernelArgs& args, int lane_, int wt_) : Common(args, lane_, wt_, D) {}

    __device__ __forceinline__ int qrow(const Rec& c, int b) const { return c.t * ROWS + 32 * (wt * NB + b); }

    __device__ __forceinline__ void walk_item(const Rec& w) {
        const size_t kvb = ((size_t)w.ks * H + w.h) * D;
        wk = slice_of((const __bf16*)a.k + kvb, w.lk, rs, D * 2);
        wv = slice_of((const __bf16*)a.v + kvb, w.lk, rs, D * 2);
        const size_t qb = ((size_t)w.qs * H + w.h) * D;
        wq = slice_of((const __bf16*)a.q + qb, w.lq, rs, D * 2);
        wo = slice_of((const __bf16*)a.dout + qb, w.lq, rs, D * 2);
        if constexpr (SM) {
            wst = slice_of(a.lse + (size_t)w.h * a.Tq + w.qs, w.lq, 4u, 4u);
            wnull = slice_of(a.lse, 0, 4u, 4u);
            wfo = slice_of((const __bf16*)a.o + qb, w.lq, rs, D * 2);
        }
        if constexpr (NORM) {
            wrq = slice_of(a.rq + (size_t)w.h * a.Tq + w.qs, w.lq, 4u, 4u);
            wrkv = slice_of(a.rkv + ((size_t)w.h * a.Tk + w.ks) * 2, w.lk, 8u, 8u);
            wnull = slice_of(a.rkv, 0, 8u, 8u);
        }
    }

    // tile rows at byte offset `off` of `t`; softmax, NORM: and the side at x_off of `xs`
    template <class RingT>
    __device__ __forceinline__ void put(RingT& g, Slice t, uint32_t off, Slice xs, uint32_t x_off) {
        if constexpr (SM || NORM)
            g.issue(t, off, xs, x_off);
        else
            g.issue(t, off);
    }

    template <class RingT>
    __device__ __forceinline__ void issue_job(RingT& g, const Rec& w, int i) {
        if (i < NSTAT) {
            // 0 Q (side: LSE or 1/rms of its rows), 1 dO, 2 O; uniform, so that the
            // descriptor chosen by it stays in scalar registers
            const int kind = __builtin_amdgcn_readfirstlane(i % K3);
            const uint32_t row0 = (uint32_t)(w.t * ROWS + 32 * (i / K3));
            if constexpr (NORM)
                put(g, kind ? wo : wq, row0 * rs, kind ? wnull : wrq, row0 * 4u);
            else if constexpr (SM) {
                if (kind == 0)
                    put(g, wq, row0 * rs, wst, row0 * 4u);
                else if (kind == 1)
                    put(g, wo, row0 * rs, wnull, 0u);
                else
                    put(g, wfo, row0 * rs, wnull, 0u);
            }
            else
                put(g, kind ? wo : wq, row0 * rs, wnull, 0u);
        } else {
            const int rel = i - NSTAT;
            const uint32_t row0 = (uint32_t)((w.s0 + (rel >> 1)) * 32);
            if constexpr (NORM)
                put(g, (rel & 1) ? wv : wk, row0 * rs, (rel & 1) ? wnull : wrkv, row0 * 8u);
            else
                put(g, (rel & 1) ? wv : wk, row0 * rs, wnull, 0u);
        }
    }

    __device__ __forceinline__ void item_begin(const Rec&) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int db = 0; db < NDB; ++db) acc[b][db] = f32x16{};
    }

    // stationary tiles i, i + 1 (jobs job, job + 1): tile u is kind u % K3 (Q, dO, O)
    // of block u / K3, owned by wave u / (K3 NB)
    template <class RingT>
    __device__ __forceinline__ void load_stat(const Rec& c, const RingT& g, int job, int i) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int tile = i + u, blk = tile / K3, kind = tile % K3;
            if (tile >= NSTAT || blk / NB != wt) continue;
            const int b = blk % NB;
            const char* tl = g.tile(job + u);
            if (kind == 0) {
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) qf[b][ks] = lds_row8<D>(tl, r, 2 * ks + hh);
                if constexpr (SM) {   // the Q job's side: LSE of this lane's q row
                    constexpr float L2E = 1.4426950408889634f;
                    l2q[b] = *(const float*)(g.side(job + u) + 4 * r) * L2E;
                }
                if constexpr (NORM) {   // the Q job's side: 1/rms of this lane's q row; the row for the norm's gradient
                    rqv[b] = *(const float*)(g.side(job + u) + 4 * r);
                    lds_acc_row<D>(tl, r, hh, qa[b]);
                }
            } else if (kind == 1) {
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) of[b][ks] = lds_row8<D>(tl, r, 2 * ks + hh);
            } else if constexpr (SM) {   // O: D = sum dO * O of this lane's row, both half-rows
                float dsum = 0.0f;
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const bf16x8 ov = lds_row8<D>(tl, r, 2 * ks + hh);
#pragma unroll
                    for (int e = 0; e < 8; ++e) dsum = __builtin_fmaf((float)of[b][ks][e], (float)ov[e], dsum);
                }
                dsum += __shfl_xor(dsum, 32);
                dq_[b] = dsum;
                // the pair the dK/dV kernel reads (chunks of a cut item write the same values)
                const int row = qrow(c, b) + r;
                if (hh == 0 && row < c.lq)
                    *(float2*)(a.stat + ((size_t)c.h * a.Tq + c.qs + row) * 2) = make_float2(l2q[b], dsum);
            }
        }
    }

    // softmax dS^T of half m (keys j0 + 16 m ..) of block b: lane column = query q0 + r,
    // element e = key j0 + 8 (e/4) + 4 hh + e % 4; keys past lk or outside the window are 0
    __device__ __forceinline__ void softmax_ds(int b, int m, int q0, int j0, int lk, const f32x16& sc,
                                               const f32x16& dp, bf16x8& dsb) const {
        constexpr float L2E = 1.4426950408889634f;
        const float c2 = scale * L2E;
        const bool tail = j0 + 32 > lk;
        const bool band = win > 0 && !band_all(q0, j0, win);
        if (tail || band) {   // one uniform branch per half, not per element
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int e = 8 * m + k;
                const float pe = fast_exp2(__builtin_fmaf(sc[e], c2, -l2q[b]));
                const int jr = 8 * (e >> 2) + 4 * hh + (e & 3);
                const int dd = q0 + r - j0 - jr;
                const bool ok = (j0 + jr < lk) & (!band | in_band(dd, win));
                dsb[k] = (__bf16)(ok ? pe * (dp[e] - dq_[b]) : 0.0f);
            }
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int e = 8 * m + k;
                const float pe = fast_exp2(__builtin_fmaf(sc[e], c2, -l2q[b]));
                dsb[k] = (__bf16)(pe * (dp[e] - dq_[b]));
            }
        }
    }

    template <class RingT>
    __device__ __forceinline__ void step(const Rec& c, int s, const RingT& g, int job) {
        if (win > 0) {   // blocks with no pair in the band add nothing: a step none of whose blocks
                         // has one is skipped (one uniform branch)
            bool dead = true;
#pragma unroll
            for (int b = 0; b < NB; ++b) dead = dead && band_none(qrow(c, b), s * 32, win);
            if (dead) return;
        }
        const char* kt = g.tile(job);
        const char* vt = g.tile(job + 1);
        bf16x8 kop[NKS], vop[NKS];
        // NORM: (1/rms of k, of v) of keys j0 + 8 j + 4 hh + {0, 1} and {2, 3}, from the K job's side
        float4 rkv[NORM ? 4 : 1][2];
        if constexpr (NORM) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                rkv[j][0] = *(const float4*)(g.side(job) + 8 * (8 * j + 4 * hh));
                rkv[j][1] = *(const float4*)(g.side(job) + 8 * (8 * j + 4 * hh) + 16);
            }
        }
        auto fk = [&](int e) -> float {
            if constexpr (NORM) return (e & 1) ? rkv[e >> 2][(e >> 1) & 1].z : rkv[e >> 2][(e >> 1) & 1].x;
            else return 1.0f;
        };
        auto fv = [&](int e) -> float {
            if constexpr (NORM) return (e & 1) ? rkv[e >> 2][(e >> 1) & 1].w : rkv[e >> 2][(e >> 1) & 1].y;
            else return 1.0f;
        };
        if constexpr (HOIST) {
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                kop[ks] = lds_row8<D>(kt, r, 2 * ks + hh);
                vop[ks] = lds_row8<D>(vt, r, 2 * ks + hh);
            }
        }
        f32x16 sc[NB], dp[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) sc[b] = dp[b] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const bf16x8 ko = HOIST ? kop[ks] : lds_row8<D>(kt, r, 2 * ks + hh);
            const bf16x8 vo = HOIST ? vop[ks] : lds_row8<D>(vt, r, 2 * ks + hh);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                sc[b] = mfma32(ko, qf[b][ks], sc[b]);
                dp[b] = mfma32(vo, of[b][ks], dp[b]);
            }
        }
        // dS^T in two halves of 16 keys (accumulator elements 8 m .. 8 m + 7), each
        // consumed by its MFMAs right away: short live ranges for the activation
        const int j0 = s * 32;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            bf16x8 dsb[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int q0 = qrow(c, b);
                if constexpr (SM) {
                    softmax_ds(b, m, q0, j0, c.lk, sc[b], dp[b], dsb[b]);
                } else if (win > 0 && !band_all(q0, j0, win)) {
                    // lane column: query q0 + r; element e: key j0 + 8 (e/4) + 4 hh + e % 4
                    const int base = q0 + r - j0 - 4 * hh;
                    const float cq = NORM ? scale * rqv[b] : scale;
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        const int e = 8 * m + k;
                        float f, gr;
                        act_fwd_grad<ACT>(sc[b][e] * cq * fk(e), f, gr);
                        const int dd = base - (8 * (e >> 2) + (e & 3));
                        dsb[b][k] = (__bf16)(in_band(dd, win) ? dp[b][e] * fv(e) * gr * fk(e) : 0.0f);
                    }
                } else {
                    const float cq = NORM ? scale * rqv[b] : scale;
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        const int e = 8 * m + k;
                        float f, gr;
                        act_fwd_grad<ACT>(sc[b][e] * cq * fk(e), f, gr);
                        dsb[b][k] = (__bf16)(dp[b][e] * fv(e) * gr * fk(e));
                    }
                }
            }
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const bf16x8 kto = lds_col8<D>(kt, 16 * m, db * 32, lane);
#pragma unroll
                for (int b = 0; b < NB; ++b) acc[b][db] = mfma32(kto, dsb[b], acc[b][db]);
            }
        }
    }

    template <class RingT>
    __device__ __forceinline__ void item_end(const Rec& c, const RingT& g, int job) {
        if constexpr (NORM) {   // through the norm (linear in dQ^, so chunks may take it separately)
            if (a.norm & 1) {
#pragma unroll
                for (int b = 0; b < NB; ++b) norm_grad<NDB>(acc[b], qa[b], rqv[b]);
            }
        }
        if (c.part >= 0) {   // one chunk of a cut item: fp32 partial block (scaled by the reduction)
#pragma unroll
            for (int b = 0; b < NB; ++b) store_partial<NDB>(acc[b], a.part, c.part, ROWS, 32 * (wt * NB + b), r, hh);
            return;
        }
        const size_t ob = ((size_t)c.qs * H + c.h) * D;
#pragma unroll
        for (int b = 0; b < NB; ++b)
            store<D>(acc[b], scale, a.dq, ob, c.lq, qrow(c, b), g.tile(job - 2 + (T > 1 ? wt : (b & 1))));
    }

    __device__ __forceinline__ void item_zero(const Rec& c) {
        const size_t ob = ((size_t)c.qs * H + c.h) * D;
#pragma unroll
        for (int b = 0; b < NB; ++b) zero<D>(a.dq, ob, c.lq, qrow(c, b));
        if constexpr (SM) {   // rows without keys: LSE -inf, O = 0, so D = 0
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int row = qrow(c, b) + r;
                if (hh == 0 && row < c.lq)
                    *(float2*)(a.stat + ((size_t)c.h * a.Tq + c.qs + row) * 2) =
                        make_float2(-__builtin_inff(), 0.0f);
            }
        }
    }
};

// =========================================================================
// dK / dV (KV-stationary)
// =========================================================================
template <int D, int T, int ACT, int NORM>
struct DkdvPol : Common {
    // stationary tiles, wave-major: (K, V) of wave 0's block, then wave 1's
    static constexpr int NSTAT = 2 * T, NSTRM = 2;
    static constexpr int NDB = D / 32, NKS = D / 16;
    static constexpr int ROWS = 32 * T;   // kv rows per item
    static constexpr bool HOIST = TeamShape<D, T, 1>::HOIST;
    static constexpr bool SM = ACT == ACT_SOFTMAX;
    Slice wk, wv, wq, wo;   // issuing side
    Slice wst, wnull;       // softmax: row statistics of the item's q rows; a zero-range side
    Slice wrq, wrkv;        // NORM: 1/rms of the item's q rows, (k, v) row pairs
    float rkl, rvl;          // NORM: 1/rms of this lane's k and v rows
    bf16x4 ka[NORM ? D / 32 : 1][4], va[NORM ? D / 32 : 1][4];   // NORM: those rows in the accumulator's layout
    bf16x8 kf[NKS], vf[NKS];
    f32x16 accK[NDB], accV[NDB];

    __device__ DkdvPol(const KernelArgs& args, int lane_, int wt_) : Common(args, lane_, wt_, D) {}

    __device__ __forceinline__ int krow(const Rec& c) const { return c.t * ROWS + 32 * wt; }

    __device__ __forceinline__ void walk_item(const Rec& w) {
        const size_t kvb = ((size_t)w.ks * H + w.h) * D;
        wk = slice_of((const __bf16*)a.k + kvb, w.lk, rs, D * 2);
        wv = slice_of((const __bf16*)a.v + kvb, w.lk, rs, D * 2);
        const size_t qb = ((size_t)w.qs * H + w.h) * D;
        wq = slice_of((const __bf16*)a.q + qb, w.lq, rs, D * 2);
        wo = slice_of((const __bf16*)a.dout + qb, w.lq, rs, D * 2);
        if constexpr (SM) {
            wst = slice_of(a.stat + ((size_t)w.h * a.Tq + w.qs) * 2, w.lq, 8u, 8u);
            wnull = slice_of(a.stat, 0, 8u, 8u);
        }
        if constexpr (NORM) {
            wrq = slice_of(a.rq + (size_t)w.h * a.Tq + w.qs, w.lq, 4u, 4u);
            wrkv = slice_of(a.rkv + ((size_t)w.h * a.Tk + w.ks) * 2, w.lk, 8u, 8u);
            wnull = slice_of(a.rkv, 0, 8u, 8u);
        }
    }

    // tile rows at byte offset `off` of `t`; softmax, NORM: and the side at x_off of `xs`
    template <class RingT>
    __device__ __forceinline__ void put(RingT& g, Slice t, uint32_t off, Slice xs, uint32_t x_off) {
        if constexpr (SM || NORM)
            g.issue(t, off, xs, x_off);
        else
            g.issue(t, off);
    }

    template <class RingT>
    __device__ __forceinline__ void issue_job(RingT& g, const Rec& w, int i) {
        if (i < NSTAT) {
            const uint32_t row0 = (uint32_t)(w.t * ROWS + 32 * (i >> 1));
            put(g, (i & 1) ? wv : wk, row0 * rs, (NORM && !(i & 1)) ? wrkv : wnull, row0 * 8u);
        } else {
            const int rel = i - NSTAT;
            const uint32_t row0 = (uint32_t)((w.s0 + (rel >> 1)) * 32);
            if constexpr (NORM)
                put(g, (rel & 1) ? wo : wq, row0 * rs, (rel & 1) ? wnull : wrq, row0 * 4u);
            else
                put(g, (rel & 1) ? wo : wq, row0 * rs, (rel & 1) ? wnull : wst, row0 * 8u);
        }
    }

    __device__ __forceinline__ void item_begin(const Rec&) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) accK[db] = accV[db] = f32x16{};
    }

    // stationary tiles i (K) and i + 1 (V), owned by wave i / 2
    template <class RingT>
    __device__ __forceinline__ void load_stat(const Rec&, const RingT& g, int job, int i) {
        if ((i >> 1) == wt) {
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                kf[ks] = lds_row8<D>(g.tile(job), r, 2 * ks + hh);
                vf[ks] = lds_row8<D>(g.tile(job + 1), r, 2 * ks + hh);
            }
            if constexpr (NORM) {   // the K job's side: (1/rms of k, of v) of this lane's row; the rows for the norm
                const float2 f = *(const float2*)(g.side(job) + 8 * r);
                rkl = f.x;
                rvl = f.y;
                lds_acc_row<D>(g.tile(job), r, hh, ka);
                lds_acc_row<D>(g.tile(job + 1), r, hh, va);
            }
        }
    }

    template <class RingT>
    __device__ __forceinline__ void step(const Rec& c, int s, const RingT& g, int job) {
        const char* qt = g.tile(job);
        const char* ot = g.tile(job + 1);
        bf16x8 qop[NKS], oop[NKS];
        // softmax: (LSE log2 e, D) of q rows i0 + 8 j + 4 hh + {0, 1} and {2, 3}, from the Q job's side
        float4 st[SM ? 4 : 1][2];
        if constexpr (SM) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                st[j][0] = *(const float4*)(g.side(job) + 8 * (8 * j + 4 * hh));
                st[j][1] = *(const float4*)(g.side(job) + 8 * (8 * j + 4 * hh) + 16);
            }
        }
        // NORM: 1/rms of q rows i0 + 8 j + 4 hh + {0..3}, from the Q job's side
        float4 rqs[NORM ? 4 : 1];
        if constexpr (NORM) {
#pragma unroll
            for (int j = 0; j < 4; ++j) rqs[j] = *(const float4*)(g.side(job) + 4 * (8 * j + 4 * hh));
        }
        auto fq = [&](int e) -> float {
            if constexpr (NORM) return rqs[e >> 2][e & 3];
            else return 1.0f;
        };
        if constexpr (HOIST) {
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                qop[ks] = lds_row8<D>(qt, r, 2 * ks + hh);
                oop[ks] = lds_row8<D>(ot, r, 2 * ks + hh);
            }
        }
        f32x16 sc = {}, dp = {};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            sc = mfma32(HOIST ? qop[ks] : lds_row8<D>(qt, r, 2 * ks + hh), kf[ks], sc);
            dp = mfma32(HOIST ? oop[ks] : lds_row8<D>(ot, r, 2 * ks + hh), vf[ks], dp);
        }
        // accumulator lane: column = kv row j0 + r, element e: q row i0 + 8 (e/4) + 4 hh + e % 4
        const int i0 = s * 32, j0 = krow(c);
        f32x16 p, ds;
        if constexpr (SM) {
            constexpr float L2E = 1.4426950408889634f;
            const float c2 = scale * L2E;
            const bool band = win > 0 && !band_all(i0, j0, win);
            const int base = i0 + 4 * hh - j0 - r;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float4& sv = st[e >> 2][(e >> 1) & 1];
                const float l2 = (e & 1) ? sv.z : sv.x, dd = (e & 1) ? sv.w : sv.y;
                p[e] = fast_exp2(__builtin_fmaf(sc[e], c2, -l2));
                ds[e] = p[e] * (dp[e] - dd);
            }
            if (band) {   // one uniform branch per block
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int k = base + 8 * (e >> 2) + (e & 3);
                    const bool ok = in_band(k, win);
                    p[e] = ok ? p[e] : 0.0f;
                    ds[e] = ok ? ds[e] : 0.0f;
                }
            }
        } else if (win > 0 && !band_all(i0, j0, win)) {
            const int base = i0 + 4 * hh - j0 - r;
            const float ck = NORM ? scale * rkl : scale, cv = NORM ? rvl : 1.0f;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                float f, gr;
                act_fwd_grad<ACT>(sc[e] * ck * fq(e), f, gr);
                const int dd = base + 8 * (e >> 2) + (e & 3);
                const bool ok = in_band(dd, win);
                p[e] = ok ? f : 0.0f;
                ds[e] = ok ? dp[e] * cv * gr * fq(e) : 0.0f;
            }
        } else {
            const float ck = NORM ? scale * rkl : scale, cv = NORM ? rvl : 1.0f;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                float f, gr;
                act_fwd_grad<ACT>(sc[e] * ck * fq(e), f, gr);
                p[e] = f;
                ds[e] = dp[e] * cv * gr * fq(e);
            }
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const bf16x8 pm = acc_to_bf16x8(p, m), dm = acc_to_bf16x8(ds, m);
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                accV[db] = mfma32(lds_col8<D>(ot, 16 * m, db * 32, lane), pm, accV[db]);
                accK[db] = mfma32(lds_col8<D>(qt, 16 * m, db * 32, lane), dm, accK[db]);
            }
        }
    }

    template <class RingT>
    __device__ __forceinline__ void item_end(const Rec& c, const RingT& g, int job) {
        if constexpr (NORM) {   // through the norms (linear in dK^, dV^, so chunks may take them separately)
            if (a.norm & 2) norm_grad<NDB>(accK, ka, rkl);
            if (a.norm & 4) norm_grad<NDB>(accV, va, rvl);
        }
        if (c.part >= 0) {   // one chunk of a cut item: fp32 partial dK, dV blocks (scaled by the reduction)
            store_partial<NDB>(accK, a.part, 2 * c.part, ROWS, 32 * wt, r, hh);
            store_partial<NDB>(accV, a.part, 2 * c.part + 1, ROWS, 32 * wt, r, hh);
            return;
        }
        const size_t ob = ((size_t)c.ks * H + c.h) * D;
        store<D>(accK, scale, a.dk, ob, c.lk, krow(c), g.tile(job - 2 + (T > 1 ? wt : 0)));
        store<D>(accV, 1.0f, a.dv, ob, c.lk, krow(c), g.tile(job - 2 + (T > 1 ? wt : 1)));
    }

    __device__ __forceinline__ void item_zero(const Rec& c) {
        const size_t ob = ((size_t)c.ks * H + c.h) * D;
        zero<D>(a.dk, ob, c.lk, krow(c));
        zero<D>(a.dv, ob, c.lk, krow(c));
    }
};

template <int D, int T, int NB, int ACT, int NORM>
__global__ __launch_bounds__((TeamShape<D, T, 2>::THREADS), (TeamShape<D, T, 2>::WPE)) void dq_bf16_kernel(
    const KernelArgs a, const Rec* __restrict__ recs, const int32_t* __restrict__ bin_ptr) {
    using RingT = Ring<D, T, TeamShape<D, T, 2>::LDS, (ACT == ACT_SOFTMAX || NORM) ? 1 : 0>;
    __shared__ __attribute__((aligned(1024))) char smem[RingT::BYTES];
    const int wt = T > 1 ? __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6) : 0;
    const int lane = threadIdx.x & 63;
    DqPol<D, T, NB, ACT, NORM> pol(a, lane, wt);
    run_team<DqPol<D, T, NB, ACT, NORM>, RingT, T>(pol, a.P, recs, bin_ptr, smem, (uint32_t)a.H * D * 2, wt, lane);
}

template <int D, int T, int ACT, int NORM>
__global__ __launch_bounds__((TeamShape<D, T, 1>::THREADS), (TeamShape<D, T, 1>::WPE)) void dkdv_bf16_kernel(
    const KernelArgs a, const Rec* __restrict__ recs, const int32_t* __restrict__ bin_ptr) {
    using RingT = Ring<D, T, TeamShape<D, T, 1>::LDS, (ACT == ACT_SOFTMAX || NORM) ? 1 : 0>;
    __shared__ __attribute__((aligned(1024))) char smem[RingT::BYTES];
    const int wt = T > 1 ? __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6) : 0;
    const int lane = threadIdx.x & 63;
    DkdvPol<D, T, ACT, NORM> pol(a, lane, wt);
    run_team<DkdvPol<D, T, ACT, NORM>, RingT, T>(pol, a.P, recs, bin_ptr, smem, (uint32_t)a.H * D * 2, wt, lane);
}

template <int T, int NB, int ACT, int NORM = 0>
const void* dq_ptr() {
    return (const void*)&dq_bf16_kernel<GDPA_D, T, NB, ACT, NORM>;
}
template <int T, int NB, int ACT, int NORM = 0>
const void* dkdv_ptr() {
    return (const void*)&dkdv_bf16_kernel<GDPA_D, T, ACT, NORM>;
}

#define GDPA_ACT_SWITCH(F, T, NB)                                                           \
    if (act & kActNorm) {   /* the RMSNorm-prologue variants */                             \
        switch (act & ~kActNorm) {                                                          \
            case ACT_GELU: return F<T, NB, ACT_GELU, 1>();                                  \
            case ACT_SILU: return F<T, NB, ACT_SILU, 1>();                                  \
            case ACT_GELU_POLY: return F<T, NB, ACT_GELU_POLY, 1>();                        \
            case ACT_GELU_TAYLOR6: return F<T, NB, ACT_GELU_TAYLOR6, 1>();                  \
            case ACT_IDENTITY: return F<T, NB, ACT_IDENTITY, 1>();                          \
        }                                                                                   \
        return nullptr;                                                                     \
    }                                                                                       \
    switch (act) {                                                                          \
        case ACT_GELU: return F<T, NB, ACT_GELU>();                                         \
        case ACT_SILU: return F<T, NB, ACT_SILU>();                                         \
        case ACT_GELU_POLY: return F<T, NB, ACT_GELU_POLY>();                               \
        case ACT_GELU_TAYLOR6: return F<T, NB, ACT_GELU_TAYLOR6>();                         \
        case ACT_IDENTITY: return F<T, NB, ACT_IDENTITY>();                                 \
    }                                                                                       \
    return nullptr;

template <int T, int NB>
const void* dq_act(int act) { GDPA_ACT_SWITCH(dq_ptr, T, NB) }
template <int T>
const void* dkdv_act(int act) { GDPA_ACT_SWITCH(dkdv_ptr, T, 1) }

}  // namespace

#define GDPA_CAT2(a, b) a##b
#define GDPA_CAT(a, b) GDPA_CAT2(a, b)

#if GDPA_BWD_PART != 2
const void* GDPA_CAT(dq_bf16_kernel_ptr_d, GDPA_D)(int team, int nb, int act) {
    if (act == ACT_SOFTMAX) {   // one-wave teams (the side buffers of the ring)
        if (team == 1 && nb == 1) return dq_ptr<1, 1, ACT_SOFTMAX>();
        if (team == 1 && nb == 2) return dq_ptr<1, 2, ACT_SOFTMAX>();
        return nullptr;
    }
    if (team == 1 && nb == 1) return dq_act<1, 1>(act);
    if (team == 1 && nb == 2) return dq_act<1, 2>(act);
#if GDPA_D == 128
    if (team == 2 && nb == 1) return dq_act<2, 1>(act);
#endif
    return nullptr;
}

#endif

#if GDPA_BWD_PART != 1
const void* GDPA_CAT(dkdv_bf16_kernel_ptr_d, GDPA_D)(int team, int nb, int act) {
    if (nb != 1) return nullptr;
#if GDPA_D == 128
    // plain activations run on the 16-row kernel (32 team rows per item: two waves
    // for a one-wave layout, four for a two-wave layout), fp8 inputs too
    const int plain = act & ~kActF8Bwd;
    if (plain >= ACT_GELU && plain <= ACT_IDENTITY) return dkdv16_kernel_ptr(32 * team, act);
    if (act & kActF8Bwd) return nullptr;
#endif
    if (act == ACT_SOFTMAX) return team == 1 ? dkdv_ptr<1, 1, ACT_SOFTMAX>() : nullptr;
    if (team == 1) return dkdv_act<1>(act);
#if GDPA_D == 128
    if (team == 2) return dkdv_act<2>(act);
#endif
    return nullptr;
}

#endif

static hipError_t launch(const void* f, const KernelArgs& a, int team, hipStream_t s) {
    if (!f) return hipErrorInvalidValue;
    if (a.P <= 0) return hipSuccess;
    KernelArgs args = a;
    const void* recs = a.items;
    const int32_t* bin_ptr = a.bin_ptr;
    void* params[] = {&args, &recs, &bin_ptr};
    return hipLaunchKernel(f, dim3(a.P), dim3(64 * team), params, 0, s);
}

#if GDPA_BWD_PART != 2
hipError_t GDPA_CAT(launch_dq_bf16_d, GDPA_D)(const KernelArgs& a, int team, int nb, int act, hipStream_t s) {
    return launch(GDPA_CAT(dq_bf16_kernel_ptr_d, GDPA_D)(team, nb, act), a, team, s);
}
#endif

#if GDPA_BWD_PART != 1
hipError_t GDPA_CAT(launch_dkdv_bf16_d, GDPA_D)(const KernelArgs& a, int team, int nb, int act, hipStream_t s) {
    const void* f = GDPA_CAT(dkdv_bf16_kernel_ptr_d, GDPA_D)(team, nb, act);
#if GDPA_D == 128
    if (f && f == dkdv16_kernel_ptr(32 * team, act)) return launch(f, a, 2 * team, s);   // 16 rows per wave
#endif
    return launch(f, a, team, s);
}
#endif

}  // namespace gdpa
