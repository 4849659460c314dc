// GDPA backward in one pass for the two shapes where one side of every sample
// fits one 32-row tile (compiled once per D with -DGDPA_D=32|64|128):
//
//   * user-ad cross-attention (every Lk <= 32): the KV-stationary pass already
//     visits all keys of a query tile in one step, so dQ of that tile is complete
//     there: dQ = dS K / sqrt(d) is formed and stored per step, next to the dK and
//     dV accumulation;
//   * PMA (every Lq <= 32): the Q-stationary pass visits all queries of a key tile
//     in one step, so dK = dS^T Q / sqrt(d) and dV = P^T dO of that tile are
//     formed and stored per step, next to the dQ accumulation.
//
// JFA (softmax attention) runs the KV-stationary pass too: with the keys of a query
// tile all in one step, D_i = sum_c dO_ic O_ic (the softmax Jacobian's row term)
// equals sum_j P_ij dP_ij over that step's keys (O_i = sum_j P_ij V_j), so the
// pass forms it from the P and dP it already holds, by a sum across the 32 lanes
// of a key column, and needs from the forward only LSE, which rides with each Q
// tile in the ring's side buffer.
//
// Either way the second kernel, and its full pass over the long side, goes away
// (GDPA page, aitrends.kr/articles/26275, "Section details": backward without the
// softmax row statistics; S is recomputed).  The products that need the other
// orientation of P or dS take it through a 32 x 32 bf16 scratch tile in LDS
// (stage_transpose32), in the slot of a streamed tile the step has finished with;
// the stationary operands of those products (K^T, or Q^T and dO^T) are read into
// registers once per item.  Rows beyond a sample's lengths are zero tiles, so only
// the local window needs a mask.
//
// With fp8 inputs (F8: Q, K and dO as OCP e4m3 bytes, one factor per tensor; V
// bf16) their tiles are one byte per element (half a slot).  S runs on the fp8
// MFMA (row reads of Q and K in either orientation); dP = dO V^T on the bf16 MFMA,
// with dO's rows widened exactly to bf16 (every e4m3 value is a bf16 value); the
// products against P and dS (dV, dK, dQ) take their fp8 tile operand through an
// 8-bit transposing read, widened the same way.  The tensors' factors are applied
// to S, to dP and to each stored gradient.
#include "bwd_common.hpp"

#ifndef GDPA_D
#error "compile with -DGDPA_D=<32|64|128>"
#endif

namespace gdpa {
namespace {

// =========================================================================
// KV-stationary: dK, dV accumulated, dQ stored per step (every Lk <= 32)
// =========================================================================
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// sum of x over the 32 lanes of each half of the wave (every lane gets its half's sum)
__device__ __forceinline__ float half_sum32(float x) {
    x += dpp_f32<0xB1>(x);    // quad_perm [1, 0, 3, 2]
    x += dpp_f32<0x4E>(x);    // quad_perm [2, 3, 0, 1]
    x += dpp_f32<0x124>(x);   // row_ror:4
    x += dpp_f32<0x128>(x);   // row_ror:8: the 16-lane row's sum
    return x + __shfl_xor(x, 16);
}

template <int D, int ACT, bool F8 = false>
struct KvFusedPol : Common {
    static constexpr int NSTAT = 2, NSTRM = 2;   // (K, V), then (Q, dO) per step
    static constexpr int NDB = D / 32, NKS = D / 16;
    static constexpr bool HOIST = TeamShape<D, 1, 2>::HOIST;
    static constexpr bool SM = ACT == ACT_SOFTMAX;
    static constexpr int XJ = SM ? 1 : 0;        // softmax: LSE of each Q tile's rows in a side buffer
    static_assert(!(F8 && SM), "fp8 inputs for the GDPA activations only");
    Slice wk, wv, wq, wo;   // issuing side
    Slice wst, wnull;       // softmax: LSE of the item's q rows; a zero-range side (F8: a zero-range tile)
    bf16x8 kf[F8 ? 1 : NKS], vf[NKS], kt[2][NDB];
    long kf8[F8 ? NKS : 1];   // F8: K rows as fp8 operands
    f32x16 accK[NDB], accV[NDB];

    __device__ KvFusedPol(const KernelArgs& args, int lane_) : Common(args, lane_, 0, D) {}

    __device__ __forceinline__ void walk_item(const Rec& w) {
        const size_t kvb = ((size_t)w.ks * H + w.h) * D;
        const size_t qb = ((size_t)w.qs * H + w.h) * D;
        if constexpr (F8) {   // one-byte rows, H D bytes apart
            wk = slice_of((const uint8_t*)a.k + kvb, w.lk, rs / 2, D);
            wv = slice_of((const __bf16*)a.v + kvb, w.lk, rs, D * 2);
            wq = slice_of((const uint8_t*)a.q + qb, w.lq, rs / 2, D);
            wo = slice_of((const uint8_t*)a.dout + qb, w.lq, rs / 2, D);
            wnull = slice_of(a.q, 0, rs / 2, D);
            return;
        }
        wk = slice_of((const __bf16*)a.k + kvb, w.lk, rs, D * 2);
        wv = slice_of((const __bf16*)a.v + kvb, w.lk, rs, D * 2);
        wq = slice_of((const __bf16*)a.q + qb, w.lq, rs, D * 2);
        wo = slice_of((const __bf16*)a.dout + qb, w.lq, rs, D * 2);
        if constexpr (SM) {
            wst = slice_of(a.lse + (size_t)w.h * a.Tq + w.qs, w.lq, 4u, 4u);
            wnull = slice_of(a.lse, 0, 4u, 4u);
        }
    }

    // tile rows at byte offset `off` of `t`; softmax: and the side at x_off of `xs`
    template <class RingT>
    __device__ __forceinline__ void put(RingT& g, Slice t, uint32_t off, Slice xs, uint32_t x_off) {
        if constexpr (SM)
            g.issue(t, off, xs, x_off);
        else
            g.issue(t, off);
    }

    template <class RingT>
    __device__ __forceinline__ void ring_ready(RingT& g, int lane_) {
        if constexpr (F8) g.init8(rs / 2, lane_);
    }

    template <class RingT>
    __device__ __forceinline__ void issue_job(RingT& g, const Rec& w, int i) {
        if constexpr (F8) {
            if (i == 0)
                g.issue8(wk, (uint32_t)(w.t * 32) * (rs / 2), wnull);
            else if (i == 1)
                g.issue(wv, (uint32_t)(w.t * 32) * rs);
            else
                g.issue8(((i - NSTAT) & 1) ? wo : wq, (uint32_t)((w.s0 + ((i - NSTAT) >> 1)) * 32) * (rs / 2),
                         wnull);
            return;
        }
        if (i < NSTAT) {
            put(g, i == 0 ? wk : wv, (uint32_t)(w.t * 32) * rs, wnull, 0u);
        } else {
            const int rel = i - NSTAT;
            const uint32_t row0 = (uint32_t)((w.s0 + (rel >> 1)) * 32);
            put(g, (rel & 1) ? wo : wq, row0 * rs, (rel & 1) ? wnull : wst, row0 * 4u);
        }
    }

    __device__ __forceinline__ void item_begin(const Rec&) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) accK[db] = accV[db] = f32x16{};
    }

    // the transposed operand of the products against P and dS (F8: widened to bf16)
    __device__ __forceinline__ bf16x8 col8(const char* tile, int row0, int col0) const {
        if constexpr (F8)
            return lds_col8_f8<D>(tile, row0, col0, lane);
        else
            return lds_col8<D>(tile, row0, col0, lane);
    }

    template <class RingT>
    __device__ __forceinline__ void load_stat(const Rec&, const RingT& g, int job, int) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            if constexpr (F8)
                kf8[ks] = lds_row8_f8<D>(g.tile(job), r, ks, hh);
            else
                kf[ks] = lds_row8<D>(g.tile(job), r, 2 * ks + hh);
            vf[ks] = lds_row8<D>(g.tile(job + 1), r, 2 * ks + hh);
        }
        // K^T, the A operand of dQ^T = K^T dS^T
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int db = 0; db < NDB; ++db) kt[m][db] = col8(g.tile(job), 16 * m, db * 32);
    }

    template <class RingT>
    __device__ __forceinline__ void step(const Rec& c, int s, const RingT& g, int job) {
        char* qt = g.tile(job);
        char* ot = g.tile(job + 1);
        f32x16 sc = {}, dp = {};
        if constexpr (F8) {   // S on the fp8 MFMA (e4m3 rows of Q against K); dP from dO's rows widened
            long qop[NKS], oop[NKS];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                qop[ks] = lds_row8_f8<D>(qt, r, ks, hh);
                oop[ks] = lds_row8_f8<D>(ot, r, ks, hh);
            }
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                sc = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(qop[ks], kf8[ks], sc, 0, 0, 0);
                dp = mfma32(widen_e4m3((int)oop[ks], (int)(oop[ks] >> 32)), vf[ks], dp);
            }
        } else {
            bf16x8 qop[NKS], oop[NKS];
            if constexpr (HOIST) {
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    qop[ks] = lds_row8<D>(qt, r, 2 * ks + hh);
                    oop[ks] = lds_row8<D>(ot, r, 2 * ks + hh);
                }
            }
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                sc = mfma32(HOIST ? qop[ks] : lds_row8<D>(qt, r, 2 * ks + hh), kf[ks], sc);
                dp = mfma32(HOIST ? oop[ks] : lds_row8<D>(ot, r, 2 * ks + hh), vf[ks], dp);
            }
        }
        const float dpm = F8 ? a.f8_dp : 1.0f;   // dP's factor (F8: s_do)
        // accumulator lane: column = key j0 + r, element e: query i0 + 8 (e/4) + 4 hh + e % 4
        const int i0 = s * 32, j0 = c.t * 32;
        const bool masked = win > 0 && !band_all(i0, j0, win);
        const int base = i0 + 4 * hh - j0 - r;
        bf16x8 pm[2], dm[2];
        if constexpr (SM) {
            // P = exp(S - LSE) (log2 units), zero for keys past the sample's length (a zero
            // K row gives S = 0, not P = 0) and outside the band; D_i = sum_j P_ij dP_ij
            constexpr float L2E = 1.4426950408889634f;
            const float c2 = scale * L2E;
            float4 ls[4];   // LSE of q rows i0 + 8 j + 4 hh + {0..3}
#pragma unroll
            for (int j = 0; j < 4; ++j) ls[j] = *(const float4*)(g.side(job) + 4 * (8 * j + 4 * hh));
            const bool key_ok = r < c.lk - j0;
            float p[16], dsum[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                float pe = fast_exp2(__builtin_fmaf(sc[e], c2, -ls[e >> 2][e & 3] * L2E));
                bool ok = key_ok;
                if (masked) ok = ok && in_band(base + 8 * (e >> 2) + (e & 3), win);
                p[e] = ok ? pe : 0.0f;
                dsum[e] = p[e] * dp[e];
            }
#pragma unroll
            for (int e = 0; e < 16; ++e) dsum[e] = half_sum32(dsum[e]);
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int e8 = 0; e8 < 8; ++e8) {
                    const int e = 8 * m + e8;
                    pm[m][e8] = (__bf16)p[e];
                    dm[m][e8] = (__bf16)(p[e] * (dp[e] - dsum[e]));
                }
        } else {
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int e8 = 0; e8 < 8; ++e8) {
                    const int e = 8 * m + e8;
                    float f, gr;
                    act_fwd_grad<ACT>(sc[e] * scale, f, gr);
                    float ds = dp[e] * (F8 ? dpm * gr : gr);
                    if (masked) {
                        const int dd = base + 8 * (e >> 2) + (e & 3);
                        const bool ok = in_band(dd, win);
                        f = ok ? f : 0.0f;
                        ds = ok ? ds : 0.0f;
                    }
                    pm[m][e8] = (__bf16)f;
                    dm[m][e8] = (__bf16)ds;
                }
        }
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                accV[db] = mfma32(col8(ot, 16 * m, db * 32), pm[m], accV[db]);
                accK[db] = mfma32(col8(qt, 16 * m, db * 32), dm[m], accK[db]);
            }
        // dQ^T = K^T dS^T for this query tile: dS^T through a scratch tile in the dO
        // slot (the products above have read it), dQ staged in the Q slot
        stage_transpose32(dm, ot, r, hh);
        bf16x8 dst[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) dst[m] = lds_col8<32>(ot, 16 * m, 0, lane);
        f32x16 dq[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            dq[db] = mfma32(kt[0][db], dst[0], f32x16{});
            dq[db] = mfma32(kt[1][db], dst[1], dq[db]);
        }
        const size_t qb = ((size_t)c.qs * H + c.h) * D;
        store<D>(dq, F8 ? a.f8_dq : scale, a.dq, qb, c.lq, i0, qt);
    }

    template <class RingT>
    __device__ __forceinline__ void item_end(const Rec& c, const RingT& g, int job) {
        if (c.part >= 0) {   // one chunk of a cut item: fp32 partial dK, dV blocks (scaled by the reduction)
            store_partial<NDB>(accK, a.part, 2 * c.part, 32, 0, r, hh);
            store_partial<NDB>(accV, a.part, 2 * c.part + 1, 32, 0, r, hh);
            return;
        }
        const size_t ob = ((size_t)c.ks * H + c.h) * D;
        store<D>(accK, F8 ? a.f8_dk : scale, a.dk, ob, c.lk, c.t * 32, g.tile(job - 2));
        store<D>(accV, F8 ? a.f8_dv : 1.0f, a.dv, ob, c.lk, c.t * 32, g.tile(job - 1));
    }

    // no queries: dK and dV are zero (the sample has no dQ rows)
    __device__ __forceinline__ void item_zero(const Rec& c) {
        const size_t ob = ((size_t)c.ks * H + c.h) * D;
        zero<D>(a.dk, ob, c.lk, c.t * 32);
        zero<D>(a.dv, ob, c.lk, c.t * 32);
    }
};

// =========================================================================
// Q-stationary: dQ accumulated, dK and dV stored per step (every Lq <= 32)
// =========================================================================
template <int D, int ACT, bool F8 = false>
struct QFusedPol : Common {
    static constexpr int NSTAT = 2, NSTRM = 2;   // (Q, dO), then (K, V) per step
    static constexpr int NDB = D / 32, NKS = D / 16;
    static constexpr bool HOIST = TeamShape<D, 1, 2>::HOIST;
    Slice wq, wo, wk, wv;   // issuing side
    Slice wnull;            // F8: a zero-range tile
    bf16x8 qf[F8 ? 1 : NKS], of[NKS], qt[2][NDB], ot[2][NDB];   // (F8: of, qt, ot widened)
    long qf8[F8 ? NKS : 1];   // F8: Q rows as fp8 operands
    f32x16 acc[NDB];

    __device__ QFusedPol(const KernelArgs& args, int lane_) : Common(args, lane_, 0, D) {}

    __device__ __forceinline__ void walk_item(const Rec& w) {
        const size_t kvb = ((size_t)w.ks * H + w.h) * D;
        const size_t qb = ((size_t)w.qs * H + w.h) * D;
        if constexpr (F8) {   // one-byte rows, H D bytes apart
            wk = slice_of((const uint8_t*)a.k + kvb, w.lk, rs / 2, D);
            wv = slice_of((const __bf16*)a.v + kvb, w.lk, rs, D * 2);
            wq = slice_of((const uint8_t*)a.q + qb, w.lq, rs / 2, D);
            wo = slice_of((const uint8_t*)a.dout + qb, w.lq, rs / 2, D);
            wnull = slice_of(a.q, 0, rs / 2, D);
            return;
        }
        wk = slice_of((const __bf16*)a.k + kvb, w.lk, rs, D * 2);
        wv = slice_of((const __bf16*)a.v + kvb, w.lk, rs, D * 2);
        wq = slice_of((const __bf16*)a.q + qb, w.lq, rs, D * 2);
        wo = slice_of((const __bf16*)a.dout + qb, w.lq, rs, D * 2);
    }

    template <class RingT>
    __device__ __forceinline__ void ring_ready(RingT& g, int lane_) {
        if constexpr (F8) g.init8(rs / 2, lane_);
    }

    template <class RingT>
    __device__ __forceinline__ void issue_job(RingT& g, const Rec& w, int i) {
        if constexpr (F8) {
            if (i < NSTAT) {
                g.issue8(i == 0 ? wq : wo, (uint32_t)(w.t * 32) * (rs / 2), wnull);
            } else {
                const int rel = i - NSTAT;
                const uint32_t row0 = (uint32_t)((w.s0 + (rel >> 1)) * 32);
                if (rel & 1)
                    g.issue(wv, row0 * rs);
                else
                    g.issue8(wk, row0 * (rs / 2), wnull);
            }
            return;
        }
        if (i < NSTAT) {
            g.issue(i == 0 ? wq : wo, (uint32_t)(w.t * 32) * rs);
        } else {
            const int rel = i - NSTAT;
            g.issue((rel & 1) ? wv : wk, (uint32_t)((w.s0 + (rel >> 1)) * 32) * rs);
        }
    }

    __device__ __forceinline__ void item_begin(const Rec&) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
    }

    // the transposed operand of the products against P and dS (F8: widened to bf16)
    __device__ __forceinline__ bf16x8 col8(const char* tile, int row0, int col0) const {
        if constexpr (F8)
            return lds_col8_f8<D>(tile, row0, col0, lane);
        else
            return lds_col8<D>(tile, row0, col0, lane);
    }

    template <class RingT>
    __device__ __forceinline__ void load_stat(const Rec&, const RingT& g, int job, int) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            if constexpr (F8) {
                qf8[ks] = lds_row8_f8<D>(g.tile(job), r, ks, hh);
                const long o8 = lds_row8_f8<D>(g.tile(job + 1), r, ks, hh);
                of[ks] = widen_e4m3((int)o8, (int)(o8 >> 32));
            } else {
                qf[ks] = lds_row8<D>(g.tile(job), r, 2 * ks + hh);
                of[ks] = lds_row8<D>(g.tile(job + 1), r, 2 * ks + hh);
            }
        }
        // Q^T and dO^T, the A operands of dK^T = Q^T dS and dV^T = dO^T P
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                qt[m][db] = col8(g.tile(job), 16 * m, db * 32);
                ot[m][db] = col8(g.tile(job + 1), 16 * m, db * 32);
            }
    }

    template <class RingT>
    __device__ __forceinline__ void step(const Rec& c, int s, const RingT& g, int job) {
        char* kt = g.tile(job);
        char* vt = g.tile(job + 1);
        f32x16 sc = {}, dp = {};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            if constexpr (F8)   // S on the fp8 MFMA (e4m3 rows of K against Q)
                sc = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(lds_row8_f8<D>(kt, r, ks, hh), qf8[ks], sc, 0, 0, 0);
            else
                sc = mfma32(lds_row8<D>(kt, r, 2 * ks + hh), qf[ks], sc);
            dp = mfma32(lds_row8<D>(vt, r, 2 * ks + hh), of[ks], dp);
        }
        const float dpm = F8 ? a.f8_dp : 1.0f;   // dP's factor (F8: s_do)
        // accumulator lane: column = query q0 + r, element e: key j0 + 8 (e/4) + 4 hh + e % 4
        const int q0 = c.t * 32, j0 = s * 32;
        const bool masked = win > 0 && !band_all(q0, j0, win);
        const int base = q0 + r - j0 - 4 * hh;
        bf16x8 pm[2], dm[2];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int e8 = 0; e8 < 8; ++e8) {
                const int e = 8 * m + e8;
                float f, gr;
                act_fwd_grad<ACT>(sc[e] * scale, f, gr);
                float ds = dp[e] * (F8 ? dpm * gr : gr);
                if (masked) {
                    const int dd = base - (8 * (e >> 2) + (e & 3));
                    const bool ok = in_band(dd, win);
                    f = ok ? f : 0.0f;
                    ds = ok ? ds : 0.0f;
                }
                pm[m][e8] = (__bf16)f;
                dm[m][e8] = (__bf16)ds;
            }
        // dQ^T += K^T dS^T
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int db = 0; db < NDB; ++db) acc[db] = mfma32(col8(kt, 16 * m, db * 32), dm[m], acc[db]);
        // dK^T = Q^T dS and dV^T = dO^T P for this key tile: dS and P through
        // 32 x 32 scratch tiles at the start of the V and K slots (every read of
        // those tiles above is done; a d = 32 slot holds exactly one), then dK
        // staged in the K slot and dV in the V slot once the scratch is read
        char* sds = vt;
        char* sp = kt;
        stage_transpose32(dm, sds, r, hh);
        stage_transpose32(pm, sp, r, hh);
        bf16x8 dsk[2], pk[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            dsk[m] = lds_col8<32>(sds, 16 * m, 0, lane);
            pk[m] = lds_col8<32>(sp, 16 * m, 0, lane);
        }
        const size_t kvb = ((size_t)c.ks * H + c.h) * D;
        if (a.out_f32) {
            f32x16 dk[NDB], dv[NDB];
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                dk[db] = mfma32(qt[1][db], dsk[1], mfma32(qt[0][db], dsk[0], f32x16{}));
                dv[db] = mfma32(ot[1][db], pk[1], mfma32(ot[0][db], pk[0], f32x16{}));
            }
            store<D>(dk, F8 ? a.f8_dk : scale, a.dk, kvb, c.lk, j0, kt);
            store<D>(dv, F8 ? a.f8_dv : 1.0f, a.dv, kvb, c.lk, j0, vt);
            return;
        }
        // one 32-column part at a time keeps the per-step accumulators small
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const f32x16 dk = mfma32(qt[1][db], dsk[1], mfma32(qt[0][db], dsk[0], f32x16{}));
            stage_part<D>(dk, db, F8 ? a.f8_dk : scale, kt, r, hh);
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const f32x16 dv = mfma32(ot[1][db], pk[1], mfma32(ot[0][db], pk[0], f32x16{}));
            stage_part<D>(dv, db, F8 ? a.f8_dv : 1.0f, vt, r, hh);
        }
        store_tile<D>(kt, slice_rsrc((const __bf16*)a.dk + kvb, c.lk, rso, D * 2), (uint32_t)j0 * rso, rso, lane);
        store_tile<D>(vt, slice_rsrc((const __bf16*)a.dv + kvb, c.lk, rso, D * 2), (uint32_t)j0 * rso, rso, lane);
    }

    template <class RingT>
    __device__ __forceinline__ void item_end(const Rec& c, const RingT& g, int job) {
        if (c.part >= 0) {   // one chunk of a cut item: fp32 partial dQ block (scaled by the reduction)
            store_partial<D / 32>(acc, a.part, c.part, 32, 0, r, hh);
            return;
        }
        const size_t ob = ((size_t)c.qs * H + c.h) * D;
        store<D>(acc, F8 ? a.f8_dq : scale, a.dq, ob, c.lq, c.t * 32, g.tile(job - 2));
    }

    // no keys: dQ is zero (the sample has no dK, dV rows)
    __device__ __forceinline__ void item_zero(const Rec& c) {
        const size_t ob = ((size_t)c.qs * H + c.h) * D;
        zero<D>(a.dq, ob, c.lq, c.t * 32);
    }
};

template <class Pol, int XJ = 0>
__device__ __forceinline__ void fused_body(const KernelArgs& a, const Rec* __restrict__ recs,
                                           const int32_t* __restrict__ bin_ptr, char* smem, int D) {
    using RingT = Ring<GDPA_D, 1, TeamShape<GDPA_D, 1, 2>::LDS, XJ>;
    const int lane = threadIdx.x & 63;
    Pol pol(a, lane);
    run_team<Pol, RingT, 1>(pol, a.P, recs, bin_ptr, smem, (uint32_t)a.H * D * 2, 0, lane);
}

template <int D, int ACT, bool F8>
__global__ __launch_bounds__((TeamShape<D, 1, 2>::THREADS), (TeamShape<D, 1, 2>::WPE)) void kv_fused_kernel(
    const KernelArgs a, const Rec* __restrict__ recs, const int32_t* __restrict__ bin_ptr) {
    constexpr int XJ = KvFusedPol<D, ACT, F8>::XJ;
    __shared__ __attribute__((aligned(1024))) char smem[Ring<D, 1, TeamShape<D, 1, 2>::LDS, XJ>::BYTES];
    fused_body<KvFusedPol<D, ACT, F8>, XJ>(a, recs, bin_ptr, smem, D);
}

template <int D, int ACT, bool F8>
__global__ __launch_bounds__((TeamShape<D, 1, 2>::THREADS), (TeamShape<D, 1, 2>::WPE)) void q_fused_kernel(
    const KernelArgs a, const Rec* __restrict__ recs, const int32_t* __restrict__ bin_ptr) {
    __shared__ __attribute__((aligned(1024))) char smem[Ring<D, 1, TeamShape<D, 1, 2>::LDS>::BYTES];
    fused_body<QFusedPol<D, ACT, F8>>(a, recs, bin_ptr, smem, D);
}

template <int ACT>
const void* kv_ptr() {
    return (const void*)&kv_fused_kernel<GDPA_D, ACT, false>;
}
template <int ACT>
const void* q_ptr() {
    return (const void*)&q_fused_kernel<GDPA_D, ACT, false>;
}
template <int ACT>
const void* kv_ptr8() {
    return (const void*)&kv_fused_kernel<GDPA_D, ACT, true>;
}
template <int ACT>
const void* q_ptr8() {
    return (const void*)&q_fused_kernel<GDPA_D, ACT, true>;
}

#define GDPA_FUSED_SWITCH(F)                                  \
    switch (act) {                                            \
        case ACT_GELU: return F<ACT_GELU>();                  \
        case ACT_SILU: return F<ACT_SILU>();                  \
        case ACT_GELU_POLY: return F<ACT_GELU_POLY>();        \
        case ACT_GELU_TAYLOR6: return F<ACT_GELU_TAYLOR6>();  \
        case ACT_IDENTITY: return F<ACT_IDENTITY>();          \
    }                                                         \
    return nullptr;

}  // namespace

#define GDPA_CAT2(a, b) a##b
#define GDPA_CAT(a, b) GDPA_CAT2(a, b)

const void* GDPA_CAT(bwd_fused_kernel_ptr_d, GDPA_D)(int kv_stationary, int act) {
    if (act & kActF8Bwd) {   // fp8 Q, K, V, dO
        act &= ~kActF8Bwd;
        if (kv_stationary) {
            GDPA_FUSED_SWITCH(kv_ptr8)
        }
        GDPA_FUSED_SWITCH(q_ptr8)
    }
    if (kv_stationary) {
        if (act == ACT_SOFTMAX) return kv_ptr<ACT_SOFTMAX>();
        GDPA_FUSED_SWITCH(kv_ptr)
    }
    GDPA_FUSED_SWITCH(q_ptr)
}

hipError_t GDPA_CAT(launch_bwd_fused_d, GDPA_D)(const KernelArgs& a, int kv_stationary, int act, hipStream_t s) {
    const void* f = GDPA_CAT(bwd_fused_kernel_ptr_d, GDPA_D)(kv_stationary, act);
    if (!f) return hipErrorInvalidValue;
    if (a.P <= 0) return hipSuccess;
    KernelArgs args = a;
    const void* recs = a.items;
    const int32_t* bin_ptr = a.bin_ptr;
    void* params[] = {&args, &recs, &bin_ptr};
    return hipLaunchKernel(f, dim3(a.P), dim3(64), params, 0, s);
}

}  // namespace gdpa
