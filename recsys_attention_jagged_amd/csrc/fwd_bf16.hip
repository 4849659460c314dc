// GDPA forward, bf16 inputs, fp32 MFMA accumulation, for one head dimension
// (compiled once per D with -DGDPA_D=32|64|128).
//
// O = act(Q K^T / sqrt(d)) V over the valid pairs of each sample, with no
// softmax and no row normalisation (GDPA page, aitrends.kr/articles/26275,
// "Key summary" and "Section details": two matrix products with a general
// activation between them; the softmax correction step is gone, so partial
// products over kv tiles simply add).
//
// Work decomposition.  A team of T waves (see ring.hpp) works on one item at a
// time: one (sample, head) and T x NB consecutive 32-row q blocks, NB per wave;
// its steps stream the sample's K and V in 32-row tiles through the team's LDS
// ring.  Per step and q block a wave computes S^T = K Q^T with MFMA (K rows from
// LDS, Q held in registers, the K operand shared by the wave's NB blocks), applies
// the activation in registers, and feeds the accumulator lanes straight back as
// the B operand of O^T += V^T P^T (V^T read from the row-major V tile with
// transposing LDS reads).  Rows beyond a sample's lengths are zero tiles, so only
// the local window needs a mask.
//
// The same kernels run jagged softmax attention (JFA, act = softmax): the block's
// scores go through an online softmax (running max and sum per q row, the O
// accumulator rescaled when the max moves) instead of the activation; there the
// keys beyond a sample's length are masked too, and the item's end divides by the
// row sum and stores the row's log-sum-exp.
//
// With the RMSNorm prologue (NORM) the kernels read the raw Q, K, V and scale by
// each row's 1 / rms instead of normalising the tensors: S_ij = r_q,i r_k,j (q_i . k_j)
// / sqrt(d), and P_ij r_v,j takes the place of P_ij (O = sum_j P_ij r_v,j v_j).  The
// factors of a tile's 32 rows (a pre-pass writes them) travel with the tile in the
// ring's side buffers: r_q with each Q tile, (r_k, r_v) pairs with each K tile.
//
// With fp8 Q and K (F8) the first product runs on the fp8 MFMA: Q and K arrive as
// OCP e4m3 bytes with one dequantisation factor per tensor (folded into the score
// scale), their tiles take half a slot, and V, P and O stay bf16 (the precision is
// chosen per product).
//
// With block-scaled fp8 Q and K (MX: OCP microscaling, one E8M0 power-of-two scale
// per 32 consecutive head columns of a row) the first product runs on gfx950's
// scaled MFMA, 32 x 32 x 64 per instruction.  Its k order pairs the halves of the
// two lane groups: lane l of group g = l / 32 holds columns 16 g + [0, 16) of the
// 64-wide block in bytes 0..15 and columns 32 + 16 g + [0, 16) in bytes 16..31, so
// the first scale block (columns 0..31) is bytes 0..15 of both groups and the second
// bytes 16..31; the scale byte of block g of row l % 32 is passed by lane l.  The
// hardware applies both operands' scales to the fp32 products.  The scale bytes of
// a tile's 32 rows ride with the tile in the ring's side buffer.
#include "kernels.hpp"
#include "ring.hpp"

#ifndef GDPA_D
#error "compile with -DGDPA_D=<32|64|128>"
#endif

namespace gdpa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// MODE: 0 plain, 1 RMSNorm prologue, 2 fp8 Q and K, 3 block-scaled fp8 (MX) Q and K
template <int D, int T, int NB, int ACT, int MODE>
struct FwdPol {
    static constexpr bool NORM = MODE == 1, MX = MODE == 3, F8 = MODE == 2 || MX;
    static constexpr int NMX = MX ? D / 64 : 1;       // MX: 64-wide k blocks (one scaled MFMA each)
    static constexpr int MXW = D / 32;                // MX: scale bytes per row, one side-load unit
    static constexpr int NSTAT = T * NB, NSTRM = 2;   // stationary tiles: wave-major q blocks
    static constexpr int NDB = D / 32, NKS = D / 16;
    static constexpr int ROWS = 32 * T * NB;          // q rows per item
    static constexpr bool HOIST = TeamShape<D, T, 0>::HOIST;

    const KernelArgs a;   // by value: kept in SGPRs, not re-read from the argument segment
    int lane, r, hh, wt, H, win;
    uint32_t rs, rso;
    float scale;
    Slice wq, wk, wv;    // issuing side: slices of the walk's current item
    Slice wrq, wrkv, wnull;   // NORM: 1/rms of the item's q rows, (k, v) row pairs; a zero-range side
    bf16x8 qf[F8 ? 1 : NB][NKS];
    long qf8[F8 && !MX ? NB : 1][NKS];   // F8: this lane's 8 fp8 values of each 16-wide k block
    i32x8 qx[MX ? NB : 1][NMX];   // MX: this lane's 32 fp8 values of each 64-wide k block
    uint32_t qsa[MX ? NB : 1][NMX];   // MX: their scale (E8M0) in the low byte
    Slice wsq, wsk;       // MX: scale bytes of the item's q rows, of its k rows
    float rqv[NB];        // NORM: 1/rms of this lane's q row
    f32x16 acc[NB][NDB];
    // softmax only: running max (log2 units) of this lane's q row and this lane's
    // share of the running sum (the other share sits in lane ^ 32)
    float mrow[NB], lrow[NB];

    __device__ FwdPol(const KernelArgs& args, int lane_, int wt_) : a(args) {
        lane = lane_;
        r = lane & 31;
        hh = lane >> 5;
        wt = wt_;
        H = a.H;
        win = a.window;
        rs = (uint32_t)H * D * 2;
        rso = (uint32_t)H * D * (a.out_f32 ? 4 : 2);
        scale = a.scale;
    }

    // first q row of this wave's block b
    __device__ __forceinline__ int qrow(const Rec& c, int b) const { return c.t * ROWS + 32 * (wt * NB + b); }
    __device__ __forceinline__ bool block_dead(const Rec& c, int b, int j0) const {
        const int q0 = qrow(c, b);
        return q0 >= c.lq || (win > 0 && band_none(q0, j0, win));
    }

    __device__ __forceinline__ void walk_item(const Rec& w) {
        const size_t kvb = ((size_t)w.ks * H + w.h) * D;
        wk = slice_of((const __bf16*)a.k + kvb, w.lk, rs, D * 2);
        wv = slice_of((const __bf16*)a.v + kvb, w.lk, rs, D * 2);
        if constexpr (F8) {   // one-byte rows, H D bytes apart
            wk = slice_of((const uint8_t*)a.k + kvb, w.lk, rs / 2, D);
            wq = slice_of((const uint8_t*)a.q + ((size_t)w.qs * H + w.h) * D, w.lq, rs / 2, D);
            wnull = slice_of(a.q, 0, rs / 2, D);
            if constexpr (MX) {   // D / 32 scale bytes per row, the rows of a head consecutive
                wsq = slice_of(a.q_mx + ((size_t)w.h * a.Tq + w.qs) * (D / 32), w.lq, D / 32, D / 32);
                wsk = slice_of(a.k_mx + ((size_t)w.h * a.Tk + w.ks) * (D / 32), w.lk, D / 32, D / 32);
            }
        } else {
            wq = slice_of((const __bf16*)a.q + ((size_t)w.qs * H + w.h) * D, w.lq, rs, D * 2);
        }
        if constexpr (NORM) {
            wrq = slice_of(a.rq + (size_t)w.h * a.Tq + w.qs, w.lq, 4u, 4u);
            wrkv = slice_of(a.rkv + ((size_t)w.h * a.Tk + w.ks) * 2, w.lk, 8u, 8u);
            wnull = slice_of(a.rkv, 0, 8u, 8u);
        }
    }

    template <class RingT>
    __device__ __forceinline__ void ring_ready(RingT& g, int lane_) {
        if constexpr (F8) g.init8(rs / 2, lane_);
    }

    template <class RingT>
    __device__ __forceinline__ void issue_job(RingT& g, const Rec& w, int i) {
        if constexpr (MX) {   // fp8 Q, K tiles with their rows' scale bytes in the side buffer
            if (i < NSTAT) {
                const uint32_t row0 = (uint32_t)(w.t * ROWS + 32 * i);
                g.template issue8<MXW>(wq, row0 * (rs / 2), wnull, wsq, row0 * (D / 32));
            } else {
                const int rel = i - NSTAT;
                const uint32_t row0 = (uint32_t)((w.s0 + (rel >> 1)) * 32);
                if (rel & 1)
                    g.issue(wv, row0 * rs, wnull, 0u);
                else
                    g.template issue8<MXW>(wk, row0 * (rs / 2), wnull, wsk, row0 * (D / 32));
            }
        } else if constexpr (F8) {
            if (i < NSTAT) {
                g.issue8(wq, (uint32_t)(w.t * ROWS + 32 * i) * (rs / 2), wnull);
            } else {
                const int rel = i - NSTAT;
                const uint32_t row0 = (uint32_t)((w.s0 + (rel >> 1)) * 32);
                if (rel & 1)
                    g.issue(wv, row0 * rs);
                else
                    g.issue8(wk, row0 * (rs / 2), wnull);
            }
        } else if (i < NSTAT) {
            const uint32_t row0 = (uint32_t)(w.t * ROWS + 32 * i);
            if constexpr (NORM)
                g.issue(wq, row0 * rs, wrq, row0 * 4u);
            else
                g.issue(wq, row0 * rs);
        } else {
            const int rel = i - NSTAT;
            const uint32_t row0 = (uint32_t)((w.s0 + (rel >> 1)) * 32);
            if constexpr (NORM)
                g.issue((rel & 1) ? wv : wk, row0 * rs, (rel & 1) ? wnull : wrkv, row0 * 8u);
            else
                g.issue((rel & 1) ? wv : wk, row0 * rs);
        }
    }

    __device__ __forceinline__ void item_begin(const Rec&) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
#pragma unroll
            for (int db = 0; db < NDB; ++db) acc[b][db] = f32x16{};
            mrow[b] = kNegBig;
            lrow[b] = 0.0f;
        }
    }

    // Online softmax of one 32 x 32 block (JFA): lane column = query q0 + r, element
    // e = key j0 + 8 (e/4) + 4 hh + e % 4.  Keys outside the sample or the window are
    // masked (zero tiles give S = 0, and exp(0) is not 0).  The reference max of a row
    // moves to the block's max only when that exceeds it by more than kLazy (log2
    // units), so P stays below 2^kLazy (exact in fp32 and bf16 up to rounding) and the
    // accumulator and running sum are rescaled only then, not whenever the max grows.
    __device__ __forceinline__ void softmax_block(int b, const f32x16& sc, int q0, int j0, int lk, f32x16& p) {
        constexpr float L2E = 1.4426950408889634f;
        const bool tail = j0 + 32 > lk;
        const bool band = win > 0 && !band_all(q0, j0, win);
        const float c2 = scale * L2E;
        float mt = kNegBig;
        // p holds the scores in log2 units first; the mask test is taken once per block
        // (a uniform branch), not per element
        if (tail || band) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int jr = 8 * (e >> 2) + 4 * hh + (e & 3);
                const int dd = q0 + r - j0 - jr;
                const bool ok = (j0 + jr < lk) & (!band | in_band(dd, win));
                p[e] = ok ? sc[e] * c2 : kNegBig;
                mt = __builtin_fmaxf(mt, p[e]);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                p[e] = sc[e] * c2;
                mt = __builtin_fmaxf(mt, p[e]);
            }
        }
        mt = __builtin_fmaxf(mt, __shfl_xor(mt, 32));
        constexpr float kLazy = 8.0f;
        const float mo = mrow[b];
        const float mn = mt > mo + kLazy ? mt : mo;   // from the sentinel: the first block with a valid key
        const float alpha = fast_exp2(mo - mn);       // 1 while the reference stays, 0 from the sentinel
        mrow[b] = mn;
        float ls = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            p[e] = p[e] > 0.5f * kNegBig ? fast_exp2(p[e] - mn) : 0.0f;
            ls += p[e];
        }
        lrow[b] = __builtin_fmaf(lrow[b], alpha, ls);
        // rescale only when some row's reference moved from a finite value (rows still at
        // the sentinel have a zero accumulator; every lane of the wave takes the same branch)
        if (__builtin_amdgcn_ballot_w64(alpha != 1.0f && mo > 0.5f * kNegBig)) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[b][db][e] *= alpha;
        }
    }

    // MX: this lane's 32 bytes of row r in 64-wide k block i8: columns 64 i8 + 16 hh
    // + [0, 16) (first scale block) and 64 i8 + 32 + 16 hh + [0, 16) (second), the
    // 16-byte chunks 4 i8 + hh and 4 i8 + 2 + hh of the fp8 tile
    __device__ __forceinline__ i32x8 mx_operand(const char* tile, int i8) const {
        const int4 lo = *(const int4*)(tile + tile8_off<D>(r, 4 * i8 + hh));
        const int4 hi = *(const int4*)(tile + tile8_off<D>(r, 4 * i8 + 2 + hh));
        return i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    }
    // MX: the scale byte this lane passes, that of block 2 i8 + hh of row r (the
    // instruction takes block hh's scale from lane group hh), from the tile's side
    // buffer, where row r's D / 32 scale bytes sit in the 4 bytes at 4 r (d = 64: two
    // bytes, zero-extended)
    __device__ __forceinline__ uint32_t mx_scale(const char* side, int i8) const {
        return (*(const uint32_t*)(side + 4 * r) >> (8 * (2 * i8 + hh))) & 0xffu;
    }

    // stationary tiles i, i + 1 (jobs job, job + 1): tile u belongs to wave u / NB, block u % NB
    template <class RingT>
    __device__ __forceinline__ void load_stat(const Rec&, const RingT& g, int job, int i) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int tile = i + u;
            if (tile < NSTAT && tile / NB == wt) {
                if constexpr (MX) {
#pragma unroll
                    for (int i8 = 0; i8 < NMX; ++i8) {
                        qx[tile % NB][i8] = mx_operand(g.tile(job + u), i8);
                        qsa[tile % NB][i8] = mx_scale(g.side(job + u), i8);
                    }
                } else if constexpr (F8) {
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks)
                        qf8[tile % NB][ks] = *(const long*)(g.tile(job + u) + tile8_off<D>(r, ks) + 8 * hh);
                } else {
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) qf[tile % NB][ks] = lds_row8<D>(g.tile(job + u), r, 2 * ks + hh);
                }
                if constexpr (NORM) rqv[tile % NB] = *(const float*)(g.side(job + u) + 4 * r);
            }
        }
    }

    template <class RingT>
    __device__ __forceinline__ void step(const Rec& c, int s, const RingT& g, int job) {
        {   // a block past the sample's last query, or with no pair inside the window band,
            // adds nothing: a step none of whose blocks adds anything is skipped (one
            // uniform branch)
            bool dead = true;
#pragma unroll
            for (int b = 0; b < NB; ++b) dead = dead && block_dead(c, b, s * 32);
            if (dead) return;
        }
        const char* kt = g.tile(job);
        const char* vt = g.tile(job + 1);
        // with one wave per SIMD all operand reads are issued up front so their
        // latency overlaps the MFMAs; with two, each is read just before use
        bf16x8 kop[NKS], vop[2][NDB];
        // NORM: (1/rms of k, of v) of keys j0 + 8 j + 4 hh + {0, 1} and {2, 3}, from the K job's side
        float4 rkv[NORM ? 4 : 1][2];
        if constexpr (NORM) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                rkv[j][0] = *(const float4*)(g.side(job) + 8 * (8 * j + 4 * hh));
                rkv[j][1] = *(const float4*)(g.side(job) + 8 * (8 * j + 4 * hh) + 16);
            }
        }
        // element e's key factors
        auto fk = [&](int e) -> float {
            if constexpr (NORM) return (e & 1) ? rkv[e >> 2][(e >> 1) & 1].z : rkv[e >> 2][(e >> 1) & 1].x;
            else return 1.0f;
        };
        auto fv = [&](int e) -> float {
            if constexpr (NORM) return (e & 1) ? rkv[e >> 2][(e >> 1) & 1].w : rkv[e >> 2][(e >> 1) & 1].y;
            else return 1.0f;
        };
        long kop8[F8 ? NKS : 1];
        if constexpr (HOIST) {
            if constexpr (!MX) {   // (MX reads its K operands next to their MFMAs)
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    if constexpr (F8)
                        kop8[ks] = *(const long*)(kt + tile8_off<D>(r, ks) + 8 * hh);
                    else
                        kop[ks] = lds_row8<D>(kt, r, 2 * ks + hh);
                }
            }
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int db = 0; db < NDB; ++db) vop[m][db] = lds_col8<D>(vt, 16 * m, db * 32, lane);
        }
        f32x16 sc[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) sc[b] = f32x16{};
        if constexpr (MX) {   // S^T = K Q^T on the scaled MFMA, 64 k per instruction
#pragma unroll
            for (int i8 = 0; i8 < NMX; ++i8) {
                const i32x8 ko = mx_operand(kt, i8);
                const uint32_t ksa = mx_scale(g.side(job), i8);
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    sc[b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ko, qx[b][i8], sc[b], 0, 0, 0, (int)ksa, 0,
                                                                           (int)qsa[b][i8]);
            }
        }
#pragma unroll
        for (int ks = 0; ks < (MX ? 0 : NKS); ++ks) {
            if constexpr (F8) {   // S^T = K Q^T on e4m3 operands, 16 k per instruction
                const long ko = HOIST ? kop8[ks] : *(const long*)(kt + tile8_off<D>(r, ks) + 8 * hh);
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    sc[b] = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(ko, qf8[b][ks], sc[b], 0, 0, 0);
                continue;
            }
            const bf16x8 ko = HOIST ? kop[ks] : lds_row8<D>(kt, r, 2 * ks + hh);
#pragma unroll
            for (int b = 0; b < NB; ++b) sc[b] = mfma32(ko, qf[b][ks], sc[b]);
        }
        const int j0 = s * 32;
        bf16x8 pb[NB][2];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int q0 = qrow(c, b);
            f32x16 p;
            if constexpr (ACT == ACT_SOFTMAX) {
                softmax_block(b, sc[b], q0, j0, c.lk, p);
            } else if (win > 0 && !band_all(q0, j0, win)) {
                // lane column: query q0 + r; element c: key j0 + 8 (c/4) + 4 hh + c % 4
                const int base = q0 + r - j0 - 4 * hh;
                const float cq = NORM ? scale * rqv[b] : scale;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int dd = base - (8 * (e >> 2) + (e & 3));
                    const float f = act_fwd<ACT>(sc[b][e] * cq * fk(e)) * fv(e);
                    p[e] = in_band(dd, win) ? f : 0.0f;
                }
            } else {
                const float cq = NORM ? scale * rqv[b] : scale;
#pragma unroll
                for (int e = 0; e < 16; ++e) p[e] = act_fwd<ACT>(sc[b][e] * cq * fk(e)) * fv(e);
            }
            pb[b][0] = acc_to_bf16x8(p, 0);
            pb[b][1] = acc_to_bf16x8(p, 1);
        }
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const bf16x8 vo = HOIST ? vop[m][db] : lds_col8<D>(vt, 16 * m, db * 32, lane);
#pragma unroll
                for (int b = 0; b < NB; ++b) acc[b][db] = mfma32(vo, pb[b][m], acc[b][db]);
            }
    }

    // this wave's blocks, staged through a slot of the last step (one slot per wave
    // in a team; blocks sharing a slot are staged one after the other)
    // softmax: this lane's row sum (both halves), the output scale 1 / sum, and the
    // row's log-sum-exp stored by the lanes of the first half (rows without keys:
    // O = 0 and LSE = -inf)
    __device__ __forceinline__ float softmax_finish(const Rec& c, int b) {
        const float l = lrow[b] + __shfl_xor(lrow[b], 32);
        const int row = qrow(c, b) + r;
        if (hh == 0 && row < c.lq)
            a.lse[(size_t)c.h * a.Tq + c.qs + row] =
                l > 0.0f ? (mrow[b] + __builtin_amdgcn_logf(l)) * 0.69314718055994531f : -__builtin_inff();
        return l > 0.0f ? 1.0f / l : 0.0f;
    }

    template <class RingT>
    __device__ __forceinline__ void item_end(const Rec& c, const RingT& g, int job) {
        if (c.part >= 0) {   // one chunk of a cut item: fp32 partial block
#pragma unroll
            for (int b = 0; b < NB; ++b) store_partial<NDB>(acc[b], a.part, c.part, ROWS, 32 * (wt * NB + b), r, hh);
            if constexpr (ACT == ACT_SOFTMAX) {   // softmax: the block is unnormalised; its rows' max and sum
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const float l = lrow[b] + __shfl_xor(lrow[b], 32);
                    if (hh == 0)
                        *(float2*)(a.part_stat + ((size_t)c.part * ROWS + 32 * (wt * NB + b) + r) * 2) =
                            make_float2(mrow[b], l);
                }
            }
            return;
        }
        const size_t ob = ((size_t)c.qs * H + c.h) * D;
        float mul[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) mul[b] = ACT == ACT_SOFTMAX ? softmax_finish(c, b) : 1.0f;
        if (a.out_f32) {
            const rsrc_t ro = slice_rsrc((const float*)a.o + ob, c.lq, rso, D * 4);
#pragma unroll
            for (int b = 0; b < NB; ++b)
                if (qrow(c, b) < c.lq) store_block_f32<NDB>(acc[b], mul[b], ro, (uint32_t)(qrow(c, b) + r) * rso, hh);
            return;
        }
        const rsrc_t ro = slice_rsrc((const __bf16*)a.o + ob, c.lq, rso, D * 2);
        const int ln = opaque(lane);   // the staging offsets are computed here, per item
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (qrow(c, b) >= c.lq) continue;   // a block past the sample's last query has no rows
            char* st = g.tile(job - 2 + (T > 1 ? wt : (b & 1)));
            stage_block<D>(acc[b], mul[b], st, ln & 31, ln >> 5);
            store_tile<D>(st, ro, (uint32_t)qrow(c, b) * rso, rso, ln);
        }
    }

    // an item without keys: its rows are zero (softmax: and their LSE -inf)
    __device__ __forceinline__ void item_zero(const Rec& c) {
        if constexpr (ACT == ACT_SOFTMAX) {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                lrow[b] = 0.0f;
                mrow[b] = kNegBig;
                (void)softmax_finish(c, b);
            }
        }
        const size_t ob = ((size_t)c.qs * H + c.h) * D;
        if (a.out_f32) {
            item_begin(c);
            const rsrc_t ro = slice_rsrc((const float*)a.o + ob, c.lq, rso, D * 4);
#pragma unroll
            for (int b = 0; b < NB; ++b) store_block_f32<NDB>(acc[b], 1.0f, ro, (uint32_t)(qrow(c, b) + r) * rso, hh);
            return;
        }
        const rsrc_t ro = slice_rsrc((const __bf16*)a.o + ob, c.lq, rso, D * 2);
#pragma unroll
        for (int b = 0; b < NB; ++b) store_zero_rows<D>(ro, (uint32_t)qrow(c, b) * rso, rso, lane);
    }
};

template <int D, int T, int NB, int ACT, int MODE>
__global__ __launch_bounds__((TeamShape<D, T, 0>::THREADS), (TeamShape<D, T, 0>::WPE)) void fwd_bf16_kernel(
    const KernelArgs a, const Rec* __restrict__ recs, const int32_t* __restrict__ bin_ptr) {
    using RingT = Ring<D, T, TeamShape<D, T, 0>::LDS, (MODE == 1 || MODE == 3) ? 1 : 0>;
    __shared__ __attribute__((aligned(1024))) char smem[RingT::BYTES];
    const int wt = T > 1 ? __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6) : 0;
    const int lane = threadIdx.x & 63;
    FwdPol<D, T, NB, ACT, MODE> pol(a, lane, wt);
    run_team<FwdPol<D, T, NB, ACT, MODE>, RingT, T>(pol, a.P, recs, bin_ptr, smem, (uint32_t)a.H * D * 2, wt,
                                                    lane);
}

template <int T, int NB, int ACT, int MODE = 0>
const void* kptr() {
    return (const void*)&fwd_bf16_kernel<GDPA_D, T, NB, ACT, MODE>;
}

template <int T, int NB>
const void* kptr_act(int act) {
    if (act & kActMX) {   // block-scaled fp8 Q and K (64-wide k blocks: d >= 64)
        if constexpr (GDPA_D >= 64) {
            switch (act & ~kActMX) {
                case ACT_GELU: return kptr<T, NB, ACT_GELU, 3>();
                case ACT_SILU: return kptr<T, NB, ACT_SILU, 3>();
                case ACT_GELU_POLY: return kptr<T, NB, ACT_GELU_POLY, 3>();
                case ACT_GELU_TAYLOR6: return kptr<T, NB, ACT_GELU_TAYLOR6, 3>();
                case ACT_IDENTITY: return kptr<T, NB, ACT_IDENTITY, 3>();
            }
        }
        return nullptr;
    }
    if (act & kActF8) {   // fp8 Q and K
        switch (act & ~kActF8) {
            case ACT_GELU: return kptr<T, NB, ACT_GELU, 2>();
            case ACT_SILU: return kptr<T, NB, ACT_SILU, 2>();
            case ACT_GELU_POLY: return kptr<T, NB, ACT_GELU_POLY, 2>();
            case ACT_GELU_TAYLOR6: return kptr<T, NB, ACT_GELU_TAYLOR6, 2>();
            case ACT_IDENTITY: return kptr<T, NB, ACT_IDENTITY, 2>();
        }
        return nullptr;
    }
    if (act & kActNorm) {   // the RMSNorm-prologue variants
        switch (act & ~kActNorm) {
            case ACT_GELU: return kptr<T, NB, ACT_GELU, 1>();
            case ACT_SILU: return kptr<T, NB, ACT_SILU, 1>();
            case ACT_GELU_POLY: return kptr<T, NB, ACT_GELU_POLY, 1>();
            case ACT_GELU_TAYLOR6: return kptr<T, NB, ACT_GELU_TAYLOR6, 1>();
            case ACT_IDENTITY: return kptr<T, NB, ACT_IDENTITY, 1>();
        }
        return nullptr;
    }
    switch (act) {
        case ACT_GELU: return kptr<T, NB, ACT_GELU>();
        case ACT_SILU: return kptr<T, NB, ACT_SILU>();
        case ACT_GELU_POLY: return kptr<T, NB, ACT_GELU_POLY>();
        case ACT_GELU_TAYLOR6: return kptr<T, NB, ACT_GELU_TAYLOR6>();
        case ACT_IDENTITY: return kptr<T, NB, ACT_IDENTITY>();
        case ACT_ONE: return kptr<T, NB, ACT_ONE>();
        case ACT_SOFTMAX: return kptr<T, NB, ACT_SOFTMAX>();
    }
    return nullptr;
}

}  // namespace

#define GDPA_CAT2(a, b) a##b
#define GDPA_CAT(a, b) GDPA_CAT2(a, b)

const void* GDPA_CAT(fwd_bf16_kernel_ptr_d, GDPA_D)(int team, int nb, int act) {
    if (team == 1 && nb == 1) return kptr_act<1, 1>(act);
    if (team == 1 && nb == 2) return kptr_act<1, 2>(act);
#if GDPA_D == 128
    if (team == 2 && nb == 1) return kptr_act<2, 1>(act);
#endif
    return nullptr;
}

hipError_t GDPA_CAT(launch_fwd_bf16_d, GDPA_D)(const KernelArgs& a, int team, int nb, int act, hipStream_t s) {
    const void* f = GDPA_CAT(fwd_bf16_kernel_ptr_d, GDPA_D)(team, nb, act);
    if (!f) return hipErrorInvalidValue;
    if (a.P <= 0) return hipSuccess;
    KernelArgs args = a;
    const void* recs = a.items;
    const int32_t* bin_ptr = a.bin_ptr;
    void* params[] = {&args, &recs, &bin_ptr};
    return hipLaunchKernel(f, dim3(a.P), dim3(64 * team), params, 0, s);
}

}  // namespace gdpa
