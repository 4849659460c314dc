// GDPA dK / dV kernel for d = 128 on the 16 x 16 x 32 bf16 MFMA, two waves per SIMD.
//
// Gradients of sum(O * dO) for O = act(S) V, S = Q K^T / sqrt(d) on the valid
// pairs (GDPA page, aitrends.kr/articles/26275, "Section details": the softmax and
// its correction step are gone, so the backward recomputes S and needs no row
// statistic): dP = dO V^T, dS = dP * act'(S), dV = P^T dO, dK = dS^T Q / sqrt(d).
//
// KV-stationary.  A workgroup is a team of two or four waves sharing one tile ring
// (ring.hpp); an item is one (sample, head) and 32 or 64 kv rows (one or two
// 32-row tiles), its steps the 32-row q tiles that hold valid pairs.  Each wave
// owns 16 of the item's kv rows:
// its K and V rows stay in registers as B operands, its dK and dV accumulate in
// registers, and both waves read every streamed Q and dO tile from the shared
// ring.  Per step and wave: S (32 q x 16 kv) and dP in eight 16 x 16 x 32 products
// each, the activation and its derivative in registers, then dV^T += dO^T P and
// dK^T += Q^T dS with P and dS taken straight from the score accumulators as B
// operands (lane l holds kv column l % 16 and q rows 4 (l / 16) + {0..3} and
// 16 + 4 (l / 16) + {0..3}; the A operands read the same q rows of dO and Q
// with transposing LDS loads).  Half the register state of a 32-row wave lets two
// waves share each SIMD, so one wave's activation overlaps the other's products.
// No atomics: every dK, dV row has one owner.
//
// With fp8 inputs (F8: Q, K and dO as e4m3 bytes, one factor per tensor; V bf16)
// their tiles are one byte per element in the first half of a slot; S runs on the
// 16 x 16 x 32 fp8 MFMA from row reads, dO's rows are widened exactly to bf16 for
// dP, and the transposed Q and dO operands come from 8-bit transposing reads,
// widened the same way.
#include "bwd_common.hpp"
#include "kernels.hpp"
#include "ring.hpp"

namespace gdpa {
namespace {

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Tiles use the 16-row swizzle (ring.hpp, SW = 1).
constexpr int SW16 = 1;

// 8 bf16 of `row`, columns [8 chunk, 8 chunk + 8)
template <int D>
__device__ __forceinline__ bf16x8 row8_16(const char* tile, int row, int chunk) {
    return *(const bf16x8*)(tile + tile_off_sw<D, SW16>(row, chunk));
}

// Transposed operand in the 16-column layout: lane l receives
// tile[row0 + 4 (l / 16) + i][col0 + l % 16], i = 0..3 (row0 a multiple of 4,
// col0 a multiple of 16).  Each 16-lane group reads one 4-row x 16-column block:
// lanes 4k .. 4k + 3 address row k's four 8-byte pieces.
template <int D>
__device__ __forceinline__ bf16x4 lds_col4_16(const char* tile, int row0, int col0, int lane) {
    const int g = lane >> 4, i = lane & 15;
    const int row = row0 + 4 * g + (i >> 2);
    const int t = i & 3;
    const int col = col0 + 4 * t;
    const int off = tile_off_sw<D, SW16>(row, col >> 3) + ((t & 1) << 3);
    const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(tile + off));
    return __builtin_bit_cast(bf16x4, v);
}

// A operand of the 8 q rows a lane group contracts over: rows row0 + 4 (l / 16) + {0..3}
// and row0 + 16 + 4 (l / 16) + {0..3}, column col0 + l % 16
template <int D>
__device__ __forceinline__ bf16x8 lds_col8_16(const char* tile, int row0, int col0, int lane) {
    const bf16x4 a = lds_col4_16<D>(tile, row0, col0, lane);
    const bf16x4 b = lds_col4_16<D>(tile, row0 + 16, col0, lane);
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// lds_col8_16 (row0 = 0) of an fp8 tile (ring.hpp's fp8 layout), widened to bf16, in
// one 8-bit transposing read: within each 16-lane group, byte i of lane j is byte
// j % 8 of the 8 bytes addressed by lane 2 i + j / 8, so lane 2 i + c addresses the
// group's i-th row (4 (l / 16) + {0..3}, then 16 + 4 (l / 16) + {0..3}) at columns
// col0 + 8 c ..  (col0 a multiple of 16)
template <int D>
__device__ __forceinline__ bf16x8 lds_col8_16_f8(const char* tile, int col0, int lane) {
    const int j = lane & 15, i = j >> 1, c = j & 1;
    const int row = 4 * (lane >> 4) + (i & 3) + 16 * (i >> 2);
    typedef int v2i __attribute__((ext_vector_type(2)));
    const v2i v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (__attribute__((address_space(3))) v2i*)(tile + tile8_off<D>(row, col0 >> 4) + 8 * c));
    return widen_e4m3(v.x, v.y);
}

// 8 e4m3 bytes of `row`, columns [8 c8, 8 c8 + 8) of an fp8 tile (the operand that
// row8_16(tile, row, c8) is for a bf16 one)
template <int D>
__device__ __forceinline__ long row8_16_f8(const char* tile, int row, int c8) {
    return lds_row8_f8<D>(tile, row, c8 >> 1, c8 & 1);
}

__device__ __forceinline__ f32x4 mfma16_f8(long a, long b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, c, 0, 0, 0);
}

template <int ACT, int T, bool F8 = false>
struct Dkdv16Pol : Common {
    static constexpr int D = 128;
    static constexpr int ROWS = 16 * T;          // kv rows per item
    static constexpr int NSTAT = ROWS / 16, NSTRM = 2;   // stationary: (K, V) of each 32-row tile
    static constexpr int NKB = D / 32;           // 32-wide head-dimension blocks (contraction of S, dP)
    static constexpr int NCB = D / 16;           // 16-wide head-dimension blocks (dK, dV columns)
    Slice wk, wv, wq, wo;                       // issuing side
    Slice wnull;                                 // F8: a zero-range tile
    bf16x8 kf[F8 ? 1 : NKB], vf[NKB];            // this wave's 16 kv rows of K and V (B operands)
    long kf8[F8 ? NKB : 1];                      // F8: the K rows as fp8 operands
    f32x4 accK[NCB], accV[NCB];                  // lane: kv row l % 16, columns 16 cb + 4 (l / 16) + {0..3}
    int l16, g4;                                 // lane % 16, lane / 16
    // exact GELU: the scale folded into the activation's constants (gelu_grad_folded), so P
    // is formed divided by the scale and dV takes the scale at its store
    static constexpr bool FOLD = ACT == ACT_GELU;
    GeluFold gf;

    __device__ Dkdv16Pol(const KernelArgs& args, int lane_, int wt_) : Common(args, lane_, wt_, D) {
        l16 = lane_ & 15;
        g4 = lane_ >> 4;
        if constexpr (FOLD) gf = gelu_fold(scale);
    }

    // P (FOLD: P / scale) and dS of one score
    __device__ __forceinline__ void act(float s, float dp, float& f, float& ds) const {
        float gr;
        if constexpr (FOLD)
            gelu_grad_folded(s, gf, f, gr);
        else
            act_fwd_grad<ACT>(s * scale, f, gr);
        ds = dp * gr;
    }
    // dV's factor at its store (FOLD: the scale P was formed without)
    __device__ __forceinline__ float dv_mul() const { return (F8 ? a.f8_dv : 1.0f) * (FOLD ? scale : 1.0f); }

    // this wave's first kv row of the item, within the sample
    __device__ __forceinline__ int krow(const Rec& c) const { return c.t * ROWS + 16 * wt; }

    __device__ __forceinline__ void walk_item(const Rec& w) {
        const size_t kvb = ((size_t)w.ks * H + w.h) * D;
        const size_t qb = ((size_t)w.qs * H + w.h) * D;
        wv = slice_of((const __bf16*)a.v + kvb, w.lk, rs, D * 2);
        if constexpr (F8) {   // one-byte rows, H D bytes apart
            wk = slice_of((const uint8_t*)a.k + kvb, w.lk, rs / 2, D);
            wq = slice_of((const uint8_t*)a.q + qb, w.lq, rs / 2, D);
            wo = slice_of((const uint8_t*)a.dout + qb, w.lq, rs / 2, D);
            wnull = slice_of(a.q, 0, rs / 2, D);
        } else {
            wk = slice_of((const __bf16*)a.k + kvb, w.lk, rs, D * 2);
            wq = slice_of((const __bf16*)a.q + qb, w.lq, rs, D * 2);
            wo = slice_of((const __bf16*)a.dout + qb, w.lq, rs, D * 2);
        }
    }

    template <class RingT>
    __device__ __forceinline__ void ring_ready(RingT& g, int lane_) {
        if constexpr (F8) g.init8(rs / 2, lane_);
    }

    template <class RingT>
    __device__ __forceinline__ void issue_job(RingT& g, const Rec& w, int i) {
        if (i < NSTAT) {   // tile i / 2 of the item: K (i even), V (i odd)
            const uint32_t row0 = (uint32_t)(w.t * ROWS + 32 * (i >> 1));
            if (F8 && !(i & 1))
                g.issue8(wk, row0 * (rs / 2), wnull);
            else
                g.issue((i & 1) ? wv : wk, row0 * rs);
        } else {
            const int rel = i - NSTAT;
            const uint32_t row0 = (uint32_t)((w.s0 + (rel >> 1)) * 32);
            if constexpr (F8)
                g.issue8((rel & 1) ? wo : wq, row0 * (rs / 2), wnull);
            else
                g.issue((rel & 1) ? wo : wq, row0 * rs);
        }
    }

    __device__ __forceinline__ void item_begin(const Rec&) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) accK[cb] = accV[cb] = f32x4{};
    }

    // the K and V tiles i / 2 (jobs job, job + 1), read by the two waves whose rows
    // they hold: row 16 (wt % 2) + l % 16, the 16-byte chunk 4 kb + l / 16 of each
    // 32-wide block kb
    template <class RingT>
    __device__ __forceinline__ void load_stat(const Rec&, const RingT& g, int job, int i) {
        if ((wt >> 1) != (i >> 1)) return;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            if constexpr (F8)
                kf8[kb] = row8_16_f8<D>(g.tile(job), 16 * (wt & 1) + l16, 4 * kb + g4);
            else
                kf[kb] = row8_16<D>(g.tile(job), 16 * (wt & 1) + l16, 4 * kb + g4);
            vf[kb] = row8_16<D>(g.tile(job + 1), 16 * (wt & 1) + l16, 4 * kb + g4);
        }
    }

    template <class RingT>
    __device__ __forceinline__ void step(const Rec& c, int s, const RingT& g, int job) {
        const int i0 = s * 32, j0 = krow(c);
        // stored dS: the block of q tile s and this wave's kv tile kt, c.pad0 + s c.pad1 +
        // (kt - js0(s)) (c.pad0 = the sample's first block of this head, c.pad1 = blocks
        // per q tile, js0(s) = the q tile's first kv tile in the band).  A 64-row item
        // also steps over q tiles that pair with its other kv tile only: no block of
        // this kv tile exists for them, and nothing is stored.
        rsrc_t rds;
        uint32_t ods = 0;
        bool has_blk = a.ds != nullptr;
        if (a.ds) {
            const int kt = c.t * (ROWS / 32) + (wt >> 1);
            const int js0 = win > 0 ? max(0, i0 - win + 1) >> 5 : 0;
            if constexpr (ROWS > 32) {
                const int a1 = min(c.lq - 1, i0 + 31);
                const int js1 = win > 0 ? min(c.lk - 1, a1 + win - 1) >> 5 : (c.lk - 1) >> 5;
                has_blk = kt >= js0 && kt <= js1;
            }
            const size_t blk = (size_t)c.pad0 + (size_t)s * (size_t)c.pad1 + (size_t)(kt - js0);
            rds = slice_rsrc(a.ds + blk * 1024, 1, 2048u, 2048u);
            ods = (uint32_t)(16 * (wt & 1) + l16) * 64u + 8u * (uint32_t)g4;   // row j, q rows 4 (l / 16) ..
        }
        // a wave whose 16 kv rows are past the sample's keys, or have no pair with this
        // q tile in the band, skips the step (its rows of a stored dS block are 0)
        if (j0 >= c.lk || (win > 0 && (j0 - (i0 + 31) >= win || i0 - (j0 + 15) >= win))) {
            if (has_blk) {
                __builtin_amdgcn_raw_buffer_store_b64(u32x2{0u, 0u}, rds, (int)ods, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b64(u32x2{0u, 0u}, rds, (int)(ods + 32u), 0, 0);
            }
            return;
        }
        const char* qt = g.tile(job);
        const char* ot = g.tile(job + 1);
        // The step's LDS reads go out in batches ahead of the products that use them
        // (the scheduling barriers keep the compiler from pairing each product with a
        // read and a wait): the Q and dO row operands, then the products for S and dP,
        // then the transposed operands of the second products, which land while the
        // activation runs.
        // S and dP: element v of block ib holds q row i0 + 16 ib + 4 (l / 16) + v, kv row j0 + l % 16
        f32x4 sc[2], dp[2];
        if constexpr (F8) {   // S on the fp8 MFMA; dP from dO's rows widened
            long qo[2][NKB], oo[2][NKB];
#pragma unroll
            for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    qo[ib][kb] = row8_16_f8<D>(qt, 16 * ib + l16, 4 * kb + g4);
                    oo[ib][kb] = row8_16_f8<D>(ot, 16 * ib + l16, 4 * kb + g4);
                }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) {
                sc[ib] = dp[ib] = f32x4{};
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    sc[ib] = mfma16_f8(qo[ib][kb], kf8[kb], sc[ib]);
                    dp[ib] = mfma16(widen_e4m3((int)oo[ib][kb], (int)(oo[ib][kb] >> 32)), vf[kb], dp[ib]);
                }
            }
        } else {
            bf16x8 qo[2][NKB], oo[2][NKB];
#pragma unroll
            for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    qo[ib][kb] = row8_16<D>(qt, 16 * ib + l16, 4 * kb + g4);
                    oo[ib][kb] = row8_16<D>(ot, 16 * ib + l16, 4 * kb + g4);
                }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ib = 0; ib < 2; ++ib) {
                sc[ib] = dp[ib] = f32x4{};
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    sc[ib] = mfma16(qo[ib][kb], kf[kb], sc[ib]);
                    dp[ib] = mfma16(oo[ib][kb], vf[kb], dp[ib]);
                }
            }
        }
        if constexpr (F8) {   // dP's factor s_do
#pragma unroll
            for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                for (int v = 0; v < 4; ++v) dp[ib][v] *= a.f8_dp;
        }
        constexpr int HC = NCB / 2;
        bf16x8 tv[HC], tk[HC];
#pragma unroll
        for (int cb = 0; cb < HC; ++cb) {
            tv[cb] = col8(ot, 16 * cb);
            tk[cb] = col8(qt, 16 * cb);
        }
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 pm, dm;
        const bool band = win > 0 && !((i0 + 31 - j0) < win && (j0 + 15 - i0) < win);
        if (band) {   // one uniform branch per step
            const int base = i0 + 4 * g4 - j0 - l16;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int ib = e >> 2, v = e & 3;
                float f, ds;
                act(sc[ib][v], dp[ib][v], f, ds);
                const bool ok = in_band(base + 16 * ib + v, win);
                pm[e] = (__bf16)(ok ? f : 0.0f);
                dm[e] = (__bf16)(ok ? ds : 0.0f);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int ib = e >> 2, v = e & 3;
                float f, ds;
                act(sc[ib][v], dp[ib][v], f, ds);
                pm[e] = (__bf16)f;
                dm[e] = (__bf16)ds;
            }
        }
        if (has_blk) {   // dS of q rows 4 (l / 16) + {0..3} and 16 + 4 (l / 16) + {0..3}, kv row j0 + l % 16
            const u32x4 w = __builtin_bit_cast(u32x4, dm);
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{w[0], w[1]}, rds, (int)ods, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{w[2], w[3]}, rds, (int)(ods + 32u), 0, 0);
        }
        // the second half's transposed operands go out before the first half's products
        bf16x8 tv2[HC], tk2[HC];
#pragma unroll
        for (int cb = 0; cb < HC; ++cb) {
            tv2[cb] = col8(ot, 16 * (cb + HC));
            tk2[cb] = col8(qt, 16 * (cb + HC));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int cb = 0; cb < HC; ++cb) {
            accV[cb] = mfma16(tv[cb], pm, accV[cb]);
            accK[cb] = mfma16(tk[cb], dm, accK[cb]);
        }
#pragma unroll
        for (int cb = 0; cb < HC; ++cb) {
            accV[cb + HC] = mfma16(tv2[cb], pm, accV[cb + HC]);
            accK[cb + HC] = mfma16(tk2[cb], dm, accK[cb + HC]);
        }
    }

    // the transposed operand of dV^T += dO^T P and dK^T += Q^T dS (F8: widened to bf16)
    __device__ __forceinline__ bf16x8 col8(const char* tile, int col0) const {
        if constexpr (F8)
            return lds_col8_16_f8<D>(tile, col0, lane);
        else
            return lds_col8_16<D>(tile, 0, col0, lane);
    }

    // this wave's 16 rows of one output (acc: kv row l % 16, columns 16 cb + 4 (l / 16) + {0..3})
    __device__ __forceinline__ void store16(const f32x4 (&acc)[NCB], float mul, void* out, size_t base, int rows,
                                            int row0, char* stage) const {
        // lane-derived offsets computed here, once per item (see opaque)
        const int ln = opaque(lane), l16 = ln & 15, g4 = ln >> 4;
        if (a.out_f32) {
            const rsrc_t ro = slice_rsrc((const float*)out + base, rows, rso, D * 4);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                u32x4 v;
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(acc[cb][i] * mul);
                buf_store16(ro, (uint32_t)(row0 + l16) * rso + (uint32_t)(16 * cb + 4 * g4) * 4u, v);
            }
            return;
        }
        // bf16: stage the 16 rows in a swizzled tile, then store whole rows, 16 bytes per lane
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            u32x2 w;
            w[0] = pack_bf16x2(acc[cb][0] * mul, acc[cb][1] * mul);
            w[1] = pack_bf16x2(acc[cb][2] * mul, acc[cb][3] * mul);
            *(u32x2*)(stage + tile_off_sw<D, SW16>(l16, 2 * cb + (g4 >> 1)) + 8 * (g4 & 1)) = w;
        }
        const rsrc_t ro = slice_rsrc((const __bf16*)out + base, rows, rso, D * 2);
        constexpr int CPR = D / 8, RPI = 64 / CPR;   // 16-byte chunks per row, rows per instruction
        const int rr = ln / CPR, cc = ln % CPR;
#pragma unroll
        for (int k = 0; k < 16 / RPI; ++k) {
            const int row = k * RPI + rr;
            buf_store16(ro, (uint32_t)(row0 + row) * rso + (uint32_t)cc * 16u, *(const u32x4*)(stage + tile_off_sw<D, SW16>(row, cc)));
        }
    }

    // a chunk's partial block: fp32 rows 16 wt + l % 16 of slot `slot` ([slots][ROWS][D])
    __device__ __forceinline__ void partial16(const f32x4 (&acc)[NCB], int slot) const {
        constexpr uint32_t RB = D * 4;
        const int ln = opaque(lane), l16 = ln & 15, g4 = ln >> 4;
        const rsrc_t ro = slice_rsrc(a.part + (size_t)slot * ROWS * D, ROWS, RB, RB);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            u32x4 v;
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(acc[cb][i]);
            buf_store16(ro, (uint32_t)(16 * wt + l16) * RB + (uint32_t)(16 * cb + 4 * g4) * 4u, v);
        }
    }

    template <class RingT>
    __device__ __forceinline__ void item_end(const Rec& c, const RingT& g, int job) {
        if (c.part >= 0) {   // one chunk of a cut item: fp32 partial dK, dV (scaled by the reduction)
            if constexpr (FOLD) {   // the scale P was formed without, before the reduction's factor
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) accV[cb][i] *= scale;
            }
            partial16(accK, 2 * c.part);
            partial16(accV, 2 * c.part + 1);
            return;
        }
        // stage through this wave's 4 KiB of the item's last two slots (free after the
        // team barrier): dK, then dV once this wave has read dK back
        char* stage = g.tile(job - 2 + (wt >> 1)) + (wt & 1) * (16 * D * 2);
        const size_t ob = ((size_t)c.ks * H + c.h) * D;
        store16(accK, F8 ? a.f8_dk : scale, a.dk, ob, c.lk, krow(c), stage);
        wait_lds();
        store16(accV, dv_mul(), a.dv, ob, c.lk, krow(c), stage);
    }

    __device__ __forceinline__ void item_zero(const Rec& c) {
        if (wt & 1) return;   // waves 0, 2 zero the item's 32-row halves
        const size_t ob = ((size_t)c.ks * H + c.h) * D;
        zero<D>(a.dk, ob, c.lk, c.t * ROWS + 16 * wt);
        zero<D>(a.dv, ob, c.lk, c.t * ROWS + 16 * wt);
    }
};

template <int ACT, int T, bool F8>
__global__ __launch_bounds__(64 * T, 2) void dkdv16_kernel(const KernelArgs a, const Rec* __restrict__ recs,
                                                          const int32_t* __restrict__ bin_ptr) {
    using RingT = Ring<128, T, 40 * 512 * T, 0, SW16>;   // 40 KiB per team of two waves
    __shared__ __attribute__((aligned(1024))) char smem[RingT::BYTES];
    const int wt = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    Dkdv16Pol<ACT, T, F8> pol(a, lane, wt);
    run_team<Dkdv16Pol<ACT, T, F8>, RingT, T>(pol, a.P, recs, bin_ptr, smem, (uint32_t)a.H * 128 * 2, wt, lane);
}

// =========================================================================
// dQ from the stored dS blocks
// =========================================================================
// dQ_i = sum_j dS_ij K_j / sqrt(d): a banded product of the dS blocks the dK/dV
// kernel stored (kv row major: block row j, 32 q columns) with K.  One wave per
// workgroup walks its bin's 32-row q items; a step streams one 32-row K tile and
// the item's dS block for that kv tile into one ring slot (ten 1 KiB loads), then
// dQ^T += K^T dS^T with both operands read from LDS by transposing loads.  No
// scores, activations or dO are touched: what the dK/dV kernel already computed
// is reused, so this kernel moves dS and K and does a quarter of the products.
// With fp8 K (F8) its tile is one byte per element in the first half of the K part
// of a slot (which keeps its bf16 size: dQ is staged there), and the K^T operand
// comes from 8-bit transposing reads widened exactly to bf16.
template <bool F8>
struct DsRing {
    static constexpr int D = 128;
    static constexpr int KT = 32 * D * 2, DT = 32 * 32 * 2, SLOT = KT + DT;
    static constexpr int KL = F8 ? KT / 2 : KT;   // bytes of K loaded per job
    static constexpr int JX = (KL + DT) / 1024;   // load instructions per job
    static constexpr int R = 4;
    static constexpr int BYTES = R * SLOT;
    uint32_t offk[KL / 1024], offd[DT / 1024];
    uint32_t base;
    char* gbase;
    int issued;

    // row_stride: bytes between K rows in memory
    __device__ __forceinline__ void init(char* slice, uint32_t row_stride, int lane) {
        gbase = slice;
        base = lds_addr(slice);
        issued = 0;
#pragma unroll
        for (int jj = 0; jj < KL / 1024; ++jj) {
            if constexpr (F8) {   // fp8 K: rows of 8 chunks, swz8<128> (ring.hpp's fp8 tiles)
                const int slot = jj * 64 + lane, row = slot / 8, pos = slot % 8;
                offk[jj] = (uint32_t)row * row_stride + (uint32_t)((pos ^ swz8<D>(row)) << 4);
            } else {   // K: rows of 16 chunks, swz<128>
                const int slot = jj * 64 + lane, row = slot / 16, pos = slot % 16;
                offk[jj] = (uint32_t)row * row_stride + (uint32_t)((pos ^ swz<D>(row)) << 4);
            }
        }
#pragma unroll
        for (int jj = 0; jj < DT / 1024; ++jj) {   // dS block: 64-byte rows of 4 chunks, swz<32>
            const int slot = jj * 64 + lane, row = slot / 4, pos = slot % 4;
            offd[jj] = (uint32_t)row * 64u + (uint32_t)((pos ^ swz<32>(row)) << 4);
        }
    }
    __device__ __forceinline__ char* ktile(int job) const { return gbase + (job % R) * SLOT; }
    __device__ __forceinline__ char* dtile(int job) const { return ktile(job) + KT; }
    // K rows [row0, row0 + 32) of the slice (k_off = row0 * stride) and the 2 KiB dS
    // block `blk` into the next slot
    __device__ __forceinline__ void issue(Slice k, uint32_t k_off, rsrc_t blk) {
        const uint32_t lds = base + (uint32_t)((issued % R) * SLOT);
        const rsrc_t rk = slice_at(k, k_off);
#pragma unroll
        for (int jj = 0; jj < KL / 1024; ++jj) dma16(rk, offk[jj], lds + (uint32_t)jj * 1024u);
#pragma unroll
        for (int jj = 0; jj < DT / 1024; ++jj) dma16(blk, offd[jj], lds + (uint32_t)(KT + jj * 1024));
        ++issued;
    }
    __device__ __forceinline__ void wait(int k) const { wait_jobs<JX>(issued - 1 - k); }
};

template <bool F8>
struct DqDsPol : Common {
    static constexpr int D = 128, NDB = D / 32;
    f32x16 acc[NDB];

    __device__ DqDsPol(const KernelArgs& args, int lane_) : Common(args, lane_, 0, D) {}

    // the job of step s of item w: K tile s and dS block w.pad0 + (s - w.s0)
    __device__ __forceinline__ void issue(DsRing<F8>& g, const Rec& w, int s) const {
        const size_t blk = (size_t)w.pad0 + (size_t)(s - w.s0);
        const rsrc_t ds = slice_rsrc(a.ds + blk * 1024, 1, 2048u, 2048u);
        const size_t kb = ((size_t)w.ks * H + w.h) * D;
        if constexpr (F8)
            g.issue(slice_of((const uint8_t*)a.k + kb, w.lk, rs / 2, D), (uint32_t)(s * 32) * (rs / 2), ds);
        else
            g.issue(slice_of((const __bf16*)a.k + kb, w.lk, rs, D * 2), (uint32_t)(s * 32) * rs, ds);
    }

    __device__ __forceinline__ void step(const DsRing<F8>& g, int job) {
        const char* kt = g.ktile(job);
        const char* dt = g.dtile(job);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            // dS^T operand: kv rows 16 m + {0..3, 8..11} + 4 (l / 32) of q column l % 32
            const bf16x8 b = lds_col8<32>(dt, 16 * m, 0, lane);
            bf16x8 kop[NDB];
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                kop[db] = F8 ? lds_col8_f8<D>(kt, 16 * m, db * 32, lane) : lds_col8<D>(kt, 16 * m, db * 32, lane);
#pragma unroll
            for (int db = 0; db < NDB; ++db) acc[db] = mfma32(kop[db], b, acc[db]);
        }
    }
};

template <bool F8>
__global__ __launch_bounds__(64, 1) void dq_from_ds_kernel(const KernelArgs a, const Rec* __restrict__ recs,
                                                          const int32_t* __restrict__ bin_ptr) {
    __shared__ __attribute__((aligned(1024))) char smem[DsRing<F8>::BYTES];
    const int lane = threadIdx.x;
    const int bin = team_bin();
    if (bin >= a.P) return;
    const int beg = bin_ptr[bin], end = bin_ptr[bin + 1];
    if (beg >= end) return;
#ifdef GDPA_BIN_CLOCK
    const unsigned long long clock0 = __builtin_amdgcn_s_memrealtime();
#endif
    DqDsPol<F8> pol(a, lane);
    DsRing<F8> ring;
    ring.init(smem, (uint32_t)a.H * 128 * (F8 ? 1 : 2), lane);
    // issuing side: the item and step of the next job (items without steps have none)
    int wi = beg, ws = 0;
    Rec wr = recs[beg];
    while (wi < end && wr.s1 < wr.s0)
        if (++wi < end) wr = recs[__builtin_amdgcn_readfirstlane(wi)];
    ws = wr.s0;
    int job = 0;
    auto pump = [&](int consumed) {
        while (wi < end && ring.issued < consumed + DsRing<F8>::R) {
            pol.issue(ring, wr, ws);
            if (++ws > wr.s1) {
                do {
                    if (++wi < end) wr = recs[__builtin_amdgcn_readfirstlane(wi)];
                } while (wi < end && wr.s1 < wr.s0);
                ws = wr.s0;
            }
        }
    };
    pump(job);
    for (int ci = beg; ci < end; ++ci) {
        const Rec c = recs[ci];
        const size_t ob = ((size_t)c.qs * pol.H + c.h) * 128;
        if (c.s1 < c.s0) {
            pol.template zero<128>(a.dq, ob, c.lq, c.t * 32);
            continue;
        }
#pragma unroll
        for (int db = 0; db < DqDsPol<F8>::NDB; ++db) pol.acc[db] = f32x16{};
        for (int s = c.s0; s <= c.s1; ++s) {
            ring.wait(job);
            wait_lds();   // this wave is done reading the slot the pump re-fills next
            pump(job);
            pol.step(ring, job);
            ++job;
        }
        wait_lds();
        if (c.part >= 0) {
            store_partial<DqDsPol<F8>::NDB>(pol.acc, a.part, c.part, 32, 0, pol.r, pol.hh);
            continue;
        }
        // staged through the K tile of the item's last step: the pump re-fills a
        // slot only at the next consume point, after that step's reads
        pol.template store<128>(pol.acc, F8 ? a.f8_dq : pol.scale, a.dq, ob, c.lq, c.t * 32, ring.ktile(job - 1));
    }
#ifdef GDPA_BIN_CLOCK
    if (a.bin_clock && lane == 0) {
        a.bin_clock[2 * bin] = clock0;
        a.bin_clock[2 * bin + 1] = __builtin_amdgcn_s_memrealtime();
    }
#endif
}

// -------------------------------------------------------------------------
// dQ from the stored dS blocks, two-wave teams over 64-row q items
// -------------------------------------------------------------------------
// The same product with two adjacent 32-row q tiles per item, one per wave: each K
// tile of the item's steps (the union of both tiles' bands) is loaded once into
// the team's slot and read by both waves, and each wave loads its own tile's dS
// block beside it.  A step costs 12 KiB of LDS for two tiles' products instead of
// 10 KiB for one, so the same LDS holds half again as much work in flight, with
// six waves per CU instead of four.  A wave whose tile has no block for a step (the
// step pairs only with the other tile, or the item's second tile lies past the
// sample's queries) loads a zero-range block (its instruction count stays the
// team's) and skips the products.  Items of this list carry (pad0, pad1) = (the
// sample's first block of this head, blocks per q tile), as the dK/dV list's do.
template <bool F8>
struct DsRing2 {
    static constexpr int D = 128;
    static constexpr int KT = 32 * D * 2, DT = 32 * 32 * 2, SLOT = KT + 2 * DT;
    static constexpr int KL = F8 ? KT / 2 : KT;   // bytes of K loaded per job
    static constexpr int JK = KL / 1024 / 2;      // K instructions per job and wave
    static constexpr int JX = JK + DT / 1024;     // instructions per job and wave
    static constexpr int R = 4;
    static constexpr int BYTES = R * SLOT;
    uint32_t offk[JK], offd[DT / 1024];
    uint32_t base;
    char* gbase;
    int wt, issued;

    __device__ __forceinline__ void init(char* slice, uint32_t row_stride, int wt_, int lane) {
        gbase = slice;
        base = lds_addr(slice);
        wt = wt_;
        issued = 0;
#pragma unroll
        for (int jj = 0; jj < JK; ++jj) {   // this wave's K instructions: 1 KiB parts 2 jj + wt
            const int slot = (2 * jj + wt) * 64 + lane;
            if constexpr (F8) {
                const int row = slot / 8, pos = slot % 8;
                offk[jj] = (uint32_t)row * row_stride + (uint32_t)((pos ^ swz8<D>(row)) << 4);
            } else {
                const int row = slot / 16, pos = slot % 16;
                offk[jj] = (uint32_t)row * row_stride + (uint32_t)((pos ^ swz<D>(row)) << 4);
            }
        }
#pragma unroll
        for (int jj = 0; jj < DT / 1024; ++jj) {
            const int slot = jj * 64 + lane, row = slot / 4, pos = slot % 4;
            offd[jj] = (uint32_t)row * 64u + (uint32_t)((pos ^ swz<32>(row)) << 4);
        }
    }
    __device__ __forceinline__ char* ktile(int job) const { return gbase + (job % R) * SLOT; }
    __device__ __forceinline__ char* dtile(int job) const { return ktile(job) + KT + wt * DT; }
    // this wave's half of K rows [row0, row0 + 32) (k_off = row0 * stride) and its own
    // 2 KiB dS block `blk` into the next slot
    __device__ __forceinline__ void issue(Slice k, uint32_t k_off, rsrc_t blk) {
        const uint32_t lds = base + (uint32_t)((issued % R) * SLOT);
        const rsrc_t rk = slice_at(k, k_off);
#pragma unroll
        for (int jj = 0; jj < JK; ++jj) dma16(rk, offk[jj], lds + (uint32_t)(2 * jj + wt) * 1024u);
#pragma unroll
        for (int jj = 0; jj < DT / 1024; ++jj) dma16(blk, offd[jj], lds + (uint32_t)(KT + wt * DT + jj * 1024));
        ++issued;
    }
    __device__ __forceinline__ void wait(int k) const { wait_jobs<JX>(issued - 1 - k); }
};

template <bool F8>
struct DqDsTeamPol : Common {
    static constexpr int D = 128, NDB = D / 32;
    f32x16 acc[NDB];

    __device__ DqDsTeamPol(const KernelArgs& args, int lane_, int wt_) : Common(args, lane_, wt_, D) {}

    // this wave's q tile of item w, and the dS block of its step s (-1: none)
    __device__ __forceinline__ int tile(const Rec& w) const { return 2 * w.t + wt; }
    __device__ __forceinline__ long block(const Rec& w, int s) const {
        const int i = tile(w);
        if (i * 32 >= w.lq) return -1;
        const int a1 = min(w.lq - 1, i * 32 + 31);
        const int js0 = win > 0 ? max(0, i * 32 - win + 1) >> 5 : 0;
        const int js1 = win > 0 ? min(w.lk - 1, a1 + win - 1) >> 5 : (w.lk - 1) >> 5;
        if (s < js0 || s > js1) return -1;
        return (long)w.pad0 + (long)i * w.pad1 + (long)(s - js0);
    }

    __device__ __forceinline__ void issue(DsRing2<F8>& g, const Rec& w, int s) const {
        const long blk = block(w, s);
        const rsrc_t ds = blk >= 0 ? slice_rsrc(a.ds + (size_t)blk * 1024, 1, 2048u, 2048u)
                                   : slice_rsrc(a.ds, 0, 2048u, 2048u);
        const size_t kb = ((size_t)w.ks * H + w.h) * D;
        if constexpr (F8)
            g.issue(slice_of((const uint8_t*)a.k + kb, w.lk, rs / 2, D), (uint32_t)(s * 32) * (rs / 2), ds);
        else
            g.issue(slice_of((const __bf16*)a.k + kb, w.lk, rs, D * 2), (uint32_t)(s * 32) * rs, ds);
    }

    // dQ^T += K^T dS^T for this wave's tile (the operands as in the one-wave kernel)
    __device__ __forceinline__ void step(const DsRing2<F8>& g, int job) {
        const char* kt = g.ktile(job);
        const char* dt = g.dtile(job);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const bf16x8 b = lds_col8<32>(dt, 16 * m, 0, lane);
            bf16x8 kop[NDB];
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                kop[db] = F8 ? lds_col8_f8<D>(kt, 16 * m, db * 32, lane) : lds_col8<D>(kt, 16 * m, db * 32, lane);
#pragma unroll
            for (int db = 0; db < NDB; ++db) acc[db] = mfma32(kop[db], b, acc[db]);
        }
    }

    // bf16 output of this wave's 32 rows, staged 64 columns at a time through its own
    // 4 KiB half of `tile` (the K part of the item's last slot)
    __device__ __forceinline__ void store_halves(float mul, size_t ob, int rows, int row0, char* tile) const {
        char* own = tile + wt * 4096;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const f32x16 part[2] = {acc[2 * hf], acc[2 * hf + 1]};
            stage_block<64>(part, mul, own, r, hh);
            store_tile<64>(own, slice_rsrc((const __bf16*)a.dq + ob + 64 * hf, rows, rso, 128),
                           (uint32_t)row0 * rso, rso, lane);
        }
    }
};

template <bool F8>
__global__ __launch_bounds__(128, 1) void dq_from_ds_team_kernel(const KernelArgs a, const Rec* __restrict__ recs,
                                                                const int32_t* __restrict__ bin_ptr) {
    __shared__ __attribute__((aligned(1024))) char smem[DsRing2<F8>::BYTES];
    const int wt = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int bin = team_bin();
    if (bin >= a.P) return;
    const int beg = bin_ptr[bin], end = bin_ptr[bin + 1];
    if (beg >= end) return;
#ifdef GDPA_BIN_CLOCK
    const unsigned long long clock0 = __builtin_amdgcn_s_memrealtime();
#endif
    DqDsTeamPol<F8> pol(a, lane, wt);
    DsRing2<F8> ring;
    ring.init(smem, (uint32_t)a.H * 128 * (F8 ? 1 : 2), wt, lane);
    // issuing side: the item and step of the next job (items without steps have none);
    // both waves walk the same jobs and issue their shares
    int wi = beg, ws = 0;
    Rec wr = recs[beg];
    while (wi < end && wr.s1 < wr.s0)
        if (++wi < end) wr = recs[__builtin_amdgcn_readfirstlane(wi)];
    ws = wr.s0;
    int job = 0;
    auto pump = [&](int consumed) {
        while (wi < end && ring.issued < consumed + DsRing2<F8>::R) {
            pol.issue(ring, wr, ws);
            if (++ws > wr.s1) {
                do {
                    if (++wi < end) wr = recs[__builtin_amdgcn_readfirstlane(wi)];
                } while (wi < end && wr.s1 < wr.s0);
                ws = wr.s0;
            }
        }
    };
    pump(job);
    for (int ci = beg; ci < end; ++ci) {
        const Rec c = recs[ci];
        const size_t ob = ((size_t)c.qs * pol.H + c.h) * 128;
        const int row0 = pol.tile(c) * 32;
        const bool own = row0 < c.lq;   // this wave's tile holds queries
        if (c.s1 < c.s0) {
            if (own) pol.template zero<128>(a.dq, ob, c.lq, row0);
            continue;
        }
#pragma unroll
        for (int db = 0; db < DqDsTeamPol<F8>::NDB; ++db) pol.acc[db] = f32x16{};
        for (int s = c.s0; s <= c.s1; ++s) {
            ring.wait(job);
            team_sync<2>();   // both waves' shares have landed and the slot the pump re-fills is read
            pump(job);
            if (pol.block(c, s) >= 0) pol.step(ring, job);
            ++job;
        }
        if (c.part >= 0) {
            if (own) store_partial<DqDsTeamPol<F8>::NDB>(pol.acc, a.part, c.part, 64, row0 - 64 * c.t, pol.r, pol.hh);
            continue;
        }
        const float mul = F8 ? a.f8_dq : pol.scale;
        if (a.out_f32) {
            if (own) pol.template store<128>(pol.acc, mul, a.dq, ob, c.lq, row0, nullptr);
            continue;
        }
        // the staging slot (the K part of the item's last step) is re-filled only at the
        // next consume point, after both waves are past this barrier's reads of it
        team_sync<2>();
        if (own) pol.store_halves(mul, ob, c.lq, row0, ring.ktile(job - 1));
    }
#ifdef GDPA_BIN_CLOCK
    if (a.bin_clock && threadIdx.x == 0) {
        a.bin_clock[2 * bin] = clock0;
        a.bin_clock[2 * bin + 1] = __builtin_amdgcn_s_memrealtime();
    }
#endif
}

}  // namespace

hipError_t launch_dq_from_ds(const KernelArgs& a, int f8, hipStream_t s) {
    if (a.P <= 0) return hipSuccess;
    if (!a.ds) return hipErrorInvalidValue;
    KernelArgs args = a;
    const void* recs = a.items;
    const int32_t* bin_ptr = a.bin_ptr;
    void* params[] = {&args, &recs, &bin_ptr};
    return hipLaunchKernel(dq_from_ds_kernel_ptr(f8), dim3(a.P), dim3(64), params, 0, s);
}

const void* dq_from_ds_kernel_ptr(int f8) {
    return f8 ? (const void*)&dq_from_ds_kernel<true> : (const void*)&dq_from_ds_kernel<false>;
}

hipError_t launch_dq_from_ds_team(const KernelArgs& a, int f8, hipStream_t s) {
    if (a.P <= 0) return hipSuccess;
    if (!a.ds) return hipErrorInvalidValue;
    KernelArgs args = a;
    const void* recs = a.items;
    const int32_t* bin_ptr = a.bin_ptr;
    void* params[] = {&args, &recs, &bin_ptr};
    return hipLaunchKernel(dq_from_ds_team_kernel_ptr(f8), dim3(a.P), dim3(128), params, 0, s);
}

const void* dq_from_ds_team_kernel_ptr(int f8) {
    return f8 ? (const void*)&dq_from_ds_team_kernel<true> : (const void*)&dq_from_ds_team_kernel<false>;
}

template <int T, bool F8>
const void* dkdv16_ptr(int act) {
    switch (act) {
        case ACT_GELU: return (const void*)&dkdv16_kernel<ACT_GELU, T, F8>;
        case ACT_SILU: return (const void*)&dkdv16_kernel<ACT_SILU, T, F8>;
        case ACT_GELU_POLY: return (const void*)&dkdv16_kernel<ACT_GELU_POLY, T, F8>;
        case ACT_GELU_TAYLOR6: return (const void*)&dkdv16_kernel<ACT_GELU_TAYLOR6, T, F8>;
        case ACT_IDENTITY: return (const void*)&dkdv16_kernel<ACT_IDENTITY, T, F8>;
    }
    return nullptr;
}

const void* dkdv16_kernel_ptr(int rows, int act) {
    const bool f8 = act & kActF8Bwd;
    act &= ~kActF8Bwd;
    if (rows == 32) return f8 ? dkdv16_ptr<2, true>(act) : dkdv16_ptr<2, false>(act);
    if (rows == 64) return f8 ? dkdv16_ptr<4, true>(act) : dkdv16_ptr<4, false>(act);
    return nullptr;
}

}  // namespace gdpa
