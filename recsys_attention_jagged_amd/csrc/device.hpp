// Device-side building blocks shared by the GDPA kernels (gfx950 only).
//
//  * Buffer resources: every global access goes through a buffer descriptor
//    that covers exactly one (sample, head) slice of a tensor, so rows beyond
//    the sample's length read as zero and stores to them are dropped by the
//    hardware range check.  This is what makes jagged tiles safe without
//    per-element predicates.
//  * MFMA: v_mfma_f32_32x32x16_bf16.  For a 32x32 output block, lane l holds
//    column (l % 32) and rows 8 j + 4 (l / 32) + i in accumulator element
//    4 j + i.  A and B operands give each lane 8 bf16 of one row (A) / column
//    (B); which 8 contraction indices a lane group supplies is our choice, as
//    long as A and B agree.
//  * Chained products: the accumulator of S (or S^T) is converted to bf16 in
//    registers and used directly as the B operand of the second product; the
//    8 contraction rows a lane then supplies are rows {0..3, 8..11} + 4 (l/32)
//    of a 16-row block, which the A operand reads with transposing LDS loads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gelu_poly.h"
#include "gelu_tail.h"

namespace gdpa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum Act { ACT_GELU = 0, ACT_SILU = 1, ACT_GELU_POLY = 2, ACT_GELU_TAYLOR6 = 3, ACT_IDENTITY = 4, ACT_ONE = 5,
           ACT_SOFTMAX = 6 };   // softmax: jagged softmax attention (JFA) through the same kernels

// running-max sentinel of the softmax kernels: finite, so that differences of two
// sentinels are 0, not NaN
constexpr float kNegBig = -1.0e30f;

// -------------------------------------------------------------------------
// buffer resources
// -------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Descriptor over rows [0, rows) of one (sample, head) slice: `base` points at
// row 0 of the head, rows are `row_bytes_stride` apart and `row_bytes` long.
__device__ __forceinline__ rsrc_t slice_rsrc(const void* base, int rows, uint32_t row_stride_bytes,
                                             uint32_t row_bytes) {
    const uint32_t n = rows > 0 ? (uint32_t)(rows - 1) * row_stride_bytes + row_bytes : 0u;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)n, 0x00020000);
}

// The same slice kept as (first byte, bytes in range), for the tile loads: each
// load builds its descriptor at the tile's first row (slice_at), so the per-lane
// offsets inside a tile never change and the range check stays exact (an offset v
// of slice_at(s, off) is in range iff off + v is in range of s).
struct Slice {
    const char* base;
    uint32_t bytes;
};

__device__ __forceinline__ Slice slice_of(const void* base, int rows, uint32_t row_stride_bytes, uint32_t row_bytes) {
    return Slice{(const char*)base, rows > 0 ? (uint32_t)(rows - 1) * row_stride_bytes + row_bytes : 0u};
}

// (the slice and the offset are uniform; readfirstlane keeps the descriptor in
// scalar registers, where the load instructions take it)
__device__ __forceinline__ rsrc_t slice_at(Slice s, uint32_t off) {
    const uint64_t a = (uint64_t)(size_t)(s.base + off);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const uint32_t n = __builtin_amdgcn_readfirstlane(s.bytes > off ? s.bytes - off : 0u);
    return __builtin_amdgcn_make_buffer_rsrc((void*)(size_t)((uint64_t)hi << 32 | lo), 0, (int)n, 0x00020000);
}

__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

__device__ __forceinline__ void buf_store16(rsrc_t r, uint32_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 0);
}

// -------------------------------------------------------------------------
// small helpers
// -------------------------------------------------------------------------
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const __bf16 a = (__bf16)lo, b = (__bf16)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// 8 consecutive accumulator elements [8 m, 8 m + 8) -> bf16x8 operand
__device__ __forceinline__ bf16x8 acc_to_bf16x8(const f32x16& c, int m) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (__bf16)c[8 * m + e];
    return r;
}

// -------------------------------------------------------------------------
// activations
// -------------------------------------------------------------------------
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Phi(-|x|) (standard normal tail) and e = exp(-x^2 / 2), with the erf
// approximation of Abramowitz & Stegun, Handbook of Mathematical Functions,
// formula 7.1.26: erf(z) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-z^2),
// t = 1/(1 + p z), z >= 0, |error| <= 1.5e-7.  One reciprocal and one
// exponential, no branches.
__device__ __forceinline__ float normal_tail(float x, float& e) {
    constexpr float p = 0.3275911f * 0.70710678118654752f;   // p / sqrt(2): z = |x| / sqrt(2)
    // a_k / 2, so that q = erfc(z) / 2 / exp(-z^2)
    constexpr float h1 = 0.5f * 0.254829592f, h2 = 0.5f * -0.284496736f, h3 = 0.5f * 1.421413741f;
    constexpr float h4 = 0.5f * -1.453152027f, h5 = 0.5f * 1.061405429f;
    const float t = fast_rcp(__builtin_fmaf(p, __builtin_fabsf(x), 1.0f));
    const float q = t * __builtin_fmaf(t, __builtin_fmaf(t, __builtin_fmaf(t, __builtin_fmaf(t, h5, h4), h3), h2), h1);
    e = fast_exp2(x * x * -0.72134752044448170f);   // exp(-x^2/2) = 2^(-x^2 log2(e) / 2)
    return q * e;
}

// GELU and GELU' of x = scale s from the raw score s, with the scale and the density's
// constant folded into the constants of the same erfc approximation (A&S 7.1.26):
//   t  = 1 / (1 + (p scale / sqrt 2) |s|),
//   e' = 2^(s^2 (-log2(e) scale^2 / 2) + log2(scale / sqrt(2 pi))) = scale phi(x),
//   Phi(-|x|) = (sum_k a_k / (2 scale / sqrt(2 pi)) t^k) e',
// so that GELU'(x) = Phi(x) + s e' is one FMA.  The value comes back divided by the
// scale, GELU(x) / scale = s Phi(x): the caller applies the scale where the value's
// products end (an output multiplier).  Two multiplies per score fewer than
// act_fwd_grad on scale s.
struct GeluFold {
    float p, k, l, h1, h2, h3, h4, h5;
};
__device__ __forceinline__ GeluFold gelu_fold(float scale) {
    GeluFold c;
    const float inv = 2.5066282746310002f / scale;   // 1 / (scale / sqrt(2 pi))
    c.p = 0.3275911f * 0.70710678118654752f * scale;
    c.k = -0.72134752044448170f * scale * scale;
    c.l = __builtin_amdgcn_logf(scale * 0.39894228040143268f);   // log2
    c.h1 = 0.5f * 0.254829592f * inv;
    c.h2 = 0.5f * -0.284496736f * inv;
    c.h3 = 0.5f * 1.421413741f * inv;
    c.h4 = 0.5f * -1.453152027f * inv;
    c.h5 = 0.5f * 1.061405429f * inv;
    return c;
}
__device__ __forceinline__ void gelu_grad_folded(float s, const GeluFold& c, float& f_over_scale, float& g) {
    const float t = fast_rcp(__builtin_fmaf(c.p, __builtin_fabsf(s), 1.0f));
    const float q = t * __builtin_fmaf(t, __builtin_fmaf(t, __builtin_fmaf(t, __builtin_fmaf(t, c.h5, c.h4), c.h3), c.h2), c.h1);
    const float e = fast_exp2(__builtin_fmaf(s * s, c.k, c.l));
    const float tail = q * e;
    const float cdf = s >= 0.0f ? 1.0f - tail : tail;
    f_over_scale = s * cdf;
    g = __builtin_fmaf(s, e, cdf);
}

// Phi(x) and exp(-x^2 / 2)
__device__ __forceinline__ void normal_cdf(float x, float& cdf, float& e) {
    const float c = normal_tail(x, e);
    cdf = x >= 0.0f ? 1.0f - c : c;
}

// Clamped polynomial GELU (value): x/2 + sum_k a_k x^(2k) on |x| <= R, else
// max(x, 0); FMAs only.  Error bound over the real line in gelu_poly.h.
__device__ __forceinline__ float gelu_poly_value(float x) {
    const float u = x * x;
    float p = kGeluPolyCoef[GDPA_GELU_POLY_DEGREE];
#pragma unroll
    for (int k = GDPA_GELU_POLY_DEGREE - 1; k >= 0; --k) p = __builtin_fmaf(p, u, kGeluPolyCoef[k]);
    return __builtin_fabsf(x) <= GDPA_GELU_POLY_R ? __builtin_fmaf(0.5f, x, p) : __builtin_fmaxf(x, 0.0f);
}

// Phi(-|x|) as 2^p(|x|), p the degree-5 fit of log2 Phi(-z) in gelu_tail.h: five
// FMAs and one exp2.  p falls without bound past its fit range, so 2^p vanishes
// faster than |x| grows and the form needs no clamp.
__device__ __forceinline__ float normal_tail_exp2(float x) {
    const float z = __builtin_fabsf(x);
    float p = kGeluTailCoef[GDPA_GELU_TAIL_DEGREE];
#pragma unroll
    for (int k = GDPA_GELU_TAIL_DEGREE - 1; k >= 0; --k) p = __builtin_fmaf(p, z, kGeluTailCoef[k]);
    return fast_exp2(p);
}

template <int ACT>
__device__ __forceinline__ float act_fwd(float x) {
    if constexpr (ACT == ACT_GELU) {
        // x Phi(x) = max(x, 0) - |x| Phi(-|x|); absolute error within GDPA_GELU_TAIL_BOUND
        return __builtin_fmaf(-__builtin_fabsf(x), normal_tail_exp2(x), __builtin_fmaxf(x, 0.0f));
    } else if constexpr (ACT == ACT_SILU) {
        return x * fast_rcp(1.0f + fast_exp2(x * -1.4426950408889634f));
    } else if constexpr (ACT == ACT_GELU_POLY) {
        return gelu_poly_value(x);
    } else if constexpr (ACT == ACT_GELU_TAYLOR6) {
        // GDPA page, code figure of the ALU-only Taylor GELU: x/2 + x^2/sqrt(2 pi)
        // - x^4/(6 sqrt(2 pi)) + x^6/(40 sqrt(2 pi)).
        const float u = x * x;
        const float c2 = 0.3989422804014327f, c4 = -0.0664903800669055f, c6 = 0.0099735570100358f;
        return __builtin_fmaf(0.5f, x, u * __builtin_fmaf(u, __builtin_fmaf(u, c6, c4), c2));
    } else if constexpr (ACT == ACT_IDENTITY) {
        return x;
    } else {
        return 1.0f;
    }
}

// act(x) and act'(x) together
template <int ACT>
__device__ __forceinline__ void act_fwd_grad(float x, float& f, float& g) {
    if constexpr (ACT == ACT_GELU) {
        float cdf, e;
        normal_cdf(x, cdf, e);
        f = x * cdf;
        g = __builtin_fmaf(x * 0.39894228040143268f, e, cdf);   // Phi(x) + x phi(x)
    } else if constexpr (ACT == ACT_SILU) {
        const float s = fast_rcp(1.0f + fast_exp2(x * -1.4426950408889634f));
        f = x * s;
        g = s * __builtin_fmaf(x, 1.0f - s, 1.0f);
    } else if constexpr (ACT == ACT_GELU_POLY) {
        // two chains with coefficients of their own; a caller that drops f
        // (the dQ kernel) evaluates only the derivative's
        f = gelu_poly_value(x);
        const float u = x * x;
        float q = kGeluPolyGradCoef[GDPA_GELU_POLY_GRAD_DEGREE];
#pragma unroll
        for (int k = GDPA_GELU_POLY_GRAD_DEGREE - 1; k >= 0; --k) q = __builtin_fmaf(q, u, kGeluPolyGradCoef[k]);
        g = __builtin_fabsf(x) <= GDPA_GELU_POLY_R ? __builtin_fmaf(x, q, 0.5f) : (x > 0.0f ? 1.0f : 0.0f);
    } else if constexpr (ACT == ACT_GELU_TAYLOR6) {
        const float u = x * x;
        const float c2 = 0.3989422804014327f, c4 = -0.0664903800669055f, c6 = 0.0099735570100358f;
        f = __builtin_fmaf(0.5f, x, u * __builtin_fmaf(u, __builtin_fmaf(u, c6, c4), c2));
        g = __builtin_fmaf(x, __builtin_fmaf(u, __builtin_fmaf(u, 6.0f * c6, 4.0f * c4), 2.0f * c2), 0.5f);
    } else if constexpr (ACT == ACT_IDENTITY) {
        f = x;
        g = 1.0f;
    } else {
        f = 1.0f;
        g = 0.0f;
    }
}

// -------------------------------------------------------------------------
// work-list records (written by the host planner)
// -------------------------------------------------------------------------
// One work item: sample rows start at qs (queries) / ks (keys) with lengths lq /
// lk, head h, stationary tile t and streaming tiles s0..s1 (none if s1 < s0);
// part >= 0: the item is one chunk of a longer one and stores its fp32 output
// block into partial slot `part` instead of the output.
// v, opaque to the compiler: values derived from it are computed where they are
// used instead of being hoisted out of the surrounding loops, where they would be
// kept in registers (or spilled to scratch) across every step.  A scratch reload is
// a vector memory load and waits behind the ring's tile loads still in flight.
__device__ __forceinline__ int opaque(int v) {
    int r;
    asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "v"(v));
    return r;
}

struct Rec {
    int32_t qs, lq, ks, lk, h, t, s0, s1, part, pad0, pad1, pad2;
};

// |dd| < win (win >= 1) as one unsigned compare, so that a mask is a select and
// not a branch: dd + win - 1 lies in [0, 2 win - 2]
__device__ __forceinline__ bool in_band(int dd, int win) {
    return (uint32_t)(dd + win - 1) <= (uint32_t)(2 * win - 2);
}

// Does no pair of the 32 x 32 block (rows i0.., columns j0..) lie inside the band
// |i - j| < win?  The block's differences j - i are the integers j0 - i0 - 31 ..
// j0 - i0 + 31, so it misses the band iff that range lies at or beyond +-win.
__device__ __forceinline__ bool band_none(int i0, int j0, int win) {
    return j0 - (i0 + 31) >= win || i0 - (j0 + 31) >= win;
}

// Does every pair of the 32 x 32 block (rows i0.., columns j0..) lie inside the
// band |i - j| < win?  (Sample lengths need no test: rows beyond a length are
// zero-filled tiles, whose products and stores vanish.)
__device__ __forceinline__ bool band_all(int i0, int j0, int win) {
    return (i0 + 31 - j0) < win && (j0 + 31 - i0) < win;
}

// -------------------------------------------------------------------------
// stores of a 32-row output block held as an MFMA accumulator: lane l holds
// output row `row` (the accumulator column) and columns d = 32 db + 8 j + 4 (l/32) + i
// in element 4 j + i of acc[db]; rows beyond the slice are dropped by the
// descriptor's range check
// -------------------------------------------------------------------------
template <int NDB>
__device__ __forceinline__ void store_block_bf16(const f32x16 (&acc)[NDB], float mul, rsrc_t ro, uint32_t row_off,
                                                 int hh) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            u32x2 w;
            w[0] = pack_bf16x2(acc[db][4 * j] * mul, acc[db][4 * j + 1] * mul);
            w[1] = pack_bf16x2(acc[db][4 * j + 2] * mul, acc[db][4 * j + 3] * mul);
            __builtin_amdgcn_raw_buffer_store_b64(w, ro, (int)(row_off + (32 * db + 8 * j + 4 * hh) * 2), 0, 0);
        }
}

template <int NDB>
__device__ __forceinline__ void store_block_f32(const f32x16 (&acc)[NDB], float mul, rsrc_t ro, uint32_t row_off,
                                                int hh);

// A chunk's 32-row block as fp32 into slot `slot` of a [slots][rows][32 NDB]
// buffer, at item row row0 (the lane's accumulator column r is row row0 + r).
template <int NDB>
__device__ __forceinline__ void store_partial(const f32x16 (&acc)[NDB], float* part, int slot, int rows, int row0,
                                              int r, int hh) {
    constexpr uint32_t RB = 32 * NDB * 4;
    const rsrc_t ro = slice_rsrc(part + (size_t)slot * rows * 32 * NDB, rows, RB, RB);
    store_block_f32<NDB>(acc, 1.0f, ro, (uint32_t)(row0 + r) * RB, hh);
}

template <int NDB>
__device__ __forceinline__ void store_block_f32(const f32x16 (&acc)[NDB], float mul, rsrc_t ro, uint32_t row_off,
                                                int hh) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            u32x4 v;
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(acc[db][4 * j + i] * mul);
            buf_store16(ro, row_off + (32 * db + 8 * j + 4 * hh) * 4, v);
        }
}

}  // namespace gdpa
