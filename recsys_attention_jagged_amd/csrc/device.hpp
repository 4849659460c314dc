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
//  * Transposed tiles: an operand that must be contracted over rows (V, K^T,
//    Q^T, dO^T) is stored in LDS as [d][row'] where row' swaps bits 2 and 3 of
//    the row index inside each 16-row block.  With that permutation the 8
//    contraction rows a lane needs for a chained MFMA (the rows an accumulator
//    lane holds) are contiguous, so every operand read is one 16-byte LDS read.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gelu_poly.h"

namespace gdpa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum Act { ACT_GELU = 0, ACT_SILU = 1, ACT_GELU_POLY = 2, ACT_GELU_TAYLOR6 = 3, ACT_IDENTITY = 4, ACT_ONE = 5 };

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

// row permutation of transposed tiles: swap bits 2 and 3
__device__ __forceinline__ int tpos(int row) { return (row & ~12) | ((row & 4) << 1) | ((row & 8) >> 1); }

// Logical bin of this workgroup.  Workgroups are dispatched round-robin over the
// 8 XCDs, so consecutive logical bins (which the planner fills with neighbouring
// items of equal cost, e.g. adjacent q tiles of one sample) are placed on the
// same XCD and share its L2.
__device__ __forceinline__ int logical_bin(int P) {
    const int w = blockIdx.x;
    if (P % 8 != 0) return w;
    return (w % 8) * (P / 8) + w / 8;
}

// -------------------------------------------------------------------------
// activations
// -------------------------------------------------------------------------
template <int ACT>
__device__ __forceinline__ float act_fwd(float x) {
    if constexpr (ACT == ACT_GELU) {
        return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f));
    } else if constexpr (ACT == ACT_SILU) {
        return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
    } else if constexpr (ACT == ACT_GELU_POLY) {
        const float u = x * x;
        float p = kGeluPolyCoef[GDPA_GELU_POLY_DEGREE];
#pragma unroll
        for (int k = GDPA_GELU_POLY_DEGREE - 1; k >= 0; --k) p = __builtin_fmaf(p, u, kGeluPolyCoef[k]);
        return __builtin_fabsf(x) <= GDPA_GELU_POLY_R ? __builtin_fmaf(0.5f, x, p) : __builtin_fmaxf(x, 0.0f);
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
        const float cdf = 0.5f * (1.0f + erff(x * 0.70710678118654752f));
        const float pdf = 0.39894228040143268f * __expf(-0.5f * x * x);
        f = x * cdf;
        g = __builtin_fmaf(x, pdf, cdf);
    } else if constexpr (ACT == ACT_SILU) {
        const float s = __builtin_amdgcn_rcpf(1.0f + __expf(-x));
        f = x * s;
        g = s * __builtin_fmaf(x, 1.0f - s, 1.0f);
    } else if constexpr (ACT == ACT_GELU_POLY) {
        const float u = x * x;
        float p = kGeluPolyCoef[GDPA_GELU_POLY_DEGREE];
        float dp = GDPA_GELU_POLY_DEGREE * kGeluPolyCoef[GDPA_GELU_POLY_DEGREE];
#pragma unroll
        for (int k = GDPA_GELU_POLY_DEGREE - 1; k >= 0; --k) {
            p = __builtin_fmaf(p, u, kGeluPolyCoef[k]);
            if (k >= 1) dp = __builtin_fmaf(dp, u, (float)k * kGeluPolyCoef[k]);
        }
        const bool in = __builtin_fabsf(x) <= GDPA_GELU_POLY_R;
        f = in ? __builtin_fmaf(0.5f, x, p) : __builtin_fmaxf(x, 0.0f);
        g = in ? __builtin_fmaf(2.0f * x, dp, 0.5f) : (x > 0.0f ? 1.0f : 0.0f);
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
// tile staging: global (one sample/head slice) -> registers -> LDS
// -------------------------------------------------------------------------
// A tile of ROWS rows x D bf16 columns is read with coalesced 16-byte loads
// (consecutive threads read consecutive 16-byte chunks of a row); each thread
// owns row pairs (2p, 2p + 1) at one chunk so that a transposed store can write
// the two rows' elements as one 32-bit word.
template <int ROWS, int D>
struct TileStage {
    static constexpr int CPR = D / 8;                 // 16-byte chunks per row
    static constexpr int PAIRS_PER_PASS = 256 / CPR;
    static constexpr int PASSES = (ROWS / 2 + PAIRS_PER_PASS - 1) / PAIRS_PER_PASS;
    u32x4 r[PASSES][2];

    // rows [row0, row0 + ROWS) of the slice; rows outside the slice read 0
    __device__ __forceinline__ void load(rsrc_t rs, int row0, uint32_t row_stride_bytes, int tid) {
        const int c = tid % CPR;
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const int row = 2 * (p * PAIRS_PER_PASS + tid / CPR);
            if (row < ROWS) {
                const uint32_t off = (uint32_t)(row0 + row) * row_stride_bytes + (uint32_t)c * 16u;
                r[p][0] = buf_load16(rs, off);
                r[p][1] = buf_load16(rs, off + row_stride_bytes);
            }
        }
    }

    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int p = 0; p < PASSES; ++p) r[p][0] = r[p][1] = u32x4{0u, 0u, 0u, 0u};
    }

    // row-major: lds[row * LDST + col]
    template <int LDST>
    __device__ __forceinline__ void store_rows(__bf16* lds, int tid) const {
        const int c = tid % CPR;
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const int row = 2 * (p * PAIRS_PER_PASS + tid / CPR);
            if (row < ROWS) {
                *(u32x4*)(lds + row * LDST + 8 * c) = r[p][0];
                *(u32x4*)(lds + (row + 1) * LDST + 8 * c) = r[p][1];
            }
        }
    }

    // transposed: lds[col * LDST + tpos(row)]
    template <int LDST>
    __device__ __forceinline__ void store_cols(__bf16* lds, int tid) const {
        const int c = tid % CPR;
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const int row = 2 * (p * PAIRS_PER_PASS + tid / CPR);
            if (row < ROWS) {
                const int pos = tpos(row);   // even; row + 1 lands at pos + 1
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const uint32_t a = r[p][0][w], b = r[p][1][w];
                    const uint32_t lo = (a & 0xffffu) | (b << 16);       // column 8c + 2w
                    const uint32_t hi = (a >> 16) | (b & 0xffff0000u);   // column 8c + 2w + 1
                    *(uint32_t*)(lds + (8 * c + 2 * w) * LDST + pos) = lo;
                    *(uint32_t*)(lds + (8 * c + 2 * w + 1) * LDST + pos) = hi;
                }
            }
        }
    }
};

// -------------------------------------------------------------------------
// flattened walk over a bin's (item, step) pairs
// -------------------------------------------------------------------------
struct ItemRec {
    int32_t b, h, t, s0, s1, pad0, pad1, pad2;
};

// All fields are uniform across the workgroup.  An item without steps
// (s1 < s0) is visited once, as a step that only writes its (zero) output.
struct StepIt {
    int idx, end;
    int b, h, t, s0, s1, s;
    int qs, lq, ks, lk;

    __device__ __forceinline__ void load(const ItemRec* items, const int32_t* q_off,
                                         const int32_t* kv_off, int i) {
        const ItemRec it = items[i];
        idx = i;
        b = it.b;
        h = it.h;
        t = it.t;
        s0 = it.s0;
        s1 = it.s1;
        s = it.s0;
        qs = q_off[b];
        lq = q_off[b + 1] - qs;
        ks = kv_off[b];
        lk = kv_off[b + 1] - ks;
    }
    __device__ __forceinline__ bool has_steps() const { return s1 >= s0; }
    __device__ __forceinline__ bool first() const { return s == s0; }
    __device__ __forceinline__ bool last() const { return s >= s1; }
    // move to the next step of this bin; false at the end
    __device__ __forceinline__ bool advance(const ItemRec* items, const int32_t* q_off,
                                            const int32_t* kv_off) {
        if (s < s1) {
            ++s;
            return true;
        }
        if (idx + 1 < end) {
            load(items, q_off, kv_off, idx + 1);
            return true;
        }
        return false;
    }
};

// Does the 32 x 32 block (rows i0.., columns j0..) of a sample with lengths
// (li, lj) hold a valid pair / only valid pairs?  win = window or a huge value.
__device__ __forceinline__ bool block_any(int i0, int j0, int li, int lj, int win) {
    return i0 < li && j0 < lj && (j0 - (i0 + 31)) < win && (i0 - (j0 + 31)) < win;
}
__device__ __forceinline__ bool block_all(int i0, int j0, int li, int lj, int win) {
    return i0 + 31 < li && j0 + 31 < lj && (i0 + 31 - j0) < win && (j0 + 31 - i0) < win;
}

}  // namespace gdpa
