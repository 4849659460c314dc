// Row statistics of jagged softmax attention (JFA): the combine of a cut forward
// item's chunks, and the backward's pre-pass.
//
// The backward of a softmax row needs two numbers per (q row, head): the row's
// log-sum-exp from the forward (to rebuild P = exp(S - LSE) without a second
// pass over the keys) and D = sum over the head dimension of dO * O, since the
// softmax Jacobian applied to dP is P * (dP - D).  This pre-pass stores both as
// one fp32 pair per (head, row), head-major, so that the 32 rows of a q tile are
// 256 consecutive bytes that one load instruction brings into LDS beside the tile.
#include "device.hpp"
#include "kernels.hpp"

namespace gdpa {
namespace {

// G = d / 8 lanes per (row, head) pair, 16 bytes of O and of dO each; grid covers
// Tq * H pairs (pair p = row * H + h: rows of [Tq, H, d] are contiguous).
template <int G>
__global__ __launch_bounds__(256) void jfa_stat_kernel(const __bf16* __restrict__ o, const __bf16* __restrict__ dout,
                                                       const float* __restrict__ lse, int Tq, int H,
                                                       float* __restrict__ stat) {
    constexpr float L2E = 1.4426950408889634f;
    const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
    const size_t pair = t / G, n = (size_t)Tq * H;
    const int c = (int)(t % G);
    float acc = 0.0f;
    if (pair < n) {
        const u32x4 x = *(const u32x4*)(o + pair * (8 * G) + 8 * c);
        const u32x4 y = *(const u32x4*)(dout + pair * (8 * G) + 8 * c);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float xl = __uint_as_float(x[w] << 16), xh = __uint_as_float(x[w] & 0xffff0000u);
            const float yl = __uint_as_float(y[w] << 16), yh = __uint_as_float(y[w] & 0xffff0000u);
            acc = __builtin_fmaf(xl, yl, acc);
            acc = __builtin_fmaf(xh, yh, acc);
        }
    }
#pragma unroll
    for (int m = G / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
    if (pair < n && c == 0) {
        const int row = (int)(pair / H), h = (int)(pair % H);
        const size_t i = (size_t)h * Tq + row;
        *(float2*)(stat + 2 * i) = make_float2(lse[i] * L2E, acc);
    }
}

// Forward chunks of a cut item (one q tile against consecutive runs of kv tiles):
// each slot j holds the unnormalised block O_j = sum over its keys of
// 2^(s - m_j) V with its rows' running max m_j (log2 units) and sum l_j.  The
// softmax over the whole row is recovered by rescaling every slot to the common
// max, the same correction the online softmax applies between steps.
// grid (ceil(rows_per_slot d / 4 / 256), cut items); a thread owns 4 columns of a row.
__global__ __launch_bounds__(256) void jfa_combine_kernel(const DevGroup* __restrict__ groups,
                                                          const float* __restrict__ part,
                                                          const float* __restrict__ pstat, int rows_per_slot, int d,
                                                          int H, int Tq, void* __restrict__ out, int out_f32,
                                                          float* __restrict__ lse) {
    const DevGroup g = groups[blockIdx.y];
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= g.rows * d / 4) return;
    const int row = 4 * i / d, col = 4 * i % d;
    const float* st = pstat + ((size_t)g.slot0 * rows_per_slot + row) * 2;
    const size_t sstep = (size_t)rows_per_slot * 2;
    float m = kNegBig;
    for (int j = 0; j < g.n; ++j) m = __builtin_fmaxf(m, st[j * sstep]);
    const float* src = part + ((size_t)g.slot0 * rows_per_slot + row) * d + col;
    const size_t ostep = (size_t)rows_per_slot * d;
    float l = 0.0f;
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int j = 0; j < g.n; ++j) {
        const float w = __builtin_amdgcn_exp2f(st[j * sstep] - m);   // 0 for a slot without keys of this row
        l = __builtin_fmaf(w, st[j * sstep + 1], l);
        const float4 x = *(const float4*)(src + j * ostep);
        acc.x = __builtin_fmaf(w, x.x, acc.x);
        acc.y = __builtin_fmaf(w, x.y, acc.y);
        acc.z = __builtin_fmaf(w, x.z, acc.z);
        acc.w = __builtin_fmaf(w, x.w, acc.w);
    }
    const float mul = l > 0.0f ? 1.0f / l : 0.0f;
    const size_t o = ((size_t)(g.row0 + row) * H + g.h) * d + col;
    if (out_f32) {
        *(float4*)((float*)out + o) = make_float4(acc.x * mul, acc.y * mul, acc.z * mul, acc.w * mul);
    } else {
        uint2 w;
        w.x = pack_bf16x2(acc.x * mul, acc.y * mul);
        w.y = pack_bf16x2(acc.z * mul, acc.w * mul);
        *(uint2*)((__bf16*)out + o) = w;
    }
    if (col == 0)
        lse[(size_t)g.h * Tq + g.row0 + row] =
            l > 0.0f ? (m + __builtin_amdgcn_logf(l)) * 0.69314718055994531f : -__builtin_inff();
}

}  // namespace

hipError_t launch_jfa_combine(const DevGroup* groups, int n_groups, const float* part, const float* part_stat,
                              int rows_per_slot, int d, int H, int Tq, void* out, int out_f32, float* lse,
                              hipStream_t s) {
    if (n_groups <= 0) return hipSuccess;
    if (!groups || !part || !part_stat || !out || !lse || rows_per_slot <= 0 || d % 4 != 0)
        return hipErrorInvalidValue;
    const int quads = rows_per_slot * d / 4;
    for (int g0 = 0; g0 < n_groups; g0 += 65535) {
        const int ng = n_groups - g0 < 65535 ? n_groups - g0 : 65535;
        hipLaunchKernelGGL(jfa_combine_kernel, dim3((quads + 255) / 256, ng), dim3(256), 0, s, groups + g0, part,
                           part_stat, rows_per_slot, d, H, Tq, out, out_f32, lse);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_jfa_stat(const void* o, const void* dout, const float* lse, int Tq, int H, int d, float* stat,
                           hipStream_t s) {
    if (Tq <= 0 || H <= 0) return hipSuccess;
    if (!o || !dout || !lse || !stat) return hipErrorInvalidValue;
    const size_t threads = (size_t)Tq * H * (d / 8);
    const dim3 grid((unsigned)((threads + 255) / 256));
    const __bf16* ob = (const __bf16*)o;
    const __bf16* db = (const __bf16*)dout;
    switch (d) {
        case 32: hipLaunchKernelGGL(jfa_stat_kernel<4>, grid, dim3(256), 0, s, ob, db, lse, Tq, H, stat); break;
        case 64: hipLaunchKernelGGL(jfa_stat_kernel<8>, grid, dim3(256), 0, s, ob, db, lse, Tq, H, stat); break;
        case 128: hipLaunchKernelGGL(jfa_stat_kernel<16>, grid, dim3(256), 0, s, ob, db, lse, Tq, H, stat); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace gdpa
