// Row statistics for the backward of jagged softmax attention (JFA).
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

}  // namespace

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
