// Pre-pass of the RMSNorm prologue: 1/rms of every (row, head) of Q, K and V.
//
// The fused kernels read the raw tensors and scale their products by these
// factors (GDPA page, "Section details", the chart comparing tanh GELU with the
// 6th-order series: RMSNorm keeps the activation's inputs in range; read as a
// per-(token, head) RMSNorm over d with no gain, applied right before GDPA).  One
// pass reads each tensor once and writes 4 bytes per row and head, in the layouts
// the kernels' side loads take: [H, Tq] for Q, [H, Tk, 2] (k, v pairs) for K and V.
#include "device.hpp"
#include "kernels.hpp"

namespace gdpa {
namespace {

// G = d / 8 lanes per (row, head) pair of x [T, H, d] bf16; pair p = row * H + h.
// out[(h * T + row) * stride + offset] = 1 / sqrt(mean(x^2) + eps), or 1 when !on.
template <int G>
__global__ __launch_bounds__(256) void rstd_kernel(const __bf16* __restrict__ x, int T, int H, int on, float eps,
                                                   float* __restrict__ out, int stride, int offset) {
    const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
    const size_t pair = t / G, n = (size_t)T * H;
    const int c = (int)(t % G);
    float acc = 0.0f;
    if (on && pair < n) {
        const u32x4 w = *(const u32x4*)(x + pair * (8 * G) + 8 * c);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float lo = __uint_as_float(w[i] << 16), hi = __uint_as_float(w[i] & 0xffff0000u);
            acc = __builtin_fmaf(lo, lo, acc);
            acc = __builtin_fmaf(hi, hi, acc);
        }
    }
#pragma unroll
    for (int m = G / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
    if (pair < n && c == 0) {
        const int row = (int)(pair / H), h = (int)(pair % H);
        out[((size_t)h * T + row) * stride + offset] = on ? 1.0f / __builtin_sqrtf(acc / (8 * G) + eps) : 1.0f;
    }
}

hipError_t launch_one(const void* x, int T, int H, int d, int on, float eps, float* out, int stride, int offset,
                      hipStream_t s) {
    if (T <= 0) return hipSuccess;
    const size_t threads = (size_t)T * H * (d / 8);
    const dim3 grid((unsigned)((threads + 255) / 256));
    const __bf16* xb = (const __bf16*)x;
    switch (d) {
        case 32: hipLaunchKernelGGL(rstd_kernel<4>, grid, dim3(256), 0, s, xb, T, H, on, eps, out, stride, offset); break;
        case 64: hipLaunchKernelGGL(rstd_kernel<8>, grid, dim3(256), 0, s, xb, T, H, on, eps, out, stride, offset); break;
        case 128: hipLaunchKernelGGL(rstd_kernel<16>, grid, dim3(256), 0, s, xb, T, H, on, eps, out, stride, offset); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_norm_rstd(const void* q, const void* k, const void* v, int Tq, int Tk, int H, int d, int norm,
                            float eps, float* rq, float* rkv, hipStream_t s) {
    if (H <= 0) return hipSuccess;
    if ((Tq > 0 && (!q || !rq)) || (Tk > 0 && (!k || !v || !rkv))) return hipErrorInvalidValue;
    hipError_t e = launch_one(q, Tq, H, d, norm & 1, eps, rq, 1, 0, s);
    if (e == hipSuccess) e = launch_one(k, Tk, H, d, (norm >> 1) & 1, eps, rkv, 2, 0, s);
    if (e == hipSuccess) e = launch_one(v, Tk, H, d, (norm >> 2) & 1, eps, rkv, 2, 1, s);
    return e;
}

}  // namespace gdpa
