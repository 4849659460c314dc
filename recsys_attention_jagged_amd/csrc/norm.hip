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

// One launch covers the tensors: blocks [0, nb0) take Q, [nb0, nb0 + nb1) K, the rest V
// (a uniform choice per block).  G = d / 8 lanes per (row, head) pair of x [T, H, d]
// bf16, pair p = row * H + h; each lane issues its U 16-byte loads (pairs U apart in
// blocks of 256 / G) before it reduces any, so that a wave keeps U KiB in flight.
// out[(h * T + row) * stride + offset] = 1 / sqrt(mean(x^2) + eps), or 1 when !on.
struct RstdTensor {
    const __bf16* x;
    float* out;
    int T, on, stride, offset, nblocks;
};
struct RstdArgs {
    RstdTensor t[3];
    int H;
    float eps;
};

constexpr int kRstdU = 4;

template <int G>
__global__ __launch_bounds__(256) void rstd_kernel(const RstdArgs a) {
    constexpr int PER = 256 / G;   // pairs per block and load round
    int blk = blockIdx.x, which = 0;
    if (blk >= a.t[0].nblocks) {
        blk -= a.t[0].nblocks;
        which = 1;
        if (blk >= a.t[1].nblocks) {
            blk -= a.t[1].nblocks;
            which = 2;
        }
    }
    const RstdTensor& t = a.t[which];
    const size_t n = (size_t)t.T * a.H;
    const size_t p0 = (size_t)blk * PER * kRstdU + threadIdx.x / G;
    const int c = threadIdx.x % G;
    u32x4 w[kRstdU];
#pragma unroll
    for (int u = 0; u < kRstdU; ++u) {
        const size_t p = p0 + (size_t)u * PER;
        w[u] = (t.on && p < n) ? *(const u32x4*)(t.x + p * (8 * G) + 8 * c) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kRstdU; ++u) {
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float lo = __uint_as_float(w[u][i] << 16), hi = __uint_as_float(w[u][i] & 0xffff0000u);
            acc = __builtin_fmaf(lo, lo, acc);
            acc = __builtin_fmaf(hi, hi, acc);
        }
#pragma unroll
        for (int m = G / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
        const size_t p = p0 + (size_t)u * PER;
        if (p < n && c == 0) {
            const int row = (int)(p / a.H), h = (int)(p % a.H);
            t.out[((size_t)h * t.T + row) * t.stride + t.offset] =
                t.on ? 1.0f / __builtin_sqrtf(acc / (8 * G) + a.eps) : 1.0f;
        }
    }
}

}  // namespace

hipError_t launch_norm_rstd(const void* q, const void* k, const void* v, int Tq, int Tk, int H, int d, int norm,
                            float eps, float* rq, float* rkv, hipStream_t s) {
    if (H <= 0) return hipSuccess;
    if ((Tq > 0 && (!q || !rq)) || (Tk > 0 && (!k || !v || !rkv))) return hipErrorInvalidValue;
    if (d != 32 && d != 64 && d != 128) return hipErrorInvalidValue;
    const int G = d / 8, per_block = (256 / G) * kRstdU;
    RstdArgs a;
    a.H = H;
    a.eps = eps;
    a.t[0] = RstdTensor{(const __bf16*)q, rq, Tq, norm & 1, 1, 0, 0};
    a.t[1] = RstdTensor{(const __bf16*)k, rkv, Tk, (norm >> 1) & 1, 2, 0, 0};
    a.t[2] = RstdTensor{(const __bf16*)v, rkv, Tk, (norm >> 2) & 1, 2, 1, 0};
    size_t total = 0;
    for (RstdTensor& t : a.t) {
        t.nblocks = (int)(((size_t)t.T * H + per_block - 1) / per_block);
        total += (size_t)t.nblocks;
    }
    if (total == 0) return hipSuccess;
    const dim3 grid((unsigned)total);
    switch (d) {
        case 32: hipLaunchKernelGGL(rstd_kernel<4>, grid, dim3(256), 0, s, a); break;
        case 64: hipLaunchKernelGGL(rstd_kernel<8>, grid, dim3(256), 0, s, a); break;
        default: hipLaunchKernelGGL(rstd_kernel<16>, grid, dim3(256), 0, s, a); break;
    }
    return hipGetLastError();
}

}  // namespace gdpa
