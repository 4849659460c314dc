// GDPA in plain fp32 arithmetic (no MFMA): one thread per (row, head).
//
// A direct evaluation of the definition (GDPA page, aitrends.kr/articles/26275,
// "Key summary" / "Section details": O = act(Q K^T / sqrt(d)) V without softmax)
// for fp32 inputs.  It is the path for small fp32 problems; it ignores the work
// lists and finds each row's sample by binary search over the offsets.
#include "device.hpp"
#include "kernels.hpp"

namespace gdpa {
namespace {

__device__ __forceinline__ int find_sample(const int32_t* off, int B, int row) {
    int lo = 0, hi = B;   // off[lo] <= row < off[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (off[mid] <= row) lo = mid; else hi = mid;
    }
    return lo;
}

template <int D, int ACT>
__global__ __launch_bounds__(256) void fwd_f32_kernel(const KernelArgs a, int Tq) {
    const int gid = blockIdx.x * 256 + threadIdx.x;
    const int H = a.H;
    if (gid >= Tq * H) return;
    const int row = gid / H, h = gid % H;
    const int b = find_sample(a.q_off, a.B, row);
    const int i = row - a.q_off[b];
    const int ks = a.kv_off[b], lk = a.kv_off[b + 1] - ks;
    const float* q = (const float*)a.q + ((size_t)row * H + h) * D;
    float qv[D], acc[D];
#pragma unroll
    for (int e = 0; e < D; ++e) {
        qv[e] = q[e];
        acc[e] = 0.0f;
    }
    int j0 = 0, j1 = lk;
    if (a.window > 0) {
        j0 = max(0, i - a.window + 1);
        j1 = min(lk, i + a.window);
    }
    for (int j = j0; j < j1; ++j) {
        const float* kr = (const float*)a.k + ((size_t)(ks + j) * H + h) * D;
        const float* vr = (const float*)a.v + ((size_t)(ks + j) * H + h) * D;
        float s = 0.0f;
#pragma unroll
        for (int e = 0; e < D; ++e) s = __builtin_fmaf(qv[e], kr[e], s);
        const float p = act_fwd<ACT>(s * a.scale);
#pragma unroll
        for (int e = 0; e < D; ++e) acc[e] = __builtin_fmaf(p, vr[e], acc[e]);
    }
    float* o = (float*)a.o + ((size_t)row * H + h) * D;
#pragma unroll
    for (int e = 0; e < D; ++e) o[e] = acc[e];
}

template <int D, int ACT>
__global__ __launch_bounds__(256) void dq_f32_kernel(const KernelArgs a, int Tq) {
    const int gid = blockIdx.x * 256 + threadIdx.x;
    const int H = a.H;
    if (gid >= Tq * H) return;
    const int row = gid / H, h = gid % H;
    const int b = find_sample(a.q_off, a.B, row);
    const int i = row - a.q_off[b];
    const int ks = a.kv_off[b], lk = a.kv_off[b + 1] - ks;
    const float* q = (const float*)a.q + ((size_t)row * H + h) * D;
    const float* go = (const float*)a.dout + ((size_t)row * H + h) * D;
    float qv[D], ov[D], acc[D];
#pragma unroll
    for (int e = 0; e < D; ++e) {
        qv[e] = q[e];
        ov[e] = go[e];
        acc[e] = 0.0f;
    }
    int j0 = 0, j1 = lk;
    if (a.window > 0) {
        j0 = max(0, i - a.window + 1);
        j1 = min(lk, i + a.window);
    }
    for (int j = j0; j < j1; ++j) {
        const float* kr = (const float*)a.k + ((size_t)(ks + j) * H + h) * D;
        const float* vr = (const float*)a.v + ((size_t)(ks + j) * H + h) * D;
        float s = 0.0f, dp = 0.0f;
#pragma unroll
        for (int e = 0; e < D; ++e) {
            s = __builtin_fmaf(qv[e], kr[e], s);
            dp = __builtin_fmaf(ov[e], vr[e], dp);
        }
        float f, g;
        act_fwd_grad<ACT>(s * a.scale, f, g);
        const float ds = dp * g;
#pragma unroll
        for (int e = 0; e < D; ++e) acc[e] = __builtin_fmaf(ds, kr[e], acc[e]);
    }
    float* dq = (float*)a.dq + ((size_t)row * H + h) * D;
#pragma unroll
    for (int e = 0; e < D; ++e) dq[e] = acc[e] * a.scale;
}

template <int D, int ACT>
__global__ __launch_bounds__(256) void dkdv_f32_kernel(const KernelArgs a, int Tk) {
    const int gid = blockIdx.x * 256 + threadIdx.x;
    const int H = a.H;
    if (gid >= Tk * H) return;
    const int row = gid / H, h = gid % H;
    const int b = find_sample(a.kv_off, a.B, row);
    const int j = row - a.kv_off[b];
    const int qs = a.q_off[b], lq = a.q_off[b + 1] - qs;
    const float* k = (const float*)a.k + ((size_t)row * H + h) * D;
    const float* v = (const float*)a.v + ((size_t)row * H + h) * D;
    float kv[D], vv[D], ak[D], av[D];
#pragma unroll
    for (int e = 0; e < D; ++e) {
        kv[e] = k[e];
        vv[e] = v[e];
        ak[e] = 0.0f;
        av[e] = 0.0f;
    }
    int i0 = 0, i1 = lq;
    if (a.window > 0) {
        i0 = max(0, j - a.window + 1);
        i1 = min(lq, j + a.window);
    }
    for (int i = i0; i < i1; ++i) {
        const float* qr = (const float*)a.q + ((size_t)(qs + i) * H + h) * D;
        const float* orow = (const float*)a.dout + ((size_t)(qs + i) * H + h) * D;
        float s = 0.0f, dp = 0.0f;
#pragma unroll
        for (int e = 0; e < D; ++e) {
            s = __builtin_fmaf(qr[e], kv[e], s);
            dp = __builtin_fmaf(orow[e], vv[e], dp);
        }
        float f, g;
        act_fwd_grad<ACT>(s * a.scale, f, g);
        const float ds = dp * g;
#pragma unroll
        for (int e = 0; e < D; ++e) {
            av[e] = __builtin_fmaf(f, orow[e], av[e]);
            ak[e] = __builtin_fmaf(ds, qr[e], ak[e]);
        }
    }
    float* dk = (float*)a.dk + ((size_t)row * H + h) * D;
    float* dv = (float*)a.dv + ((size_t)row * H + h) * D;
#pragma unroll
    for (int e = 0; e < D; ++e) {
        dk[e] = ak[e] * a.scale;
        dv[e] = av[e];
    }
}


template <int D>
const void* fwd_ptr(int act) {
    switch (act) {
        case ACT_GELU: return (const void*)&fwd_f32_kernel<D, ACT_GELU>;
        case ACT_SILU: return (const void*)&fwd_f32_kernel<D, ACT_SILU>;
        case ACT_GELU_POLY: return (const void*)&fwd_f32_kernel<D, ACT_GELU_POLY>;
        case ACT_GELU_TAYLOR6: return (const void*)&fwd_f32_kernel<D, ACT_GELU_TAYLOR6>;
        case ACT_IDENTITY: return (const void*)&fwd_f32_kernel<D, ACT_IDENTITY>;
        case ACT_ONE: return (const void*)&fwd_f32_kernel<D, ACT_ONE>;
    }
    return nullptr;
}

template <int D>
void bwd_ptrs(int act, const void** dq, const void** dkdv) {
    *dq = *dkdv = nullptr;
    switch (act) {
#define GDPA_CASE(A)                                    \
    case A:                                             \
        *dq = (const void*)&dq_f32_kernel<D, A>;        \
        *dkdv = (const void*)&dkdv_f32_kernel<D, A>;    \
        break;
        GDPA_CASE(ACT_GELU)
        GDPA_CASE(ACT_SILU)
        GDPA_CASE(ACT_GELU_POLY)
        GDPA_CASE(ACT_GELU_TAYLOR6)
        GDPA_CASE(ACT_IDENTITY)
#undef GDPA_CASE
    }
}

hipError_t launch_rows(const void* f, const KernelArgs& a, int rows, hipStream_t s) {
    if (!f) return hipErrorInvalidValue;
    const long long n = (long long)rows * a.H;
    if (n == 0) return hipSuccess;
    KernelArgs args = a;
    int r = rows;
    void* params[] = {&args, &r};
    return hipLaunchKernel(f, dim3((unsigned)((n + 255) / 256)), dim3(256), params, 0, s);
}

}  // namespace

hipError_t launch_fwd_f32(const KernelArgs& a, int Tq, int d, int act, hipStream_t s) {
    const void* f = d == 32 ? fwd_ptr<32>(act) : d == 64 ? fwd_ptr<64>(act) : d == 128 ? fwd_ptr<128>(act) : nullptr;
    return launch_rows(f, a, Tq, s);
}

hipError_t launch_bwd_f32(const KernelArgs& a, int Tq, int Tk, int d, int act, hipStream_t s) {
    const void *fdq = nullptr, *fkv = nullptr;
    if (d == 32) bwd_ptrs<32>(act, &fdq, &fkv);
    else if (d == 64) bwd_ptrs<64>(act, &fdq, &fkv);
    else if (d == 128) bwd_ptrs<128>(act, &fdq, &fkv);
    if (!fdq || !fkv) return hipErrorInvalidValue;
    hipError_t e = launch_rows(fdq, a, Tq, s);
    if (e != hipSuccess) return e;
    return launch_rows(fkv, a, Tk, s);
}

}  // namespace gdpa
