// Reduction of chunk partial outputs.
//
// The planner may cut a long Q-stationary item (one stationary tile and a long
// run of streaming tiles) into chunks that run in different bins; each chunk
// stores its fp32 output block into its own slot, and this kernel adds the slots
// of one item in slot order, scales the sum and stores the rows of the item.  No
// atomics: every output row has one writer, and the order of the additions is
// fixed, so the result does not depend on scheduling.
#include "device.hpp"
#include "kernels.hpp"

namespace gdpa {
namespace {

// grid (ceil(quads / 256), cut items): a thread owns 4 consecutive columns of one
// row of one item (a "quad") and adds that quad over the item's slots.
// Block b of slot s is at part + (stride s + offset) * rows_per_slot * d: one output
// per slot (stride 1) or dK, dV interleaved (stride 2, offset 0 or 1).
__global__ __launch_bounds__(256) void partial_sum_kernel(const DevGroup* __restrict__ groups,
                                                          const float* __restrict__ part, int rows_per_slot,
                                                          int stride, int offset, int d, int H, float mul,
                                                          void* __restrict__ out, int out_f32) {
    const DevGroup g = groups[blockIdx.y];
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= g.rows * d / 4) return;
    const int row = 4 * i / d, col = 4 * i % d;
    const size_t step = (size_t)stride * rows_per_slot * d;   // floats between consecutive slots
    const float* src = part + ((size_t)stride * g.slot0 + offset) * rows_per_slot * d + (size_t)row * d + col;
    float4 acc = *(const float4*)src;
    int j = 1;
    // four loads in flight, added in slot order
    for (; j + 4 <= g.n; j += 4) {
        const float4 x0 = *(const float4*)(src + (size_t)j * step);
        const float4 x1 = *(const float4*)(src + (size_t)(j + 1) * step);
        const float4 x2 = *(const float4*)(src + (size_t)(j + 2) * step);
        const float4 x3 = *(const float4*)(src + (size_t)(j + 3) * step);
        acc.x = (((acc.x + x0.x) + x1.x) + x2.x) + x3.x;
        acc.y = (((acc.y + x0.y) + x1.y) + x2.y) + x3.y;
        acc.z = (((acc.z + x0.z) + x1.z) + x2.z) + x3.z;
        acc.w = (((acc.w + x0.w) + x1.w) + x2.w) + x3.w;
    }
    for (; j < g.n; ++j) {
        const float4 x = *(const float4*)(src + (size_t)j * step);
        acc.x += x.x;
        acc.y += x.y;
        acc.z += x.z;
        acc.w += x.w;
    }
    const size_t o = ((size_t)(g.row0 + row) * H + g.h) * d + col;
    if (out_f32) {
        *(float4*)((float*)out + o) = make_float4(acc.x * mul, acc.y * mul, acc.z * mul, acc.w * mul);
    } else {
        uint2 w;
        w.x = pack_bf16x2(acc.x * mul, acc.y * mul);
        w.y = pack_bf16x2(acc.z * mul, acc.w * mul);
        *(uint2*)((__bf16*)out + o) = w;
    }
}

}  // namespace

hipError_t launch_partial_sum(const DevGroup* groups, int n_groups, const float* part, int rows_per_slot,
                              int stride, int offset, int d, int H, float mul, void* out, int out_f32,
                              hipStream_t s) {
    if (n_groups <= 0) return hipSuccess;
    if (!groups || !part || !out || rows_per_slot <= 0 || d % 4 != 0 || stride < 1 || offset < 0 ||
        offset >= stride)
        return hipErrorInvalidValue;
    // a group has at most rows_per_slot rows; at most 65535 groups per launch (grid y)
    const int quads = rows_per_slot * d / 4;
    for (int g0 = 0; g0 < n_groups; g0 += 65535) {
        const int ng = n_groups - g0 < 65535 ? n_groups - g0 : 65535;
        hipLaunchKernelGGL(partial_sum_kernel, dim3((quads + 255) / 256, ng), dim3(256), 0, s, groups + g0, part,
                           rows_per_slot, stride, offset, d, H, mul, out, out_f32);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace gdpa
