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

// one workgroup per cut item; a thread handles 4 consecutive columns of a row
// Block b of slot s is at part + (stride s + offset) * rows_per_slot * d: one output
// per slot (stride 1) or dK, dV interleaved (stride 2, offset 0 or 1).
__global__ __launch_bounds__(256) void partial_sum_kernel(const DevGroup* __restrict__ groups,
                                                          const float* __restrict__ part, int rows_per_slot,
                                                          int stride, int offset, int d, int H, float mul,
                                                          void* __restrict__ out, int out_f32) {
    const DevGroup g = groups[blockIdx.x];
    const int quads = g.rows * d / 4;
    const size_t slot_elems = (size_t)rows_per_slot * d;
    for (int i = threadIdx.x; i < quads; i += blockDim.x) {
        const int row = 4 * i / d, col = 4 * i % d;
        const float* src = part + ((size_t)stride * g.slot0 + offset) * slot_elems + (size_t)row * d + col;
        float4 acc = *(const float4*)src;
        for (int j = 1; j < g.n; ++j) {
            const float4 x = *(const float4*)(src + (size_t)j * stride * slot_elems);
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
}

}  // namespace

hipError_t launch_partial_sum(const DevGroup* groups, int n_groups, const float* part, int rows_per_slot,
                              int stride, int offset, int d, int H, float mul, void* out, int out_f32,
                              hipStream_t s) {
    if (n_groups <= 0) return hipSuccess;
    if (!groups || !part || !out || rows_per_slot <= 0 || d % 4 != 0 || stride < 1 || offset < 0 ||
        offset >= stride)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(partial_sum_kernel, dim3(n_groups), dim3(256), 0, s, groups, part, rows_per_slot, stride,
                       offset, d, H, mul, out, out_f32);
    return hipGetLastError();
}

}  // namespace gdpa
