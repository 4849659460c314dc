// LDS access-pattern probe for reading the SQ_LDS_BANK_CONFLICT counter: one kernel per access
// pattern of the d = 128 kernels (and linear accesses of each width for calibration), every lane's
// offset inside an 8 KiB tile (32 rows x 256 B), the instruction repeated in a loop.
//
//   hipcc -O3 --offload-arch=gfx950 -Xclang -target-feature -Xclang -packed-fp32-ops lds_patterns.hip -o lds_patterns
//   rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS GRBM_GUI_ACTIVE -- ./lds_patterns
//
// Kernel probe<P>: 0 linear 16-byte reads, 1 the 16-row dK/dV kernel's row operand reads, 2 its
// 16-column transposing reads, 3 its output staging writes, 4 its staged rows read back, 5 the 32-row
// kernels' transposing reads, 6 linear 8-byte reads, 7 linear transposing reads.
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdint>
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16_t;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
constexpr int ITERS = 4096;

__device__ __forceinline__ int swz16(int row) { return ((row & 7) << 1) | ((row >> 3) & 1); }   // 16-row kernel's tiles
__device__ __forceinline__ int off16(int row, int chunk) { return row * 256 + ((chunk ^ swz16(row)) << 4); }

template <int PAT>
__global__ __launch_bounds__(64) void probe(unsigned* out, int kb_in) {
    __shared__ __attribute__((aligned(1024))) char tile[8192];
    const int lane = threadIdx.x;
    for (int i = lane; i < 8192 / 4; i += 64) ((unsigned*)tile)[i] = i;
    __syncthreads();
    unsigned acc = 0;
    const int l16 = lane & 15, g4 = lane >> 4;
    for (int it = 0; it < ITERS; ++it) {
        int kb = (kb_in + it) & 3;
        asm volatile("" : "+v"(kb));
        if constexpr (PAT == 0) {   // linear b128 (baseline)
            const u32x4 v = *(const u32x4*)(tile + lane * 16 + kb * 1024);
            acc ^= v.x;
        } else if constexpr (PAT == 1) {   // 16-row kernel: row operand b128, rows 16 ib + l % 16, chunk 4 kb + l / 16
            const u32x4 v = *(const u32x4*)(tile + off16(16 * (kb & 1) + l16, 4 * kb + g4));
            acc ^= v.x;
        } else if constexpr (PAT == 2) {   // 16-row kernel: transposed tr16 read (lds_col4_16, row0 = 0 or 16, col0 = 16 cb)
            const int g = lane >> 4, i = lane & 15;
            const int row = 16 * (kb & 1) + 4 * g + (i >> 2);
            const int t = i & 3;
            const int col = 16 * (kb + (kb >> 1)) + 4 * t;   // col0 = 16 cb, cb = 0..5
            const int off = off16(row, col >> 3) + ((t & 1) << 3);
            const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(tile + off));
            acc ^= (unsigned)v.x;
        } else if constexpr (PAT == 3) {   // 16-row kernel: output staging b64 write
            u32x2 w = {acc, (unsigned)it};
            const int cb = kb;
            *(u32x2*)(tile + off16(l16, 2 * cb + (g4 >> 1)) + 8 * (g4 & 1)) = w;
        } else if constexpr (PAT == 4) {   // 16-row kernel: staged rows read back, b128, row = k * 4 + lane / 16, chunk lane % 16
            const int row = kb * 4 + (lane >> 4), cc = lane & 15;
            const u32x4 v = *(const u32x4*)(tile + off16(row, cc));
            acc ^= v.x;
        } else if constexpr (PAT == 5) {   // 32-row layout (swz<128>: row & 15 ^ ...) transposed tr16 read, for comparison
            const int g = lane >> 4, i = lane & 15;
            const int row = 8 * (kb & 1) + 4 * (g >> 1) + (i >> 2);
            const int t = i & 3;
            const int col = 32 * (kb >> 1) + 16 * (g & 1) + 4 * t;
            const int off = row * 256 + (((col >> 3) ^ ((row & 15) ^ ((row & 3) << 2))) << 4) + ((t & 1) << 3);
            const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(tile + off));
            acc ^= (unsigned)v.x;
        } else if constexpr (PAT == 6) {   // b64 linear read (baseline for 8-byte accesses)
            const u32x2 v = *(const u32x2*)(tile + lane * 8 + kb * 512);
            acc ^= v.x;
        } else if constexpr (PAT == 7) {   // tr16 with linear addresses (each lane 8 B at lane * 8)
            const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(tile + lane * 8 + kb * 512));
            acc ^= (unsigned)v.x;
        }
    }
    out[blockIdx.x * 64 + lane] = acc;
}

int main() {
    unsigned* d;
    if (hipMalloc(&d, 256 * 64 * 4) != hipSuccess) return 1;
    hipLaunchKernelGGL(probe<0>, dim3(256), dim3(64), 0, 0, d, 0);
    hipLaunchKernelGGL(probe<1>, dim3(256), dim3(64), 0, 0, d, 0);
    hipLaunchKernelGGL(probe<2>, dim3(256), dim3(64), 0, 0, d, 0);
    hipLaunchKernelGGL(probe<3>, dim3(256), dim3(64), 0, 0, d, 0);
    hipLaunchKernelGGL(probe<4>, dim3(256), dim3(64), 0, 0, d, 0);
    hipLaunchKernelGGL(probe<5>, dim3(256), dim3(64), 0, 0, d, 0);
    hipLaunchKernelGGL(probe<6>, dim3(256), dim3(64), 0, 0, d, 0);
    hipLaunchKernelGGL(probe<7>, dim3(256), dim3(64), 0, 0, d, 0);
    if (hipDeviceSynchronize() != hipSuccess) return 1;
    printf("probe done\n");
    return 0;
}
