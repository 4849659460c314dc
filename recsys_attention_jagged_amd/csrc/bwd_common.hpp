// State and output helpers shared by the backward kernels (bf16 inputs).
#pragma once

#include "kernels.hpp"
#include "ring.hpp"

namespace gdpa {

// Per-wave constants of a backward kernel and its output stores.
struct Common {
    const KernelArgs a;   // by value: kept in SGPRs, not re-read from the argument segment
    int lane, r, hh, wt, H, win;
    uint32_t rs, rso;
    float scale;

    __device__ Common(const KernelArgs& args, int lane_, int wt_, int D) : a(args) {
        lane = lane_;
        r = lane & 31;
        hh = lane >> 5;
        wt = wt_;
        H = a.H;
        win = a.window;
        rs = (uint32_t)H * D * 2;
        rso = (uint32_t)H * D * (a.out_f32 ? 4 : 2);
        scale = a.scale;
    }

    // store a 32-row output block: fp32 directly from the accumulator, bf16 staged
    // through `tile` (a slot of the item's last step) and written as whole rows
    template <int D>
    __device__ __forceinline__ void store(const f32x16 (&acc)[D / 32], float mul, void* out, size_t base, int rows,
                                          int row0, char* tile) const {
        if (a.out_f32) {
            store_block_f32<D / 32>(acc, mul, slice_rsrc((const float*)out + base, rows, rso, D * 4),
                                    (uint32_t)(row0 + r) * rso, hh);
        } else {
            stage_block<D>(acc, mul, tile, r, hh);
            store_tile<D>(tile, slice_rsrc((const __bf16*)out + base, rows, rso, D * 2), (uint32_t)row0 * rso, rso,
                          lane);
        }
    }

    // zero rows row0 .. row0 + 31 of an output slice
    template <int D>
    __device__ __forceinline__ void zero(void* out, size_t base, int rows, int row0) const {
        if (a.out_f32) {
            f32x16 z[D / 32];
#pragma unroll
            for (int db = 0; db < D / 32; ++db) z[db] = f32x16{};
            store_block_f32<D / 32>(z, 1.0f, slice_rsrc((const float*)out + base, rows, rso, D * 4),
                                    (uint32_t)(row0 + r) * rso, hh);
        } else {
            store_zero_rows<D>(slice_rsrc((const __bf16*)out + base, rows, rso, D * 2), (uint32_t)row0 * rso, rso,
                               lane);
        }
    }
};


}  // namespace gdpa
