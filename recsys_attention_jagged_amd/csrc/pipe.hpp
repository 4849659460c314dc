// Multi-stage LDS pipeline shared by the GDPA kernels (gfx950).
//
// Tiles are copied global -> LDS with buffer_load_dwordx4 ... lds (no VGPR
// staging): the 64 lanes of one instruction write 1 KiB of consecutive LDS.
// A tile of R rows x D bf16 is stored row-major without padding; the 16-byte
// chunk c of row r sits at chunk position c ^ swz<D>(r).  The swizzle makes both
// read patterns bank-conflict free:
//   * row-major operand reads: 16 rows at one chunk (ds_read_b128);
//   * transposed operand reads: 4 consecutive rows x 4 consecutive chunks
//     (ds_read_b64_tr_b16), where lane i of each 16-lane group receives column
//     i of a 4-row block whose rows are addressed by lanes 4k .. 4k+3.
// Rows outside the (sample, head) slice are out of the buffer descriptor's
// range and arrive as zeros.
//
// Each wave counts the DMA instructions it issued per stage; since loads
// complete in issue order, waiting for the oldest stage is `s_waitcnt vmcnt(n)`
// with n = the instructions of the later stages.  A stage only loads what its
// step needs (the stationary tile only when the step starts an item).  The DMA is
// issued from inline assembly: the compiler then neither sees the asynchronous
// LDS writes nor inserts full `vmcnt(0)` waits before LDS reads; ordering is
// kept by the explicit waits and barriers below (all with memory clobbers).
#pragma once

#include "device.hpp"

namespace gdpa {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16_t;

template <int D>
__device__ __forceinline__ int swz(int row) {
    if constexpr (D == 128) {
        return (row & 15) ^ ((row & 3) << 2);
    } else if constexpr (D == 64) {
        const int u = row >> 1;
        return (u & 7) ^ ((u & 1) << 2);
    } else {
        return (row >> 2) & 3;
    }
}

// byte offset of (row, 16-byte chunk) inside a swizzled tile
template <int D>
__device__ __forceinline__ int tile_off(int row, int chunk) {
    return row * (D * 2) + ((chunk ^ swz<D>(row)) << 4);
}

// 8 bf16 of `row`, columns [8 chunk, 8 chunk + 8)
template <int D>
__device__ __forceinline__ bf16x8 lds_row8(const char* tile, int row, int chunk) {
    return *(const bf16x8*)(tile + tile_off<D>(row, chunk));
}

// Transposed operand: lane l receives the 4 values tile[row0 + 4 (l/32) + i][col0 + l % 32],
// i = 0..3 (row0 a multiple of 4, col0 a multiple of 32).
template <int D>
__device__ __forceinline__ bf16x4 lds_col4(const char* tile, int row0, int col0, int lane) {
    const int g = lane >> 4, i = lane & 15;
    const int row = row0 + 4 * (g >> 1) + (i >> 2);
    const int t = i & 3;
    const int col = col0 + 16 * (g & 1) + 4 * t;
    const int off = tile_off<D>(row, col >> 3) + ((t & 1) << 3);
    const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(tile + off));
    return __builtin_bit_cast(bf16x4, v);
}

// A operand of 8 contraction rows for the chained MFMA: rows
// row0 + {0..3} + 4 (l/32) and row0 + 8 + {0..3} + 4 (l/32), column col0 + l % 32.
template <int D>
__device__ __forceinline__ bf16x8 lds_col8(const char* tile, int row0, int col0, int lane) {
    const bf16x4 a = lds_col4<D>(tile, row0, col0, lane);
    const bf16x4 b = lds_col4<D>(tile, row0 + 8, col0, lane);
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// -------------------------------------------------------------------------
// async tiles
// -------------------------------------------------------------------------
// LDS byte address of a pointer into a __shared__ array
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(size_t)(const __attribute__((address_space(3))) char*)p;
}

// One wave instruction: lane l's 16 bytes at byte offset `voff` of the buffer
// land at LDS address lds + 16 l (lds uniform).  The whole offset is in the
// VGPR: the hardware range check covers the VGPR offset, not the scalar one.
__device__ __forceinline__ void dma16(rsrc_t rs, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(rs)
                 : "memory", "m0");
}

template <int ROWS, int D>
struct AsyncTile {
    static constexpr int CPR = D / 8;                 // chunks per row
    static constexpr int WINSTR = ROWS * CPR / 64;    // wave instructions for the tile
    static constexpr int PER_WAVE = (WINSTR + 3) / 4; // issued by each of the 4 waves
    static constexpr int BYTES = PER_WAVE * 4 * 1024; // LDS footprint incl. padding
    static_assert(ROWS * CPR % 64 == 0, "tile must be a whole number of wave loads");

    // per-lane byte offsets inside the slice for this wave's instructions
    uint32_t off[PER_WAVE];

    __device__ __forceinline__ void init(uint32_t row_stride_bytes, int wave, int lane) {
#pragma unroll
        for (int j = 0; j < PER_WAVE; ++j) {
            const int slot = (wave + 4 * j) * 64 + lane;
            const int row = (slot / CPR) % ROWS, pos = slot % CPR;
            off[j] = (uint32_t)row * row_stride_bytes + (uint32_t)((pos ^ swz<D>(row)) << 4);
        }
    }

    // rows [row0, row0 + ROWS) of the slice described by `rs`; row_off = row0 * stride;
    // tile = LDS address of the tile.  Returns the number of DMA instructions
    // this wave issued (uniform).
    __device__ __forceinline__ int issue(rsrc_t rs, uint32_t row_off, uint32_t tile, int wave) const {
        const int w = __builtin_amdgcn_readfirstlane(wave);
        int n = 0;
#pragma unroll
        for (int j = 0; j < PER_WAVE; ++j) {
            const int ins = w + 4 * j;   // uniform
            if (ins < WINSTR) {
                dma16(rs, off[j] + row_off, tile + (uint32_t)ins * 1024u);
                ++n;
            }
        }
        return n;
    }
};

// Wait until at most n vector-memory instructions of this wave are in flight
// (n uniform; the count needs an immediate, hence the switch), then barrier.
__device__ __forceinline__ void wait_vm_barrier(int n) {
    switch (n) {
        case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
        case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
        case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
        case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
        case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
        case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
        case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
        case 7: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
        case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
        case 9: asm volatile("s_waitcnt vmcnt(9)" ::: "memory"); break;
        case 10: asm volatile("s_waitcnt vmcnt(10)" ::: "memory"); break;
        case 11: asm volatile("s_waitcnt vmcnt(11)" ::: "memory"); break;
        case 12: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
        case 13: asm volatile("s_waitcnt vmcnt(13)" ::: "memory"); break;
        case 14: asm volatile("s_waitcnt vmcnt(14)" ::: "memory"); break;
        case 15: asm volatile("s_waitcnt vmcnt(15)" ::: "memory"); break;
        case 16: asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); break;
        case 17: asm volatile("s_waitcnt vmcnt(17)" ::: "memory"); break;
        case 18: asm volatile("s_waitcnt vmcnt(18)" ::: "memory"); break;
        case 19: asm volatile("s_waitcnt vmcnt(19)" ::: "memory"); break;
        case 20: asm volatile("s_waitcnt vmcnt(20)" ::: "memory"); break;
        case 21: asm volatile("s_waitcnt vmcnt(21)" ::: "memory"); break;
        case 22: asm volatile("s_waitcnt vmcnt(22)" ::: "memory"); break;
        case 23: asm volatile("s_waitcnt vmcnt(23)" ::: "memory"); break;
        case 24: asm volatile("s_waitcnt vmcnt(24)" ::: "memory"); break;
        case 25: asm volatile("s_waitcnt vmcnt(25)" ::: "memory"); break;
        case 26: asm volatile("s_waitcnt vmcnt(26)" ::: "memory"); break;
        case 27: asm volatile("s_waitcnt vmcnt(27)" ::: "memory"); break;
        case 28: asm volatile("s_waitcnt vmcnt(28)" ::: "memory"); break;
        case 29: asm volatile("s_waitcnt vmcnt(29)" ::: "memory"); break;
        case 30: asm volatile("s_waitcnt vmcnt(30)" ::: "memory"); break;
        case 31: asm volatile("s_waitcnt vmcnt(31)" ::: "memory"); break;
        case 32: asm volatile("s_waitcnt vmcnt(32)" ::: "memory"); break;
        case 33: asm volatile("s_waitcnt vmcnt(33)" ::: "memory"); break;
        case 34: asm volatile("s_waitcnt vmcnt(34)" ::: "memory"); break;
        case 35: asm volatile("s_waitcnt vmcnt(35)" ::: "memory"); break;
        case 36: asm volatile("s_waitcnt vmcnt(36)" ::: "memory"); break;
        case 37: asm volatile("s_waitcnt vmcnt(37)" ::: "memory"); break;
        case 38: asm volatile("s_waitcnt vmcnt(38)" ::: "memory"); break;
        case 39: asm volatile("s_waitcnt vmcnt(39)" ::: "memory"); break;
        case 40: asm volatile("s_waitcnt vmcnt(40)" ::: "memory"); break;
        case 41: asm volatile("s_waitcnt vmcnt(41)" ::: "memory"); break;
        case 42: asm volatile("s_waitcnt vmcnt(42)" ::: "memory"); break;
        case 43: asm volatile("s_waitcnt vmcnt(43)" ::: "memory"); break;
        case 44: asm volatile("s_waitcnt vmcnt(44)" ::: "memory"); break;
        case 45: asm volatile("s_waitcnt vmcnt(45)" ::: "memory"); break;
        case 46: asm volatile("s_waitcnt vmcnt(46)" ::: "memory"); break;
        case 47: asm volatile("s_waitcnt vmcnt(47)" ::: "memory"); break;
        case 48: asm volatile("s_waitcnt vmcnt(48)" ::: "memory"); break;
        case 49: asm volatile("s_waitcnt vmcnt(49)" ::: "memory"); break;
        case 50: asm volatile("s_waitcnt vmcnt(50)" ::: "memory"); break;
        case 51: asm volatile("s_waitcnt vmcnt(51)" ::: "memory"); break;
        case 52: asm volatile("s_waitcnt vmcnt(52)" ::: "memory"); break;
        case 53: asm volatile("s_waitcnt vmcnt(53)" ::: "memory"); break;
        case 54: asm volatile("s_waitcnt vmcnt(54)" ::: "memory"); break;
        case 55: asm volatile("s_waitcnt vmcnt(55)" ::: "memory"); break;
        case 56: asm volatile("s_waitcnt vmcnt(56)" ::: "memory"); break;
        case 57: asm volatile("s_waitcnt vmcnt(57)" ::: "memory"); break;
        case 58: asm volatile("s_waitcnt vmcnt(58)" ::: "memory"); break;
        case 59: asm volatile("s_waitcnt vmcnt(59)" ::: "memory"); break;
        case 60: asm volatile("s_waitcnt vmcnt(60)" ::: "memory"); break;
        case 61: asm volatile("s_waitcnt vmcnt(61)" ::: "memory"); break;
        case 62: asm volatile("s_waitcnt vmcnt(62)" ::: "memory"); break;
        default: asm volatile("s_waitcnt vmcnt(63)" ::: "memory"); break;
    }
    asm volatile("s_barrier" ::: "memory");
}

__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// all waves have finished their LDS accesses up to here
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// -------------------------------------------------------------------------
// the persistent, flattened, multi-stage loop
// -------------------------------------------------------------------------
// A step of a bin's walk: the item's planner record and the streaming tile.
// All fields are uniform across the workgroup.
struct Step {
    Rec r;
    int s;
    bool valid;
    __device__ __forceinline__ bool has_steps() const { return r.s1 >= r.s0; }
    __device__ __forceinline__ bool first() const { return s == r.s0; }
    __device__ __forceinline__ bool last() const { return s >= r.s1; }
};

// Pol provides: NS (stages), STAGE_BYTES, new_item(step) (per-item descriptors
// for issuing), issue(step, stage LDS address) -> DMA instructions this wave
// issued,
// item_start(step, stage), compute(step, stage), epilogue(step, stage) (may use
// the whole stage).  The issuing walk runs NS steps ahead of the computing one;
// the computing side receives each step's record through a shift register, so
// the work list is read once per item, with one scalar load and no dependent
// loads.
template <class Pol>
__device__ __forceinline__ void run_pipeline(Pol& pol, int P, const Rec* __restrict__ recs,
                                             const int32_t* __restrict__ bin_ptr, char* smem) {
    constexpr int NS = Pol::NS;
    const int bin = logical_bin(P);
    int idx = bin_ptr[bin];
    const int end = bin_ptr[bin + 1];
    if (idx >= end) return;

    Step is;
    is.r = recs[idx];
    is.s = is.r.s0;
    is.valid = true;
    pol.new_item(is);
    Rec next = recs[idx + 1 < end ? idx + 1 : idx];   // prefetched one item ahead

    const uint32_t base = lds_addr(smem);
    Step pipe[NS];
    int cnt[NS];   // DMA instructions this wave issued for each stage in flight
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        pipe[j] = is;
        cnt[j] = pol.issue(is, base + j * Pol::STAGE_BYTES);
        // advance the issuing walk
        if (is.valid) {
            if (is.s < is.r.s1) {
                ++is.s;
            } else if (++idx < end) {
                is.r = next;
                is.s = is.r.s0;
                pol.new_item(is);
                next = recs[idx + 1 < end ? idx + 1 : idx];
            } else {
                is.valid = false;
            }
        }
    }
    int stage = 0;
    for (;;) {
        // loads complete in issue order: the oldest stage has landed once no more
        // than the later stages' instructions remain (stores only make this stricter)
        int later = 0;
#pragma unroll
        for (int j = 1; j < NS; ++j) later += cnt[j];
        wait_vm_barrier(later);
        const Step cur = pipe[0];
        char* st = smem + stage * Pol::STAGE_BYTES;
        if (cur.first()) pol.item_start(cur, st);
        pol.compute(cur, st);
        lds_barrier();
        if (cur.last()) {
            pol.epilogue(cur, st);
            lds_barrier();
        }
        const int issued = pol.issue(is, base + stage * Pol::STAGE_BYTES);
#pragma unroll
        for (int j = 0; j + 1 < NS; ++j) {
            pipe[j] = pipe[j + 1];
            cnt[j] = cnt[j + 1];
        }
        pipe[NS - 1] = is;
        cnt[NS - 1] = issued;
        if (is.valid) {
            if (is.s < is.r.s1) {
                ++is.s;
            } else if (++idx < end) {
                is.r = next;
                is.s = is.r.s0;
                pol.new_item(is);
                next = recs[idx + 1 < end ? idx + 1 : idx];
            } else {
                is.valid = false;
            }
        }
        if (!pipe[0].valid) break;
        stage = (stage + 1 == NS) ? 0 : stage + 1;
    }
    wait_vm_all();   // no DMA may land after the workgroup's LDS is released
}

template <int STAGE_BYTES>
struct Stages {
    static constexpr int LDS_MAX = 160 * 1024;
    static constexpr int N = (LDS_MAX / STAGE_BYTES) > 4 ? 4 : (LDS_MAX / STAGE_BYTES);
    static_assert(N >= 2, "a stage must fit twice in LDS");
};

}  // namespace gdpa
