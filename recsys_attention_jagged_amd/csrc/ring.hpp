// Tile ring and persistent walk shared by the bf16 GDPA kernels (gfx950).
//
// A workgroup is a team of T waves (T = 1 or 2) that owns one planner bin and
// one slice of LDS, and synchronises only with itself.  The slice is a ring of R
// slots, each holding one 32-row tile of one tensor (32 x D bf16).  The team walks
// its bin's items as one flattened sequence of tile loads ("jobs"): for each item
// its stationary tiles, then for each step its streaming tiles.  The issuing side
// runs up to R jobs ahead of the computing side, across item boundaries, so short
// items do not drain the pipeline (GDPA page, aitrends.kr/articles/26275,
// "Section details": pipelining moved to the outer loop; loop flattening).  With
// two waves per SIMD (two teams, or two one-wave workgroups, per SIMD) one wave's
// loads overlap the other's arithmetic.
//
// Loads are buffer_load_dwordx4 ... lds: the 64 lanes of one instruction write
// 1 KiB of consecutive LDS, without VGPR staging; each wave of a team issues its
// share of a tile's instructions.  A tile is stored row-major without padding,
// the 16-byte chunk c of row r at chunk position c ^ swz<D>(r); the swizzle is
// applied on the global side (each lane fetches the chunk that belongs at its LDS
// position) and makes both read patterns bank-conflict free:
//   * row operands: 16 rows at one chunk (ds_read_b128);
//   * transposed operands: 4 consecutive rows x 4 consecutive chunks
//     (ds_read_b64_tr_b16), where lane i of each 16-lane group receives column
//     i of a 4-row block whose rows are addressed by lanes 4k .. 4k+3.
// Rows outside the (sample, head) slice are outside the buffer descriptor's
// range and arrive as zeros; a job of an empty slice writes a zero tile.
//
// Synchronisation: a wave's load instructions complete in issue order, so "job k
// has landed" is `s_waitcnt vmcnt(JX * (jobs issued after k))` per wave (JX load
// instructions per job and wave, the same for every job), followed
// by a workgroup barrier when T > 1 so that every wave's share is visible.  Slots
// are re-filled only after such a barrier (and this wave's `s_waitcnt
// lgkmcnt(0)`), i.e. after every wave has finished reading them.  The loads are
// issued from inline assembly, so the compiler neither sees the asynchronous LDS
// writes nor inserts waits of its own for them; stores are left to the compiler
// and are not counted (a wait then only becomes stricter).
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

// A second swizzle for d = 128 (SW = 1), for kernels whose waves own 16-row
// blocks: s(r) = ((r & 7) << 1) | ((r >> 3) & 1).  Over 16 rows it is a
// permutation (16 rows x one chunk, the row operands, are conflict free), and
// the chunk pairs {s(r) ^ 2m, s(r) ^ (2m + 1)} of any 8 consecutive rows 0..7 or
// 8..15 are disjoint (8 rows x two adjacent chunks, the 16-column transposed
// operands read by each half of a wave, are conflict free).
template <int D, int SW>
__device__ __forceinline__ int swz_sel(int row) {
    if constexpr (SW == 1) {
        static_assert(D == 128, "the 16-row swizzle is for d = 128");
        return ((row & 7) << 1) | ((row >> 3) & 1);
    } else {
        return swz<D>(row);
    }
}

template <int D, int SW>
__device__ __forceinline__ int tile_off_sw(int row, int chunk) {
    return row * (D * 2) + ((chunk ^ swz_sel<D, SW>(row)) << 4);
}

// fp8 tiles (32 rows of D one-byte values, in the first half of a slot): the
// 16-byte chunk c of row r sits at chunk position c ^ swz8<D>(r).  Operand reads
// take 8 bytes of one chunk in each of 32 rows; rows share a 256-byte bank window
// 256 / D at a time, and the swizzle spreads the rows of one window over distinct
// chunk positions (at most two-way bank conflicts).
template <int D>
__device__ __forceinline__ int swz8(int row) {
    if constexpr (D == 128) {
        return (row >> 1) & 7;
    } else if constexpr (D == 64) {
        return (row >> 2) & 3;
    } else {
        return (row >> 3) & 1;
    }
}

template <int D>
__device__ __forceinline__ int tile8_off(int row, int chunk) {
    return row * D + ((chunk ^ swz8<D>(row)) << 4);
}

// fp8 tiles: the 8 e4m3 bytes of `row`, columns [16 ks + 8 half, + 8): the fp8
// MFMA's operand for 16-wide k block ks, lane group `half` (the bf16 operand
// lds_row8(tile, row, 2 ks + half) holds the same columns)
template <int D>
__device__ __forceinline__ long lds_row8_f8(const char* tile, int row, int ks, int half) {
    return *(const long*)(tile + tile8_off<D>(row, ks) + 8 * half);
}

// 8 e4m3 values (bytes 0..3 of lo, then of hi) as bf16; exact, since every e4m3
// value is a bf16 value
__device__ __forceinline__ bf16x8 widen_e4m3(int lo, int hi) {
    const auto a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
    const auto b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
    const auto c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
    const auto e = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
    return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], e[0], e[1]};
}

// lds_col8 of an fp8 tile, widened to bf16: lane l receives rows row0 + {0..3} +
// 4 (l/32), then row0 + 8 + {0..3} + 4 (l/32), of column col0 + l % 32 (col0 a
// multiple of 32), in one 8-bit transposing read.  Within each 16-lane group of
// that read, byte i of lane j is byte j % 8 of the 8 bytes addressed by lane
// 2 i + j / 8, so lane 2 i + c addresses the group's i-th row at the columns
// col0 + 16 (group % 2) + 8 c ..
template <int D>
__device__ __forceinline__ bf16x8 lds_col8_f8(const char* tile, int row0, int col0, int lane) {
    const int grp = lane >> 4, j = lane & 15;
    const int i = j >> 1, c = j & 1;
    const int row = row0 + 4 * (lane >> 5) + (i & 3) + 8 * (i >> 2);
    const int off = tile8_off<D>(row, (col0 >> 4) + (grp & 1)) + 8 * c;
    typedef int v2i __attribute__((ext_vector_type(2)));
    const v2i v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i*)(tile + off));
    return widen_e4m3(v.x, v.y);
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

// LDS byte address of a pointer into a __shared__ array
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(size_t)(const __attribute__((address_space(3))) char*)p;
}

// One wave instruction: lane l's 16 bytes at byte offset `voff` of the buffer
// land at LDS address lds + 16 l (lds uniform).  The whole offset is in the
// VGPR: the hardware range check covers the VGPR offset, not the scalar one.
// No memory clobber: LDS reads of other slots may move across it; ordering
// against the waits below is kept because volatile asm statements stay in order.
// The copy takes its LDS base from m0, which the compiler reserves (it cannot be
// declared clobbered), so the statement saves m0 in a scratch SGPR and restores
// it after issuing the load: whatever the compiler keeps in m0 survives.
__device__ __forceinline__ void dma16(rsrc_t rs, uint32_t voff, uint32_t lds) {
    uint32_t keep;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
                 "s_mov_b32 m0, %0"
                 : "=&s"(keep)
                 : "s"(lds), "v"(voff), "s"(rs));
}

// One wave instruction: lane l's 4 bytes at byte offset `voff` land at LDS
// address lds + 4 l (256 bytes per instruction); m0 kept as in dma16.
__device__ __forceinline__ void dma4(rsrc_t rs, uint32_t voff, uint32_t lds) {
    uint32_t keep;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tbuffer_load_dword %2, %3, 0 offen lds\n\t"
                 "s_mov_b32 m0, %0"
                 : "=&s"(keep)
                 : "s"(lds), "v"(voff), "s"(rs));
}

// One wave instruction: lane l's 2 bytes at byte offset `voff` land, zero-extended to
// 4 bytes, at LDS address lds + 4 l; the range check is per 2-byte unit (a unit past
// the end of the range reads as zero).  m0 kept as in dma16.
__device__ __forceinline__ void dma2(rsrc_t rs, uint32_t voff, uint32_t lds) {
    uint32_t keep;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tbuffer_load_ushort %2, %3, 0 offen lds\n\t"
                 "s_mov_b32 m0, %0"
                 : "=&s"(keep)
                 : "s"(lds), "v"(voff), "s"(rs));
}

// s_waitcnt vmcnt(J m) for a uniform m in [0, MMAX] (the count is an immediate)
template <int J>
__device__ __forceinline__ void wait_jobs(int m) {
    constexpr int MMAX = (63 / J) > 15 ? 15 : (63 / J);
#define GDPA_WJ(M) \
    case M: if constexpr (M <= MMAX) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(J * M) : "memory"); break;
    switch (m) {
        GDPA_WJ(0) GDPA_WJ(1) GDPA_WJ(2) GDPA_WJ(3) GDPA_WJ(4) GDPA_WJ(5) GDPA_WJ(6) GDPA_WJ(7)
        GDPA_WJ(8) GDPA_WJ(9) GDPA_WJ(10) GDPA_WJ(11) GDPA_WJ(12) GDPA_WJ(13) GDPA_WJ(14) GDPA_WJ(15)
        default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    }
#undef GDPA_WJ
}

// this wave's LDS reads (and scalar loads) have completed
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Geometry of a team's ring: T waves share LDS_BYTES of LDS.  With XJ = 1 every
// slot also has a 256-byte side buffer, filled by one more instruction per job and
// wave (per-row statistics that travel with a tile), so that every job still counts
// the same number of instructions.  In a two-wave team both waves load the same 256
// bytes into the same side buffer: the second write stores the values the first
// did, and the buffer is read only after the team barrier that follows both.
template <int D, int T, int LDS_BYTES, int XJ = 0>
struct RingGeom {
    static constexpr int TILE = 32 * D * 2;            // bytes of one 32-row tile
    static constexpr int SIDE = 256 * XJ;              // side bytes per slot
    static constexpr int J = TILE / 1024;              // wave instructions per tile
    static constexpr int JW = J / T;                   // issued by each wave of the team
    static constexpr int JX = JW + XJ;                 // instructions per job and wave
    static constexpr int RMAX = (63 / JX) + 1 > 16 ? 16 : (63 / JX) + 1;   // vmcnt is 6 bits
    static constexpr int RFIT = LDS_BYTES / (TILE + SIDE);
    static constexpr int R = RFIT > RMAX ? RMAX : RFIT;   // slots
    static constexpr int BYTES = R * (TILE + SIDE);
    static_assert(J % T == 0, "a tile's instructions are split evenly over the team");
    // a consume point takes at most 2 jobs and the ring runs R - 2 jobs past the
    // previous one, so R >= 4 keeps every awaited job issued
    static_assert(R >= 4, "the ring needs a step plus look-ahead");
};

template <int D, int T, int LDS_BYTES, int XJ = 0, int SW = 0>
struct Ring : RingGeom<D, T, LDS_BYTES, XJ> {
    using G = RingGeom<D, T, LDS_BYTES, XJ>;
    static constexpr int CPR = D / 8;   // 16-byte chunks per row
    uint32_t off[G::JW];                // lane offsets of this wave's instructions inside a tile
    uint32_t base;                      // LDS address of slot 0 (uniform)
    char* gbase;                        // the same slot 0 as a generic pointer
    int wt;                             // this wave's index in the team (uniform)
    int issued;                         // jobs issued so far (uniform)
    uint32_t xlane;                     // this lane's byte offset in a side load
    uint32_t off8[G::JW / 2 > 0 ? G::JW / 2 : 1];   // lane offsets of an fp8 tile's instructions

    __device__ __forceinline__ void init(char* slice, uint32_t row_stride_bytes, int wt_, int lane) {
        gbase = slice;
        base = lds_addr(slice);
        wt = wt_;
        issued = 0;
        xlane = 4u * (uint32_t)lane;
#pragma unroll
        for (int jj = 0; jj < G::JW; ++jj) {
            const int slot = (jj * T + wt) * 64 + lane;
            const int row = slot / CPR, pos = slot % CPR;
            off[jj] = (uint32_t)row * row_stride_bytes + (uint32_t)((pos ^ swz_sel<D, SW>(row)) << 4);
        }
    }

    // fp8 tiles: lane offsets for a tensor whose rows are row_stride8 bytes apart
    __device__ __forceinline__ void init8(uint32_t row_stride8, int lane) {
        constexpr int CPR8 = D / 16;   // 16-byte chunks per fp8 row
#pragma unroll
        for (int jj = 0; jj < G::JW / 2; ++jj) {
            const int slot = (jj * T + wt) * 64 + lane;
            const int row = slot / CPR8, pos = slot % CPR8;
            off8[jj] = (uint32_t)row * row_stride8 + (uint32_t)((pos ^ swz8<D>(row)) << 4);
        }
    }

    __device__ __forceinline__ int slot_of(int job) const { return job % G::R; }
    __device__ __forceinline__ char* tile(int job) const { return gbase + slot_of(job) * G::TILE; }
    // side buffer of job's slot (XJ = 1)
    __device__ __forceinline__ const char* side(int job) const {
        return gbase + G::R * G::TILE + slot_of(job) * G::SIDE;
    }

    // this wave's share of loading rows [row0, row0 + 32) of the slice `rs`
    // (row_off = row0 * stride) into the next slot
    __device__ __forceinline__ void issue(Slice rs, uint32_t row_off) {
        static_assert(XJ == 0, "jobs of a ring with side buffers carry a side load");
        const uint32_t lds = base + (uint32_t)(slot_of(issued) * G::TILE);
        {
            const rsrc_t rt = slice_at(rs, row_off);
#pragma unroll
            for (int jj = 0; jj < G::JW; ++jj) dma16(rt, off[jj], lds + (uint32_t)(jj * T + wt) * 1024u);
        }
        ++issued;
    }

    // issue() plus 256 bytes at byte offset x_off of `xs` into the slot's side
    // buffer (a zero-range `xs` fills it with zeros)
    __device__ __forceinline__ void issue(Slice rs, uint32_t row_off, Slice xs, uint32_t x_off) {
        static_assert(XJ == 1, "side loads need side buffers");
        const int slot = slot_of(issued);
        const uint32_t lds = base + (uint32_t)(slot * G::TILE);
        {
            const rsrc_t rt = slice_at(rs, row_off);
#pragma unroll
            for (int jj = 0; jj < G::JW; ++jj) dma16(rt, off[jj], lds + (uint32_t)(jj * T + wt) * 1024u);
        }
        dma4(slice_at(xs, x_off), xlane, base + (uint32_t)(G::R * G::TILE + slot * G::SIDE));
        ++issued;
    }

    // an fp8 tile (32 rows, D bytes each, rows row_off8 / stride on) into the first half
    // of the next slot; the other half of this wave's instructions load a zero-range
    // descriptor (`none`), so an fp8 job counts as many instructions as a bf16 one
    __device__ __forceinline__ void issue8(Slice rs, uint32_t row_off8, Slice none) {
        static_assert(XJ == 0, "fp8 tiles without side buffers");
        static_assert(G::JW % 2 == 0, "an fp8 tile takes half of a bf16 tile's instructions");
        const uint32_t lds = base + (uint32_t)(slot_of(issued) * G::TILE);
        const rsrc_t rt = slice_at(rs, row_off8), rz = slice_at(none, 0u);
#pragma unroll
        for (int jj = 0; jj < G::JW / 2; ++jj) dma16(rt, off8[jj], lds + (uint32_t)(jj * T + wt) * 1024u);
#pragma unroll
        for (int jj = G::JW / 2; jj < G::JW; ++jj) dma16(rz, 0u, lds + (uint32_t)(jj * T + wt) * 1024u);
        ++issued;
    }

    // issue8() plus a side load from byte offset x_off of `xs` into the slot's side
    // buffer: XW = 4, 256 bytes (lane l's 4 bytes at 4 l); XW = 2, lane l's 2 bytes
    // at 2 l, zero-extended into the 4 bytes at 4 l (units of 2 bytes range-checked
    // one by one, for rows of 2 bytes)
    template <int XW = 4>
    __device__ __forceinline__ void issue8(Slice rs, uint32_t row_off8, Slice none, Slice xs, uint32_t x_off) {
        static_assert(XJ == 1, "side loads need side buffers");
        static_assert(G::JW % 2 == 0, "an fp8 tile takes half of a bf16 tile's instructions");
        const int slot = slot_of(issued);
        const uint32_t lds = base + (uint32_t)(slot * G::TILE);
        const rsrc_t rt = slice_at(rs, row_off8), rz = slice_at(none, 0u);
#pragma unroll
        for (int jj = 0; jj < G::JW / 2; ++jj) dma16(rt, off8[jj], lds + (uint32_t)(jj * T + wt) * 1024u);
#pragma unroll
        for (int jj = G::JW / 2; jj < G::JW; ++jj) dma16(rz, 0u, lds + (uint32_t)(jj * T + wt) * 1024u);
        static_assert(XW == 4 || XW == 2, "side loads of 4 or 2 bytes per lane");
        if constexpr (XW == 4)
            dma4(slice_at(xs, x_off), xlane, base + (uint32_t)(G::R * G::TILE + slot * G::SIDE));
        else
            dma2(slice_at(xs, x_off), xlane >> 1, base + (uint32_t)(G::R * G::TILE + slot * G::SIDE));
        ++issued;
    }

    // wait until this wave's share of job k has landed
    __device__ __forceinline__ void wait(int k) const { wait_jobs<G::JX>(issued - 1 - k); }
};

// Launch shape of a team (KIND: 0 forward, 1 dK/dV, 2 dQ): waves per SIMD the
// register budget is sized for (WPE), and the team's LDS (160 KiB per CU shared
// by the resident teams).  Two waves per SIMD (8 per CU) where the registers fit
// and it measured faster: the forward kernel (d <= 64: one-wave teams with 20 KiB;
// d = 128: two-wave teams with 40 KiB) and the d <= 64 dQ kernel.  Otherwise one
// wave per SIMD with 40 KiB per wave (80 KiB for a two-wave d = 128 backward
// team).  With two waves per SIMD, operands are read from LDS just before use
// (the other wave hides the latency); with one, all of a step's operand reads are
// issued up front.
template <int D, int T, int KIND>
struct TeamShape {
    static_assert(T == 1 || T == 2, "teams of one or two waves");
    static constexpr int THREADS = 64 * T;
    static constexpr bool TWO = KIND == 0 ? (D < 128 || T == 2) : (KIND == 2 && D < 128);
    static constexpr int WPE = TWO ? 2 : 1;
    static constexpr int LDS = (TWO ? 20 * 1024 : 40 * 1024) * T;
    static constexpr bool HOIST = WPE == 1;
};

// this wave's LDS reads have completed and, for a team, every wave has arrived
template <int T>
__device__ __forceinline__ void team_sync() {
    if constexpr (T > 1)
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else
        wait_lds();
}

// -------------------------------------------------------------------------
// output blocks: staged through LDS, stored as whole rows
// -------------------------------------------------------------------------
// Stage a 32-row output block held as an MFMA accumulator (lane (r, hh) holds
// output row r and columns 32 db + 8 j + 4 hh + i in element 4 j + i of acc[db])
// as bf16 into a swizzled 32 x D tile.
template <int D>
__device__ __forceinline__ void stage_block(const f32x16 (&acc)[D / 32], float mul, char* tile, int r, int hh) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            u32x2 w;
            w[0] = pack_bf16x2(acc[db][4 * j] * mul, acc[db][4 * j + 1] * mul);
            w[1] = pack_bf16x2(acc[db][4 * j + 2] * mul, acc[db][4 * j + 3] * mul);
            *(u32x2*)(tile + tile_off<D>(r, 4 * db + j) + 8 * hh) = w;
        }
}

// One 32-column part (db) of stage_block.
template <int D>
__device__ __forceinline__ void stage_part(const f32x16& acc, int db, float mul, char* tile, int r, int hh) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        u32x2 w;
        w[0] = pack_bf16x2(acc[4 * j] * mul, acc[4 * j + 1] * mul);
        w[1] = pack_bf16x2(acc[4 * j + 2] * mul, acc[4 * j + 3] * mul);
        *(u32x2*)(tile + tile_off<D>(r, 4 * db + j) + 8 * hh) = w;
    }
}

// Write a 32 x 32 block held as two bf16x8 halves of an accumulator (lane (r, hh)
// holds column r and rows 8 j + 4 hh + i, element 8 m + 4 (j % 2) + i of half m
// = j / 2) into a swizzled 32 x 32 scratch tile as rows r (row r, columns
// 8 j + 4 hh + i): reading it back with lds_col8<32>(tile, 16 m, 0, lane) then
// gives lane l the values of rows 16 m + {0..3, 8..11} + 4 (l / 32) of column
// l % 32 of the block, i.e. the block's transpose in the chained operand layout.
__device__ __forceinline__ void stage_transpose32(const bf16x8 (&half)[2], char* tile, int r, int hh) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const bf16x8& h = half[j >> 1];
        const int o = 4 * (j & 1);
        const bf16x4 v = {h[o], h[o + 1], h[o + 2], h[o + 3]};
        *(bf16x4*)(tile + tile_off<32>(r, j) + 8 * hh) = v;
    }
}

// Store a staged 32 x D bf16 tile as rows row0 .. row0 + 31 of the slice `ro`
// (row_off0 = row0 * rso): each instruction writes whole rows, 16 bytes per lane.
template <int D>
__device__ __forceinline__ void store_tile(const char* tile, rsrc_t ro, uint32_t row_off0, uint32_t rso, int lane) {
    constexpr int CPR = D / 8, RPI = 64 / CPR;   // chunks per row, rows per instruction
    const int rr = lane / CPR, c = lane % CPR;
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
        const int row = i * RPI + rr;
        buf_store16(ro, row_off0 + (uint32_t)row * rso + (uint32_t)c * 16u,
                    *(const u32x4*)(tile + tile_off<D>(row, c)));
    }
}

// Zero rows row0 .. row0 + 31 of the bf16 slice `ro` (whole rows per instruction).
template <int D>
__device__ __forceinline__ void store_zero_rows(rsrc_t ro, uint32_t row_off0, uint32_t rso, int lane) {
    constexpr int CPR = D / 8, RPI = 64 / CPR;
    const int rr = lane / CPR, c = lane % CPR;
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i)
        buf_store16(ro, row_off0 + (uint32_t)(i * RPI + rr) * rso + (uint32_t)c * 16u, u32x4{0u, 0u, 0u, 0u});
}

// The issuing walk over a bin's items (every wave of a team runs the same walk
// and issues its share of each job).  Pol provides NSTAT (stationary tiles per
// item with steps), NSTRM (streaming tiles per step), walk_item(rec) (per-item
// descriptors of the issuing side) and issue_job(ring, rec, i) for the i-th job
// of the item (i < NSTAT: stationary tile i; else step s0 + (i - NSTAT) / NSTRM,
// tile (i - NSTAT) % NSTRM).  Items without steps have no jobs.
struct Walk {
    Rec r;
    int idx, end, pos, njobs;
    bool valid;
};

template <class Pol, class RingT>
__device__ __forceinline__ void walk_settle(Pol& pol, Walk& w, const Rec* __restrict__ recs) {
    // skip items without jobs
    while (w.valid && w.njobs == 0) {
        if (++w.idx < w.end) {
            // a uniform index, so that the record comes through the scalar cache: a vector
            // load here would make the compiler wait for vmcnt(0), i.e. for every tile
            // still in flight, each time the walk moves on to the next item
            w.r = recs[__builtin_amdgcn_readfirstlane(w.idx)];
            w.pos = 0;
            w.njobs = w.r.s1 >= w.r.s0 ? Pol::NSTAT + Pol::NSTRM * (w.r.s1 - w.r.s0 + 1) : 0;
        } else {
            w.valid = false;
        }
    }
    if (w.valid && w.pos == 0) pol.walk_item(w.r);
}

// Issue jobs until the ring is full (consumed = jobs the computing side has freed).
template <class Pol, class RingT>
__device__ __forceinline__ void pump(Pol& pol, Walk& w, RingT& ring, int consumed, const Rec* __restrict__ recs) {
    while (w.valid && ring.issued < consumed + RingT::R) {
        pol.issue_job(ring, w.r, w.pos);
        if (++w.pos == w.njobs) {
            w.njobs = 0;
            walk_settle<Pol, RingT>(pol, w, recs);
        }
    }
}

// A policy may set up the ring once it is initialised (fp8 tile offsets): it does
// so with a member ring_ready(ring, lane), which is called when present.
template <class Pol, class RingT>
__device__ __forceinline__ auto ring_ready(Pol& p, RingT& g, int lane, int) -> decltype(p.ring_ready(g, lane), void()) {
    p.ring_ready(g, lane);
}
template <class Pol, class RingT>
__device__ __forceinline__ void ring_ready(Pol&, RingT&, int, long) {}

// This team's bin: workgroups are dispatched round-robin over the 8 XCDs, so the
// workgroup index is remapped to make consecutive logical workgroups (whose bins
// the planner fills with neighbouring items of equal cost, e.g. the q tiles of one
// sample) share an XCD and its L2.
__device__ __forceinline__ int team_bin() {
    const int G = gridDim.x, w = blockIdx.x;
    return (G % 8 == 0) ? (w % 8) * (G / 8) + w / 8 : w;
}

// Items claimed at run time (one-wave teams, a.claim set).  The workgroups of the
// launch take items in the planner's order a.order: the first P (one per workgroup,
// P = the grid) without a claim, item r by the workgroup of logical bin r, where the
// planner's deal puts its first round (so that neighbouring items share an XCD as
// they do there); every further item from one counter, P + (the counter's value).
// A claim is a vector atomic from one lane whose value is used at once, so it waits
// for the tiles still in flight (the counter orders them): the planner claims only
// lists whose items are long against that wait.  The walk hands
// every claimed item to the computing side through a queue held one entry per lane
// of a register; it claims only while fewer than kClaimQueue items are unfinished
// (entry k lives in lane k % 64 until the computing side has read it), and the
// computing side runs the walk again whenever it has emptied the queue.  A workgroup
// adds itself to a.claim[1] after its last claim, and the last one to do so sets
// both counters back to 0 for the next launch.
constexpr int kClaimQueue = 48;

struct ClaimWalk {
    Rec r;
    int pos, njobs;   // the walk's item: jobs issued, jobs (pos == njobs: claim the next)
    bool valid;       // false once a claim has found the list exhausted
    bool first;       // this workgroup's first item (no claim) is still to be taken
    int queue;        // lane (k % 64): the k-th claimed item
    int n;            // items claimed so far (uniform)
};

template <class Pol>
__device__ __forceinline__ void claim_one(Pol& pol, ClaimWalk& w, const Rec* __restrict__ recs, int lane) {
    int k;
    if (w.first) {
        k = team_bin();
        w.first = false;
    } else {
        k = 0;
        if (lane == 0) k = __hip_atomic_fetch_add(pol.a.claim, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        k = (int)gridDim.x + __builtin_amdgcn_readfirstlane(k);
    }
    if (k >= pol.a.n_items) {
        w.valid = false;
        return;
    }
    const int idx = __builtin_amdgcn_readfirstlane(pol.a.order[k]);
    w.queue = lane == (w.n & 63) ? idx : w.queue;
    ++w.n;
    w.r = recs[idx];
    w.pos = 0;
    w.njobs = w.r.s1 >= w.r.s0 ? Pol::NSTAT + Pol::NSTRM * (w.r.s1 - w.r.s0 + 1) : 0;
    if (w.njobs > 0) pol.walk_item(w.r);
}

// issue jobs until the ring is full, claiming items as the walk needs them (done:
// items the computing side has finished)
template <class Pol, class RingT>
__device__ __forceinline__ void claim_pump(Pol& pol, ClaimWalk& w, RingT& ring, int consumed, int done,
                                          const Rec* __restrict__ recs, int lane) {
    while (w.valid && ring.issued < consumed + RingT::R) {
        if (w.pos == w.njobs) {
            if (w.n - done >= kClaimQueue) return;
            claim_one(pol, w, recs, lane);
            continue;
        }
        pol.issue_job(ring, w.r, w.pos);
        ++w.pos;
    }
}

template <class Pol, class RingT>
__device__ __forceinline__ void run_claimed(Pol& pol, const Rec* __restrict__ recs, char* slice, uint32_t row_stride,
                                            int lane) {
#ifdef GDPA_BIN_CLOCK
    const unsigned long long clock0 = __builtin_amdgcn_s_memrealtime();
#endif
    RingT ring;
    ring.init(slice, row_stride, 0, lane);
    ring_ready(pol, ring, lane, 0);
    ClaimWalk w;
    w.queue = 0;
    w.n = 0;
    w.pos = w.njobs = 0;
    w.valid = true;
    w.first = true;
    int job = 0, ci = 0;
    claim_pump<Pol, RingT>(pol, w, ring, job, ci, recs, lane);
    for (;;) {
        if (ci == w.n) {   // every claimed item is done: claim more, or stop
            if (!w.valid) break;
            claim_pump<Pol, RingT>(pol, w, ring, job, ci, recs, lane);
            continue;
        }
        const Rec c = recs[__builtin_amdgcn_readlane(w.queue, ci & 63)];
        if (c.s1 < c.s0) {
            pol.item_zero(c);
            ++ci;
            continue;
        }
        // every job before this item's first is consumed: the walk (on this item or
        // past it) issues at least the jobs of the item's first consume point
        claim_pump<Pol, RingT>(pol, w, ring, job, ci, recs, lane);
        pol.item_begin(c);
#pragma unroll
        for (int i = 0; i < Pol::NSTAT; i += 2) {
            const int n = (Pol::NSTAT - i) < 2 ? 1 : 2;
            ring.wait(job + n - 1);
            wait_lds();
            claim_pump<Pol, RingT>(pol, w, ring, job, ci, recs, lane);
            pol.load_stat(c, ring, job, i);
            job += n;
        }
        for (int s = c.s0;; ++s) {
            ring.wait(job + 1);
            wait_lds();
            claim_pump<Pol, RingT>(pol, w, ring, job, ci, recs, lane);
            pol.step(c, s, ring, job);
            job += 2;
            if (s == c.s1) break;
        }
        wait_lds();
        pol.item_end(c, ring, job);
        ++ci;
    }
    if (lane == 0) {
        const int fin = __hip_atomic_fetch_add(pol.a.claim + 1, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        if (fin == (int)gridDim.x - 1) {   // every workgroup has made its last claim
            __hip_atomic_store(pol.a.claim, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(pol.a.claim + 1, 0, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
#ifdef GDPA_BIN_CLOCK
    if (pol.a.bin_clock && lane == 0) {
        const int bin = team_bin();
        pol.a.bin_clock[2 * bin] = clock0;
        pol.a.bin_clock[2 * bin + 1] = __builtin_amdgcn_s_memrealtime();
    }
#endif
}

// The computing side.  Pol also provides:
//   item_begin(rec)                 zero the accumulators
//   load_stat(rec, ring, job, i)    stationary tiles i, i + 1 (jobs job, job + 1; only
//                                   tile i if i + 1 == NSTAT) -> the owning wave's registers
//   step(rec, s, ring, job)         one streaming step (jobs job, job + 1)
//   item_end(rec, ring, job)        store this wave's outputs, staged through a slot of
//                                   the item's last step (jobs job - 2, job - 1), which
//                                   is re-filled only after the next barrier
//   item_zero(rec)                  store this wave's outputs of an item without steps
// Every consume point waits for its jobs, synchronises the team and only then
// re-fills the slots the team has finished with.
template <class Pol, class RingT, int T>
__device__ __forceinline__ void run_team(Pol& pol, int P, const Rec* __restrict__ recs,
                                         const int32_t* __restrict__ bin_ptr, char* slice, uint32_t row_stride,
                                         int wt, int lane) {
    static_assert(Pol::NSTRM == 2, "a step streams two tiles");
    if constexpr (T == 1) {
        if (pol.a.claim) {
            run_claimed<Pol, RingT>(pol, recs, slice, row_stride, lane);
            return;
        }
    }
    const int bin = team_bin();
    if (bin >= P) return;
    const int beg = bin_ptr[bin], end = bin_ptr[bin + 1];
    if (beg >= end) return;
#ifdef GDPA_BIN_CLOCK
    const unsigned long long clock0 = __builtin_amdgcn_s_memrealtime();
#endif

    RingT ring;
    ring.init(slice, row_stride, wt, lane);
    ring_ready(pol, ring, lane, 0);
    Walk w;
    w.idx = beg;
    w.end = end;
    w.r = recs[beg];
    w.pos = 0;
    w.njobs = w.r.s1 >= w.r.s0 ? Pol::NSTAT + Pol::NSTRM * (w.r.s1 - w.r.s0 + 1) : 0;
    w.valid = true;
    walk_settle<Pol, RingT>(pol, w, recs);
    int job = 0;   // next job the computing side consumes
    pump<Pol, RingT>(pol, w, ring, job, recs);

    for (int ci = beg; ci < end; ++ci) {
        const Rec c = recs[ci];
        if (c.s1 < c.s0) {
            pol.item_zero(c);
            continue;
        }
        pol.item_begin(c);
#pragma unroll
        for (int i = 0; i < Pol::NSTAT; i += 2) {
            const int n = (Pol::NSTAT - i) < 2 ? 1 : 2;
            ring.wait(job + n - 1);
            team_sync<T>();
            pump<Pol, RingT>(pol, w, ring, job, recs);
            pol.load_stat(c, ring, job, i);
            job += n;
        }
        for (int s = c.s0;; ++s) {
            ring.wait(job + 1);
            team_sync<T>();
            pump<Pol, RingT>(pol, w, ring, job, recs);
            pol.step(c, s, ring, job);
            job += 2;
            if (s == c.s1) break;
        }
        team_sync<T>();   // every wave is done with the last step's slots
        pol.item_end(c, ring, job);
    }
#ifdef GDPA_BIN_CLOCK
    if (pol.a.bin_clock && wt == 0 && lane == 0) {
        pol.a.bin_clock[2 * bin] = clock0;
        pol.a.bin_clock[2 * bin + 1] = __builtin_amdgcn_s_memrealtime();
    }
#endif
}

}  // namespace gdpa
