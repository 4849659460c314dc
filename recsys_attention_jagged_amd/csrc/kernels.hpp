// Kernel arguments and launchers shared between the HIP kernels and the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.hpp"

namespace gdpa {

// Arguments common to every kernel.  Tensors are [T, H, d] row-major; a work
// list is (items, bin_ptr) over P bins, one per persistent workgroup.
struct KernelArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* dout;
    void* o;    // forward output
    void* dq;
    void* dk;
    void* dv;
    const int32_t* q_off;
    const int32_t* kv_off;
    const void* items;          // device work-list records (Rec), bin-major
    const int32_t* bin_ptr;
    float* part;                // fp32 partial-output slots of chunks, [slots][blocks][rows per item][d]
                                // (one block per slot; two, dK then dV, for the dK/dV list)
    float* part_stat;           // softmax forward chunks: per slot row (running max in log2 units, row sum),
                                // [slots][rows per item][2]
    int P;          // bins = persistent workgroups
    int B;          // samples
    int H;
    int window;     // 0 = none
    float scale;    // 1 / sqrt(d)
    int out_f32;    // outputs stored as fp32 instead of bf16
    // softmax attention (JFA) only: per-row log-sum-exp, fp32 [H, Tq] (head-major),
    // written by the forward (and read by the backward's dQ kernel, with the forward's
    // O in `o`); per (head, q row) the pair (LSE log2(e), D = sum of dO * O over the
    // row), fp32 [H, Tq, 2], written by the dQ kernel and read by the dK/dV kernel
    float* lse;
    float* stat;
    int Tq;
    // RMSNorm prologue only: 1/rms per (head, row) of Q, fp32 [H, Tq], and of K and V
    // as pairs, fp32 [H, Tk, 2] (1 for a tensor left raw); `norm` says which of Q (1),
    // K (2), V (4) are normalised (their gradients go through the norm)
    const float* rq;
    const float* rkv;
    int Tk;
    int norm;
    // stored dS (d = 128 two-kernel backward): 32 x 32 bf16 blocks (kv row major)
    // that the dK/dV kernel writes and the dQ kernel reads; records locate them
    // (see DsLayout)
    __bf16* ds;
    // block-scaled fp8 forward (MX): one E8M0 scale byte per 32 consecutive head
    // columns of each Q and K row, head-major [H, Tq, d / 32] and [H, Tk, d / 32]
    const uint8_t* q_mx;
    const uint8_t* k_mx;
    // fp8 backward (Q, K, dO as e4m3 with one factor per tensor, V bf16): `scale` is
    // then the score factor s_q s_k / sqrt(d); dP is the product times f8_dp = s_do;
    // the stored dQ, dK, dV are their products times f8_dq = s_k / sqrt(d),
    // f8_dk = s_q / sqrt(d), f8_dv = s_do
    float f8_dp, f8_dq, f8_dk, f8_dv;
    // items claimed at run time (one-wave teams; claim == nullptr: each workgroup walks
    // its bin): claim k takes item order[k] of `items`, k < n_items; claim[0] counts
    // the claims of the launch, claim[1] the workgroups that have finished, and the
    // last to finish sets both back to 0
    const int32_t* order;
    int* claim;
    int n_items;
#ifdef GDPA_BIN_CLOCK
    // clock-probe builds only: per bin, the real-time stamps (100 MHz) of the start and
    // the end of its walk, [P][2]
    unsigned long long* bin_clock;
#endif
};

// the activation code of the softmax (JFA) variant of the bf16 kernels (device
// enum Act::ACT_SOFTMAX); the public activations are gdpa_act
constexpr int kActSoftmax = 6;

// flag on an activation code: the RMSNorm-prologue variant of a GDPA kernel
constexpr int kActNorm = 16;

// flag on an activation code: the forward with fp8 (OCP e4m3) Q and K
constexpr int kActF8 = 32;
// or'ed into the act code: the forward with block-scaled fp8 (MX) Q and K
constexpr int kActMX = 64;
// or'ed into the act code of a backward kernel: Q, K and dO as fp8 (e4m3)
constexpr int kActF8Bwd = 128;

// bf16 MFMA kernels, one translation unit per head dimension.  A workgroup is a
// team of `team` waves (1, or 2 for d = 128) working on one bin (P bins, P
// workgroups); nb = 32-row stationary blocks per wave (forward and dQ: 1 or 2,
// dK/dV: 1), so an item holds 32 * team * nb stationary rows.
#define GDPA_DECLARE_LAUNCHERS(D)                                                                      \
    hipError_t launch_fwd_bf16_d##D(const KernelArgs& a, int team, int nb, int act, hipStream_t s);    \
    hipError_t launch_dq_bf16_d##D(const KernelArgs& a, int team, int nb, int act, hipStream_t s);     \
    hipError_t launch_dkdv_bf16_d##D(const KernelArgs& a, int team, int nb, int act, hipStream_t s);   \
    const void* fwd_bf16_kernel_ptr_d##D(int team, int nb, int act);                                   \
    const void* dq_bf16_kernel_ptr_d##D(int team, int nb, int act);                                    \
    const void* dkdv_bf16_kernel_ptr_d##D(int team, int nb, int act);
GDPA_DECLARE_LAUNCHERS(32)
GDPA_DECLARE_LAUNCHERS(64)
GDPA_DECLARE_LAUNCHERS(128)
#undef GDPA_DECLARE_LAUNCHERS

// d = 128 dK/dV kernel on the 16 x 16 x 32 MFMA for kv items of `rows` = 32 or 64
// rows (the dK/dV list's layouts team 1 and team 2, one block): a workgroup of
// rows / 16 waves, 16 kv rows per wave, two waves per SIMD.  Plain GDPA
// activations only, with kActF8Bwd for fp8 Q, K, dO (nullptr otherwise).
const void* dkdv16_kernel_ptr(int rows, int act);

// d = 128 dQ from the stored dS blocks: dQ = dS K / sqrt(d) over the dQ list of
// 32-row q items (one wave per workgroup); a.ds, a.items: that list, a.part its
// slots; f8: K as fp8 (e4m3)
hipError_t launch_dq_from_ds(const KernelArgs& a, int f8, hipStream_t s);
const void* dq_from_ds_kernel_ptr(int f8 = 0);
// the same over 64-row q items in two-wave teams (items carry the dS layout's head
// base and blocks per q tile in pad0, pad1)
hipError_t launch_dq_from_ds_team(const KernelArgs& a, int f8, hipStream_t s);
const void* dq_from_ds_team_kernel_ptr(int f8 = 0);

// One-pass backward (one-wave teams, one block per wave): kv_stationary = 1 runs
// over the dK/dV list when every Lk <= 32 (dQ stored per step), 0 over the dQ
// list when every Lq <= 32 (dK, dV stored per step).
#define GDPA_DECLARE_FUSED(D)                                                                         \
    hipError_t launch_bwd_fused_d##D(const KernelArgs& a, int kv_stationary, int act, hipStream_t s);   \
    const void* bwd_fused_kernel_ptr_d##D(int kv_stationary, int act);
GDPA_DECLARE_FUSED(32)
GDPA_DECLARE_FUSED(64)
GDPA_DECLARE_FUSED(128)
#undef GDPA_DECLARE_FUSED

// Output rows of cut items: out = mul * (sum of the item's slots, in slot order),
// stored as bf16 (out_f32 = 0) or fp32.  A slot holds `stride` blocks of
// rows_per_slot x d floats; block `offset` of each slot is summed (O and dQ:
// stride 1; dK, dV: stride 2, offsets 0 and 1).
hipError_t launch_partial_sum(const DevGroup* groups, int n_groups, const float* part, int rows_per_slot,
                              int stride, int offset, int d, int H, float mul, void* out, int out_f32,
                              hipStream_t s);

// RMSNorm prologue pre-pass: rq[h, i] = 1 / sqrt(mean_c q[i, h, c]^2 + eps) for
// i < Tq when norm & 1 (else 1); rkv[h, j] = (the same of k, of v) for j < Tk when
// norm & 2, norm & 4 (else 1); inputs bf16 [T, H, d]
hipError_t launch_norm_rstd(const void* q, const void* k, const void* v, int Tq, int Tk, int H, int d, int norm,
                            float eps, float* rq, float* rkv, hipStream_t s);

// JFA forward chunks: per row of each cut item, O = (sum_j 2^(m_j - m) O_j) / l and
// LSE = (m + log2 l) ln 2, with m = max_j m_j and l = sum_j 2^(m_j - m) l_j over the
// item's slots j in slot order (out bf16 or fp32 [Tq, H, d]; lse [H, Tq])
hipError_t launch_jfa_combine(const DevGroup* groups, int n_groups, const float* part, const float* part_stat,
                              int rows_per_slot, int d, int H, int Tq, void* out, int out_f32, float* lse,
                              hipStream_t s);

// JFA backward pre-pass: stat[h, i] = (lse[h, i] log2(e), sum_c dout[i, h, c] o[i, h, c])
// for the Tq rows of o, dout ([Tq, H, d] bf16)
hipError_t launch_jfa_stat(const void* o, const void* dout, const float* lse, int Tq, int H, int d, float* stat,
                           hipStream_t s);

// Bytes of the fixed device scratch array that the no-allocation entry points
// use (per GPU, for the life of the process), and its address on the current
// device (looked up once per device).
constexpr size_t kNoallocScratchBytes = (size_t)32 << 20;
hipError_t noalloc_scratch(void** out);

// plain fp32 kernels (no MFMA): forward, dQ, dK/dV over the offsets directly
hipError_t launch_fwd_f32(const KernelArgs& a, int Tq, int d, int act, hipStream_t s);
hipError_t launch_bwd_f32(const KernelArgs& a, int Tq, int Tk, int d, int act, hipStream_t s);

}  // namespace gdpa
