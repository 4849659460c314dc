/*
 * gdpa.h - C ABI of a jagged Generalized Dot-Product Attention (GDPA) library for
 * AMD Instinct MI355X (gfx950).
 *
 * What is computed (GDPA page: aitrends.kr/articles/26275, "Generalized
 * Dot-Product Attention (GDPA): kernel optimisation for real recommendation-system
 * training loads"; "Key summary" and "Section details", diagram "Self-attention,
 * PMA and pFFN unified as GDPA", and the paragraph on removing the softmax
 * correction step):  for every sample b and head h, over the valid pairs
 * (i, j) with 0 <= i < Lq_b, 0 <= j < Lk_b and, if window > 0, |i - j| < window,
 *
 *     S_ij = <Q_i, K_j> / sqrt(d),   P_ij = act(S_ij),   O_i = sum_j P_ij V_j
 *
 * with no softmax and no row normalisation.  The backward pass returns dQ, dK,
 * dV of the loss sum(O * dO), recomputing S inside the kernels (no O and no
 * row statistics are kept).  The three shapes of the GEM page (techlist.io,
 * "GEM training: ...", section on why high GPU utilisation is hard): jagged
 * self-attention with an optional short window, user-ad cross-attention (long
 * Q, short K/V) and PMA (short Q, long K/V) are all served by the same calls.
 *
 * Data layout.  Q, dO, O, dQ are [Tq, H, d] and K, V, dK, dV are [Tk, H, d],
 * dense, row-major (d fastest, then heads, then tokens).  Offsets are int32
 * [B + 1], non-decreasing, off[0] = 0, off[B] = T; sample b owns rows
 * off[b] .. off[b+1]-1.  bf16 is IEEE bfloat16.
 *
 * Ownership.  The caller owns every tensor and offset buffer and keeps them
 * alive until the stream work that uses them has finished.  A plan owns its
 * host and device work lists; gdpa_plan_destroy frees them.  A plan's work lists
 * are immutable after creation and any stream may run it, but calls on one plan
 * must not overlap in time: items cut into chunks keep their partial outputs in
 * the plan's slot buffer (see gdpa_plan_create).
 *
 * Asynchrony.  gdpa_fwd / gdpa_bwd validate their arguments on the host, then
 * only enqueue kernels on `stream` (NULL = the null stream); they never
 * synchronise.  A fault during execution shows up at the caller's next
 * synchronisation.  The launch path makes no allocation, memset or copy, so the
 * calls can be captured into a HIP graph (except with GDPA_DEBUG=1, whose offset
 * re-check copies the device offsets to the host).
 *
 * Errors.  Every call returns a gdpa_status; no call throws.  Arguments are
 * validated before anything is enqueued.  gdpa_last_error() returns a
 * thread-local message describing the most recent failure on this thread.
 *
 * Determinism.  No atomics: every output row is written by exactly one work
 * item, so results are bitwise identical from run to run.
 */
#ifndef GDPA_H
#define GDPA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDPA_OK = 0,
    GDPA_ERR_INVALID_ARG = 1,   /* null pointer, bad size, B/H/d/window out of range */
    GDPA_ERR_BAD_OFFSETS = 2,   /* offsets not [0, .., T] non-decreasing, or a window with Lq != Lk */
    GDPA_ERR_UNSUPPORTED = 3,   /* d not in {32, 64, 128}, activation/dtype combination not built */
    GDPA_ERR_PLAN_MISMATCH = 4, /* B/H/d/window differ from the plan's, or a host-only plan */
    GDPA_ERR_HIP = 5,           /* a HIP runtime call failed (message in gdpa_last_error) */
    GDPA_ERR_NOMEM = 6          /* host or device allocation failed */
} gdpa_status;

/* Activations.  GELU is the exact erf form x * Phi(x), evaluated to within 7e-7
 * absolute (forward: a fitted exp2 tail; backward: Abramowitz & Stegun 7.1.26's
 * erfc, |error| <= 1.5e-7).  GELU_POLY is an
 * ALU-only clamped polynomial fit of it (FMA only; absolute error bounds
 * gdpa_gelu_poly_bound() for the value, gdpa_gelu_poly_grad_bound() for the
 * derivative).  GELU_TAYLOR6 is the GDPA page's series (code figure
 * "ALU-only 6th-order Taylor GELU"), accurate only near 0.  IDENTITY and ONE
 * (P = 1 on valid pairs) are test probes; ONE has no backward. */
typedef enum {
    GDPA_ACT_GELU = 0,
    GDPA_ACT_SILU = 1,
    GDPA_ACT_GELU_POLY = 2,
    GDPA_ACT_GELU_TAYLOR6 = 3,
    GDPA_ACT_IDENTITY = 4,
    GDPA_ACT_ONE = 5
} gdpa_act;

/* Storage types.  BF16: bf16 inputs and outputs, fp32 accumulation (MFMA).
 * BF16_F32OUT: bf16 inputs, fp32 outputs (O, dQ, dK, dV).  F32: fp32 in and
 * out, plain fp32 arithmetic (no MFMA; a correctness path for small inputs). */
typedef enum { GDPA_F32 = 0, GDPA_BF16 = 1, GDPA_BF16_F32OUT = 2 } gdpa_dtype;

/* Work lists of a plan, for gdpa_plan_export / gdpa_plan_stats.  DQ_TEAM: dQ from
 * stored dS in two-wave teams (gdpa_plan_stats: dq_team 2), export only. */
typedef enum { GDPA_LIST_FWD = 0, GDPA_LIST_DKDV = 1, GDPA_LIST_DQ = 2, GDPA_LIST_DQ_TEAM = 3 } gdpa_list;

/* Planning options.  All-zero (or a NULL pointer) selects the defaults. */
typedef struct {
    int host_only;   /* 1: plan on the host only (export / stats); no device memory is
                        allocated and gdpa_fwd / gdpa_bwd reject the plan */
    int bins[3];     /* bins per list (GDPA_LIST_*), one per persistent workgroup; 0 = as
                        many workgroups as the device holds resident (host_only: 1024) */
    int team[3];     /* waves per workgroup sharing one tile ring: 0 = automatic, 1, or 2
                        (d = 128 only) */
    int blocks[3];   /* 32-row stationary blocks per wave: 0 = automatic, 1 or 2 (dK/dV
                        and two-wave teams: 1).  An item holds 32 * team * blocks
                        stationary rows */
    int deal;        /* how sorted items go to bins: 0 greedy (each item to the bin of
                        least cost so far), 1 zigzag (snake), 2 round robin */
    int no_split;    /* 1: never cut an item into chunks (see gdpa_plan_create) */
    int unfused;     /* 1: gdpa_bwd always runs the two backward kernels (see gdpa_bwd) */
    int no_ds;       /* 1: gdpa_bwd recomputes dS in its dQ kernel instead of storing it
                        (no dS buffer; see gdpa_plan_create) */
    int claim;       /* how workgroups get items: 0 automatic (claimed at run time, in the
                        planner's order, where the list's kernel runs one-wave teams and its
                        items average 64 steps or more; else the planner's bins), 1 the
                        planner's bins only, 2 claimed wherever the kernel runs one-wave
                        teams.  A claim waits for the loads in flight (about one memory
                        latency).  Results do not depend on it (bit for bit) */
    int slot_time;   /* 0 automatic: where a list has automatic bins and its kernel is one
                        measured for it (the d = 128 two-wave forward and 16-row dK/dV
                        kernels at four workgroups per CU, the d = 64 forward at eight, dQ
                        from stored dS in two-wave teams at three), the
                        greedy deal weighs each bin's cost by a time factor of its dispatch
                        round on its CU (workgroups placed early on a CU ran up to 12 %
                        faster than later ones), so earlier-placed bins get more work; 1 every
                        bin is dealt by plain cost.  Results do not depend on it (bit for
                        bit) */
    int dq_team;     /* dQ from stored dS (see ds_bytes): 0 automatic, two-wave teams over
                        64-row q items (a work list of its own, list 3 of
                        gdpa_plan_export; each K tile read once for two q tiles); 1 one-wave
                        workgroups over the dQ list.  Results equal bit for bit unless
                        items are cut into chunks (their chunks then differ) */
} gdpa_plan_opts;

/* Summary numbers of a plan. */
typedef struct {
    int64_t Tq, Tk;          /* total query / key rows */
    int64_t valid_pairs;     /* sum over samples of the valid (i, j) pairs */
    int32_t n_items[3];      /* work items per list */
    int32_t n_steps[3];      /* streaming steps per list (a step-less item counts 0) */
    int32_t bins[3];         /* bins (persistent workgroups) per list */
    int32_t tile_stat[3];    /* stationary tile rows per list */
    int32_t tile_strm[3];    /* streaming tile rows per list */
    int64_t bin_cost_max[3]; /* per-bin cost extremes (planner cost units) */
    int64_t bin_cost_min[3];
    int32_t bwd_fused;       /* what gdpa_bwd runs: 0 the two kernels, 1 one KV-stationary
                                pass (every Lk <= 32), 2 one Q-stationary pass (every Lq <= 32) */
    int32_t n_parts[3];      /* partial-output slots per list (chunks of cut items; 0 for
                                the dK/dV list) */
    int64_t ds_bytes;        /* bytes of the plan's dS buffer (0: gdpa_bwd does not store dS) */
    int32_t claimed[3];      /* 1: the list's items are claimed at run time (see claim) */
    int32_t slot_weighted[3];/* 1: the list's deal took the dispatch-slot time factors */
    int32_t dq_team;         /* dQ from stored dS: 0 none (ds_bytes 0), 1 one-wave workgroups
                                over the dQ list, 2 two-wave teams over list 3 */
    int32_t dq_team_items;   /* list 3 (dq_team 2): work items, bins, cut items' chunk slots */
    int32_t dq_team_bins;
    int32_t dq_team_parts;
    int32_t dq_team_slot_weighted; /* 1: list 3's deal took the dispatch-slot time factors */
} gdpa_plan_stats_t;

typedef struct gdpa_plan_s* gdpa_plan;

/*
 * gdpa_plan_create - enumerate the non-empty tiles on the host and deal them to
 * persistent workgroups (GDPA page, "Section details": the CPU precomputes the
 * valid tiles, sorts them and assigns them to processors in a zigzag order; here
 * the sorted items go by default each to the least-loaded bin, which balances
 * better than the fixed snake, and zigzag remains an option).
 *
 *   q_off_host, kv_off_host : host int32 [B + 1] offsets (read during the call only)
 *   B >= 0 samples, H >= 1 heads, d in {32, 64, 128}
 *   window >= 0             : 0 = every in-range pair; w > 0 keeps |i - j| < w and
 *                             requires Lq_b == Lk_b for every b
 *   dtype                   : storage type the plan will be used with
 *   opts                    : NULL or planning options
 *   stream                  : a hipStream_t (NULL = the null stream) on which the
 *                             work lists are copied to the device; ignored for a
 *                             host_only plan
 *   out                     : receives the plan (NULL on failure)
 *
 * For d = 128 bf16 plans whose gdpa_bwd runs the two backward kernels (and unless
 * opts->no_ds, or a layout other than one block per wave in the dK/dV list and
 * the automatic one-wave, one-block dQ list is asked for), the plan also owns a dS
 * buffer: each sample gives each of its 32-row q tiles as many 32 x 32 bf16 blocks
 * (2 KiB) as the most 32-row kv tiles any of its q tiles has a valid pair with,
 * per head (gdpa_plan_stats reports its size).  gdpa_bwd's dK/dV kernel stores dS there and
 * its dQ kernel computes dQ = dS K / sqrt(d) from it instead of recomputing the
 * scores and the activation's derivative.
 *
 * Items of the Q-stationary lists (forward, dQ) whose cost exceeds the mean
 * per-bin cost are cut into chunks of consecutive streaming tiles (unless
 * opts->no_split); each chunk stores an fp32 partial output block into the plan's
 * slot buffer and a small reduction kernel, enqueued right after the main kernel,
 * adds the chunks of each cut item in a fixed order (no atomics).  Calls that use
 * one plan therefore must not overlap in time (e.g. on two streams).
 *
 * Unless opts->host_only, allocates the device work lists and the slot buffers
 * (n_parts * tile_stat * w * 4 bytes per list, w = d + 2 for the forward list,
 * 2 d for dK/dV, d for dQ) on the current device with hipMalloc, stages the
 * lists in a pinned host buffer that the plan owns, and enqueues their copies on
 * `stream` without waiting for them: the call never synchronises the device.
 * Work that uses the plan must be ordered after those copies (enqueued on the
 * same stream, or after an event or a synchronisation of it).  Planning itself
 * runs on the host during the call (the GDPA page, "Section details": the tiles
 * are precomputed on the CPU).  Errors: INVALID_ARG, BAD_OFFSETS, UNSUPPORTED,
 * HIP, NOMEM.
 */
gdpa_status gdpa_plan_create(const int32_t* q_off_host, const int32_t* kv_off_host, int B, int H,
                             int d, int window, gdpa_dtype dtype, const gdpa_plan_opts* opts,
                             void* stream, gdpa_plan* out);

/*
 * gdpa_fwd - O = act(Q K^T / sqrt(d)) V over the valid pairs (see top).
 *
 *   q [Tq,H,d], k [Tk,H,d], v [Tk,H,d] : device inputs of the plan's dtype
 *   q_off_dev, kv_off_dev              : device int32 [B + 1], equal to the plan's
 *                                        host offsets (precondition; GDPA_DEBUG=1 in
 *                                        the environment re-checks it with a copy)
 *   B, H, d, window                    : must equal the plan's
 *   act                                : activation
 *   o [Tq,H,d]                         : device output (bf16, or fp32 for F32 /
 *                                        BF16_F32OUT); every row is written, rows
 *                                        with no valid key as 0
 *   stream                             : a hipStream_t (NULL = null stream)
 *
 * Errors: INVALID_ARG, PLAN_MISMATCH, UNSUPPORTED, HIP (launch failure).
 */
gdpa_status gdpa_fwd(gdpa_plan plan, const void* q, const void* k, const void* v,
                     const int32_t* q_off_dev, const int32_t* kv_off_dev, int B, int H, int d,
                     gdpa_act act, int window, void* o, void* stream);

/*
 * gdpa_fwd_noalloc - gdpa_fwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  It makes no device or pinned allocation and calls no allocating
 * library routine; instead of the plan's device work list and chunk slot buffer
 * it uses the library's fixed scratch array of 32 MiB per GPU (a static device
 * array, resident until the process ends): the call copies the plan's forward
 * work list from the plan's host memory into it (hipMemcpyAsync on `stream`)
 * and the kernels keep the chunk partial outputs there.
 *
 *   plan : any bf16 plan, in particular one made with opts->host_only = 1, which
 *          owns no device memory at all (its bins, team and block layout are used
 *          as planned; F32 plans: UNSUPPORTED).  It must stay alive until the
 *          enqueued work has finished (the copy reads its host memory).
 *   other arguments, outputs and errors as gdpa_fwd; the result is the one
 *   gdpa_fwd computes with the same plan layout.
 *
 * A plan whose forward list (records, bin pointers, chunk groups and slots) needs
 * more than the 32 MiB is rejected with INVALID_ARG before anything is enqueued.
 * Every call on one GPU shares that GPU's array and overwrites it, so calls that
 * overlap in time on one GPU (e.g. on two streams) race; calls on one stream are
 * ordered.  Nothing in the array needs to start at zero.
 */
gdpa_status gdpa_fwd_noalloc(gdpa_plan plan, const void* q, const void* k, const void* v,
                             const int32_t* q_off_dev, const int32_t* kv_off_dev, int B, int H, int d,
                             gdpa_act act, int window, void* o, void* stream);

/*
 * gdpa_bwd - gradients of sum(O * dO): dQ [Tq,H,d], dK and dV [Tk,H,d].
 *
 * dS = (dO V^T) * act'(S) on valid pairs; dV = P^T dO, dK = dS^T Q / sqrt(d),
 * dQ = dS K / sqrt(d).  S is recomputed; O is not needed.  Arguments as for
 * gdpa_fwd plus dout [Tq,H,d] (input) and dq, dk, dv (outputs, fully written;
 * rows with no valid partner are 0).  act = GDPA_ACT_ONE is rejected
 * (UNSUPPORTED).  Enqueues up to two kernels on `stream`: one KV-stationary pass
 * when every sample has at most 32 keys (and no sample has queries but no keys),
 * else one Q-stationary pass when every sample has at most 32 queries (and none
 * has keys but no queries), else a KV-stationary dK/dV kernel and a
 * Q-stationary dQ kernel (always, with opts->unfused).
 */
gdpa_status gdpa_bwd(gdpa_plan plan, const void* q, const void* k, const void* v, const void* dout,
                     const int32_t* q_off_dev, const int32_t* kv_off_dev, int B, int H, int d,
                     gdpa_act act, int window, void* dq, void* dk, void* dv, void* stream);

/*
 * gdpa_bwd_dkdv - only dK and dV (one KV-stationary kernel); same arguments and
 * errors as gdpa_bwd without dq.  For callers whose queries are frozen or who
 * schedule the two halves of the backward pass separately.  On a plan with a dS
 * buffer (gdpa_plan_stats: ds_bytes > 0) it also stores dS there, for
 * gdpa_bwd_dq.
 */
gdpa_status gdpa_bwd_dkdv(gdpa_plan plan, const void* q, const void* k, const void* v, const void* dout,
                          const int32_t* q_off_dev, const int32_t* kv_off_dev, int B, int H, int d,
                          gdpa_act act, int window, void* dk, void* dv, void* stream);

/*
 * gdpa_bwd_dq - only dQ (one Q-stationary kernel); same arguments and errors as
 * gdpa_bwd without dk and dv.  gdpa_bwd == gdpa_bwd_dkdv followed by gdpa_bwd_dq.
 * On a plan with a dS buffer it computes dQ from the dS that the last
 * gdpa_bwd_dkdv on this plan stored, so it must follow that call, on the same
 * inputs and ordered after it; a caller that needs dQ alone creates the plan with
 * opts->no_ds (the kernel then recomputes dS).
 */
gdpa_status gdpa_bwd_dq(gdpa_plan plan, const void* q, const void* k, const void* v, const void* dout,
                        const int32_t* q_off_dev, const int32_t* kv_off_dev, int B, int H, int d,
                        gdpa_act act, int window, void* dq, void* stream);

/*
 * gdpa_jfa_fwd - jagged softmax attention (JFA) on a GDPA plan: over the same valid
 * pairs, P_ij = exp(S_ij - LSE_i) with LSE_i = log sum_j exp(S_ij) over row i's valid
 * keys, O = P V (the softmax's row max, row sum and rescale that GDPA drops; GDPA
 * page, "Section details"; GEM page on jagged attention kernels).  Arguments as
 * gdpa_fwd without act, plus
 *   lse : device fp32 [H, Tq] (head-major), written: LSE of each row, -inf for rows
 *         with no valid key (their O rows are 0).
 * The plan must be bf16 (UNSUPPORTED otherwise).  A cut forward item's chunks
 * store unnormalised partial rows with their running max and sum; a combine
 * kernel rescales them to the common max and divides by the total sum (in slot
 * order, so the result does not depend on scheduling).  Errors as gdpa_fwd.
 */
gdpa_status gdpa_jfa_fwd(gdpa_plan plan, const void* q, const void* k, const void* v, const int32_t* q_off_dev,
                         const int32_t* kv_off_dev, int B, int H, int d, int window, void* o, float* lse,
                         void* stream);

/*
 * gdpa_jfa_bwd - gradients of sum(O * dO) for gdpa_jfa_fwd: with the forward's
 * O and LSE, P_ij = exp(S_ij - LSE_i) on the valid pairs, D_i = sum_c dO_ic O_ic,
 * dS = P * (dO V^T - D_i) (the softmax Jacobian; GEM page on jagged attention
 * kernels, backward of the fused attention), dV = P^T dO, dK = dS^T Q / sqrt(d),
 * dQ = dS K / sqrt(d).  Arguments as gdpa_bwd without act, plus
 *   o, lse : the forward's outputs (bf16 [Tq,H,d]; fp32 [H,Tq]), read;
 *   stat   : device fp32 [H, Tq, 2], caller-owned scratch, written: per (head, q
 *            row) the pair (LSE_i log2(e), D_i).
 * Enqueues the Q-stationary dQ kernel, which also forms D from O and dO and writes
 * stat, then the KV-stationary dK/dV kernel, which reads stat, plus the chunk
 * reductions of cut items.  On a plan whose every sample has Lk <= 32
 * (gdpa_plan_stats: bwd_fused = 1) it runs one KV-stationary pass instead: all keys
 * of a query tile are in one step there, so D_i = sum_j P_ij dP_ij (which equals
 * sum_c dO_ic O_ic for the exact O) is formed in the pass from P and dP; O and stat
 * are neither read nor written (both may be NULL).  The plan must be GDPA_BF16
 * (O is read as bf16; a GDPA_BF16_F32OUT plan, whose gdpa_jfa_fwd writes fp32 O,
 * and an F32 plan are rejected with UNSUPPORTED) with one-wave dQ and dK/dV teams
 * (the automatic layouts; UNSUPPORTED otherwise).
 * Errors as gdpa_bwd.  On the other plans gdpa_jfa_bwd == gdpa_jfa_bwd_dq, then
 * gdpa_jfa_bwd_dkdv (the parts always run the two kernels).
 */
gdpa_status gdpa_jfa_bwd(gdpa_plan plan, const void* q, const void* k, const void* v, const void* o,
                         const float* lse, const void* dout, const int32_t* q_off_dev, const int32_t* kv_off_dev,
                         int B, int H, int d, int window, float* stat, void* dq, void* dk, void* dv, void* stream);

/*
 * The parts of gdpa_jfa_bwd, for callers who schedule them separately:
 *   gdpa_jfa_bwd_dq   - dQ, and stat written from o, lse and dout;
 *   gdpa_jfa_bwd_dkdv - dK, dV, reading a stat written for the same o, lse, dout
 *                       (by gdpa_jfa_bwd_dq or gdpa_jfa_bwd_stat);
 *   gdpa_jfa_bwd_stat - only stat, from o, lse and dout (one pass over O and dO;
 *                       H and d must match the plan), so that dK/dV can run first.
 * Arguments and errors as gdpa_jfa_bwd.
 */
gdpa_status gdpa_jfa_bwd_dq(gdpa_plan plan, const void* q, const void* k, const void* v, const void* o,
                            const float* lse, const void* dout, const int32_t* q_off_dev, const int32_t* kv_off_dev,
                            int B, int H, int d, int window, float* stat, void* dq, void* stream);
gdpa_status gdpa_jfa_bwd_dkdv(gdpa_plan plan, const void* q, const void* k, const void* v, const void* dout,
                              const int32_t* q_off_dev, const int32_t* kv_off_dev, int B, int H, int d, int window,
                              const float* stat, void* dk, void* dv, void* stream);
gdpa_status gdpa_jfa_bwd_stat(gdpa_plan plan, const void* o, const float* lse, const void* dout, int H, int d,
                              float* stat, void* stream);

/*
 * GDPA with a fused RMSNorm prologue: the inputs named by `norm` (a combination of
 * 1 = Q, 2 = K, 4 = V) go through a per-(token, head) RMSNorm over d,
 * x^ = x / sqrt(mean(x^2) + 1e-6) with no gain, before the attention (GDPA page,
 * "Section details", chart of tanh GELU against the 6th-order series: RMSNorm keeps
 * the activation's inputs in range).  The kernels read the raw tensors and scale by
 * each row's 1/rms, so no normalised copy is written, and the backward returns the
 * gradients of the RAW inputs, dx = r (dx^ - x^ mean(dx^ x^)) for a normalised
 * input (dx^ otherwise).  bf16 plans only; act = GDPA_ACT_ONE is rejected
 * (UNSUPPORTED).
 *
 *   gdpa_norm_rstd - the pre-pass: writes rstd, device fp32 scratch of
 *                    H * (Tq + 2 Tk) floats: [H, Tq] (1/rms of Q's rows), then
 *                    [H, Tk, 2] (1/rms of K's and V's rows as pairs); 1 for a
 *                    tensor not in `norm`.  H and d must match the plan.
 *   gdpa_norm_fwd  - O [Tq,H,d] from raw q, k, v and the rstd that gdpa_norm_rstd
 *                    wrote for the same q, k, v and norm (read-only here);
 *                    arguments otherwise as gdpa_fwd.
 *   gdpa_norm_bwd  - raw-input gradients dq, dk, dv (arguments as gdpa_bwd plus
 *                    norm and that rstd): the dK/dV kernel, then the dQ kernel
 *                    (never the one-pass kernels), plus chunk reductions;
 *                    == gdpa_norm_bwd_dkdv followed by gdpa_norm_bwd_dq.
 * Errors as gdpa_fwd / gdpa_bwd; norm outside 0..7 or a NULL rstd: INVALID_ARG.
 */
gdpa_status gdpa_norm_rstd(gdpa_plan plan, const void* q, const void* k, const void* v, int H, int d, int norm,
                           float* rstd, void* stream);
gdpa_status gdpa_norm_fwd(gdpa_plan plan, const void* q, const void* k, const void* v, const int32_t* q_off_dev,
                          const int32_t* kv_off_dev, int B, int H, int d, gdpa_act act, int window, int norm,
                          const float* rstd, void* o, void* stream);
gdpa_status gdpa_norm_bwd(gdpa_plan plan, const void* q, const void* k, const void* v, const void* dout,
                          const int32_t* q_off_dev, const int32_t* kv_off_dev, int B, int H, int d, gdpa_act act,
                          int window, int norm, const float* rstd, void* dq, void* dk, void* dv, void* stream);
gdpa_status gdpa_norm_bwd_dkdv(gdpa_plan plan, const void* q, const void* k, const void* v, const void* dout,
                               const int32_t* q_off_dev, const int32_t* kv_off_dev, int B, int H, int d,
                               gdpa_act act, int window, int norm, const float* rstd, void* dk, void* dv,
                               void* stream);
gdpa_status gdpa_norm_bwd_dq(gdpa_plan plan, const void* q, const void* k, const void* v, const void* dout,
                             const int32_t* q_off_dev, const int32_t* kv_off_dev, int B, int H, int d, gdpa_act act,
                             int window, int norm, const float* rstd, void* dq, void* stream);

/*
 * gdpa_fp8_fwd - GDPA forward with 8-bit Q and K (GEM page, section on the custom
 * kernels and precision: mixed ultra-low precision, MXFP8 among it, for attention,
 * with the precision chosen per operation).  q8 [Tq,H,d] and
 * k8 [Tk,H,d] are OCP FP8 E4M3 bytes (the e4m3fn encoding: bias 7, max 448, no
 * infinities) standing for q8 * q_scale and k8 * k_scale; S = (q8 . k8) q_scale
 * k_scale / sqrt(d) is computed by the fp8 MFMA with fp32 accumulation.  V is
 * bf16, P is rounded to bf16 for the second product, O is bf16 (fp32 for a
 * GDPA_BF16_F32OUT plan).  Arguments otherwise as gdpa_fwd; q_scale and k_scale
 * finite and > 0 (INVALID_ARG otherwise).  bf16 plans only; act = GDPA_ACT_ONE is
 * rejected (UNSUPPORTED).  The gradients: gdpa_bwd on bf16 inputs, or
 * gdpa_fp8_bwd on fp8 ones.
 */
gdpa_status gdpa_fp8_fwd(gdpa_plan plan, const void* q8, const void* k8, const void* v, const int32_t* q_off_dev,
                         const int32_t* kv_off_dev, int B, int H, int d, gdpa_act act, int window, float q_scale,
                         float k_scale, void* o, void* stream);

/*
 * gdpa_fp8_bwd - GDPA backward with 8-bit Q, K and dO (GEM page, section on the
 * custom kernels and precision: mixed ultra-low precision for attention, the
 * precision chosen per operation).  q8, dout8 [Tq,H,d] and k8 [Tk,H,d] are OCP FP8
 * E4M3 bytes (e4m3fn) standing for q8 * q_scale, dout8 * do_scale and
 * k8 * k_scale; v [Tk,H,d] is bf16, as in gdpa_fp8_fwd.  S = (q8 . k8) q_scale
 * k_scale / sqrt(d) runs on the fp8 MFMA with fp32 accumulation, dP = (dout8 . v)
 * do_scale on the bf16 MFMA with dout8 widened to bf16 (exactly: every e4m3
 * value is a bf16 value); P = act(S) and dS = dP act'(S) in fp32, rounded to bf16
 * as operands of dV = P^T dout, dK = dS^T q / sqrt(d) and dQ = dS k / sqrt(d),
 * whose fp8 operand is widened the same way; each gradient takes its input's
 * factor and is stored as bf16 (fp32 for a GDPA_BF16_F32OUT plan), as gdpa_bwd
 * stores them.  Runs on plans whose backward is one pass (gdpa_plan_stats.bwd_fused
 * = 1 or 2: every Lk <= 32 or every Lq <= 32) or, at d = 128, the dK/dV kernel
 * storing dS followed by dQ from the stored blocks (gdpa_plan_stats.ds_bytes > 0);
 * UNSUPPORTED otherwise.  bf16 plans only; act = GDPA_ACT_ONE UNSUPPORTED; factors
 * finite and > 0 (INVALID_ARG otherwise).  Arguments otherwise as gdpa_bwd.
 */
gdpa_status gdpa_fp8_bwd(gdpa_plan plan, const void* q8, const void* k8, const void* v, const void* dout8,
                         const int32_t* q_off_dev, const int32_t* kv_off_dev, int B, int H, int d, gdpa_act act,
                         int window, float q_scale, float k_scale, float do_scale, void* dq, void* dk, void* dv,
                         void* stream);

/*
 * gdpa_mx_fwd - GDPA forward with block-scaled fp8 Q and K (OCP microscaling, MXFP8:
 * the GEM page's section on custom kernels and precision names MXFP8 for attention).
 * q8 [Tq,H,d] and k8 [Tk,H,d] are OCP FP8 E4M3 bytes (e4m3fn); q_scale [H,Tq,d/32]
 * and k_scale [H,Tk,d/32] (head-major: the rows of one head consecutive) are E8M0
 * bytes, one per 32 consecutive head columns of a row, each standing for 2^(byte -
 * 127) (255 is NaN).  The element at column c of a row stands for its e4m3 value
 * times its block's scale; S = (q . k) / sqrt(d) is computed on gfx950's scaled
 * MFMA (32 x 32 x 64, the scales applied in hardware, fp32 accumulation).  V is
 * bf16, P is rounded to bf16 for the second product, O is bf16 (fp32 for a
 * GDPA_BF16_F32OUT plan).  Arguments otherwise as gdpa_fwd.  bf16 plans with
 * d = 64 or 128 only (UNSUPPORTED otherwise, and for act = GDPA_ACT_ONE); the
 * gradients run on bf16 inputs (gdpa_bwd).
 */
gdpa_status gdpa_mx_fwd(gdpa_plan plan, const void* q8, const void* q_scale, const void* k8, const void* k_scale,
                        const void* v, const int32_t* q_off_dev, const int32_t* kv_off_dev, int B, int H, int d,
                        gdpa_act act, int window, void* o, void* stream);

/*
 * pFFN as GDPA (GDPA page, "Section details", diagram of self-attention, PMA and
 * pFFN unified as GDPA).  The page gives no formula; read here as: per head,
 * weight matrices W_K, W_V [M, H, d] shared by every query row of the batch,
 *     O_i = sum_{j < M} act(Q_i . W_K,j / sqrt(d)) W_V,j,
 * with the weight gradients dW_K, dW_V summed over all Tq query rows.  Samples do
 * not interact, so this is GDPA on one sample of Tq queries and M keys; the
 * planner's chunks spread the weight-gradient reduction over the device.
 *
 * gdpa_pffn_plan_create - a plan for Tq >= 0 query rows and M >= 0 weight rows
 *   (H, d, dtype, opts, stream as for gdpa_plan_create).  Also keeps device copies
 *   of the offsets, so the pFFN calls take none.  Errors as gdpa_plan_create.
 * gdpa_pffn_fwd - O [Tq, H, d] from q [Tq, H, d], wk, wv [M, H, d]; act as gdpa_fwd.
 * gdpa_pffn_bwd - dQ [Tq, H, d], dW_K and dW_V [M, H, d] for the loss sum(O * dO).
 *   Both: device pointers in the plan's dtype; errors as gdpa_fwd / gdpa_bwd, and
 *   PLAN_MISMATCH for a plan not made by gdpa_pffn_plan_create.
 */
gdpa_status gdpa_pffn_plan_create(int Tq, int M, int H, int d, gdpa_dtype dtype, const gdpa_plan_opts* opts,
                                  void* stream, gdpa_plan* out);
gdpa_status gdpa_pffn_fwd(gdpa_plan plan, const void* q, const void* wk, const void* wv, gdpa_act act, void* o,
                          void* stream);
gdpa_status gdpa_pffn_bwd(gdpa_plan plan, const void* q, const void* wk, const void* wv, const void* dout,
                          gdpa_act act, void* dq, void* dwk, void* dwv, void* stream);

/*
 * gdpa_plan_export - serialise one work list as int32 values:
 *   [P, n_items, tile_stat, tile_strm, team, blocks, bin_ptr[0..P], then per item in
 *    bin order (b, h, t, s0, s1, part)]
 * where t is the stationary tile, [s0, s1] the streaming tiles (s1 < s0: no
 * steps, the item writes zeros) and part the chunk's partial-output slot (-1 for
 * an item that stores its outputs itself).  With buf == NULL, *n receives the length;
 * otherwise *n is the capacity of buf on entry and the length on return.
 * Errors: INVALID_ARG (bad list, list 3 on a plan without it, or capacity too small).
 */
gdpa_status gdpa_plan_export(gdpa_plan plan, int list, int32_t* buf, size_t* n);

/* gdpa_plan_stats - summary numbers of a plan.  Errors: INVALID_ARG. */
gdpa_status gdpa_plan_stats(gdpa_plan plan, gdpa_plan_stats_t* out);

/* gdpa_plan_destroy - free a plan (NULL is ignored).  The caller must make sure
 * no enqueued work still uses it. */
void gdpa_plan_destroy(gdpa_plan plan);

/* gdpa_status_string - static name of a status code. */
const char* gdpa_status_string(gdpa_status s);

/* gdpa_last_error - thread-local description of the last failure ("" if none). */
const char* gdpa_last_error(void);

/* gdpa_gelu_poly_bound - max |GELU_POLY(x) - x Phi(x)| over all real x, as
 * derived when the polynomial was fitted (the larger of the fp64 and the
 * device-order fp32 evaluations, and the tail beyond the clamp). */
double gdpa_gelu_poly_bound(void);

/* gdpa_gelu_poly_grad_bound - the same for the derivative the backward kernels
 * use, max |GELU_POLY'(x) - (Phi(x) + x phi(x))|; the derivative has its own
 * polynomial, fitted to GELU' directly. */
double gdpa_gelu_poly_grad_bound(void);

#ifdef __cplusplus
}
#endif

#endif /* GDPA_H */
