/*
 * zb.h -- C ABI of the split-backward pipeline stage library (libzb.so) for
 * AMD Instinct MI355X (gfx950).
 *
 * One pipeline stage of a transformer, with the backward pass split in two
 * (the split is the subject of "Zero-Bubble Pipeline Parallelism Guide for
 * LLMs", section "Core Innovation 1: Mathematical Decomposition of the
 * Backward Pass", and of the arXiv abstract page "Zero Bubble Pipeline
 * Parallelism"):
 *
 *   F : Y  = X . W^T                  (forward; stashes what B and W need)
 *   B : dX = dY . W  (+ activation backward)   critical path, sent upstream
 *   W : dW += dY^T . X  (fp32, in place)       local, deferrable
 *
 * The stage API mirrors the Guide's "Step-by-Step Implementation" listing
 * (forward_microbatch / backward_input_bx / backward_weight_bw); the schedule
 * generator follows the Guide's scheduler listing and "Core Innovation 2".
 *
 * Conventions for every call below
 * --------------------------------
 * - Pointers named "device" point to HIP device memory the CALLER owns and
 *   keeps alive for as long as the library may touch it (weights, dW,
 *   workspace: until zb_stage_destroy; x/y/dx/dy: until the stream work of
 *   the call has finished).  The library allocates no device memory.
 * - Weights are stored [out, in], row-major (PyTorch's linear layout); the
 *   Guide's Y = X.W uses W_eq = W^T.  Activations are [tokens, features],
 *   row-major, contiguous.  bf16 is IEEE bfloat16 bit patterns.
 * - "stream" is a hipStream_t passed as void* (NULL = the null stream).
 *   Compute calls only enqueue work and return; errors that are known when
 *   the call is made are returned at once and nothing is enqueued.
 *   Device-side failures surface as ZB_EHIP from a later call.
 * - zb_last_error() returns a thread-local message for the last failure.
 * - A zb_stage is not thread safe: issue its calls from one host thread.
 */
#ifndef ZB_H_
#define ZB_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct zb_stage zb_stage;

enum {
    ZB_OK = 0,
    ZB_EINVAL = -1,        /* bad argument or unsupported shape              */
    ZB_ESTATE = -2,        /* op out of order for this microbatch            */
    ZB_ERING_FULL = -3,    /* F would exceed the stash ring (memory limit)   */
    ZB_EHIP = -4,          /* a HIP runtime call failed                      */
    ZB_ENOMEM = -5         /* workspace smaller than zb_stage_workspace_bytes */
};

/* Element types.  A stage's dtype is ZB_F32, ZB_BF16 or ZB_FP8; ZB_E4M3 and
 * ZB_I32 only describe stashed tensors (zb_stage_stash_tensor).
 *  ZB_FP8  (ZB_LLAMA only) bf16 weights, activations and gradients at the
 *          boundary, fp32 dW; every linear product of F, B and W runs on
 *          E4M3 operands (OCP 8-bit float, 3 mantissa bits) with one
 *          power-of-two scale per tensor, 2^e with e the smallest integer such
 *          that max|x| <= 448 * 2^e, values rounded to nearest even, fp32
 *          accumulation ("The Ghost in the Machine ...", "Memory Pressure":
 *          FP8 halves buffers and makes room for the deferred-W stash).  The
 *          stash keeps the W-only operands as E4M3 codes, transposed so
 *          that every product has a K-contiguous operand pair.  hidden and
 *          ffn must be multiples of 128. */
enum { ZB_F32 = 0, ZB_BF16 = 1, ZB_FP8 = 2, ZB_E4M3 = 3, ZB_I32 = 4 };

/* Stage kinds.
 *  ZB_LINEAR   one layer Y = X W^T; in = hidden, out = ffn.  Weight list: {W[ffn,hidden]}.
 *  ZB_MLP_GELU fc1 -> GeLU(tanh) -> fc2, no bias.  Weights {W1[ffn,hidden], W2[hidden,ffn]}.
 *  ZB_LLAMA    n_layers pre-norm decoder layers: RMSNorm, causal GQA
 *              attention (no RoPE), residual, RMSNorm, SwiGLU MLP, residual.
 *              tokens must be a multiple of 128 (the attention kernels'
 *              query and key blocks), head_dim 128, hidden <= 8192.
 *              Weights per layer l, in this order:
 *                Wqkv[(n_heads+2*n_kv_heads)*head_dim, hidden] (rows: q | k | v),
 *                Wo[hidden, n_heads*head_dim], Wgu[2*ffn, hidden] (rows: gate | up),
 *                Wd[hidden, ffn], g1[hidden], g2[hidden] (RMSNorm gains). */
enum { ZB_LINEAR = 0, ZB_MLP_GELU = 1, ZB_LLAMA = 2 };

typedef struct {
    int32_t kind;        /* ZB_LINEAR / ZB_MLP_GELU / ZB_LLAMA                    */
    int32_t dtype;       /* ZB_F32 (ZB_LINEAR only), ZB_BF16, ZB_FP8 (ZB_LLAMA only) */
    int32_t n_layers;    /* ZB_LLAMA: decoder layers; otherwise 1                  */
    int32_t tokens;      /* T = batch * sequence length of one microbatch          */
    int32_t hidden;      /* model width h                                         */
    int32_t ffn;         /* MLP width (ZB_LINEAR: output width)                   */
    int32_t n_heads;     /* ZB_LLAMA: query heads                                  */
    int32_t n_kv_heads;  /* ZB_LLAMA: key/value heads; n_heads % n_kv_heads == 0    */
    int32_t head_dim;    /* ZB_LLAMA: must be 128                                  */
    float rms_eps;       /* ZB_LLAMA: RMSNorm epsilon (inside the square root)     */
    int32_t ring_slots;  /* R: microbatches whose activations may be stashed at once */
} zb_stage_desc;

/* Number of weight tensors of a stage (and of dW buffers): 1, 2 or 6*n_layers. */
int32_t zb_stage_num_weights(const zb_stage_desc* desc);

/* Bytes of device workspace zb_stage_create needs: the stash ring
 * (ring_slots slots) plus per-pass scratch.  The B scratch of a Llama stage
 * includes the attention backward's dS^T, n_heads * tokens^2 bf16 values
 * (1.07 GB at 32 heads and 4096 tokens); GPT-MLP stages add fp32 split-K
 * partial sums to the F and B scratch.  Returns 0 for an invalid desc
 * (zb_last_error says why). */
size_t zb_stage_workspace_bytes(const zb_stage_desc* desc);

/* Create a stage.  weights[i] / dw[i] are device pointers in the weight order
 * of the kind (see above); weights are ZB_BF16 (or ZB_F32 for an fp32 linear
 * stage), dw buffers are always fp32 of the same shape.  workspace is device
 * memory of at least zb_stage_workspace_bytes(desc) bytes, 256-byte aligned.
 * The library keeps the pointers (not copies).  dW is NOT cleared: call
 * zb_stage_zero_grad before the first W of an iteration.
 * Errors: ZB_EINVAL (desc/shape), ZB_ENOMEM (ws_bytes too small), ZB_EHIP. */
int32_t zb_stage_create(const zb_stage_desc* desc, void* const* weights, float* const* dw,
                        void* workspace, size_t ws_bytes, zb_stage** out);

/* Release host state (events).  Waits for no device work: synchronize the
 * streams first.  NULL is accepted. */
void zb_stage_destroy(zb_stage* st);

/* F for microbatch mb (Guide listing: forward_microbatch).  x: device [T, hidden]
 * (caller's, read during the call's stream work), y: device [T, out]
 * (out = hidden, or ffn for ZB_LINEAR).  Stashes into ring slot mb % R
 * everything B and W need (a copy of x included).
 * Errors: ZB_EINVAL (mb < 0, NULL pointers); ZB_ESTATE (F(mb) already issued
 * or mb not the next in ascending order); ZB_ERING_FULL (slot mb % R still
 * holds a microbatch whose W has not been issued -- the memory ceiling of
 * the Guide's "Memory Management & Activation Rollback").  If the slot's
 * previous W was issued on another stream, F waits for it on the device. */
int32_t zb_fwd(zb_stage* st, int32_t mb, const void* x, void* y, void* stream);

/* B for microbatch mb (Guide listing: backward_input_bx).  dy: device
 * [T, out] output gradient, dx: device [T, hidden] input gradient.  Fuses the
 * activation backward (GeLU / SwiGLU) and, for ZB_LLAMA, RMSNorm and
 * attention backward.  Stashes the output gradients W needs.
 * Errors: ZB_ESTATE unless F(mb) was issued and B(mb) was not. */
int32_t zb_bwd_input(zb_stage* st, int32_t mb, const void* dy, void* dx, void* stream);

/* W for microbatch mb (Guide listing: backward_weight_bw):
 * dW[i] += (this microbatch's weight gradient), fp32, deterministic (no
 * atomics; calls add in issue order).  Frees ring slot mb % R once the
 * device work has completed.  W must be issued in ascending mb order.
 * Errors: ZB_ESTATE unless B(mb) was issued and W(mb) was not, or mb is not
 * the next W in ascending order. */
int32_t zb_bwd_weight_accum(zb_stage* st, int32_t mb, void* stream);

/* zb_bwd_weight_accum for callers that cannot allocate memory (code under
 * HIP graph capture, tight loops, harnesses that forbid allocation): the
 * same work, state rules, errors and bit-identical results, with the W pass's
 * only scratch (the fp32 RMSNorm dgamma partials: ceil(tokens / 64) * hidden
 * floats, Llama stages only) in a fixed device array of
 * ZB_NOALLOC_SCRATCH_BYTES inside the library instead of the stage's
 * workspace.  Each GPU holds its own copy of that array until the process
 * ends; it is looked up on the first call on a device.  Calls no allocating
 * routine.  All calls on one GPU share the array: calls that may overlap in
 * time on one GPU (other stages, other streams without ordering between
 * them) race and must be serialized by the caller.
 * Errors: as zb_bwd_weight_accum, plus ZB_EINVAL when the stage needs more
 * scratch than ZB_NOALLOC_SCRATCH_BYTES or the stage's device is not the
 * current one. */
#define ZB_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
int32_t zb_bwd_weight_accum_noalloc(zb_stage* st, int32_t mb, void* stream);

/* W for microbatches mb and mb + 1 in one pass.  The weight-gradient pass is
 * deferrable and needs only the stashed activations and output gradients
 * (Guide, "Core Innovation 1": the weight gradient does not feed any other
 * computation), so two ready microbatches may be combined: each product runs
 * once with K spanning both microbatches' tokens, and dW is read and written
 * once for the pair instead of twice.  Mathematically equal to
 * zb_bwd_weight_accum(mb) then zb_bwd_weight_accum(mb + 1); the fp32
 * rounding differs (the two microbatches' contributions are summed before
 * they are added to dW), within 1e-5 relative.  RMSNorm dgamma is reduced per
 * microbatch exactly as by two W calls.  Frees both ring slots once the
 * device work has completed.  Stages whose products cannot take the
 * two-segment kernel (fp32 linear stages, tokens not a multiple of 32) run
 * it as the two single calls.
 * Errors: ZB_ESTATE unless B was issued and W was not for both microbatches,
 * or mb is not the next W in ascending order. */
int32_t zb_bwd_weight_accum_pair(zb_stage* st, int32_t mb, void* stream);

/* Set every dW buffer to 0 (a fill kernel on stream) and reset the
 * microbatch counters for a new iteration.  Errors: ZB_ESTATE if a
 * microbatch is still in flight (F issued, W not). */
int32_t zb_stage_zero_grad(zb_stage* st, void* stream);

/* Device pointer of a stashed tensor, for inspection by tests: ring slot of
 * microbatch mb, decoder layer (0 for the other kinds), tensor index
 * (kind-specific, see the library's stash table).  Writes rows/cols/dtype.
 * Valid between F(mb) (or B(mb) for gradients) and W(mb). */
int32_t zb_stage_stash_tensor(zb_stage* st, int32_t mb, int32_t layer, int32_t which,
                              void** ptr, int32_t* rows, int32_t* cols, int32_t* dtype);

/* Device pointers of the E4M3 copies of linear weight i of a ZB_FP8 stage
 * (for inspection by tests): q [out][in] (used by F), qt [in][out] (used by
 * B), and e, the int32 exponent of their common scale.  They are refreshed
 * by the first F after zb_stage_create or zb_stage_sgd_step.  ZB_EINVAL for
 * another dtype or an index that is not a linear weight. */
int32_t zb_stage_fp8_weight(zb_stage* st, int32_t i, void** q, void** qt, void** e);

/* Optimizer step of the stage, closing an iteration (the op ZB_OP_O of
 * zb_schedule_generate_iters): for every weight, w -= lr * dW elementwise
 * (fp32 product and difference, each rounded once, then rounded once to the
 * weight's type, round to nearest even), after every issued W has completed
 * on the device; then dW is cleared and the stage is reset for a new
 * iteration as by zb_stage_zero_grad.  The next F, on whatever stream it is
 * issued, waits for the step on the device.  A plain SGD step: the pages name an
 * optimizer step per iteration but no optimizer.  lr must be finite.
 * Errors: ZB_EINVAL, ZB_ESTATE if a microbatch is in flight (its W not
 * issued). */
int32_t zb_stage_sgd_step(zb_stage* st, float lr, void* stream);

/* The stage keeps copies of its linear weights that its passes read instead
 * of the caller's: E4M3 codes in a ZB_FP8 stage (refreshed by its first F),
 * transposed bf16 copies [in][out] in a bf16 ZB_LLAMA stage (refreshed by its
 * first B; the B pass multiplies by them so that its products have both
 * operands K-contiguous).  They are refreshed after zb_stage_create and
 * zb_stage_sgd_step; a caller that writes the weights itself calls this
 * before the next F and B.  ZB_EINVAL for a NULL stage. */
int32_t zb_stage_weights_changed(zb_stage* st);

/* Learning rate of the optimizer steps zb_stage_run_schedule issues for
 * ZB_OP_O ops (default 0: the weights are left unchanged).  ZB_EINVAL if lr
 * is not finite. */
int32_t zb_stage_set_lr(zb_stage* st, float lr);

/* Debug aids.  The pages define none; they check the ring discipline the
 * split relies on (the Guide's "Memory Management & Activation Rollback": a
 * microbatch's stash is freed only once its W has run, so a slot is reused
 * only after that W).  The host already enforces that order when calls are
 * issued (ZB_ESTATE, ZB_ERING_FULL); these check it where the work runs.
 *  ZB_DEBUG_SLOT_TAGS  every pass checks, on the device and in stream order
 *                      with its kernels, the tag of its microbatch's ring
 *                      slot, then updates it: tag = 4 mb + 1 after F(mb),
 *                      + 2 after B(mb), + 3 after W(mb), -1 unused.  F needs
 *                      an unused slot or one whose W is done, B(mb) needs
 *                      4 mb + 1, W(mb) needs 4 mb + 2.  A mismatch is
 *                      counted and recorded (zb_stage_debug_report); nothing
 *                      traps.  Enabling the flag resets every tag to unused
 *                      (after the stage's issued work), so microbatches in
 *                      flight at that moment report at their next pass.
 *  ZB_DEBUG_SERIALIZE  every op (F, B, W, W pair, optimizer step) ends with
 *                      hipDeviceSynchronize; a device fault is then reported
 *                      (ZB_EHIP) by the op that caused it.  Timing figures of
 *                      zb_stage_run_schedule are meaningless in this mode.
 * w_delay_us (0 .. 1000000): each W pass (single or pair) first waits that
 * long on its stream (a device-clock wait kernel), to test that nothing
 * overwrites a slot before a slow W has read it.  ZB_EINVAL for an unknown
 * flag or a delay out of range. */
enum { ZB_DEBUG_SLOT_TAGS = 1, ZB_DEBUG_SERIALIZE = 2 };
int32_t zb_stage_set_debug(zb_stage* st, int32_t flags, int32_t w_delay_us, void* stream);

/* Waits for the device, then returns the number of slot-tag mismatches
 * since the tags were enabled (>= 0) and, if info is non-NULL, writes the
 * last one: info[0..4] = {op type (ZB_OP_F/B/W), mb, slot, tag found, tag
 * expected (-2: unused or W done)}.  ZB_ESTATE if slot tags are not
 * enabled. */
int32_t zb_stage_debug_report(zb_stage* st, int32_t* info);

/* ------------------------------------------------------------ schedules -- */

/* Op of a per-stage schedule (the Guide scheduler listing's task types). */
enum { ZB_OP_F = 0, ZB_OP_B = 1, ZB_OP_W = 2,
       ZB_OP_O = 3 /* optimizer step closing an iteration (zb_schedule_generate_iters) */ };
typedef struct { int32_t type; int32_t mb; } zb_op;

/* Schedule kinds: GPipe and 1F1B with the backward kept whole (each B is
 * followed at once by its W), and the memory-limited zero-bubble greedy. */
enum { ZB_SCHED_GPIPE = 0, ZB_SCHED_1F1B = 1, ZB_SCHED_ZB = 2 };

typedef struct {
    int64_t makespan;      /* pipeline makespan (all stages), cost units   */
    int64_t busy;          /* this stage's busy time                       */
    int64_t first_start;   /* this stage's first op start                  */
    int64_t last_end;      /* this stage's last op end                     */
    int32_t peak_active;   /* most microbatches stashed at once            */
    int32_t n_ops;         /* 3 * m                                        */
} zb_sched_stats;

/* Generate stage `stage`'s op order for a p-stage, m-microbatch iteration by
 * integer-time simulation of the whole pipeline (no communication cost).
 *   GPIPE: all F, then all backwards ("1. The GPipe Bubble").
 *   1F1B : min(p-1-stage, m) warm-up F, then F/B pairs, then the remaining
 *          backwards ("2. The 1F1B Schedule").
 *   ZB   : at every completion time each idle stage takes the lowest ready
 *          B; else the lowest ready F if fewer than mem_limit microbatches
 *          are stashed; else the lowest ready W (which releases one); else
 *          waits ("Core Innovation 2" and the scheduler listing, without its
 *          unconditional-forward fallback, which would break the ceiling).
 * Costs cF, cB >= 1; cW >= 0 (>= 1 for ZB).  Host only, no GPU needed.
 * Outputs (each may be NULL): ops[3m], start[3m], end[3m] of this stage;
 * arrive_f[m] = end of F(stage-1, j) (0 on stage 0), arrive_b[m] = end of the
 * downstream backward of j (B for ZB, the whole backward otherwise; 0 on the
 * last stage); stats.  cap = capacity of ops/start/end.
 * Returns the number of ops (3m) or ZB_EINVAL (bad arguments, cap < 3m,
 * mem_limit too small to make progress). */
int32_t zb_schedule_generate(int32_t kind, int32_t p, int32_t m, int32_t mem_limit,
                             int32_t cF, int32_t cB, int32_t cW, int32_t stage,
                             zb_op* ops, int64_t* start, int64_t* end, int32_t cap,
                             int64_t* arrive_f, int64_t* arrive_b, zb_sched_stats* stats);

/* Several iterations back to back (kind ZB_SCHED_ZB or ZB_SCHED_1F1B).
 * Each stage closes iteration it with an optimizer step (op ZB_OP_O,
 * mb = it, cost c_opt >= 1) as soon as all of its own W of that iteration
 * have completed; its first F of iteration it+1 waits for that step and for
 * the upstream F, and for nothing else.  The abstract page "Zero Bubble
 * Pipeline Parallelism" says the method bypasses the optimizer step's
 * synchronizations; this is read as no barrier across stages.
 *   ZB  : a ready step is taken before any B, F or W; otherwise the rules of
 *         ZB above apply with the global microbatch index g = it * m + j.
 *   1F1B: each stage's 1F1B sequence of every iteration, the step after it.
 * F, B, W ops carry g.  Outputs as for zb_schedule_generate, with
 * 3 m n_iter + n_iter ops and arrivals indexed by g (arrive_f / arrive_b of
 * m * n_iter entries; arrive_b the downstream B for ZB, the downstream
 * whole backward for 1F1B).  Returns the number of ops or ZB_EINVAL. */
int32_t zb_schedule_generate_iters(int32_t kind, int32_t p, int32_t m, int32_t mem_limit, int32_t cF, int32_t cB,
                                   int32_t cW, int32_t c_opt, int32_t n_iter, int32_t stage,
                                   zb_op* ops, int64_t* start, int64_t* end, int32_t cap,
                                   int64_t* arrive_f, int64_t* arrive_b, zb_sched_stats* stats);

/* Op of a schedule over several model chunks per stage (interleaved 1F1B):
 * the op type, the chunk of this stage it runs on, the microbatch. */
typedef struct { int32_t type; int32_t chunk; int32_t mb; } zb_chunk_op;

/* Interleaved 1F1B, the virtual-stage variant of 1F1B that the Guide's
 * "2. The 1F1B Schedule" and its "Quantitative Comparison" table (v = 2)
 * compare against: each of the p stages holds v model chunks, chunk c of
 * stage i being virtual stage c*p + i of a v*p-stage pipeline, so a
 * microbatch's forward visits every stage v times.  The pages give no
 * algorithm; this is the published interleaved schedule (microbatches in
 * groups of p, chunk-major within a group), with (p-1-stage) + (v-1)p
 * warm-up forwards, the fewest that cannot deadlock, then (forward, whole
 * backward) pairs, then the remaining backwards; backwards stay whole (B then
 * W at once), as in 1F1B.  Costs are per chunk.  With v = 1 it is
 * ZB_SCHED_1F1B.  Its bubble over the makespan is (p-1)/(v m + p-1).
 * Outputs as for zb_schedule_generate, with 3 v m ops of type F, B, W
 * (ops, start, end: capacity cap >= 3 v m) and arrivals of v m entries
 * indexed [chunk * m + mb]: arrive_f = end of the forward of the previous
 * virtual stage (0 for virtual stage 0), arrive_b = end of the whole
 * backward of the next virtual stage (0 for the last).  stats->peak_active
 * counts chunk-microbatches stashed at once.  Host only.
 * Returns the number of ops or ZB_EINVAL (p, m, v < 1; v > 1 with m not a
 * multiple of p; bad costs or stage; cap too small). */
int32_t zb_schedule_generate_interleaved(int32_t p, int32_t m, int32_t v, int32_t cF, int32_t cB, int32_t cW,
                                         int32_t stage, zb_chunk_op* ops, int64_t* start, int64_t* end,
                                         int32_t cap, int64_t* arrive_f, int64_t* arrive_b, zb_sched_stats* stats);

/* ------------------------------------------------------------- executor -- */

enum {
    ZB_EXEC_ORDERED = 0,  /* ops start strictly in list order (W on lo_stream,
                             chained to its neighbours by events)            */
    ZB_EXEC_FILLER = 1    /* W runs on lo_stream as soon as its B is done,
                             alongside F/B on hi_stream                       */
};

typedef struct {
    double t_first_start_ms;  /* relative to the executor's time origin      */
    double t_last_end_ms;
    double window_ms;         /* t_last_end - t_first_start                   */
    double busy_ms;           /* union of op intervals                         */
    double in_window_idle;    /* (window - busy) / window                      */
    double wait_late_ms;      /* sum over waits of (wait end - deadline) > 0   */
} zb_run_stats;

/* Run one iteration of a stage schedule on the GPU (the "list of ops, then
 * run" shape of the Ghost page's conceptual scheduler).  ops[n] as produced
 * by zb_schedule_generate.  Before F(j) the high stream waits until
 * t0 + arrive_f[j] * unit_ms, before B(j) until t0 + arrive_b[j] * unit_ms,
 * where t0 is taken on the device when the run starts; the waits are timed
 * with the GPU's constant-rate wall clock and always end.  x[j], dy[j] are
 * the per-microbatch inputs, y[j], dx[j] the outputs (device, caller-owned).
 * Both streams must be default-priority HIP streams (NULL = create and
 * destroy private ones).  op_ms (may be NULL) receives 2*n doubles: start and
 * end of each op in ms since t0.  Blocks until the run has finished.
 * Several iterations (ops of zb_schedule_generate_iters): F, B, W ops carry
 * the global microbatch index g (into x, y, dy, dx and the arrivals, which
 * then have one entry per microbatch of every iteration); a ZB_OP_O op runs
 * zb_stage_sgd_step with the rate of zb_stage_set_lr on the high stream,
 * after every W issued before it, and the next F restarts the stage's own
 * numbering at 0.
 * Each op's start stamp is taken after its dependency waits (its pass's
 * previous op, its microbatch's previous op, the W that frees a reused ring
 * slot) and its arrival wait, so op intervals and the idle figure count only
 * time in which the op could run.
 * Errors: as the compute calls, plus ZB_EINVAL for a malformed op list (an
 * op type outside F, B, W, O, a negative index, or an op of an iteration an
 * optimizer step has already closed), a unit_ms that is not finite or < 0,
 * or an arrival more than 30 s (the wait kernel's cap) after the start, all
 * detected before any work is issued (the op list and the times are checked
 * before the stage pointer). */
int32_t zb_stage_run_schedule(zb_stage* st, const zb_op* ops, int32_t n,
                              const double* arrive_f, const double* arrive_b, double unit_ms,
                              const void* const* x, void* const* y,
                              const void* const* dy, void* const* dx,
                              void* hi_stream, void* lo_stream, int32_t mode,
                              zb_run_stats* stats, double* op_ms);

/* zb_stage_run_schedule for a stage made of v model chunks (interleaved
 * 1F1B, zb_schedule_generate_interleaved): chunks[c] is the zb_stage object
 * of chunk c (distinct objects, each with its own weights and stash ring),
 * ops[k].chunk selects the object an op runs on, and x, y, dy, dx and the
 * arrivals hold v * m entries indexed [chunk * m + mb] (the input of chunk
 * c comes from the previous virtual stage, emulated like any arrival).  An
 * optimizer-step op steps every chunk.  Timing, streams, modes, stamps,
 * stats and errors as for zb_stage_run_schedule, plus ZB_EINVAL for an op
 * whose chunk is outside [0, v) or whose microbatch is >= m, or a stage
 * object given twice. */
int32_t zb_run_schedule_chunks(zb_stage* const* chunks, int32_t v, const zb_chunk_op* ops, int32_t n, int32_t m,
                               const double* arrive_f, const double* arrive_b, double unit_ms,
                               const void* const* x, void* const* y, const void* const* dy, void* const* dx,
                               void* hi_stream, void* lo_stream, int32_t mode, zb_run_stats* stats, double* op_ms);

/* ------------------------------------------------------------- kernels --- */

/* One GEMM through the stage's kernels, for kernel-level tests and timing.
 *   C[M,N] (op)= opA(A)[M,K] . opB(B)[K,N]
 *   a_kmajor: 1 -> A[m*lda + k], 0 -> A[k*lda + m];
 *   b_kmajor: 1 -> B[n*ldb + k], 0 -> B[k*ldb + n];
 *   dtype ZB_BF16: A, B bf16; out_f32 = 0 -> C bf16 (C = acc),
 *                  out_f32 = 1 -> C fp32 and C += acc (the W-pass epilogue).
 *   dtype ZB_F32: A, B, C fp32; out_f32 must be 1; accumulate = C += acc, else C = acc.
 * M, N, K >= 1; bf16 needs K, and M (if a_kmajor == 0), N (if b_kmajor == 0),
 * and every leading dimension to be multiples of 8.  Errors: ZB_EINVAL. */
int32_t zb_gemm(int32_t dtype, int32_t M, int32_t N, int32_t K,
                const void* A, int64_t lda, int32_t a_kmajor,
                const void* B, int64_t ldb, int32_t b_kmajor,
                void* C, int64_t ldc, int32_t out_f32, int32_t accumulate, void* stream);

/* Per-tensor E4M3 quantization of a bf16 matrix x [rows, cols] (leading
 * dimension ld, elements) as the ZB_FP8 stage quantizes its operands:
 * *e_out (device int32) = the smallest e with max|x| <= 448 * 2^e (0 for an
 * all-zero x); the codes of x * 2^-e, rounded to nearest even, row-major
 * into q ([rows][ldq] bytes) and/or transposed into qt ([cols][ldqt]); q or
 * qt may be NULL.  part: device scratch of 512 floats.  rows, cols, ldq,
 * ldqt multiples of 16, ld of 8, pointers 16-byte aligned.  Errors:
 * ZB_EINVAL. */
int32_t zb_quantize_e4m3(const void* x, int32_t rows, int32_t cols, int64_t ld, void* q, int64_t ldq, void* qt,
                         int64_t ldqt, void* e_out, void* part, void* stream);

/* One fp8 product through the ZB_FP8 stage's kernel, for kernel tests:
 * C[M,N] (op)= (A . B^T) * 2^(*ea + *eb), A [M][lda], B [N][ldb] E4M3
 * codes (K contiguous in both), ea / eb device int32.  out_f32 = 0: C bf16
 * (C = result); out_f32 = 1: C fp32 and C += result.  K a multiple of 128,
 * lda, ldb multiples of 16.  Errors: ZB_EINVAL. */
int32_t zb_gemm_fp8(int32_t M, int32_t N, int32_t K, const void* A, int64_t lda, const void* ea, const void* B,
                    int64_t ldb, const void* eb, void* C, int64_t ldc, int32_t out_f32, void* stream);

/* The ZB_FP8 stage's W-pass launch for kernel timing and tests: for
 * i < count, C_i[M_i, N_i] (fp32) += (A_i . B_i^T) * 2^(*ea_i + *eb_i) with
 * E4M3 codes A_i [M_i][lda_i], B_i [N_i][ldb_i] (K contiguous), up to 16
 * products per launch; each product obeys zb_gemm_fp8's rules.  Errors:
 * ZB_EINVAL. */
int32_t zb_gemm_fp8_wgrad_group(int32_t count, const int32_t* M, const int32_t* N, const int32_t* K,
                                const void* const* A, const int64_t* lda, const void* const* ea,
                                const void* const* B, const int64_t* ldb, const void* const* eb,
                                void* const* C, const int64_t* ldc, void* stream);

/* A group of weight-gradient products in one launch ([Guide] "Core
 * Innovation 1": W is each layer's weight gradient, and the products of one
 * microbatch are independent of each other once B has run).  For i < count:
 *   C_i[M_i, N_i] (fp32) += opA_i(A_i)[M_i, K_i] . opB_i(B_i)[K_i, N_i]
 * with bf16 A_i, B_i, the same operand orientations (a_kmajor, b_kmajor, as
 * in zb_gemm) for every product, and host arrays of length count (1..256).
 * Each product obeys zb_gemm's rules; the C_i must not overlap.  Products
 * that do not fit the single-launch kernel run one launch each.  The result
 * is bit-identical to count zb_gemm calls.  Errors: ZB_EINVAL. */
int32_t zb_gemm_wgrad_group(int32_t count, const int32_t* M, const int32_t* N, const int32_t* K,
                            const void* const* A, const int64_t* lda, int32_t a_kmajor,
                            const void* const* B, const int64_t* ldb, int32_t b_kmajor,
                            void* const* C, const int64_t* ldc, void* stream);

/* Thread-local description of the last error (never NULL). */
const char* zb_last_error(void);

/* Library version string. */
const char* zb_version(void);

#ifdef __cplusplus
}
#endif
#endif /* ZB_H_ */
