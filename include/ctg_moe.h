/*
 * ctg_moe.h -- C-ABI of one MI355X's share of an expert-parallel MoE layer.
 *
 * The layer has three steps, each an entry point below, plus one call that runs
 * all three:
 *
 *   moe_dispatch      tokens arriving from S source ranks are pushed, with no
 *                     metadata exchanged first, into rank-major receive buffers
 *                     ("windows") in this GPU's HBM.  Source s owns window rows
 *                     [s*T_s*k, (s+1)*T_s*k) and lays its (token, slot) pairs out
 *                     sorted by expert using only its own counts.
 *                     ["One-Sided Expert-Parallel All-to-All for Mixture-of-Experts
 *                     Inference over NVLink", abstract: one-sided push into
 *                     rank-major buffers without a metadata exchange; "Relay Buffer
 *                     Independent Communication over Pooled HBM for Efficient MoE
 *                     Inference on Ascend", abstract: direct placement into
 *                     destination expert windows, counts/offsets/sync state only.]
 *   moe_grouped_gemm  per local expert, the windows are read in place by an FP8
 *                     (or MXFP4) block-scaled grouped GEMM with the SwiGLU
 *                     activation and the FP8 requantisation of its output fused,
 *                     followed by the down projection; an optional shared expert
 *                     runs over every token, reading the source buffers in place.
 *                     ["One-Sided ... over NVLink", abstract: grouped GEMMs read
 *                     the buffers in place; "GC-MoE: Overlapping Expert-Parallel
 *                     Token Dispatch with FP8/FP4 Grouped GEMM via CUDA Green
 *                     Contexts", full text: block-scaled MMA with fused SwiGLU,
 *                     requantization and optional shared experts.]
 *   moe_combine       every token's k expert outputs are read back from the
 *                     windows, weighted by its top-k gate weights and summed in
 *                     token order (plus the shared expert's output).
 *                     ["Relay Buffer Independent Communication ...", abstract:
 *                     direct reading from expert windows, less output restoration.]
 *
 * Synchronisation between dispatch and GEMM follows one of two schedules
 * ["One-Sided ... over NVLink", abstract: Fence for throughput, Sentinel for
 * latency].  FENCE: the steps run in stream order.  SENTINEL (moe_layer): dispatch
 * and GEMM1 run at the same time.  Each source publishes an epoch tag once its
 * counts and offsets are written and another once all of its window rows are; a
 * GEMM1 workgroup polls the first kind for every source, builds its expert's row
 * table, issues its weight-scale loads, and then waits only for the sources that
 * hold rows of its expert (the device-side counter handshake of "GC-MoE", full
 * text, and of "GC-MoE: Decoupling MoE Communication and Computation with CUDA
 * Green Contexts", section "Three-Node CUDA Graph and token-ring Handshake").
 * Epoch tags grow monotonically, so no clean pass is needed between calls.
 * Two forms, chosen by dispatch_cus:
 *   0   the dispatch runs inside the GEMM1 launch itself: each of its first
 *       workgroups issues its first weight loads, runs one dispatch chunk, and only
 *       then waits (one queue; workgroups are placed in index order, and a chunk
 *       waits for nothing, so every flag awaited is published by a running workgroup);
 *   >0  the dispatch kernel runs on a stream restricted to dispatch_cus CUs and
 *       GEMM1 on a stream holding the other CUs (the partition of the "GC-MoE"
 *       pages); GEMM2 and the combine run on the caller's stream after both
 *       streams join.  Each fork and join is a wait between hardware queues.
 * SENTINEL applies to the FP8/MXFP4 decode kernels; the tiled prefill GEMM, the
 * fp32 path, the persistent GEMM and the separate stage calls run in stream
 * order (FENCE).
 *
 * Conventions
 *   - Every data pointer is a DEVICE pointer owned by the caller, except the
 *     arrays of per-source pointers (x, x_scale), which are HOST arrays of S
 *     device pointers.  The context owns its workspace (windows, control state).
 *   - Row-major layouts; FP8 is OCP e4m3 ("e4m3fn": bias 7, max 448, no inf);
 *     FP4 is OCP e2m1 with element 2i in the low nibble of byte i; e8m0 scale
 *     bytes mean 2^(b-127).
 *   - Block scales are fp32 multipliers (real value = code value * scale):
 *     activations 1x128 along the hidden dimension; FP8 weights 128x128 over
 *     (output row, input column); MXFP4 weights e8m0 per 1x32 along the input.
 *   - The layer calls (moe_dispatch, moe_grouped_gemm, moe_combine, moe_combine_fp8,
 *     moe_layer) and the gate calls are asynchronous on the given stream (0 = the null
 *     stream) and allocate nothing; moe_get_routing and moe_copy_buffer enqueue copies.
 *     Allocation happens only in moe_create (the workspace) and moe_set_timing (its
 *     events); moe_last_device_error, moe_read_timing, moe_set_timing and the
 *     MOE_OPT_EPOCH option wait for the device.  A context is not thread-safe; calls on
 *     one context must be issued on one stream (or be ordered by the caller).
 *   - Arguments are validated on the host before any work is enqueued; a
 *     non-OK status means nothing was enqueued, and moe_last_error_message()
 *     gives the reason.  Conditions found on the device (an expert id outside
 *     [-1, E), a sentinel wait that timed out) are latched in a device error
 *     word read by moe_last_device_error().
 */
#ifndef CTG_MOE_H
#define CTG_MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_MAX_SRC 32      /* simulated source ranks */
#define MOE_MAX_EXPERTS 256 /* local routed experts */
#define MOE_MAX_TOPK 16
#define MOE_MAX_DIM 16384   /* hidden, inter and shared_inter: multiples of 128 up to this */

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* bad pointer, size, alignment or dtype combination */
  MOE_ERR_UNSUPPORTED = 2, /* valid request the library does not implement */
  MOE_ERR_HIP = 3,         /* a HIP runtime call failed (no device, out of memory, ...) */
  MOE_ERR_DEVICE = 4       /* a device-side condition was latched; see moe_last_device_error */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2, MOE_FP4_E2M1 = 3 } moe_dtype;

typedef enum { MOE_SCHED_FENCE = 0, MOE_SCHED_SENTINEL = 1 } moe_schedule;

/* device error bits (moe_last_device_error) */
#define MOE_DEVERR_BAD_ID 0x1u  /* an expert id outside [-1, E); that pair was dropped */
#define MOE_DEVERR_TIMEOUT 0x2u /* a sentinel wait gave up; the GEMM output is invalid */

typedef struct moe_config {
  int32_t n_src;          /* S: simulated source ranks, 1..MOE_MAX_SRC */
  int32_t max_tokens;     /* capacity T_cap: largest tokens-per-source of any call */
  int32_t hidden;         /* H, multiple of 128 */
  int32_t inter;          /* I of the routed experts, multiple of 128 */
  int32_t n_experts;      /* E local routed experts, 1..MOE_MAX_EXPERTS */
  int32_t topk;           /* k, 1..MOE_MAX_TOPK */
  int32_t shared_inter;   /* I of the one shared expert, multiple of 128; 0 = none */
  moe_dtype act;          /* MOE_FP8_E4M3 (with 1x128 scales), MOE_BF16 (the W4A16 variant:
                             MXFP4 weights, bf16 activations and h) or MOE_F32 */
  moe_dtype weight;       /* MOE_FP8_E4M3 or MOE_FP4_E2M1 (with MOE_FP8_E4M3 act), MOE_FP4_E2M1
                             (with MOE_BF16 act), or MOE_F32 */
  moe_dtype out;          /* MOE_BF16 (FP8 or BF16 act) or MOE_F32 (F32 act) */
  moe_schedule sched;     /* FENCE or SENTINEL */
  int32_t dispatch_cus;   /* SENTINEL: 0 = dispatch inside the GEMM1 launch; else the
                             CUs of a separate dispatch stream, a multiple of 8 (the
                             mask spreads over the 8 XCDs) below the GPU's CU count */
} moe_config;

/*
 * Expert weights, all device pointers, row-major:
 *   FP8:   w13 u8  [E][2I][H]   s13 f32 [E][2I/128][H/128]
 *          w2  u8  [E][H][I]    s2  f32 [E][H/128][I/128]
 *   MXFP4: w13 u8  [E][2I][H/2] s13 u8 (e8m0) [E][2I][H/32]
 *          w2  u8  [E][H][I/2]  s2  u8 (e8m0) [E][H][I/32]
 *   F32:   w13 f32 [E][2I][H], w2 f32 [E][H][I], s13 = s2 = NULL
 * Rows 0..I-1 of W13[e] are the gate projection, rows I..2I-1 the up projection.
 * The shared expert (sh_*) has the same layout with E = 1 and I = shared_inter;
 * its pointers are ignored when shared_inter = 0.
 * packed = 0: the row-major layouts above.  packed = 1: buffers written by
 * moe_pack_weights (FP8 and MXFP4 only), the order in which the GEMM streams them.
 */
typedef struct moe_weights {
  const void *w13, *s13, *w2, *s2;
  const void *sh_w13, *sh_s13, *sh_w2, *sh_s2;
  int32_t packed;
} moe_weights;

typedef struct moe_ctx moe_ctx;

/* Internal buffers that moe_copy_buffer can read (parity tests of intermediate steps). */
typedef enum {
  MOE_BUF_WINDOW = 0,   /* dispatched rows: [R][H] in the activation dtype (e4m3, bf16 or f32), R = S*T_s*k */
  MOE_BUF_WSCALE = 1,   /* their scales: f32 [R][H/128] (FP8 act only) */
  MOE_BUF_H = 2,        /* SwiGLU output [R + T][max(I, shared_I)] in the activation dtype; rows R.. = shared expert */
  MOE_BUF_HSCALE = 3,   /* its 1x128 scales: f32 [R + T][I/128] (FP8 act only) */
  MOE_BUF_Y = 4         /* expert outputs: [R + T][H] in the output dtype; rows R.. = shared expert */
} moe_buffer;

/* Creates a context on the current HIP device and allocates all of its workspace
 * (sized by cfg->max_tokens).  On success *out owns the context. */
moe_status moe_create(const moe_config* cfg, moe_ctx** out);

/* Frees the context and its workspace (waits for the device first). NULL is a no-op. */
moe_status moe_destroy(moe_ctx* ctx);

/*
 * Dispatch [S sources x T_s tokens x k slots] into the windows.
 *   tokens_per_src  T_s, 0..max_tokens (0 = nothing to do)
 *   x               host array [S] of device pointers; x[s] -> [T_s][H] in the activation
 *                   dtype (e4m3 bytes, bf16 or f32), 16-byte aligned
 *   x_scale         host array [S] of device pointers; x_scale[s] -> f32 [T_s][H/128]
 *                   (FP8 act); NULL for BF16 and F32 act
 *   ids             device int32 [S][T_s][k]: local expert id of each slot, -1 = not
 *                   routed to this GPU; ids outside [-1, E) set MOE_DEVERR_BAD_ID and
 *                   the pair is dropped
 * The rows, counts and offsets it writes stay valid until the next dispatch.  The
 * x buffers must stay valid until the following moe_grouped_gemm has run when a
 * shared expert is configured (it reads them in place).
 */
moe_status moe_dispatch(moe_ctx* ctx, int32_t tokens_per_src, const void* const* x,
                        const float* const* x_scale, const int32_t* ids, hipStream_t stream);

/* Grouped GEMM over the windows written by the last moe_dispatch (and the shared
 * expert over the last dispatch's x).  Experts with no rows read no weights. */
moe_status moe_grouped_gemm(moe_ctx* ctx, const moe_weights* w, hipStream_t stream);

/*
 * Combine: out[s][t][:] = sum_j topk_w[s][t][j] * y[dst_row[s][t][j]] (+ shared y),
 * accumulated in fp32 in slot order, for the tokens of the last dispatch.
 *   topk_w  device f32 [S][T_s][k]
 *   out     device [S][T_s][H] in the output dtype, 16-byte aligned
 */
moe_status moe_combine(moe_ctx* ctx, const float* topk_w, void* out, hipStream_t stream);

/*
 * The same combine with its output requantised as the next layer's FP8 input (the
 * requantisation the layer fuses [GC-MoE feed, full text], here also applied to the
 * layer's output): the fp32 slot-order sums of moe_combine, then per token row and
 * 128-element block s = fl32(amax / 448) (1 when amax = 0) and code = e4m3 of
 * clamp(fl32(v / s), +-448), nearest even -- the rule of the h requantisation.
 * Any configuration (y bf16 or fp32).
 *   out        device u8 [S][T_s][H] e4m3 codes, 16-byte aligned
 *   out_scale  device f32 [S][T_s][H/128], 4-byte aligned
 * NULL or misaligned pointers return MOE_ERR_INVALID_ARG; before any dispatch likewise.
 */
moe_status moe_combine_fp8(moe_ctx* ctx, const float* topk_w, uint8_t* out, float* out_scale,
                           hipStream_t stream);

/*
 * The whole layer: dispatch, grouped GEMM and combine, synchronised per cfg.sched.
 *
 * Graph replay (the decode step as one submitted graph [GC-MoE explainer, "Three-Node
 * CUDA Graph and token-ring Handshake"]): under the FENCE schedule the call only
 * enqueues kernels on `stream` (no allocation, memset, copy or host wait) and every
 * buffer it reads is rewritten by an earlier step of the same call, so it may be
 * captured into a HIP graph (stream capture) and the graph replayed; each replay
 * computes the layer on what x, ids and topk_w hold at that time, with the sizes and
 * pointers of the captured call.  moe_dispatch, moe_grouped_gemm and moe_combine may
 * be captured likewise.  A call that takes the SENTINEL handshake (its flags carry a
 * per-call epoch set on the host) or records timing events returns MOE_ERR_INVALID_ARG
 * when `stream` is capturing.
 */
moe_status moe_layer(moe_ctx* ctx, int32_t tokens_per_src, const void* const* x,
                     const float* const* x_scale, const int32_t* ids, const float* topk_w,
                     const moe_weights* w, void* out, hipStream_t stream);

/*
 * Copies the last dispatch's control state to caller device buffers (any may be NULL):
 *   cnt [S][E], off [S][E] (exclusive prefix of cnt[s] over e),
 *   dst_row [S][T_s][k] (window row of each pair, -1 if not routed),
 *   row_src [S*T_s*k] (flattened pair s*T_s*k + t*k + j filling each row, -1 if unused).
 */
moe_status moe_get_routing(moe_ctx* ctx, int32_t* cnt, int32_t* off, int32_t* dst_row,
                           int32_t* row_src, hipStream_t stream);

/* Copies the first `bytes` of an internal buffer to device memory `dst` (stream-ordered). */
moe_status moe_copy_buffer(moe_ctx* ctx, moe_buffer which, void* dst, size_t bytes,
                           hipStream_t stream);

/*
 * Weight packing (a one-time preparation, as at model load): the grouped GEMM streams
 * each expert's weights from HBM once per call, and streams them fastest when every
 * wavefront's share is one contiguous run in the order it is consumed.
 * moe_packed_sizes gives the byte size of each of the 8 moe_weights buffers of the
 * packed form, in field order (w13, s13, w2, s2, sh_w13, sh_s13, sh_w2, sh_s2; 0 for
 * unused fields).  moe_pack_weights rewrites the row-major set src into the caller's
 * buffers dst (which must have those sizes, dst->packed = 1, no overlap with src);
 * FP8 block scales are copied unchanged, MXFP4 e8m0 scales are permuted with their
 * weights.  Stream-ordered; F32 weights return MOE_ERR_UNSUPPORTED.
 */
moe_status moe_packed_sizes(const moe_config* cfg, size_t sizes[8]);
moe_status moe_pack_weights(moe_ctx* ctx, const moe_weights* src, const moe_weights* dst,
                            hipStream_t stream);

/*
 * Tuning options of a context (each defaults to automatic):
 *   MOE_OPT_PERSISTENT_GEMM  0: two kernels, one workgroup per work item (default);
 *                            1: both GEMMs in one persistent kernel fed by work queues,
 *                            GEMM2 items waiting on per-expert counters (the cross-XCD
 *                            hand-off of h costs an L2 write-back per item).  The W4A16
 *                            variant always runs two kernels.
 *   MOE_OPT_TOKEN_TILES      0: automatic; 2..6: most 16-row token tiles per GEMM pass
 *                            (kernels take at most 4 for FP8 and 5 for MXFP4 weights).
 *   MOE_OPT_QUEUE            0: automatic; 1: one work queue per XCD (an expert's items
 *                            stay on one XCD); 2: one queue for the whole GPU.
 *   MOE_OPT_TILED_GEMM       0: automatic (LDS-tiled MFMA kernels from 192 mean rows per
 *                            expert, FP8 weights); 1: always tiled (FP8 weights);
 *                            2: never (the weight-streaming kernels).
 *   MOE_OPT_SENTINEL_SPIN    SENTINEL: polls of one flag before a GEMM1 workgroup gives
 *                            up (latching MOE_DEVERR_TIMEOUT); 0: default (2^20).
 *   MOE_OPT_SENTINEL_STALL   1: GEMM1 waits for an epoch the dispatch never publishes,
 *                            so every routed wait times out -- a test of the failure
 *                            path (the layer output is then invalid); 0: off.
 *   MOE_OPT_TILED_MFMA       the LDS-tiled kernels' MFMA: 0: 16x16x128 (default);
 *                            1: 32x32x64, the two 64-deep halves of a 128-deep scale block
 *                            chained before one promotion (results agree with 0 to fp32
 *                            rounding of the block sums, not bit for bit).
 *   MOE_OPT_FUSED_COMBINE    1: moe_layer forms the top-k weighted combine in the epilogue
 *                            of the decode GEMM2 (the weight-streaming kernels, two-kernel
 *                            or persistent, bf16 out): the item that brings a token's last
 *                            contribution to a block of 256 output columns sums that block
 *                            (per-token counters at agent scope, reset by that item), with
 *                            the combine kernel's arithmetic, so the output is
 *                            bit-identical; the tiled and fp32 paths keep the combine
 *                            kernel; 0: the combine kernel (default).
 * Test aids for the handshake and the reuse of the workspace without a clean pass:
 *   MOE_OPT_POISON           1: every moe_layer call first fills the windows, their scales,
 *                            h, its scales and y (all rows of the capacity) with NaN codes
 *                            of their formats (a kernel, enqueued on the call's stream), so
 *                            that reading a row the call has not written shows; 0: off.
 *   MOE_OPT_EPOCH            sets the SENTINEL epoch counter to (uint32_t)value (the next
 *                            call uses the value after it, skipping 0) and clears the flags;
 *                            waits for the device.  For calls across the counter's wrap.
 *   MOE_OPT_DISPATCH_DELAY   SENTINEL: every dispatch chunk waits this many microseconds
 *                            (0..10000) after publishing the counts and before writing its
 *                            window rows, so GEMM1 workgroups wait on the row flags; 0: off.
 * Unknown options or values return MOE_ERR_INVALID_ARG.
 */
typedef enum {
  MOE_OPT_PERSISTENT_GEMM = 0,
  MOE_OPT_TOKEN_TILES = 1,
  MOE_OPT_QUEUE = 2,
  MOE_OPT_TILED_GEMM = 3,
  MOE_OPT_SENTINEL_SPIN = 4,
  MOE_OPT_SENTINEL_STALL = 5,
  MOE_OPT_TILED_MFMA = 6,
  MOE_OPT_POISON = 7,
  MOE_OPT_EPOCH = 8,
  MOE_OPT_DISPATCH_DELAY = 9,
  MOE_OPT_FUSED_COMBINE = 10
} moe_option;
moe_status moe_set_option(moe_ctx* ctx, moe_option opt, int32_t value);

/*
 * Gating ahead of dispatch.  Each token goes to the experts its gating result names
 * ["GC-MoE: Decoupling MoE Communication and Computation with CUDA Green Contexts",
 * "Why Expert Parallelism Is Inefficient in MoE Decoding"]; the gate is the
 * sparsely-gated MoE layer's ["Relay Buffer Independent Communication over Pooled HBM
 * for Efficient MoE Inference on Ascend", "Builds on"]: the k largest logits of a
 * token (ties to the lower expert id; slot 0 holds the largest), weights = softmax
 * over the kept logits.  Neither call needs a context; neither allocates.
 *
 * moe_router_logits: logits[t][e] = sum_h x[t][h] * wr[e][h] for T tokens and E
 *   experts; x [T][H] and wr [E][H] bf16 (16-byte aligned), H a multiple of 32,
 *   E <= MOE_MAX_GATE_EXPERTS; logits [T][E] fp32 (caller-owned).  fp32 accumulation
 *   (MFMA); the order of the sum is the kernel's.
 * moe_topk_softmax: from logits [T][E] fp32 to ids [T][k] int32 (descending logit)
 *   and w [T][k] fp32 (sums to 1 per token); k <= min(E, MOE_MAX_TOPK).  The
 *   selection compares the given fp32 values exactly, so it is reproducible: the
 *   same logits always give the same ids.
 * T = 0 is a no-op.  Invalid sizes or pointers return MOE_ERR_INVALID_ARG before any
 * work is enqueued.
 */
#define MOE_MAX_GATE_EXPERTS 256
moe_status moe_router_logits(int32_t T, int32_t H, int32_t E, const void* x, const void* wr, float* logits,
                             hipStream_t stream);
moe_status moe_topk_softmax(int32_t T, int32_t E, int32_t k, const float* logits, int32_t* ids, float* w,
                            hipStream_t stream);

/*
 * moe_gate: the two steps above in one call, for the latency of small batches: the router's
 * K reduction is split over workgroups so that a few hundred tokens still occupy every CU.
 * Partial sums go to `workspace` (device, 16-byte aligned, caller-owned, at least
 * moe_gate_workspace_bytes(T, H, E) bytes given in workspace_bytes; its contents on entry
 * do not matter and are overwritten) and are added in a fixed order, so the result does
 * not depend on timing.  logits [T][E] fp32 receives the sums when not NULL; ids and w are
 * as for moe_topk_softmax, and are the top-k of exactly those sums.  Same argument rules
 * as the two calls; a short workspace is MOE_ERR_INVALID_ARG.  The sums' order differs
 * from moe_router_logits', so the two may differ in the last bits.
 * moe_gate_workspace_bytes returns 0 for empty or invalid sizes.
 */
size_t moe_gate_workspace_bytes(int32_t T, int32_t H, int32_t E);
moe_status moe_gate(int32_t T, int32_t H, int32_t E, int32_t k, const void* x, const void* wr, void* workspace,
                    size_t workspace_bytes, float* logits, int32_t* ids, float* w, hipStream_t stream);

/*
 * moe_gate_noalloc: moe_gate without a caller workspace and without any allocation, for
 * callers that cannot allocate device memory -- code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  The router's partial sums go to a
 * fixed scratch array of MOE_GATE_NOALLOC_MAX_BYTES in the library's device code (one per
 * GPU, held until the process ends); a shape whose moe_gate_workspace_bytes exceeds it
 * (beyond 4096 tokens at 256 experts) returns MOE_ERR_INVALID_ARG before any work is
 * enqueued.  The first call on a device looks up that device's copy of the array (no
 * allocation).  Results are bit-identical to moe_gate's for the same arguments.  Every
 * call on one GPU uses the same array: calls that overlap on one GPU (different streams
 * with no order between them, or different threads) race and give undefined results.
 * Other arguments and rules as for moe_gate.
 */
#define MOE_GATE_NOALLOC_MAX_BYTES (4u << 20)
moe_status moe_gate_noalloc(int32_t T, int32_t H, int32_t E, int32_t k, const void* x, const void* wr, float* logits,
                            int32_t* ids, float* w, hipStream_t stream);

/*
 * Measurement aid, not part of the layer: launches `blocks` workgroups that issue only
 * FP8 MFMAs (v_mfma_scale_f32_16x16x128_f8f6f4, operands in registers, no memory
 * traffic) `iters` times per chain, and returns the flops the launch performs (-1 on
 * invalid arguments: sink NULL or not 4-byte aligned, blocks or iters < 1).  sink:
 * device fp32 [4], caller-owned, accumulated into (its contents are not meaningful).
 * The caller times the launch on `stream`; flops / time is the sustained FP8 MFMA rate,
 * reported beside the published peak.
 */
int64_t moe_mfma_fp8_probe(float* sink, int32_t blocks, int32_t iters, hipStream_t stream);

/*
 * Verification aid, not part of the layer: one v_mfma_scale_f32_16x16x128_f8f6f4 with unit
 * scales -- the instruction the FP8 and MXFP4 GEMMs use -- so that tests can check how it
 * accumulates.  a: 16 rows of 128 codes in a_fmt (MOE_FP8_E4M3, or MOE_FP4_E2M1 with one
 * code in the low 4 bits of each byte), b: 16 columns of 128 e4m3 codes; each row or column
 * is 128 consecutive bytes.  out: fp32 [16][16] with out[i][j] = the instruction's sum over
 * k of a[i][k] * b[j][k].  All three are caller-owned device buffers.  Another a_fmt, NULL
 * pointers or a misaligned out return MOE_ERR_INVALID_ARG.
 */
moe_status moe_mfma_dot16x16(moe_dtype a_fmt, const uint8_t* a, const uint8_t* b, float* out, hipStream_t stream);

/* Waits for the device, returns the latched device error bits and clears them.  After a
 * timeout (MOE_DEVERR_TIMEOUT) the calls since the last check produced invalid output, and
 * a persistent GEMM that skipped work may have left the combine counters of
 * MOE_OPT_FUSED_COMBINE part-counted: this call then also resets them. */
moe_status moe_last_device_error(moe_ctx* ctx, uint32_t* bits);

/*
 * Per-stage timing with HIP events, for measurement.  moe_set_timing(ctx, n) keeps
 * events for up to n moe_layer calls (0 turns timing off); moe_read_timing waits for
 * them and returns, for the calls recorded since the last read, the summed
 * milliseconds of [0] dispatch, [1] GEMM1 (+SwiGLU+requant), [2] GEMM2, [3] combine,
 * [4] whole layer, and the number of calls in *n_calls.  With the persistent GEMM
 * kernel or the tiled GEMM, [1] holds both GEMMs and [2] is 0.  Under SENTINEL,
 * [0] is the dispatch on its own stream, [1] runs from the end of the dispatch to
 * the end of GEMM1 (the part of GEMM1 not hidden behind it) and [2] includes the
 * join of the two streams; in the fused form [0] is 0 and [1] holds the launch
 * that runs both.
 */
moe_status moe_set_timing(moe_ctx* ctx, int32_t max_calls);
moe_status moe_read_timing(moe_ctx* ctx, float* ms_sum5, int32_t* n_calls);

const char* moe_status_str(moe_status s);
/* Detail text of the last non-OK status returned on this thread. */
const char* moe_last_error_message(void);

#ifdef __cplusplus
}
#endif
#endif /* CTG_MOE_H */
