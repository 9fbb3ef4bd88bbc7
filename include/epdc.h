/*
 * epdc.h -- C ABI of the MI355X (gfx950) MoE expert-parallel dispatch/combine
 * hot path.
 *
 * The operations mirror the methods of MORI's EpDispatchCombineOp (MORI
 * "Communication APIs" page, MORI-EP section, methods table):
 *   dispatch(input, weights, scales, indices)
 *       -> (output, weights, scales, indices, recv_count)
 *   combine(input, weights, indices) -> (output, weights)
 *   reset()
 *   get_dispatch_src_token_pos()
 * on one GPU, for one GPU's share of the tokens, with the destination ranks
 * of an intra-node EP group modelled as contiguous segments of one receive
 * buffer in HBM.
 *
 * Received layout.  Every (token t, k) pair with a valid expert index gets one
 * received row ("slot").  Slots are grouped by expert, experts ascending, and
 * inside an expert ordered by the pair index p = t*K + k.  Virtual rank r owns
 * experts [r*E/R, (r+1)*E/R), i.e. the slots [rank_off[r], rank_off[r+1]).
 * recv_count[r] = rank_off[r+1] - rank_off[r] is produced by dispatch itself,
 * zero included (same page, "AsyncLL v2 SDMA overlap" section: a peer's
 * count arrives even when it is zero, and the dispatch kernels compute it).
 *
 * Conventions for every entry point:
 *  - Pointers marked "device" are HBM addresses on the op's device; the
 *    caller allocates and owns all of them, including the op's workspace.  The
 *    library never allocates device memory.  "host" pointers are read or
 *    written before the call returns.
 *  - `stream` is a hipStream_t passed as void*; NULL is the null stream.  The
 *    work is enqueued on it and the call returns without waiting; results are
 *    valid once that work completes (same page, AsyncLL section: payload
 *    and counts may be used once the stream has finished the receive step).
 *  - Row-major layouts; no padding between rows.  Payload rows (input, out,
 *    output) start 16-byte aligned, every other array 4-byte aligned;
 *    misaligned pointers give EPDC_ERR_INVALID_ARGS.
 *  - A non-SUCCESS status leaves no work enqueued, except EPDC_ERR_GPU_OP
 *    after a failed launch.  epdc_last_error() gives a thread-local message.
 *  - An op is not thread-safe and its calls must be ordered (one stream, or
 *    ordered streams): the workspace holds the routing between calls.
 * Status names follow MORI-IO's StatusCode enum (same page, MORI-IO section).
 */
#ifndef EPDC_H
#define EPDC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum epdc_status {
    EPDC_SUCCESS = 0,
    EPDC_ERR_INVALID_ARGS = -1,  /* bad pointer, size or configuration */
    EPDC_ERR_BAD_STATE = -2,     /* e.g. combine with no dispatch recorded */
    EPDC_ERR_GPU_OP = -3,        /* a HIP call failed (message says which) */
    EPDC_ERR_UNSUPPORTED = -4,   /* device is not gfx950 */
    EPDC_ERR_NOT_FOUND = -5      /* unknown kernel id */
} epdc_status;

/* Payload kind of dispatch's `input`.  RAW rows are opaque bytes that are
 * copied unchanged, e.g. already-quantized FP8/FP4 payloads ("Choosing an EP
 * API and backend" page, "EP paths" table, HIP row). */
typedef enum epdc_input_kind {
    EPDC_IN_BF16 = 0,            /* [T, hidden] bfloat16 */
    EPDC_IN_RAW = 1              /* [T, raw_row_bytes] bytes */
} epdc_input_kind;

/* On-the-fly quantization applied by dispatch to BF16 input ("Choosing an EP
 * API and backend" page, EPv2 restrictions list: OCP E4M3 on gfx950; FP4 via
 * gfx950's pair-at-a-time scaled convert family). */
typedef enum epdc_quant {
    EPDC_QUANT_NONE = 0,
    /* OCP E4M3 codes [N, H] + fp32 scales [N, H/128]; per block of 128:
     * scale = amax/448 (fp32 division), code = E4M3(x/scale) rounded to
     * nearest even, saturated to +-448; amax == 0 gives scale 0, codes 0. */
    EPDC_QUANT_FP8_E4M3_B128 = 1,
    /* MXFP4: E2M1 codes two per byte (element 2m in the low nibble of byte
     * m) [N, H/2] + E8M0 scales [N, H/32]; per block of 32 the shared
     * exponent is floor(log2(amax)) - 2 clamped to [-127, 127] (-127 for an
     * all-zero block); codes round to nearest even and saturate to +-6. */
    EPDC_QUANT_MXFP4_B32 = 2
} epdc_quant;

/* Fixed at creation. */
typedef struct epdc_config {
    int32_t max_tokens;      /* T_max >= 0: largest num_tokens of a dispatch */
    int32_t hidden;          /* H in (0, 2^24], multiple of 8 (bf16 rows of
                                16-byte vectors); multiple of 128 for FP8, 32
                                for MXFP4 */
    int32_t topk;            /* K in [1, 16] */
    int32_t num_experts;     /* E in [1, 512] */
    int32_t num_ranks;       /* R >= 1 with E % R == 0 */
    int32_t input_kind;      /* epdc_input_kind */
    int32_t quant;           /* epdc_quant; != NONE requires EPDC_IN_BF16 */
    int32_t raw_row_bytes;   /* EPDC_IN_RAW: bytes per row, in (0, 2^25], multiple
                                of 16 */
    int32_t scale_row_bytes; /* bytes per carried scale row, multiple of 4,
                                0 = dispatch carries no scales; must be 0 when
                                quant != NONE (scales are then produced) */
} epdc_config;

typedef struct epdc_op epdc_op;

/* Kernel ids for the profiling calls below. */
enum {
    EPDC_KERNEL_ROUTE = 0,         /* per-tile histograms + stable in-tile ranks,
                                      and the scan to expert/rank offsets + tile
                                      bases (by the last block to finish, or by
                                      the scatter blocks for a small tile table;
                                      a dispatch of at most 1024 pairs routes
                                      inside its scatter launch instead, so it
                                      records only the scatter kernel) */
    EPDC_KERNEL_ROUTE_SCAN = 1,    /* reserved: the scan has no launch of its own */
    EPDC_KERNEL_SCATTER = 2,       /* slot + row copy (bf16 or raw) */
    EPDC_KERNEL_SCATTER_FP8 = 3,   /* slot + E4M3 quantize + copy */
    EPDC_KERNEL_SCATTER_MXFP4 = 4, /* slot + MXFP4 quantize + copy */
    EPDC_KERNEL_COMBINE = 5,       /* gather + weighted fp32 sum */
    EPDC_KERNEL_UNITS_TO_EXPERTS = 6, /* unit rows -> expert rows (conversion) */
    EPDC_KERNEL_EXPERTS_TO_UNITS = 7, /* weighted sum of a unit's expert rows */
    EPDC_KERNEL_COMBINE_UNITS = 8,    /* sum of a token's unit rows */
    EPDC_KERNEL_COMBINE_PUSH = 9,     /* scatter combine: weighted rows -> staging */
    EPDC_KERNEL_COMBINE_REDUCE = 10,  /* scatter combine: staging -> token rows */
    EPDC_KERNEL_CHECK_INDICES = 11,   /* debug check of combine's indices */
    EPDC_NUM_KERNELS = 12
};

/* What the caller knows about combine's input rows (epdc_set_combine_hint):
 * only how epdc_combine launches and stores depends on it, never a result. */
enum {
    /* default: the input was written long before (HBM-resident) */
    EPDC_COMBINE_INPUT_COLD = 0,
    /* the input rows were written just before the combine (by the expert
     * computation, or the dispatch itself for identity experts), so part of
     * them sits dirty in the last-level cache */
    EPDC_COMBINE_INPUT_RECENT = 1
};

/* Debug switches (epdc_set_debug). */
enum {
    /* combine and combine_scatter check a non-NULL `indices` against the
     * recorded routing before combining (one extra launch) */
    EPDC_DEBUG_CHECK_INDICES = 1
};

/* Bytes of device workspace an op with this config needs (host only, no GPU
 * call).  Returns EPDC_ERR_INVALID_ARGS for an invalid config. */
epdc_status epdc_workspace_bytes(const epdc_config *cfg, size_t *bytes);

/* Bytes per received row of dispatch's `out` and `out_scales` for this config
 * (host only): bf16 2H, RAW raw_row_bytes, FP8 H, MXFP4 H/2; scales
 * scale_row_bytes, 4*H/128 for FP8, H/32 for MXFP4. */
epdc_status epdc_row_bytes(const epdc_config *cfg, size_t *payload_bytes,
                           size_t *scale_bytes);

/* Create an op on the current HIP device.  `workspace` (device, >= the size
 * from epdc_workspace_bytes, 256-byte aligned) stays owned by the caller and
 * must outlive the op; the op clears its control words synchronously.
 * EPDC_ERR_UNSUPPORTED if the current device is not gfx950. */
epdc_status epdc_create(const epdc_config *cfg, void *workspace,
                        size_t workspace_bytes, epdc_op **op);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the op of
 * the current device whose workspace is the library's own static device
 * array of 8 MiB (EPDC_STATIC_WORKSPACE_BYTES), one array and one op per
 * device, both held until the process ends.  No workspace argument, and no
 * allocation of any kind: the first call on a device looks up that device's
 * copy of the array, and every call configures the device's op in place for
 * `cfg` and returns it (the same handle each time).  EPDC_ERR_INVALID_ARGS
 * when epdc_workspace_bytes(cfg) exceeds the array (about 25 bytes per
 * (token, k) pair: max_tokens*topk above roughly 300,000); otherwise as
 * epdc_create, and every other entry point works on the op unchanged.
 * Because there is one workspace per device, a call re-configures the op for
 * everyone holding the handle: the recorded routing and any unreceived send
 * are forgotten and the control words (the sticky error flag) cleared.
 * Calls on the op must be ordered (one stream or ordered streams);
 * overlapping calls race.  epdc_destroy on it forgets its state and releases
 * its timing events but keeps the op and the array.
 */
#define EPDC_STATIC_WORKSPACE_BYTES (8u << 20)
epdc_status epdc_create_static(const epdc_config *cfg, epdc_op **op);

/* Free the host-side op (the workspace is the caller's). NULL is allowed. */
epdc_status epdc_destroy(epdc_op *op);

/*
 * dispatch: route num_tokens tokens to their top-K experts' slots.
 *   input       device [T, H] bf16 (EPDC_IN_BF16) or [T, raw_row_bytes] (RAW)
 *   weights     device [T, K] fp32, or NULL (then out_weights must be NULL)
 *   scales      device [T, scale_row_bytes] carried unchanged, or NULL; must
 *               be NULL when scale_row_bytes == 0 or quant != NONE
 *   indices     device [T, K] int32 expert ids.  An id outside [0, E) is a
 *               precondition violation: that pair gets no slot, the device
 *               error flag is raised (epdc_get_device_error), nothing is
 *               written out of bounds.  (Flag bit 1; bit 2 marks a slot
 *               outside [0, num_tokens*K), which a consistent routing table
 *               never produces: such a pair is dropped, not written.)
 *   out         device [T_max*K, payload row] (epdc_row_bytes)
 *   out_weights device [T_max*K, K] fp32 (each slot carries its token's row)
 *   out_scales  device [T_max*K, scale row]; required when quant != NONE or
 *               scales != NULL, else ignored
 *   out_indices device [T_max*K, K] int32, or NULL
 *   recv_count  device [R] int32 (rows per virtual rank; sum = valid pairs)
 * With num_tokens == 0 only out and recv_count are required (recv_count and
 * the offsets are written as zeros).
 * Only rows [0, n_valid) of the outputs are written, n_valid = expert_off[E].
 * Records the routing for the next combine and for the getters below.
 */
epdc_status epdc_dispatch(epdc_op *op, void *stream, int32_t num_tokens,
                          const void *input, const float *weights,
                          const void *scales, const int32_t *indices,
                          void *out, float *out_weights, void *out_scales,
                          int32_t *out_indices, int32_t *recv_count);

/*
 * combine: for every token t of the last dispatch,
 *   output[t, :] = bf16_rne( sum_{k=0..K-1} w(t,k) * input[slot(t,k), :] )
 * accumulated in fp32 in k order (a separate multiply and add per term,
 * starting from +0), with w(t,k) = weights[slot(t,k), k] (1 if weights is
 * NULL).  Pairs without a slot contribute nothing and report weight 0.
 *   input       device [rows, H] bf16 in the received layout; only rows below
 *               n_valid <= num_tokens*K of the last dispatch are read
 *   weights     device [rows, K] fp32 in the received layout, or NULL
 *   indices     device [rows, K] int32 or NULL.  The op keeps the routing, so
 *               combine does not need them; with EPDC_DEBUG_CHECK_INDICES on
 *               (epdc_set_debug) a non-NULL `indices` is checked first: row
 *               s < n_valid must hold, in entry k of its row (k of the pair
 *               it came from), the expert whose rows contain s.  A mismatch
 *               raises bit 4 of the device error flag (epdc_get_device_error)
 *               and the combine still runs.
 *   output      device [num_tokens, H] bf16
 *   out_weights device [num_tokens, K] fp32 = w(t,k), or NULL
 * EPDC_ERR_BAD_STATE if no dispatch is recorded (none yet, or reset).
 */
epdc_status epdc_combine(epdc_op *op, void *stream, const void *input,
                         const float *weights, const int32_t *indices,
                         void *output, float *out_weights);

/*
 * Scatter combine ("Choosing an EP API and backend" page, "EP paths" table,
 * FlyDSL row: gather/scatter combine).  Reading implemented here: the expert
 * side pushes each received row, multiplied by its weight in fp32, to the
 * fp32 staging row of the (token, k) pair it came from, and the token side
 * adds its K staging rows in k order.  No two rows share a staging row, so no
 * atomics are needed and the result is bit-identical to epdc_combine (same
 * products, same order).  Arguments as epdc_combine, plus staging: caller
 * device memory of max_tokens * topk rows of hidden fp32 values (16-byte
 * aligned); it holds the weighted products afterwards.  On one GPU this
 * moves 8 more bytes per element than the gather; it is the form a push
 * across GPUs would take.
 */
epdc_status epdc_combine_scatter(epdc_op *op, void *stream, const void *input,
                                 const float *weights, const int32_t *indices,
                                 float *staging, void *output, float *out_weights);

/*
 * Rank-deduplicated dispatch and the standard-MoE conversion.
 *
 * The pages name a standard-MoE conversion for the intra-node path ("Choosing
 * an EP API and backend" page, "EP paths" table) and an intra-node kernel
 * type ("Communication APIs" page, kernel types table) without defining
 * them.  Reading implemented here: a token travels once to each destination
 * rank that hosts at least one of its valid experts ("unit" (t, r)); the
 * receiving rank expands its unit rows into the expert-contiguous rows of
 * epdc_dispatch (epdc_units_to_experts) for the grouped expert GEMM; on the
 * way back it sums the weighted outputs of each unit's experts into one bf16
 * unit row (epdc_experts_to_units), and the source adds its token's unit
 * rows (epdc_combine_units).  On several GPUs only unit rows would cross the
 * links, min(K, R) per token at most instead of K.
 *
 * Unit rows: U = sum(recv_count) <= T * min(K, R); rank r owns rows
 * [unit_off[r], unit_off[r+1]), ordered by token.  Unit row buffers need
 * capacity U_cap = max_tokens * min(topk, num_ranks) rows.
 */

/* Like epdc_dispatch, with one received row per unit: out, out_weights,
 * out_scales and out_indices are [U_cap, ...] in the unit layout (each unit
 * carries its token's full weights / indices / scales rows), recv_count[r]
 * = unit rows of rank r.  The pair routing (expert offsets, slot of each
 * pair, source positions) is recorded as well, so epdc_combine,
 * epdc_get_routing and epdc_get_dispatch_src_token_pos work after it as after
 * epdc_dispatch, and epdc_dispatch_replay replays the unit rows. */
epdc_status epdc_dispatch_dedup(epdc_op *op, void *stream, int32_t num_tokens,
                                const void *input, const float *weights,
                                const void *scales, const int32_t *indices,
                                void *out, float *out_weights, void *out_scales,
                                int32_t *out_indices, int32_t *recv_count);

/* Device pointers of the last rank-deduplicated dispatch's unit routing:
 * unit_off [R+1], unit_of [T*K] (unit row of each pair, -1 for an invalid
 * expert id), unit_src [U] (token of each unit row).  Any output may be
 * NULL.  BAD_STATE if the last dispatch was not rank-deduplicated. */
epdc_status epdc_get_unit_routing(epdc_op *op, const int32_t **unit_off,
                                  const int32_t **unit_of, const int32_t **unit_src);

/* Conversion to the standard MoE layout: every unit row (payload bytes of
 * the config, and the carried weights / scales / indices rows where given) is
 * copied to the expert rows of its pairs, giving exactly the rows
 * epdc_dispatch writes for the same input.  input [U_cap, P] (P = payload
 * bytes per row as epdc_row_bytes reports), out [N_cap, P]; each carried
 * array needs its input and output, or neither; scale rows must be a
 * multiple of 4 bytes.  Reads the unit count on the device (no host wait).
 * BAD_STATE if the last dispatch was not rank-deduplicated. */
epdc_status epdc_units_to_experts(epdc_op *op, void *stream, const void *input,
                                  const float *in_weights, const void *in_scales,
                                  const int32_t *in_indices, void *out,
                                  float *out_weights, void *out_scales,
                                  int32_t *out_indices);

/* Conversion back: unit row u of token t = bf16_rne(sum over k = 0..K-1 of
 * the pairs of t in u of w(t,k) * in[slot(t,k)]) in fp32, separate multiply
 * and add, w(t,k) = weights[slot(t,k)][k] (1 when weights is NULL).  input
 * [N_cap, H] bf16 expert rows, weights [N_cap, K] fp32 or NULL, output
 * [U_cap, H] bf16.  BAD_STATE if the last dispatch was not rank-deduplicated. */
epdc_status epdc_experts_to_units(epdc_op *op, void *stream, const void *input,
                                  const float *weights, void *output);

/* Combine of unit rows: output[t] = bf16_rne(sum of the token's unit rows in
 * ascending row order, i.e. ascending rank) in fp32 from +0 (+0 for a token
 * with no valid pair); out_weights[t][k] = unit_weights[unit of (t,k)][k] (1
 * when unit_weights is NULL, 0 for an invalid pair) or NULL.  input
 * [U_cap, H] bf16, unit_weights [U_cap, K] fp32 or NULL, output [T, H].  It
 * differs from epdc_combine on the same expert rows only by the bf16
 * rounding of each unit's partial sum.  BAD_STATE as above. */
epdc_status epdc_combine_units(epdc_op *op, void *stream, const void *input,
                               const float *unit_weights, void *output,
                               float *out_weights);

/*
 * Routing replay: dispatch a new payload with the routing recorded by the last
 * dispatch (same tokens, same expert ids), skipping the histogram, scan and
 * ranking ("Choosing an EP API and backend" page, "EP paths" table: routing
 * replay).  Writes the payload, carried weights and scales rows to the same
 * slots; out_indices, recv_count, the offsets and src_token_pos are those of
 * the recorded dispatch and are not rewritten.  Arguments as in
 * epdc_dispatch, for num_tokens = the recorded dispatch's; after
 * epdc_dispatch_dedup the rows written are unit rows.  BAD_STATE if no
 * dispatch is recorded.
 */
epdc_status epdc_dispatch_replay(epdc_op *op, void *stream, const void *input,
                                 const float *weights, const void *scales, void *out,
                                 float *out_weights, void *out_scales);

/*
 * Split phases for overlapping other work with dispatch and combine
 * ("Communication APIs" page, methods table: dispatch_send / dispatch_recv,
 * combine_send / combine_recv; "AsyncLL v2 SDMA overlap" section: payload
 * and counts may be used once the stream has finished the receive step).  On one
 * GPU the send phase is the whole operation enqueued on `stream` (typically a
 * side stream) followed by a completion marker owned by the op; the receive
 * phase makes `stream` (typically the compute stream) wait for that marker,
 * without a host wait.  *_send takes the arguments of epdc_dispatch /
 * epdc_combine; *_recv returns BAD_STATE without a matching send.
 */
epdc_status epdc_dispatch_send(epdc_op *op, void *stream, int32_t num_tokens,
                               const void *input, const float *weights,
                               const void *scales, const int32_t *indices,
                               void *out, float *out_weights, void *out_scales,
                               int32_t *out_indices, int32_t *recv_count);
epdc_status epdc_dispatch_recv(epdc_op *op, void *stream);
epdc_status epdc_combine_send(epdc_op *op, void *stream, const void *input,
                              const float *weights, const int32_t *indices,
                              void *output, float *out_weights);
epdc_status epdc_combine_recv(epdc_op *op, void *stream);

/* Device pointer to src_token_pos [T_max*K] int32 of the last dispatch: for
 * slot s < n_valid, the pair index p = t*K + k it came from (the methods
 * table's get_dispatch_src_token_pos, which reports where each received
 * token came from, for checking a dispatch).
 * *count = num_tokens*K of that dispatch (host).  BAD_STATE if none. */
epdc_status epdc_get_dispatch_src_token_pos(epdc_op *op, const int32_t **dev_ptr,
                                            int32_t *count);

/* Device pointers into the workspace for the last dispatch: expert_off [E+1]
 * and rank_off [R+1] (exclusive prefix sums of the expert and rank counts;
 * rank r's rows are [rank_off[r], rank_off[r+1])).  Either may be NULL.
 * BAD_STATE if no dispatch is recorded. */
epdc_status epdc_get_offsets(epdc_op *op, const int32_t **expert_off,
                             const int32_t **rank_off);

/* Device pointers into the workspace for the last dispatch: expert_off [E+1],
 * rank_off [R+1] (exclusive prefix sums), slot_of [num_tokens*K] (slot of
 * pair p, -1 if none).  Any may be NULL.  BAD_STATE if none. */
epdc_status epdc_get_routing(epdc_op *op, const int32_t **expert_off,
                             const int32_t **rank_off, const int32_t **slot_of);

/* Tell epdc_combine how recently its input rows were written
 * (EPDC_COMBINE_INPUT_*; COLD is the default).  A performance hint, measured
 * on MI355X: with RECENT the combine's output takes stores that allocate in
 * the caches, 6-7% faster when the input is still partly in the last-level
 * cache and 7-12% slower when it is not, and batches of more than 1024
 * pairs run with at most three 4-wave blocks per CU (up to 2% faster).  With
 * COLD, batches of more than 1024 pairs use nontemporal stores and, for rows
 * whose byte size is not a power of two, a form that writes groups of up to
 * four output rows at once (6-7% faster at hidden 7168), else fewer waves per
 * CU once the input rows span 768 MiB or more (3-6% faster).  Results are
 * identical in every case.  Host state only; INVALID_ARGS for an unknown
 * value. */
epdc_status epdc_set_combine_hint(epdc_op *op, int32_t hint);

/* Switch debug checks on or off for this op (EPDC_DEBUG_* bits; 0 = none,
 * the default).  Host state only.  INVALID_ARGS for an unknown bit. */
epdc_status epdc_set_debug(epdc_op *op, int32_t flags);

/* Wait for `stream`, then return (host) and clear the sticky device error
 * flag: nonzero if some call since the last read raised it.  Bits: 1 = a
 * dispatch saw an expert id outside [0, E); 2 = a slot outside the call's
 * rows (never produced by a consistent routing; the pair was dropped);
 * 4 = the debug check found combine indices that disagree with the
 * recorded routing.  Synchronizes; not for use under graph capture. */
epdc_status epdc_get_device_error(epdc_op *op, void *stream, int32_t *flag);

/* Forget the recorded routing and any unreceived send ("Reset internal state
 * between iterations").  No device work: counts need no clearing because
 * dispatch writes them. */
epdc_status epdc_reset(epdc_op *op);

/* Thread-local message for the last non-SUCCESS status ("" if none). */
const char *epdc_last_error(void);

/* Kernel name for an EPDC_KERNEL_* id, NULL if unknown. */
const char *epdc_kernel_name(int32_t kernel_id);

/* Per-kernel timing with HIP events recorded on the launch stream around
 * each kernel the op launches.  The events are created without the
 * system-scope release at their timestamps (hipEventDisableSystemFence), so
 * a pair times the launch, not an L2 write-back after it; they order
 * nothing and make no memory visible to the host.  begin: allocate events
 * for up to max_launches launches (host-side event objects, no device
 * memory).  end:
 * wait for the last recorded event, write (host) the summed milliseconds and
 * the launch count per kernel id into ms[EPDC_NUM_KERNELS] and
 * launches[EPDC_NUM_KERNELS], and release the events. */
epdc_status epdc_profile_begin(epdc_op *op, int32_t max_launches);
epdc_status epdc_profile_end(epdc_op *op, float *ms, int32_t *launches);

#ifdef __cplusplus
}
#endif

#endif /* EPDC_H */
