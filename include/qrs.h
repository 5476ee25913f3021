/*
 * qrs.h -- C ABI for one GPU's share of a quantized reduce-scatter on MI355X
 * (gfx950).
 *
 * The operation (page "aclnnQuantReduceScatter", Function description): the
 * output is a reduction, over the data arriving from the different ranks, of
 * the all-to-all'ed scales multiplied by the all-to-all'ed quantized x. On
 * one GPU the all-to-all has already happened: the caller passes W rank
 * slices of x codes, each [rows, H] with rows = BS / W, and their scales.
 * For every row i and column c, with G the group size of the scale layout:
 *
 *     p_r      = fp32( decode(x_r[i][c]) * decode(scale_r[i][c / G]) )
 *     acc      = p_0;  acc = fp32(acc + p_r)  for r = 1 .. W-1, in rank order
 *     out[i][c] = acc                 (QRS_OUT_F32)
 *     out[i][c] = bf16_rne(acc)       (QRS_OUT_BF16)
 *     out[i][c] = f16_rne(acc)        (QRS_OUT_F16)
 *
 * Products and sums are separate binary32 operations rounded to nearest-even
 * (no fused multiply-add), subnormals are kept, NaN and infinity propagate.
 * The fixed rank order makes the result deterministic.
 *
 * The calls follow the page's two-phase form (Prototype): a first call
 * checks the parameters and prepares the computation (qrs_plan, host only),
 * a second runs it on a stream (qrs_run). Both return a status code. The
 * parameter and error tables of the page did not survive, so names and codes
 * here are this library's own.
 *
 * Ownership: the caller owns every device buffer and the stream; the library
 * owns only the plan. No call allocates device memory; the workspace size is
 * always 0. A plan is immutable and may be used by any number of concurrent
 * qrs_run calls on different streams. The launching calls (qrs_run,
 * qrs_run_all_shares, qrs_run_strided, qrs_quantize) enqueue kernels only --
 * no allocation, memset or synchronisation -- so they may be captured in a
 * HIP graph.
 *
 * Errors: every call returns a qrs_status. On failure, qrs_last_error()
 * returns a human-readable message for the calling thread.
 *
 * Throughput note: one launch has a fixed cost of a few microseconds (ramp
 * up and drain); on MI355X one W=8, H=8192 MX share (172 MB) runs at about
 * 6.4 TB/s and the 514 MB W=8, H=5120 share at about 6.7 TB/s. A caller
 * with independent shares (different batches or buckets) can alternate them
 * over two streams of the same priority to overlap the fixed cost, or hand
 * a whole group to qrs_run_all_shares (one launch).
 */
#ifndef QRS_H_
#define QRS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qrs_status {
  QRS_OK = 0,
  QRS_ERR_INVALID_ARG = 1, /* a parameter breaks a documented constraint   */
  QRS_ERR_UNSUPPORTED = 2, /* a format the library does not implement      */
  QRS_ERR_HIP = 3,         /* the HIP runtime reported an error at launch  */
  QRS_ERR_OUT_OF_MEMORY = 4, /* a host allocation (plan, launch handle) failed */
  /* Range markers, not statuses: they make every int a value of the type,
   * so a caller may pass any int and the library rejects it as a value. */
  QRS_STATUS_RANGE_MIN_ = -2147483647 - 1,
  QRS_STATUS_RANGE_MAX_ = 2147483647
} qrs_status;

/* Element format of x (page "aclnnQuantReduceScatter", Constraints).
 * FP8 formats are the OCP 8-bit float formats. HIFLOAT8 is listed by the page
 * but never defined there, so it is reserved and always rejected with
 * QRS_ERR_UNSUPPORTED. */
typedef enum qrs_x_dtype {
  QRS_X_INT8 = 0,       /* two's complement byte                         */
  QRS_X_FP8_E4M3FN = 1, /* OCP E4M3 "FN": bias 7, no inf, max 448        */
  QRS_X_FP8_E5M2 = 2,   /* OCP E5M2: bias 15, inf/NaN, max 57344         */
  QRS_X_HIFLOAT8 = 3,   /* reserved                                      */
  QRS_X_DTYPE_RANGE_MIN_ = -2147483647 - 1, /* range markers, not formats  */
  QRS_X_DTYPE_RANGE_MAX_ = 2147483647
} qrs_x_dtype;

/* Scale layout (same page, Constraints). Groups and blocks run along H
 * within one token, so slice r's scales are row-major:
 *   QRS_SCALE_F32_GROUP128: float32 [rows, H/128], per-token-per-group mode,
 *                           for INT8, E4M3FN or E5M2 x;
 *   QRS_SCALE_E8M0_BLOCK32: uint8 E8M0 [rows, H/32] (value 2^(code-127),
 *                           code 255 = NaN), MX mode, for E4M3FN or E5M2 x.
 * The block of 32 is fixed by the page's MX scales size (one byte per 32
 * elements of x). */
typedef enum qrs_scale_layout {
  QRS_SCALE_F32_GROUP128 = 0,
  QRS_SCALE_E8M0_BLOCK32 = 1,
  QRS_SCALE_LAYOUT_RANGE_MIN_ = -2147483647 - 1, /* range markers, not layouts */
  QRS_SCALE_LAYOUT_RANGE_MAX_ = 2147483647
} qrs_scale_layout;

/* Output type. The page's output dtype table did not survive extraction;
 * fp32 and bf16 are the types the workloads use, fp16 is the other 16-bit
 * output a half-precision consumer takes. Both 16-bit types are the
 * round-to-nearest-even of the fp32 accumulator (fp16: values from 65520 up
 * become infinity, subnormals are kept). */
typedef enum qrs_out_dtype {
  QRS_OUT_F32 = 0,  /* float32 [rows, H]                                 */
  QRS_OUT_BF16 = 1, /* bfloat16 [rows, H], round-to-nearest-even of fp32 */
  QRS_OUT_F16 = 2,  /* IEEE binary16 [rows, H], round-to-nearest-even    */
  QRS_OUT_DTYPE_RANGE_MIN_ = -2147483647 - 1, /* range markers, not types  */
  QRS_OUT_DTYPE_RANGE_MAX_ = 2147483647
} qrs_out_dtype;

typedef struct qrs_plan_s* qrs_plan_t;

/*
 * Phase 1: check the problem and prepare a plan. Host only, no GPU work.
 *
 *   world_size  W, the communicator size: 2, 4 or 8 (Constraints).
 *   bs          tokens per rank before the all-to-all (x is [BS, H] on each
 *               rank, Constraints); must be > 0 (no empty input) and a
 *               multiple of W. This GPU's share has rows = bs / W, and
 *               rows * h may not exceed 2^40 elements.
 *   h           hidden size: a multiple of 128 in [1024, 8192] (Constraints).
 *   x_dtype, scale_layout, out_dtype
 *               a pair that selects a mode of the page: MX needs an FP8 x;
 *               INT8 with E8M0 is QRS_ERR_INVALID_ARG; HIFLOAT8 is
 *               QRS_ERR_UNSUPPORTED.
 *   plan_out    receives the plan (non-null). Free it with qrs_plan_destroy.
 *   workspace_bytes_out
 *               receives the device workspace size, always 0 (non-null).
 *
 * Returns QRS_OK, QRS_ERR_INVALID_ARG, QRS_ERR_UNSUPPORTED or
 * QRS_ERR_OUT_OF_MEMORY. On error *plan_out is set to NULL (when plan_out is
 * non-null).
 */
qrs_status qrs_plan(int world_size, int64_t bs, int64_t h, qrs_x_dtype x_dtype, qrs_scale_layout scale_layout,
                    qrs_out_dtype out_dtype, qrs_plan_t* plan_out, size_t* workspace_bytes_out);

/*
 * Phase 2: run the planned share on a stream. Asynchronous: no host
 * synchronisation, no allocation.
 *
 *   x_slices      HOST array of W DEVICE pointers; x_slices[r] is rank r's
 *                 uint8 codes [rows, H], contiguous row-major, 16-byte
 *                 aligned. One [W, rows, H] buffer is the case of equally
 *                 spaced pointers.
 *   scale_slices  HOST array of W DEVICE pointers to rank r's scales in the
 *                 plan's layout, contiguous row-major; fp32 scales 4-byte
 *                 aligned.
 *   out           DEVICE buffer [rows, H] of the plan's output type, 16-byte
 *                 aligned, not overlapping any input.
 *   workspace, workspace_bytes
 *                 unused (the plan needs none); any value is accepted.
 *   stream        a hipStream_t (NULL = the default stream).
 *
 * A share of more than 2^34 elements runs as consecutive launches over
 * consecutive 2^34-element ranges (a HIP grid holds fewer than 2^32
 * work-items along a dimension); the results are the same bits as one
 * launch's. The environment variable QRS_MAX_LAUNCH_ELEMS, read once per
 * process, may lower that bound to a multiple of 4096 elements (this and
 * every other call that launches reduce or quantize kernels); any other
 * value makes those calls return QRS_ERR_INVALID_ARG.
 *
 * Returns QRS_ERR_INVALID_ARG for a null plan or pointer, a misaligned
 * pointer or an output that overlaps an input, and QRS_ERR_HIP if a kernel
 * launch fails (every launch of a split share is checked before the first is
 * enqueued). Inputs are not validated element by element: NaN or infinite
 * codes and scales propagate as in IEEE 754.
 */
qrs_status qrs_run(qrs_plan_t plan, const void* const* x_slices, const void* const* scale_slices, void* out,
                   void* workspace, size_t workspace_bytes, void* stream);

typedef struct qrs_launch_s* qrs_launch_t;

/*
 * Phase 2 split in two, for callers that run the same share again and again
 * on fixed buffers and one stream (serving loops, benchmarks): the page's
 * two-phase interface (Prototype) carried one step further.
 * qrs_launch_create makes every check qrs_run makes (same arguments, same
 * errors) and chooses the kernel, grid and residency cap for the device of
 * `stream` (for each launch of a share split as qrs_run splits it), then
 * keeps them in *launch_out (host memory; no GPU work, no device
 * allocation). qrs_launch_enqueue then enqueues that launch on that
 * stream with no further checks: asynchronous, no host synchronisation, no
 * allocation; the same results as qrs_run with the same arguments.
 *
 *   launch_out  receives the handle (non-null); NULL on error.
 *
 * The handle copies what it needs from the plan (which may be destroyed
 * afterwards) but not the buffers or the stream: they must stay valid while
 * enqueues may use them. The handle is read-only after creation, so
 * enqueues from several threads are safe (they race on the output like any
 * two launches on one buffer). qrs_launch_destroy frees the handle (NULL is
 * accepted); it does not wait for enqueued work, which keeps running.
 *
 * qrs_launch_create returns what qrs_run returns, or QRS_ERR_OUT_OF_MEMORY;
 * qrs_launch_enqueue returns QRS_ERR_INVALID_ARG for a NULL handle and
 * QRS_ERR_HIP if the launch fails.
 */
qrs_status qrs_launch_create(qrs_plan_t plan, const void* const* x_slices, const void* const* scale_slices, void* out,
                             void* stream, qrs_launch_t* launch_out);
qrs_status qrs_launch_enqueue(qrs_launch_t launch);
qrs_status qrs_launch_destroy(qrs_launch_t launch);

/*
 * The whole reduce-scatter of a W-rank group computed on this GPU: every
 * rank's share, from the ranks' inputs as they are BEFORE the all-to-all.
 * Page "aclnnQuantReduceScatter", Function description: the data and scales
 * are all-to-all'ed, then reduced. The all-to-all splits each rank's [BS, H]
 * rows into W row blocks of rows = BS/W and delivers block j of every rank
 * to rank j (in rank order); here that index map is applied by addressing,
 * with no copy, so share j is
 *
 *     out_shares[j] = Reduce_r( scales_r[block j] * x_r[block j] )
 *
 * with the same arithmetic as qrs_run. Up to about 300 MB of algorithmic
 * bytes per share one launch covers all W shares; larger shares are
 * enqueued as W launches, one per share, on the same stream (measured
 * faster on MI355X at those sizes). Shares of more than 2^34 elements are
 * further split into launches over element ranges, as qrs_run splits them.
 * Either way the call only enqueues work, and the results are the same.
 *
 *   x_full        HOST array of W DEVICE pointers; x_full[r] is rank r's
 *                 uint8 codes [BS, H], contiguous, 16-byte aligned.
 *   scale_full    HOST array of W DEVICE pointers to rank r's scales for all
 *                 BS rows in the plan's layout ([BS, H/128] fp32, 4-byte
 *                 aligned, or [BS, H/32] E8M0).
 *   out_shares    HOST array of W DEVICE pointers; out_shares[j] is share
 *                 j's [BS/W, H] output, 16-byte aligned, overlapping neither
 *                 an input nor another share.
 *   workspace, workspace_bytes, stream: as for qrs_run.
 *
 * Errors as for qrs_run.
 */
qrs_status qrs_run_all_shares(qrs_plan_t plan, const void* const* x_full, const void* const* scale_full,
                              void* const* out_shares, void* workspace, size_t workspace_bytes, void* stream);

/*
 * qrs_run for slices and an output whose rows are not adjacent: row i of
 * rank r's x slice starts i * x_row_stride bytes after x_slices[r], row i of
 * its scales i * scale_row_stride scale elements after scale_slices[r], and
 * row i of the output i * out_row_stride output elements after out. This
 * covers slices that are row ranges of wider buffers (for example a column
 * range [.., c0:c0+H] of a [BS, H_total] tensor) and padded rows. Same
 * arithmetic and result as qrs_run on the same values.
 *
 *   x_row_stride      bytes, >= h, a multiple of 16 (rows stay 16-byte
 *                     aligned; x_slices[r] 16-byte aligned).
 *   scale_row_stride  elements, >= h / G (fp32 scale pointers 4-byte
 *                     aligned).
 *   out_row_stride    elements, >= h, spanning a multiple of 16 bytes; out
 *                     16-byte aligned.
 *
 * Each row stride, in bytes, must be below 4 GiB, the plan's rows per
 * share below 2^32, and one slice's scales, from its first row's start to
 * its last row's end, must span less than 4 GiB. The output's address span,
 * from its first to the last element written, must not overlap the address
 * span of any input slice. A share of more than 2^34 elements runs as
 * launches over consecutive row ranges of at most 2^34 elements (at least
 * one row each), as qrs_run splits contiguous shares. Errors as for qrs_run.
 */
qrs_status qrs_run_strided(qrs_plan_t plan, const void* const* x_slices, int64_t x_row_stride,
                           const void* const* scale_slices, int64_t scale_row_stride, void* out,
                           int64_t out_row_stride, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Producer side: quantize bf16 activations into the x codes and scales that
 * the reduce consumes, in one of the page's modes (page
 * "aclnnQuantReduceScatter", Constraints: per-token-per-group with 128
 * columns and fp32 scales, or MX with 32 elements and E8M0 scales). The page
 * does not say how scales are chosen; this library uses
 *   MX:        the OCP Microscaling v1.0 conversion -- shared exponent
 *              floor(log2(amax)) - emax of the element format (8 for E4M3,
 *              15 for E5M2), limited to [-127, 127]; each element divided by
 *              the scale (exact), clamped to the largest normal, rounded to
 *              nearest-even; an all-zero block gets code 0;
 *   per-group: scale = amax / qmax (qmax = 127, 448 or 57344), codes =
 *              round-to-nearest-even(clamp(v * (qmax / amax), +-qmax)); the
 *              scale is kept at or above 2^-126 (then the multiplier is
 *              2^126), which also covers all-zero groups.
 * Every step is a single binary32 operation (amax, the per-group division,
 * the per-element product), so results are deterministic bit for bit.
 *
 *   tokens, h   x is [tokens, h] bf16, row-major; tokens > 0; h a multiple
 *               of 128 in [1024, 8192] (as for qrs_plan).
 *   x_dtype, scale_layout
 *               a mode of the page (HIFLOAT8: QRS_ERR_UNSUPPORTED; INT8 with
 *               E8M0: QRS_ERR_INVALID_ARG).
 *   x_bf16      DEVICE bf16 [tokens, h], 16-byte aligned, finite values
 *               (NaN / infinity inputs give unspecified codes).
 *   x_codes     DEVICE uint8 [tokens, h], 16-byte aligned.
 *   scales      DEVICE [tokens, h/128] fp32 (4-byte aligned) or [tokens, h/32]
 *               uint8 E8M0.
 *   stream      a hipStream_t (NULL = the default stream).
 *
 * The three buffers must not overlap. Asynchronous; allocates nothing.
 * More than 2^34 elements run as consecutive launches over 2^34-element
 * ranges, under the same bound as qrs_run (QRS_MAX_LAUNCH_ELEMS included).
 */
qrs_status qrs_quantize(int64_t tokens, int64_t h, qrs_x_dtype x_dtype, qrs_scale_layout scale_layout,
                        const void* x_bf16, void* x_codes, void* scales, void* stream);

/* Free a plan. NULL is accepted. Plans in use by queued runs may be freed:
 * qrs_run copies what the kernel needs into its launch arguments. */
qrs_status qrs_plan_destroy(qrs_plan_t plan);

/* Shape of a plan's share: rows = bs / world_size and h. Either out-pointer
 * may be NULL. */
qrs_status qrs_plan_shape(qrs_plan_t plan, int64_t* rows_out, int64_t* h_out);

/*
 * Recommended placement when the W rank slices of x (and of the scales)
 * share one allocation, for example the receive buffer of the all-to-all:
 * slice r at byte offset r * x_pitch (scales: r * scale_pitch). What the
 * W concurrent read streams see of each other is the pitch modulo 4 MiB:
 * near a multiple of 4 MiB the same offset of every slice falls in the same
 * HBM bank group and the streams evict each other's DRAM rows (measured on
 * MI355X: 16 MiB slices back to back 31.5 us, staggered 28.9 us; 7 MiB
 * slices at a pitch of 0.25 MiB modulo 4 MiB 14.75 us, at 1.25 MiB 13.95
 * us). The x pitch is the slice size rounded up to 64 KiB, plus the
 * smallest stagger that makes it 1.25 MiB modulo 4 MiB; the scale pitch is
 * the scale slice rounded up to 4 KiB plus 40 KiB. Any placement gives the
 * same results; this only affects speed. Offsets are multiples of 64 KiB
 * (x) and 4 KiB (scales), so alignment requirements hold.
 *
 *   x_pitch_out, scale_pitch_out  receive the pitches in bytes; either may be
 *                                 NULL.
 *   full_inputs                   0: pitches for this GPU's slices ([rows, H]
 *                                 each, for qrs_run); 1: for the ranks' whole
 *                                 inputs ([BS, H] each, for
 *                                 qrs_run_all_shares).
 */
qrs_status qrs_slice_pitch(qrs_plan_t plan, int full_inputs, size_t* x_pitch_out, size_t* scale_pitch_out);

/*
 * The launch qrs_run makes for this plan on the device of `stream` (a
 * hipStream_t; NULL = the current device), reported without launching
 * anything. Host only; the library reads the device's sizes with
 * hipDeviceGetAttribute (once per device) but enqueues no work.
 *
 *   launches           kernel launches qrs_run makes: 1, or more for shares
 *                      of more than 2^34 elements (see qrs_run); the other
 *                      fields describe the first launch, and every launch
 *                      but the last is alike;
 *   blocks             work-groups in the grid;
 *   threads_per_block  threads per work-group;
 *   dynamic_lds_bytes  unused LDS requested per work-group so that at most
 *                      blocks_per_cu_cap work-groups reside on one CU (large
 *                      contiguous shares only; 0 = no cap);
 *   blocks_per_cu_cap  that cap (0 = none);
 *   device_cus, device_lds_per_cu, device_lds_per_block
 *                      the device sizes the cap is derived from (CU count,
 *                      LDS bytes per CU, LDS bytes one work-group may use);
 *                      0 if they could not be read (then no cap).
 *
 * Returns QRS_ERR_INVALID_ARG for a null plan or info pointer.
 */
typedef struct qrs_launch_info {
  uint64_t blocks;
  uint32_t threads_per_block;
  uint32_t dynamic_lds_bytes;
  uint32_t blocks_per_cu_cap;
  uint32_t device_cus;
  uint32_t device_lds_per_cu;
  uint32_t device_lds_per_block;
  uint32_t launches;
} qrs_launch_info;

qrs_status qrs_run_launch_info(qrs_plan_t plan, void* stream, qrs_launch_info* info_out);

/* Static, never-null name of a status code. */
const char* qrs_status_string(qrs_status status);

/* Message describing the calling thread's most recent failing call (empty
 * if none). Valid until that thread's next call into the library. */
const char* qrs_last_error(void);

/*
 * Utility, not part of the operation: copy `bytes` bytes from src to dst on
 * `stream` with the same 16-byte streaming loads and stores the reduction
 * uses. It is the reference stream for bandwidth and traffic-counter
 * calibration. bytes must be a positive multiple of 16, both pointers
 * 16-byte aligned device pointers, and the ranges must not overlap. More
 * than 2^35 bytes run as consecutive launches of 2^35 bytes.
 */
qrs_status qrs_stream_copy(const void* src, void* dst, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QRS_H_ */
