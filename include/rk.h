/*
 * rk.h -- device-wide mapreduce for AMD Instinct MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels.  It computes the mapped reductions
 * described on the AcceleratedKernels.jl pull-request pages:
 *
 *   - PR #139, "Finish whole-array reductions on the device": a whole array
 *     is reduced in at most two launches (a grid-capped first pass whose
 *     blocks stride over tiles, then a one-block second pass); the last pass
 *     applies `init`, or folds into the output's previous value, or leaves a
 *     bare partial that the host finishes (sections "What changes" and
 *     "Compatibility").
 *   - PR #176, strided reductions along dims: one selector picks among one
 *     thread per output, a tiled 2-d block and a split columns kernel, and
 *     the columns kernel also takes runs of contiguous outputs such as the
 *     middle dim of a 3-d array (section "This PR").
 *   - a two-input source f(a_i, b_i) on the whole-array passes
 *     (rk_reduce_all2), and scans, the prefix folds of PR #202 (rk_scan,
 *     rk_scan_dims).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Arrays are column-major (Julia semantics).  `shape[d]` is the extent of
 * dim d and `strides[d]` its stride in ELEMENTS (>= 0); a contiguous
 * (d1, d2, d3) array has strides (1, d1, d1*d2).  Bit d of `reduce_mask`
 * marks dim d (0-based) as reduced, so Julia's `dims=k` is bit k-1.  The
 * outputs are the kept dims, stored contiguously in column-major order (the
 * reduced dims behave as extent 1).
 *
 * The result for each output is  R = s (+) f(x_0) (+) f(x_1) (+) ...  where
 * (+) is the op, f the map applied after widening an element to the
 * accumulator type, and s the starting value chosen by the mode:
 *   RK_MODE_OVERWRITE  s = *init (the op's identity when init is NULL); the
 *                      result is stored into the device array `out`;
 *   RK_MODE_FOLD       s = the previous value of out[o], read back into the
 *                      accumulator type; `init` is ignored, so an init that
 *                      was applied by an earlier call is not applied again;
 *   RK_MODE_HOST       s = *init (or identity); the GPU leaves a bare
 *                      accumulator-typed partial in a small pinned host
 *                      buffer the library keeps per host thread (or, without
 *                      one, in the workspace, copied back), and the host
 *                      finishes it; `out` is a HOST pointer and the call
 *                      returns after the stream has drained.  Valid only when
 *                      there is a single output.  Setting the environment
 *                      variable RK_HOST_COPY before the first host-mode call
 *                      of a thread selects the copy.
 * `init` is applied exactly once.  Partial results keep the accumulator type
 * until the final store, which converts once to the output type (round to
 * nearest even for floating point, two's-complement wrap for integers).  The
 * output is never used to hold intermediate values.  The association order
 * is the library's own, so floating-point results may differ from a
 * sequential loop by rounding.  Identities: 0 for sum, -inf / the
 * accumulator's minimum integer for max, +inf / its maximum for min.  max
 * and min propagate NaN.
 *
 * Dtype combinations: the input and accumulator are both floating point or
 * both integer, and the accumulator is at least as wide as the input
 * (f32 -> f32|f64, bf16 -> f32|f64, f16 -> f32|f64, f64 -> f64,
 * i32 -> i32|i64, i64 -> i64).  The output has the accumulator's kind and any
 * width of that kind; it may be narrower than the accumulator.
 *
 * Ownership: the caller owns every buffer (`ptr`, `out`, `workspace`).  The
 * library allocates and frees no device memory; its per-stream slots are
 * static device memory of its code objects (about 42 MB per device, loaded
 * with the library).  Kernels are enqueued on
 * `stream` (a hipStream_t; NULL is the null stream) of the current device.
 * OVERWRITE and FOLD calls are asynchronous: buffers must stay alive until
 * the stream's work has completed.  Between calls the library keeps only
 * cached device properties and, per (device, stream), a slot of state in its
 * own device memory, so a reduction split across blocks finishes inside its
 * one launch: a whole-array pass's blocks store their partials tagged with
 * the call's number and block 0 collects them; split dims reductions count
 * arrivals on counters that return to zero by themselves.  Calls from several host threads are
 * safe; two calls that share a workspace must be ordered by the caller.
 *
 * Graph capture: OVERWRITE and FOLD calls enqueue kernels only (no memset,
 * no copy, no allocation), so they may be captured into a HIP graph and the
 * graph replayed.  Captured kernels keep the slot of the stream they were
 * captured on: replays of one graph must not overlap each other or calls on
 * that capture stream.  HOST mode waits on the stream and cannot be captured.
 *
 * Errors: every argument is validated before any launch; a rejected call
 * returns a non-zero rk_status and writes nothing.  A HIP launch failure is
 * reported as RK_ERR_HIP.  The library prints nothing unless the environment
 * variable RK_DEBUG is set.
 *
 * Waits inside a launch: block 0 of a whole-array pass waits for the other
 * blocks' partials, and a scan tile waits for its predecessors' prefixes.  No
 * block waits on the block that waits for it, so these waits end; as a
 * safety net each is bounded (about a second).  A wait that gives up stores
 * no result (out keeps its previous contents; a scan's outputs after that
 * tile are wrong) and is counted: HOST mode then returns RK_ERR_HIP, and
 * rk_stream_timeouts reports the count for OVERWRITE, FOLD and scan calls.
 */
#ifndef RK_H
#define RK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    RK_OK = 0,
    RK_ERR_INVALID_ARGUMENT = 1, /* bad pointer, size, shape, mask, mode or alignment */
    RK_ERR_UNSUPPORTED = 2,      /* dtype combination outside the table above */
    RK_ERR_HIP = 3,              /* the HIP runtime reported an error */
    RK_ERR_TOO_LARGE = 4         /* rk_reduce_dims_no_workspace: the call needs more than the scratch */
} rk_status;

typedef enum { RK_OP_SUM = 0, RK_OP_MAX = 1, RK_OP_MIN = 2 } rk_op;

/* Element map f, applied after widening to the accumulator type (the `f` of
 * mapreduce(f, op, A); PR #139, opening section).  Integer maps wrap in the
 * accumulator type. */
typedef enum { RK_MAP_IDENTITY = 0, RK_MAP_SQUARE = 1, RK_MAP_ABS = 2 } rk_map;

/* Two-input map f(a, b) of a fused source (rk_reduce_all2), applied after
 * widening both elements to the accumulator type; integer forms wrap in the
 * accumulator type. */
typedef enum { RK_MAP2_MUL = 0, RK_MAP2_SQDIFF = 1, RK_MAP2_ABSDIFF = 2 } rk_map2;

typedef enum {
    RK_F32 = 0, RK_BF16 = 1, RK_F16 = 2, RK_F64 = 3, RK_I32 = 4, RK_I64 = 5
} rk_dtype;

typedef enum { RK_MODE_OVERWRITE = 0, RK_MODE_FOLD = 1, RK_MODE_HOST = 2 } rk_mode;

/*
 * Bytes of device workspace that rk_reduce_all (ndim = 1, reduce_mask = 1,
 * strides[0] = 1, shape[0] = n) or rk_reduce_dims needs for this layout on the
 * current device.  For a whole array this is one accumulator per first-pass
 * block plus one for the bare final partial (PR #139, "What changes": the
 * workspace holds target_blocks + 1 partial results) and a 4-byte word for
 * host mode's copied-back result, rounded up to 256
 * bytes; for a dims reduction split across blocks it is split * n_out
 * accumulators; otherwise 0.  The contents need not be initialised and the
 * same workspace may be reused by later calls of any shape and type.
 * Returns 0 for invalid arguments as well.
 */
size_t rk_workspace_size(int in_dtype, int acc_dtype, int ndim, const int64_t *shape,
                         const int64_t *strides, uint32_t reduce_mask);

/*
 * Whole-array mapped reduction of n contiguous elements at `ptr` (device
 * pointer, aligned to its element size; it need not be 16-byte aligned, so
 * offset views work).  PR #139, "What changes": at most two launches, one
 * launch when the input fits one block.  Here a larger input also takes one
 * launch: the last first-pass block to arrive folds the partials (it falls
 * back to the one-block second launch when its stream has no counter slot).
 *   init      host pointer to one accumulator-typed value, or NULL.
 *   mode      RK_MODE_OVERWRITE / RK_MODE_FOLD: `out` is a device pointer to
 *             one out-typed element; RK_MODE_HOST: `out` is a host pointer to
 *             one out-typed element, written before the call returns.
 *   workspace device pointer to >= rk_workspace_size bytes, aligned to 8
 *             bytes (may be NULL only if that size is 0).
 *   stream    hipStream_t or NULL.
 * n = 0 gives the starting value s.  Returns an rk_status.
 */
int rk_reduce_all(int op, int map, int in_dtype, int acc_dtype, int out_dtype,
                  const void *ptr, int64_t n, const void *init, int mode, void *out,
                  void *workspace, void *stream);

/*
 * Whole-array reduction of a fused two-input source: R = s (+) f(a_0, b_0)
 * (+) f(a_1, b_1) (+) ..., f one of rk_map2 -- a dot product, a squared or an
 * absolute distance.  PR #139, "What changes": the whole-array path takes a
 * lazy broadcast as its source, and the page's test list covers fused
 * sources; this is the broadcast of two arrays through f, read in one pass
 * with nothing materialised.
 *   a, b      device pointers to n contiguous in_dtype elements each, aligned
 *             to the element size; they may be the same array.  When both sit
 *             at the same offset from a 16-byte boundary the pass uses 16-byte
 *             loads, otherwise element loads (slower; rk_plan_all2 reports
 *             vec = 1).
 *   workspace >= rk_workspace_size(in_dtype, acc_dtype, 1, &n, &one, 1) bytes
 *             (the one-input whole-array size for n elements), aligned to 8.
 * op, dtypes, init, mode, out and stream as for rk_reduce_all; `out` must not
 * alias a or b.  n = 0 gives s.  Returns an rk_status.
 */
int rk_reduce_all2(int op, int map2, int in_dtype, int acc_dtype, int out_dtype,
                   const void *a, const void *b, int64_t n, const void *init, int mode,
                   void *out, void *workspace, void *stream);

/*
 * Mapped reduction along the dims in `reduce_mask` of a strided column-major
 * view with 1 <= ndim <= 4 dims (PR #176, section "This PR"; a single output
 * with a contiguous source takes the whole-array path, PR #139 "What
 * changes").  `ptr` is the device address of element (0,...,0), aligned to
 * its element size; `out` holds prod(kept extents) out-typed elements,
 * contiguous, column-major over the kept dims (device pointer; a host pointer
 * to one element in RK_MODE_HOST, which requires a single output).  `out`
 * must not alias the input.  Other arguments as for rk_reduce_all.
 */
int rk_reduce_dims(int op, int map, int in_dtype, int acc_dtype, int out_dtype,
                   const void *ptr, int ndim, const int64_t *shape, const int64_t *strides,
                   uint32_t reduce_mask, const void *init, int mode, void *out,
                   void *workspace, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * rk_reduce_dims without the workspace argument.  Same arguments, results
 * and errors as rk_reduce_dims, and the same kernels, but the partials go to
 * a scratch array of the library's own (static device memory of 2 MiB per
 * GPU, held until the process ends) instead of a workspace; the call
 * allocates nothing (HOST mode copies its result back from that scratch
 * rather than using the pinned host buffer).  Every call on one GPU shares
 * that GPU's scratch: calls on one stream are ordered and safe, but calls
 * that may overlap on one GPU (different streams, or host threads without
 * ordering) race on it and must be ordered by the caller.  The scratch keeps
 * the last call's contents; no call reads what it did not write.  Returns
 * RK_ERR_TOO_LARGE, before any launch, when the call's plan needs more
 * workspace than the scratch holds (rk_workspace_size above 2 MiB; no plan
 * on a 256-CU GPU does).
 */
int rk_reduce_dims_no_workspace(int op, int map, int in_dtype, int acc_dtype, int out_dtype,
                                const void *ptr, int ndim, const int64_t *shape,
                                const int64_t *strides, uint32_t reduce_mask, const void *init,
                                int mode, void *out, void *stream);

/* ------------------------------------------------------------------------
 * Scans (prefix folds).  PR #202 (tile scans), opening paragraph:
 * accumulate! over a whole array or along one dim.  Every line -- the
 * elements whose indices differ only along the scan dim -- is scanned on its
 * own: with x_0, x_1, ... its elements in order and s = *init (the op's
 * identity when init is NULL), output k of the line is
 *   inclusive = 1:  s (+) x_0 (+) ... (+) x_k
 *   inclusive = 0:  s (+) x_0 (+) ... (+) x_(k-1)   (output 0 is s)
 * with elements widened to the accumulator type, running values kept in it,
 * and each output converted once to out_dtype (nearest even / wrap).  The
 * association order is the library's own, so floating-point outputs may
 * differ from a sequential loop by rounding.  The dtype table, ops and
 * identities are those of the reductions; there is no map.
 * ---------------------------------------------------------------------- */

/*
 * Bytes of device workspace rk_scan_dims (or rk_scan: ndim = 1, strides[0] =
 * 1, dim = 0) needs for this layout on the current device: the tile state of
 * a look-back scan (a 256-byte header; per tile a flag and two accumulators,
 * or two per line of a tile for a strided scan dim; neighbouring tiles'
 * state in different 128-byte lines), rounded up to 256 bytes; 0 when the
 * layout takes a kernel without tiles.  Contents need not be
 * initialised; the call clears what it uses.  After a look-back scan the
 * first two 32-bit words hold the number of tiles and a timeout word, which
 * is nonzero only if a bounded wait between tiles ever gave up (then the
 * outputs are not valid).  Returns 0 for invalid arguments as well.
 */
size_t rk_scan_workspace_size(int in_dtype, int acc_dtype, int ndim, const int64_t *shape,
                              const int64_t *strides, int dim);

/*
 * Scan along dim `dim` (0-based: Julia's dims=k is dim = k-1) of a strided
 * column-major view with 1 <= ndim <= 4 dims.  `ptr` is the device address
 * of element (0,...,0), aligned to its element size; `out` is a device
 * pointer to prod(shape) out-typed elements, the view's shape stored
 * contiguously in column-major order.  `out` may be `ptr` itself when the
 * view is contiguous and the two dtypes have the same size (an in-place
 * scan); any other overlap is rejected.  init: host pointer to one
 * accumulator-typed value, or NULL.  inclusive: 1 or 0.  workspace: device
 * pointer to >= rk_scan_workspace_size bytes, aligned to 8 (NULL allowed
 * when that size is 0); a workspace must not be shared by calls that may run
 * at the same time.  stream: hipStream_t or NULL; asynchronous.  A line
 * contiguous along the scan dim and at least one tile long (or contiguous on
 * one side only, input or output, the other side's elements then moved one
 * by one; or a strided scan dim over runs of contiguous lines; or a view
 * whose input and output are contiguous along different axes) is scanned in
 * one pass with decoupled look-back between tiles.  The tiles' counter and flags (along contiguous
 * lines: all of the per-tile state) live in the library's per-stream slot
 * when they fit one (4096 tiles along contiguous lines, 8192 for a strided
 * scan dim; the last block of the call zeroes them again), otherwise in the
 * workspace, cleared by a small launch first.  Returns an rk_status.
 */
int rk_scan_dims(int op, int in_dtype, int acc_dtype, int out_dtype, const void *ptr, int ndim,
                 const int64_t *shape, const int64_t *strides, int dim, const void *init,
                 int inclusive, void *out, void *workspace, void *stream);

/* Scan of n contiguous elements: rk_scan_dims with ndim = 1, shape = {n},
 * strides = {1}, dim = 0. */
int rk_scan(int op, int in_dtype, int acc_dtype, int out_dtype, const void *ptr, int64_t n,
            const void *init, int inclusive, void *out, void *workspace, void *stream);

/* Static, human-readable name of an rk_status value. */
const char *rk_status_string(int status);

/* ------------------------------------------------------------------------
 * Diagnostics and hooks for tests and benchmarks: which kernel a call takes
 * and its plan (these launch nothing), timing of a call's first pass, the
 * device's read ceiling, and the finishing tags of a stream's slot.
 * ---------------------------------------------------------------------- */

/* Kernels a call can take.  The dims selector (PR #176, "This PR" item 1)
 * chooses among THREAD, TILED and COLUMNS for a strided reduced dim with
 * contiguous runs of outputs (in the output's order, or else in storage
 * order, each output then stored at its own place); ROW serves a contiguous
 * reduced dim, GENERIC any other layout, and a single output takes the
 * whole-array path. */
typedef enum {
    RK_KERNEL_NONE = 0,         /* nothing to compute (no outputs) */
    RK_KERNEL_ALL = 1,          /* whole-array first pass (+ one-block second pass) */
    RK_KERNEL_ALL_STRIDED = 2,  /* whole-array passes over a non-contiguous single-output view */
    RK_KERNEL_THREAD = 3,       /* one thread per output (or per 16-byte group of outputs) */
    RK_KERNEL_TILED = 4,        /* 2-d block over a narrow tile of outputs, one pass */
    RK_KERNEL_COLUMNS = 5,      /* 2-d block over a wide tile of outputs, split along the reduced dim */
    RK_KERNEL_ROW = 6,          /* one wave per output over a contiguous reduced dim */
    RK_KERNEL_GENERIC = 7,      /* one block per output, any layout */
    RK_KERNEL_ALL2 = 8,         /* whole-array passes over a two-input source (rk_reduce_all2) */
    RK_KERNEL_SCAN_TILE = 9,    /* scan: tiles of lines contiguous along the scan dim (in input and output,
                                   or on one side for a few lines), decoupled look-back (+ a clearing launch) */
    RK_KERNEL_SCAN_ROWWAVE = 10,/* scan: one wave per contiguous line shorter than a tile */
    RK_KERNEL_SCAN_LINES = 11,  /* scan: one thread per line along a strided scan dim */
    RK_KERNEL_SCAN_COLUMNS = 12,/* scan: tiles of contiguous lines x scan positions, look-back along
                                   a strided scan dim (+ a clearing launch) */
    RK_KERNEL_SCAN_TRANSPOSE = 13 /* scan: input and output contiguous along different axes (a
                                   transposed or permuted view): tiles of lines x scan positions
                                   staged through LDS, look-back along the scan dim (+ a clearing
                                   launch) */
} rk_kernel;

typedef struct {
    int kernel;               /* rk_kernel */
    int launches;             /* kernel launches the call makes: 0, 1 or 2 (1 when a split
                                 reduction finishes inside its first launch) */
    int64_t grid;             /* blocks of the first launch */
    int block;                /* threads per block of the first launch */
    int split;                /* blocks sharing one output's reduction (1 = no second pass) */
    int vec;                  /* elements per load in the first launch */
    int tile_outputs;         /* outputs per block tile (tile kernels) */
    int64_t n_out;            /* number of outputs */
    int64_t reduce_len;       /* elements folded into each output */
    size_t workspace_bytes;   /* what rk_workspace_size returns for this layout */
} rk_plan_info;

/* Plan of rk_reduce_all / rk_reduce_all2 / rk_reduce_dims for `num_cus` compute units (0 =
 * the current device), without launching.  `ptr` only matters through its
 * alignment.  Returns an rk_status. */
int rk_plan_all(int in_dtype, int acc_dtype, const void *ptr, int64_t n, int num_cus,
                rk_plan_info *info);
int rk_plan_all2(int in_dtype, int acc_dtype, const void *a, const void *b, int64_t n, int num_cus,
                 rk_plan_info *info);
int rk_plan_dims(int in_dtype, int acc_dtype, const void *ptr, int ndim, const int64_t *shape,
                 const int64_t *strides, uint32_t reduce_mask, int num_cus,
                 rk_plan_info *info);
/* Plan of rk_scan_dims: kernel is one of the RK_KERNEL_SCAN_* values (NONE
 * for an empty view), split is the tiles along each line, tile_outputs the
 * elements per tile, n_out the number of outputs and reduce_len the line
 * length. */
int rk_plan_scan(int in_dtype, int acc_dtype, int out_dtype, const void *ptr, const void *out, int ndim,
                 const int64_t *shape, const int64_t *strides, int dim, int num_cus,
                 rk_plan_info *info);

/* Whether a split reduction may finish inside its first launch (block 0
 * collecting tagged partials, or the last block to arrive; the default)
 * instead of a second launch.  Both give the same
 * results; tests switch it off to cover the second-launch path.  Process-
 * wide.  Returns the previous setting (1 or 0). */
int rk_debug_set_fused_finish(int enable);

/* Benchmark hook: while both are non-NULL, every later rk_reduce_*, rk_scan*
 * and rk_debug_stream_read call made by this host thread records hipEvent_t
 * `begin` when its first kernel starts and `end` when it ends, on the call's
 * stream (the events ride on that kernel's dispatch packet).  Pass NULLs to
 * stop.  Returns an rk_status. */
int rk_debug_set_launch_events(void *begin, void *end);

/* Test hook: make the last whole-array finishing tag of `stream`'s slot `e`
 * (every kernel translation unit), so a test can run calls across the wrap
 * of the tags: e = 2^32 - 2 makes the next call the one that wraps.  Enqueued
 * on `stream`.  Returns an rk_status: RK_ERR_INVALID_ARGUMENT for e above
 * 2^32 - 2, RK_ERR_UNSUPPORTED when the stream gets no slot. */
int rk_debug_set_finish_tag(void *stream, uint32_t e);

/* Benchmark hook: the device's read-bandwidth ceiling.  Enqueues on `stream`
 * one kernel that loads each of the nbytes / 16 vectors at `ptr` once
 * (16-byte non-temporal loads, `grid` blocks of 256 threads, 0 = 2048) and
 * does one integer operation per word; it computes nothing a caller can use.
 * `ptr`: device memory, 16-byte aligned; nbytes: a multiple of 16.  `sink`:
 * one 4-byte device word that the kernel may overwrite with an unspecified
 * value.  Asynchronous.  Honours rk_debug_set_launch_events like the
 * reductions, so both are timed on their own dispatch packets.  Returns an
 * rk_status. */
int rk_debug_stream_read(const void *ptr, int64_t nbytes, int grid, void *sink, void *stream);

/* The current device's compute units, memory clock (kHz) and memory bus
 * width (bits), as the HIP runtime reports them.  Returns an rk_status
 * (RK_ERR_HIP without a usable device). */
int rk_debug_device_info(int64_t *num_cus, int64_t *mem_clock_khz, int64_t *mem_bus_bits);

/* How many waits inside launches gave up (see "Waits inside a launch" above)
 * in calls on `stream` since the last query, plus those of calls on streams
 * that have no library slot; the counts are cleared.  It waits for `stream`
 * to drain (hipStreamSynchronize), then reads the library's counts with
 * synchronous copies, so it must not be called during graph capture.  After
 * a whole-array wait gave up it also clears the stream's tagged partials,
 * so a block of that call that had not even started when the wait gave up
 * cannot be taken for one of a later call.  `*count` receives the number
 * (0 in every normal run).  Returns an rk_status: RK_ERR_INVALID_ARGUMENT
 * for a NULL count, RK_ERR_HIP when the stream or a copy fails. */
int rk_stream_timeouts(void *stream, uint64_t *count);

/* Test hook: with polls >= 0, every later whole-array collection (split
 * whole-array calls that finish in one launch) and scan look-back waits for
 * a tag or flag that never comes and gives up after `polls` polls, as a real
 * wait would after its bound; polls < 0 restores normal waits.  Every kernel
 * still ends; the calls store no result or wrong scan outputs, and count
 * their waits for rk_stream_timeouts.  Process-wide.  Returns an rk_status. */
int rk_debug_force_wait_timeout(int64_t polls);

/* Test hook: the next `count` reduction or scan calls that pass validation
 * return RK_ERR_HIP where they would launch their first kernel, and launch
 * nothing (out and workspace untouched), as after a launch the runtime
 * rejected.  Process-wide; 0 switches it off.  Returns an rk_status. */
int rk_debug_fail_launches(int count);

#ifdef __cplusplus
}
#endif

#endif /* RK_H */
