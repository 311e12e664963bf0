/*
 * distgemm.h -- C ABI of the MI355X (gfx950) TP-step GEMM library.
 *
 * The library computes, on one GPU, that GPU's share of a tensor-parallel
 * GEMM
 *
 *     D = alpha * (scale_a * A) * (scale_b * B) + beta * C  (+ bias)
 *
 * as the sequence of TP steps that one of the Distributed GEMM schedules
 * prescribes (CUTLASS Distributed GEMM example page, "Trying out other
 * schedules": AllGather1D_TilingCD_RotatingA / _RotatingB,
 * ReduceScatter1D_TilingA_RotatingC / _TilingB_RotatingC; TP = number of
 * GPUs = number of steps).  Per the Distributed GEMM pull-request page, the
 * operand that would arrive from a peer at each step is moved by the copy
 * engine while the GEMM of the previous step runs, and each step's GEMM
 * waits for its operand before it starts.  On one GPU the peer's shard is a
 * region of the caller's full operand; the library copies it device to
 * device into the same region of a gathered image of that operand (the
 * plan's, or the caller's gathered output, see dist_gemm_run_ag), and the
 * step GEMM reads it from there.  By default one persistent kernel per run
 * does both: its workgroups copy the shards in pieces ahead of use and
 * compute the tiles of the monolithic tile grid, a tile that reads a staged
 * shard starting once a device-side counter shows the 256 rows (or columns)
 * of the gathered operand that it reads complete (DIST_GEMM_OPT_EXECUTION =
 * 1).  The alternative (= 0) launches the step GEMMs separately and copies
 * on side streams, ordered by events.
 *
 * Layouts (all row-major, element strides, batch index outermost):
 *   A : L x M x K   (K contiguous, lda = K, batch stride M*K)
 *   B : L x N x K   (the logical K x N operand stored K-contiguous,
 *                    ldb = K, batch stride N*K)
 *   C : L x M x N   (ldc = N, batch stride M*N)
 *   D : L x M x N   (ldd = N, batch stride M*N)
 * All pointers passed to dist_gemm_run are device pointers on the plan's
 * device; the caller owns them.  Element types are fixed by the plan's
 * dtype (see enum dist_gemm_dtype).
 *
 * Errors: every call returns DIST_GEMM_OK (0) or a negative code from enum
 * dist_gemm_status.  A failed call leaves no work enqueued by that call
 * except where noted, and records a message readable with
 * dist_gemm_last_error(plan) (or dist_gemm_last_error(NULL) when there is
 * no plan).  The library never exits or aborts the process.
 *
 * Threads: calls on one plan must not run concurrently; different plans may
 * be used from different host threads.
 */
#ifndef DISTGEMM_H_
#define DISTGEMM_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct dist_gemm_plan_s* dist_gemm_plan_t;

enum dist_gemm_status {
  DIST_GEMM_OK = 0,
  DIST_GEMM_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, unknown enum */
  DIST_GEMM_ERR_SHAPE = -2,       /* divisibility / alignment / size limit violated */
  DIST_GEMM_ERR_UNSUPPORTED = -3, /* valid request this build cannot run */
  DIST_GEMM_ERR_OOM = -4,         /* device allocation of plan resources failed */
  DIST_GEMM_ERR_HIP = -5          /* a HIP runtime call failed (message holds hipError_t) */
};

/* Schedules.  Rank r = 0 (one GPU).  S = TP steps.
 *   AG_ROT_A: step s consumes A row shard j = (r+s) mod S (rows
 *     [j*M/S, (j+1)*M/S)) and writes those rows of D for all N columns.
 *     Step 0 reads the local shard in place; steps 1..S-1 read a copy.
 *   AG_ROT_B: step s consumes B column shard j = (r+s) mod S (rows
 *     [j*N/S, (j+1)*N/S) of the N x K storage) and writes those columns of D.
 *   RS_TILE_A_ROT_C: step s produces row chunk j = (r+s+1) mod S (own chunk
 *     last): D[chunk] = alpha*A[chunk]*B + beta*C[chunk], where C[chunk] is
 *     the rotating partial that arrives from the previous GPU; step 0 reads
 *     it in place, steps 1..S-1 from a copy.  beta is normally 1.
 *   RS_TILE_B_ROT_C: the same over column chunks of width N/S.
 *   MONOLITHIC: one GEMM over the whole problem, no copies (the
 *     single-device GEMM the pages' reference check compares against).
 * The rotation orders are those of the PyTorch symmetric-memory page
 * (_pipelined_all_gather_and_consume, _pipelined_produce_and_all2all). */
enum dist_gemm_schedule {
  DIST_GEMM_AG_ROT_A = 0,
  DIST_GEMM_AG_ROT_B = 1,
  DIST_GEMM_RS_TILE_A_ROT_C = 2,
  DIST_GEMM_RS_TILE_B_ROT_C = 3,
  DIST_GEMM_MONOLITHIC = 4
};

/* Element types (A/B in -> C/D out).  Accumulation is always fp32.
 *   F32       : A,B fp32;            C,D fp32
 *   BF16_F32  : A,B bf16;            C,D fp32
 *   BF16_BF16 : A,B bf16;            C,D bf16 (round to nearest even)
 *   E4M3_BF16 : A,B OCP e4m3fn;      C,D bf16; per-tensor scales apply
 *   E4M3_F32  : A,B OCP e4m3fn;      C,D fp32; per-tensor scales apply
 *   E4M3_E4M3 : A,B OCP e4m3fn;      C,D OCP e4m3fn (round to nearest even,
 *               saturating at +-448; NaN stays NaN); per-tensor scales and
 *               the result scale apply
 * The scaled fp8 form follows _scaled_mm's scale_a / scale_b / scale_result
 * / out_dtype on the PyTorch symmetric-memory page
 * (fused_all_gather_scaled_matmul, fused_scaled_matmul_reduce_scatter). */
enum dist_gemm_dtype {
  DIST_GEMM_F32 = 0,
  DIST_GEMM_BF16_F32 = 1,
  DIST_GEMM_BF16_BF16 = 2,
  DIST_GEMM_E4M3_BF16 = 3,
  DIST_GEMM_E4M3_F32 = 4,
  DIST_GEMM_E4M3_E4M3 = 5
};

/* One row of the step table (host data). */
typedef struct dist_gemm_step {
  int32_t step;     /* s */
  int32_t shard;    /* shard / chunk index j */
  int32_t staged;   /* 1: operand arrives by a copy into the gathered image */
  int32_t slot;     /* position of that copy in the gathered image, in shards
                       (= shard; -1 when not staged) */
  int64_t m0, m1;   /* row range of D written by this step */
  int64_t n0, n1;   /* column range of D written by this step */
} dist_gemm_step;

/* Build the step table on the host, with no device work.  Validates exactly
 * as dist_gemm_plan does.  Writes min(*n_steps on entry, TP) rows to `out`
 * (which may be NULL when *n_steps is 0) and sets *n_steps to the number of
 * steps.  Limits: 1 <= M, N <= 2^31-1; 1 <= L <= 65535; K >= 1 with
 * K * element_size a multiple of 16 bytes; 256 * K * element_size < 2^31;
 * 1 <= TP <= 1024; S | M (AG_ROT_A, RS_TILE_A_ROT_C) or S | N (AG_ROT_B,
 * RS_TILE_B_ROT_C).  MONOLITHIC ignores TP for the step count (1 step). */
int dist_gemm_step_table(int64_t M, int64_t N, int64_t K, int64_t L, int TP, int schedule,
                         int dtype, dist_gemm_step* out, int* n_steps);

/* The single launch's work and copy tables (dist_gemm_run's default
 * execution), computed on the host with no device work, for checking the
 * schedule's bookkeeping on a CPU: exactly the tables a plan with these
 * options builds for a device running n_wg workgroups (the plan uses one
 * per CU, rounded down to a multiple of the queues).  Validates the
 * problem as dist_gemm_step_table does and the options as
 * dist_gemm_set_option does (SHARED_A, QUEUES, STEP_GROUP, COPY_AHEAD,
 * COPY_CHUNK); UNSUPPORTED for MONOLITHIC or one step.  `info` is
 * required; each array may be NULL (call once with NULLs to size them):
 *   segs   [n_segs][4]: first strip-list position, strips, tiles per batch,
 *          quota (list-0 pieces each tile claims before its GEMM);
 *   steps  [TP][7]: piece size (bytes; column strips: rows), first
 *          strip-list position, strips, pieces per strip (a strip's counter
 *          target per batch), pieces (strips x batches x pieces per strip),
 *          1 if its tiles wait for their strip, first piece in claim order;
 *   strips [2 n_strips + TP]: the strip list (step by step), the step of
 *          each position, the steps in claim order (1 .. TP-1, then 0);
 *   seg    [queues][n_segs + 1]: the first item of each segment in each
 *          queue (items of a queue: its share of each segment's tile order,
 *          batch by batch), then the queue's item count.
 * Claim lists (the gathered image not returned): list 0 is pieces
 * [0, n_list0) of the claim order, list 1 [n_list0, n_list0 + n_list1);
 * step 0's n_local pieces follow and join the last nonempty list when the
 * gathered image is returned. */
typedef struct dist_gemm_fused_info {
  int32_t n_strips;       /* strips (256 rows or columns) per batch of the gathered operand */
  int32_t n_segs;         /* queue segments */
  int32_t LG;             /* batches of the gathered image */
  int32_t cols;           /* 1: a strip is a tile column, else a tile row */
  int32_t strided;        /* 1: a strip is 256 columns of every row (RS_TILE_B_ROT_C) */
  int32_t loop;           /* 1: list 1 is copied inside K loops, one piece per starting tile */
  int32_t n_list0, n_list1, n_local;
  int32_t reserved;
  int64_t strip_bytes;    /* bytes of a full strip of one batch */
  int64_t ext;            /* rows (row strips) or columns (column strips) of the operand */
  int64_t row_bytes;      /* row strips: bytes per row; column strips: element bytes */
  int64_t height;         /* column strips: rows per batch */
  int64_t loop_capacity;  /* bytes one tile's K loop copies at most */
} dist_gemm_fused_info;
int dist_gemm_fused_tables(int64_t M, int64_t N, int64_t K, int64_t L, int TP, int schedule, int dtype,
                           int shared_a, int queues, int step_group, int copy_ahead, int64_t copy_chunk,
                           int n_wg, dist_gemm_fused_info* info, int32_t* segs, int64_t* steps,
                           int32_t* strips, int32_t* seg);

/* Create a plan on the current HIP device: validates the problem (same
 * rules as dist_gemm_step_table), builds the step table, allocates the
 * gathered image of the rotating operand (A for AG_ROT_A, B for AG_ROT_B,
 * C for the reduce-scatter schedules; L batches, same layout as the
 * operand; none for MONOLITHIC or TP = 1), the single-launch tables and
 * counters, one side stream for copies, one second compute stream, and the
 * events that order them.  *out receives the handle (NULL on failure). */
int dist_gemm_plan(int64_t M, int64_t N, int64_t K, int64_t L, int TP, int schedule, int dtype,
                   dist_gemm_plan_t* out);

/* Per-tensor dequantisation scales for the E4M3 dtypes (default 1.0 each).
 * The epilogue multiplies the fp32 accumulator by alpha*scale_a*scale_b.
 * Returns INVALID_ARG for a NULL plan or non-finite scales. */
int dist_gemm_set_scales(dist_gemm_plan_t plan, float scale_a, float scale_b);

/* Result scale of the scaled matmul with an fp8 output (the `scale_result`
 * argument that the fused scaled ops of the PyTorch symmetric-memory page
 * pass to _scaled_mm): runs after this call compute, for dtype E4M3_E4M3,
 *   D = cast_e4m3(scale_result * (alpha*scale_a*scale_b*(A B) + beta*C + bias))
 * the product, C and bias summed in fp32, then multiplied, then cast once.
 * Default 1.0.  INVALID_ARG for a NULL plan or a non-finite scale;
 * UNSUPPORTED for a scale other than 1.0 on a plan whose output is not
 * E4M3 (the result scale exists for fp8 outputs). */
int dist_gemm_set_result_scale(dist_gemm_plan_t plan, float scale_result);

/* Bias of the scaled matmul (the `bias` argument of _scaled_mm in the op
 * schemas of the PyTorch symmetric-memory page): runs after this call compute
 *   D = alpha*scale_a*scale_b*(A B) + beta*C + bias[j]
 * for every row i and batch of column j.  `bias` is a device pointer to N
 * values of the output element type (fp32, bf16 or e4m3), read by every later run
 * of the plan, so it must stay allocated while those runs may execute; the
 * plan does not own it.  NULL (the default) removes the bias.  16-byte
 * alignment (fp32 output) or 8-byte alignment (bf16 output) keeps the
 * vectorised epilogue; any alignment of the element is accepted.  Returns
 * INVALID_ARG for a NULL plan. */
int dist_gemm_set_bias(dist_gemm_plan_t plan, const void* bias);

/* Tuning options (host state of the plan; take effect at the next run).
 * Returns INVALID_ARG for a NULL plan, an unknown option or a value out of
 * range; the plan is unchanged then.
 *   DIST_GEMM_OPT_COMPUTE_STREAMS: 1 = all step GEMMs on the caller's
 *     stream; 2 (default) = steps alternate between the caller's stream and
 *     the plan's second compute stream by step parity, so the tail of one
 *     step's launch overlaps the next step (the alternation the PyTorch
 *     symmetric-memory page uses for its all-gather consumer).
 *   DIST_GEMM_OPT_COPY_ENGINE: 0 = SDMA copy engine
 *     (hipMemcpyDeviceToDeviceNoCU); 1 = the runtime's device copy
 *     (hipMemcpyDeviceToDevice, a copy kernel); 2 (default) = the library's
 *     streaming copy kernel (16-byte non-temporal loads and stores).
 *     Measured on MI355X: SDMA copies run at about 1 TB/s alone but several
 *     times slower while the step GEMMs load memory, and then gate the
 *     launches that wait for them; a copy kernel finishes in the gaps
 *     between GEMM workgroups.
 *   DIST_GEMM_OPT_STEP_TIMING: V > 0 = record a HIP event pair around every
 *     step GEMM on the stream it is launched on, keeping the pairs of the
 *     last V runs (V <= 4096); read with dist_gemm_step_times.  0 (default)
 *     = off.  Setting it waits for the plan's last run and clears the record.
 *   DIST_GEMM_OPT_COPY_STREAMS: n in 1..8 side streams carry the shard
 *     copies; staged copy k (k = 0 .. S-2, in step order) goes to side
 *     stream k mod n.  An all-gather pulls step s's shard from peer
 *     (r+s) mod S, so on a fully connected xGMI node every step's transfer
 *     has a link of its own and the transfers of different steps run
 *     concurrently; n copy streams stand in for n such links.  Default 2
 *     (with the two compute streams, four streams: the hardware queues a
 *     process gets by default).
 *   DIST_GEMM_OPT_STEP_GROUP: g in 1..1024.  Mode 0: at most g consecutive
 *     staged steps run as one GEMM launch once all of their shards have
 *     arrived.  Consecutive steps consume adjacent shards (rows of A,
 *     columns of B or of the partial) that sit side by side in the gathered
 *     image, so their GEMMs are one GEMM over the union; every output
 *     element is computed exactly as by its own step.  The step that uses
 *     the local shard launches alone.  Mode 1: the tiles of g consecutive
 *     staged steps form one queue segment, ordered and split over the work
 *     queues together (step 1 always alone, so that the launch's first
 *     round of tiles waits for as little as it can).  1 = one launch /
 *     segment per step; default 2.
 *   DIST_GEMM_OPT_EXECUTION: how a run with more than one step executes.
 *     0 = step launches and side-stream copies (the options above apply);
 *     1 (default) = one persistent launch on the caller's stream does
 *     the whole run on the monolithic tile grid: its workgroups take the
 *     tiles step by step and copy the staged shards in pieces handed out
 *     in step order by device counters (a tile whose strip is not yet
 *     complete copies pieces while it waits; a tile that starts its GEMM
 *     copies one piece of a later step inside its K loop, see COPY_AHEAD),
 *     and a tile that reads a staged shard starts once
 *     a device-side counter shows complete the strip it reads -- the 256
 *     rows (AG_ROT_A, RS_TILE_A_ROT_C) or columns (AG_ROT_B,
 *     RS_TILE_B_ROT_C) of the gathered operand that one tile row or column
 *     uses (the per-step ready barrier of the Distributed GEMM pull-request
 *     page, kept on the device per tile row or column; a strip that
 *     straddles two shards waits for both).  Every element is computed
 *     exactly as by the monolithic GEMM and by mode 0 (same kernel tile,
 *     same K order).  Single-launch runs on one device are ordered after
 *     one another, also across plans (their workgroups should not wait on
 *     each other), except inside a graph capture.
 *   DIST_GEMM_OPT_QUEUES (mode 1): 8 (default) = one work queue per XCD,
 *     each XCD runs contiguous ranges of every step's tile order; 1 = one
 *     queue for the chip.
 *   DIST_GEMM_OPT_COPY_CHUNK (mode 1, quota form below): the largest copy
 *     piece, in bytes, a multiple of 16 in [4096, 2^28]; default 2 MiB.
 *     Pieces are about a quarter of the copy bytes per claiming workgroup,
 *     whole 32 KiB above that size, at least 4 KiB, capped by this (column
 *     strips: whole rows of the strip).  The plan's device tables are
 *     rebuilt (synchronously) when it changes.
 *   DIST_GEMM_OPT_WAIT_LIMIT_US (mode 1): how long one wait for a strip
 *     may last, in microseconds, in [0, 10^8]; default 10^6.  A wait that
 *     runs out is counted (dist_gemm_device_errors) and the waiting
 *     workgroup copies the strip into the gathered image itself (the same
 *     bytes its claimers write), so the result stays correct; it only costs
 *     time.  Waits run out when the launch cannot keep a workgroup running
 *     on every work queue (other kernels holding the device's CUs), never
 *     in an unshared device; 0 makes every wait copy its own strip.
 *   DIST_GEMM_OPT_COPY_AHEAD (mode 1): D in 0..64; default 0.  The staged
 *     shards are copied in pieces from two lists: list 0, the steps the
 *     launch's first round of tiles reads, and list 1, the later steps.
 *     Every tile of the first D segments (D = 1: the local step's, which
 *     wait for nothing) claims a quota of list 0 before its GEMM (list 0 /
 *     (those tiles + the staged tiles of the first round)); a tile whose
 *     strip is not complete copies pieces while it waits (with D = 0 those
 *     tiles copy all of list 0, and the local step's start at once).  For row strips
 *     (AG_ROT_A, AG_ROT_B, RS_TILE_A_ROT_C) whose rows are a multiple of 16
 *     bytes, with K of at least 6 slabs (over 640 bytes of a row of A) and
 *     steps left after those the first round reads, list 1 is copied
 *     inside K loops: every tile that starts its GEMM while pieces are left
 *     copies one (16 KiB per 128-byte K slab, loads and stores behind the
 *     slab's operand loads; pieces an equal share of a strip, no larger
 *     than one K loop carries, as small as the steps' deadlines allow).
 *     Otherwise list 0 holds every staged step.  Workgroups with no tiles
 *     left copy whatever remains, and unaligned operand or image pointers
 *     send in-loop pieces to them too.
 *   DIST_GEMM_OPT_SHARED_A: 1 = A holds one M x K matrix that every one of
 *     the L batches multiplies (B, C, D keep their L batches): the several-B
 *     form of the PyTorch symmetric-memory page's fused all-gather matmul
 *     (one gathered A, one output per B, e.g. the gate and up projections).
 *     With AG_ROT_A the A shards are rotated once for all L products.
 *     0 (default) = A has L batches like the other operands.  Waits for the
 *     plan's last run when it changes.
 *   DIST_GEMM_OPT_FAST_ACCUM: 0 (default) or 1, the use_fast_accum flag of
 *     the fused scaled ops on the PyTorch symmetric-memory page.  It trades
 *     accumulation precision for speed on parts whose fp8 matrix units
 *     accumulate in reduced precision unless asked not to; gfx950's
 *     f8f6f4 MFMA accumulates in fp32 at full rate, so both settings run the
 *     same kernel and give the same bits.
 *   DIST_GEMM_OPT_HALF_TILES: 1 (default) or 0.  When the last round of
 *     an XCD's (mode 1: a work queue's) tiles would fill at most half of
 *     its CUs, each of those tiles runs as two 128 x 256 half-height tiles
 *     on two CUs, so the round takes about half as long.  Every element of
 *     D is computed by the same instructions in the same order either way,
 *     so the result is the same bit for bit.
 *   DIST_GEMM_OPT_COPY_DELAY_US: a test hook that holds back every shard
 *     copy by this many microseconds, in [0, 10^6] (default 0): in mode 1
 *     each workgroup starts its first copy piece no earlier than this long
 *     after it started; in mode 0 each side stream first runs a one-thread
 *     kernel that waits this long.  The consumers must wait for the late
 *     copies, so a run with a delay must equal the run without bit for bit.
 * Options that rebuild the single-launch tables (QUEUES, COPY_CHUNK,
 * COPY_AHEAD, STEP_GROUP, SHARED_A) return UNSUPPORTED, and leave the plan
 * unchanged, once a run of the plan has been captured into a graph: the
 * graph's kernel arguments hold the tables' sizes. */
enum dist_gemm_option {
  DIST_GEMM_OPT_COMPUTE_STREAMS = 0,
  DIST_GEMM_OPT_COPY_ENGINE = 1,
  DIST_GEMM_OPT_STEP_TIMING = 2,
  DIST_GEMM_OPT_COPY_STREAMS = 3,
  DIST_GEMM_OPT_STEP_GROUP = 4,
  DIST_GEMM_OPT_EXECUTION = 5,
  DIST_GEMM_OPT_QUEUES = 6,
  DIST_GEMM_OPT_COPY_CHUNK = 7,
  DIST_GEMM_OPT_WAIT_LIMIT_US = 8,
  DIST_GEMM_OPT_COPY_AHEAD = 9,
  DIST_GEMM_OPT_SHARED_A = 10,
  DIST_GEMM_OPT_COPY_DELAY_US = 11,
  DIST_GEMM_OPT_FAST_ACCUM = 12,
  DIST_GEMM_OPT_HALF_TILES = 13
};
int dist_gemm_set_option(dist_gemm_plan_t plan, int option, int64_t value);

/* Enqueue the whole TP-step schedule on `stream` (a hipStream_t; NULL = the
 * null stream) and return without waiting.  Completion of every step, copy
 * and side-stream operation is ordered before any later work on `stream`.
 *   A, B, D: required device pointers.  C: may be NULL iff beta == 0 (C is
 *   not read when beta == 0; a reduce-scatter schedule with beta == 0 then
 *   has no partial to rotate and copies nothing).  D may alias C exactly
 *   (same pointer) for the RS schedules and MONOLITHIC; no other overlap
 *   between D and A, B or C is allowed.  A and B are only read.
 * Buffers must stay allocated until the work completes on `stream`.  A run
 * on another stream first waits for the plan's previous run.
 * A reduce-scatter that averages over the ranks (the reduce_op "avg" of the
 * fused matmul + reduce-scatter on the PyTorch symmetric-memory page, which
 * averages the ranks' scaled-matmul outputs, bias included) is every rank
 * scaling its whole contribution by 1/TP before the partials are summed:
 * alpha = 1/TP and, with a bias, a bias vector divided by TP (the bias is
 * added once per step, so the sum reduction passes it unscaled).
 * Any element alignment is correct; D and C with 16-byte aligned base and
 * row pitch (fp32 output), or D with 8-byte aligned base and row pitch (bf16
 * output, beta == 0), take the vectorised epilogue, other layouts an
 * element-wise one.
 * Errors: INVALID_ARG (NULL plan/A/B/D, C NULL with beta != 0, non-finite
 * alpha/beta); HIP if an enqueue fails (earlier steps may be enqueued).
 * Graph capture: with DIST_GEMM_OPT_STEP_TIMING = 0 and the plan's previous
 * run (if any) on the same stream, a run enqueues only copies, kernel
 * launches and event record / wait pairs that fork from and join back into
 * `stream` (a single-launch run: one kernel launch), so it can be captured
 * into a HIP graph.  A captured single-launch run is not ordered against
 * single-launch runs of other plans: do not replay it while one of those
 * may run on the device (a wait that then runs out costs time, not
 * correctness; see DIST_GEMM_OPT_WAIT_LIMIT_US).  The graph uses the plan's
 * gathered image and device tables: its replays must not overlap other
 * runs of the plan, the plan must outlive the graph, and once captured the
 * plan refuses the options that rebuild its tables. */
int dist_gemm_run(dist_gemm_plan_t plan, const void* A, const void* B, const void* C, void* D,
                  float alpha, float beta, void* stream);

/* dist_gemm_run that also returns the gathered operand (the fused
 * all-gather matmul of the PyTorch symmetric-memory page returns the
 * all-gathered A beside the products): for AG_ROT_A, `ag_out` receives A
 * (L x M x K, or M x K with DIST_GEMM_OPT_SHARED_A) and for AG_ROT_B it
 * receives B (L x N x K), in the operand's layout.  `ag_out` replaces the
 * plan's gathered image for this run: every staged shard is copied into
 * it and the steps that consume a copied shard read it from there, and the
 * local shard is copied into it too, so on completion it equals the
 * operand bit for bit.  The caller owns `ag_out` (device memory on the
 * plan's device, not overlapping A, B, C or D) and keeps it allocated until
 * the run completes on `stream`.  INVALID_ARG for a NULL `ag_out` or a
 * reduce-scatter or MONOLITHIC plan (nothing is gathered there); otherwise
 * as dist_gemm_run. */
int dist_gemm_run_ag(dist_gemm_plan_t plan, const void* A, const void* B, const void* C, void* D,
                     void* ag_out, float alpha, float beta, void* stream);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation: one run
 * of the problem (M, N, K, L, TP, schedule, dtype; same validation and
 * layouts as dist_gemm_plan and dist_gemm_run) with no plan, computing
 *   D = alpha*scale_a*scale_b*(A B) + beta*C
 * exactly as a plan's default single-launch run does (bit for bit), with
 * scale_a / scale_b as dist_gemm_set_scales (ignored unless the dtype is an
 * E4M3 one; pass 1.0f).  It allocates nothing: the gathered image, the
 * single-launch tables and the counters live in one file-scope device array
 * of 32 MiB + 256 KiB that every GPU running this call holds until the
 * process ends (its address taken on each device's first call, which also
 * creates the event that orders single-launch runs on the device).  Limits
 * (UNSUPPORTED, with a message, beyond them): at most 16 steps, at most 128
 * strips of 256 rows (AG_ROT_A, RS_TILE_A_ROT_C) or columns (AG_ROT_B,
 * RS_TILE_B_ROT_C), a gathered rotating operand of at most 32 MiB
 * (L x M x K, L x N x K or L x M x N elements), and L x (strips + steps) at
 * most 61440.  MONOLITHIC or TP = 1 runs one GEMM and uses no scratch.
 * Calls on one GPU share the array, which keeps the last call's contents
 * (each call rewrites its tables and clears its counters first): calls that
 * overlap on one GPU race, so issue them on one stream, or order them; the
 * library orders uncaptured calls on a device after one another anyway.
 * Errors: as dist_gemm_plan plus dist_gemm_run; the message is read with
 * dist_gemm_last_error(NULL). */
int dist_gemm_run_noalloc(int64_t M, int64_t N, int64_t K, int64_t L, int TP, int schedule, int dtype,
                          const void* A, const void* B, const void* C, void* D, float alpha, float beta,
                          float scale_a, float scale_b, void* stream);

/* Query the plan's step table (same contents as dist_gemm_step_table). */
int dist_gemm_plan_steps(dist_gemm_plan_t plan, dist_gemm_step* out, int* n_steps);

/* With DIST_GEMM_OPT_STEP_TIMING = V set: wait for the last run to finish and
 * write the step GEMM durations in milliseconds of the last R = min(runs, V)
 * timed runs, oldest run first, steps in order (R * steps values, at most *n
 * written); *n receives R * steps.  Steps that ran as one launch share its
 * duration equally.  UNSUPPORTED if no timed run exists. */
int dist_gemm_step_times(dist_gemm_plan_t plan, float* ms, int* n);

/* With DIST_GEMM_OPT_STEP_TIMING set: wait for the last run to finish and
 * write its timeline, three values per step in step order, in milliseconds
 * since the run was enqueued on its stream: [3s] = the moment the step's
 * shard copy completed (-1 for a step that consumes no copy), [3s+1] = the
 * GEMM work of the step began, [3s+2] = it ended.  Step launches (mode 0):
 * event times of the copy and of the launch that computed the step.  One
 * launch (mode 1): the device's own wall-clock stamps -- the last strip of
 * the step complete, the first tile of the step starting after its wait,
 * the last tile of the step done -- placed on the run's time line by the
 * launch's start event (-1 where a step has no copy or no tile of its own:
 * strips that straddle two shards count for the later step).  At most *n
 * values are written; *n receives 3 * steps.  UNSUPPORTED if no timed run
 * exists. */
int dist_gemm_step_timeline(dist_gemm_plan_t plan, float* ms, int* n);

/* Wait for the plan's last run and write to *count the number of device-side
 * strip waits that ran out of time (DIST_GEMM_OPT_WAIT_LIMIT_US) in all
 * single-launch runs of the plan so far; each such workgroup copied its
 * strip itself, so results stay correct.  0 on an unshared device.
 * INVALID_ARG for NULL arguments; HIP if the read fails. */
int dist_gemm_device_errors(dist_gemm_plan_t plan, int64_t* count);

/* Synchronise the plan's streams, free its staging, streams and events, and
 * the handle.  NULL is accepted (no-op). */
int dist_gemm_destroy(dist_gemm_plan_t plan);

/* Message of the last failure on `plan` (NULL: the last failure of a call
 * without a plan, per thread).  Never NULL; valid until the next call. */
const char* dist_gemm_last_error(dist_gemm_plan_t plan);

/* Static name of a status code. */
const char* dist_gemm_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* DISTGEMM_H_ */
