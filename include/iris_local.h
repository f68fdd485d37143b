/*
 * iris_local: one GPU's share of Iris-style fused communication + GEMM ops
 * on AMD Instinct MI355X (gfx950). C ABI.
 *
 * Sources of the operation definitions:
 *   [DOCS]   Iris docs, "Fused Communication and Compute Operations":
 *            entries all_gather_matmul, matmul_reduce_scatter,
 *            matmul_all_reduce (signatures: output, inputs, optional bias of
 *            length M or N, optional FusedConfig, optional workspace).
 *   [PR544]  ROCm/iris PR "Add iris.concurrent (concurrent, independent,
 *            fused comm+gemm)": description (persistent work-stealing
 *            kernels, the GEMM/comm split `gemm_wgs` and the GEMM tile are
 *            the knobs; fused = one persistent kernel with two work-stealing
 *            queues) and review answer (the GEMM and the collective are
 *            independent).
 *   [PR506]  ROCm/iris PR "Add auto-config selection for fused AG+matmul
 *            with 28 tuned HBM buffer configs": summary (config=None selects
 *            a configuration automatically; only the NN layout is supported).
 *
 * One GPU's share: the other ranks' shards and partial buffers are stand-in
 * buffers already resident in this GPU's memory, passed by pointer. There is
 * no communication between GPUs here.
 *
 * Data conventions (all entry points):
 *   - fp16 is IEEE binary16, stored as 2-byte elements.
 *   - Matrices are row-major and contiguous (the NN layout of [PR506]).
 *   - Every matrix and vector pointer is a DEVICE pointer, 16-byte aligned.
 *     Pointer ARRAYS (A_shards, partials, comm_in) are HOST arrays of device
 *     pointers; the library copies them before returning.
 *   - Row lengths must be multiples of 8 elements (16 bytes): K_local (or K)
 *     and N for the GEMM, N/W for reduce_scatter.
 *   - Outputs must not overlap inputs.
 *   - bias may be NULL. It has N entries (added to every row), or M entries
 *     (added to every column) when IRIS_FLAG_BIAS_ALONG_M is set.
 *   - Accumulation is fp32; every fp16 output is rounded once, to nearest
 *     even.
 *
 * Ownership: the caller owns every buffer. The library keeps no caller
 * pointer after the work it enqueued has run. If `workspace` is NULL the
 * library uses a workspace of its own per (device, stream), allocated on
 * first use and released by iris_finalize().
 *
 * Synchronisation: every op only enqueues work on `stream` (a hipStream_t
 * passed as void*; NULL is the default stream) and returns without waiting.
 * Two calls that share one workspace must not run concurrently.
 *
 * Errors: every function returns an iris_status (0 = IRIS_OK). Arguments are
 * validated before any HIP call; on error nothing is enqueued. A
 * human-readable message for the last error on the calling thread is
 * returned by iris_last_error_message().
 */
#ifndef IRIS_LOCAL_H
#define IRIS_LOCAL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define IRIS_MAX_W 16

typedef enum iris_status {
  IRIS_OK = 0,
  IRIS_ERR_INVALID_ARG = 1,   /* NULL pointer, bad size, W out of range, ... */
  IRIS_ERR_UNSUPPORTED = 2,   /* a valid request this build does not serve */
  IRIS_ERR_CONFIG = 3,        /* tile shape / gemm_wgs / mode not allowed */
  IRIS_ERR_ALIGNMENT = 4,     /* pointer not 16-byte aligned or row length % 8 */
  IRIS_ERR_NO_MEMORY = 5,     /* internal workspace allocation failed */
  IRIS_ERR_HIP = 6,           /* a HIP runtime call failed (message has it) */
  IRIS_ERR_WORKSPACE = 7,     /* caller workspace smaller than required */
  IRIS_ERR_NO_DEVICE = 8,     /* no usable gfx950 device */
  IRIS_ERR_DEVICE_TIMEOUT = 9 /* a bounded device-side wait expired */
} iris_status;

/*
 * Every device-side wait (a GEMM tile for its gathered rows, a reduce unit
 * for its tiles) polls at most a bounded number of times, then records an
 * error in the workspace and goes on, so every launch ends. The last
 * workgroup of the launch folds that error into the workspace's status word,
 * which keeps it until iris_check_device_error() reads and clears it. An op
 * call itself does not wait for its kernels, so it returns IRIS_OK even when
 * one of its waits later gives up: call iris_check_device_error() after the
 * ops whose outputs you rely on. With the environment variable
 * IRIS_LOCAL_DEBUG set, every op makes that check itself before returning
 * (synchronizing its stream). IRIS_LOCAL_SPIN_LIMIT=n (n >= 0) sets the poll
 * bound (default 2^24), so that the error path can be exercised.
 */

/* execution modes ([PR544] description) */
#define IRIS_MODE_FUSED 0      /* one persistent kernel, two work queues */
#define IRIS_MODE_SEQUENTIAL 1 /* comm kernel and GEMM kernel, one after the
                                  other on the same stream, each on the whole
                                  GPU (the unfused baseline); an all_gather
                                  larger than 256 MiB runs its copy on the
                                  persistent kernel's copy workgroups alone */
#define IRIS_MODE_TWO_STREAM 2 /* GEMM kernel on gemm_wgs workgroups on the
                                  caller's stream, comm kernel beside it on a
                                  second stream of the library's; only for ops
                                  whose GEMM and collective are independent
                                  (iris_concurrent, iris_mm_ag_local), others
                                  give IRIS_ERR_CONFIG ([PR544]: mode
                                  "concurrent", separate persistent kernels on
                                  different streams) */

/* config flags */
#define IRIS_FLAG_NO_STEAL 1     /* workgroups stay on their first queue */
#define IRIS_FLAG_BIAS_ALONG_M 2 /* bias has M entries instead of N */
#define IRIS_FLAG_NO_LOCKSTEP 4  /* GEMM rounds of an XCD queue may overlap (no
                                    wait for the previous round's tiles);
                                    same results, for measuring what the
                                    lockstep saves */

/* op ids (workspace sizing, tuning) */
#define IRIS_OP_AG_MM 1
#define IRIS_OP_MM_RS 2
#define IRIS_OP_MM_AR 3
#define IRIS_OP_CONCURRENT 4
#define IRIS_OP_MM_AG 5

/* collectives for iris_concurrent ([PR544] description: all_gather,
 * all_reduce, reduce_scatter, all_to_all, broadcast) */
#define IRIS_COLL_ALL_REDUCE 1
#define IRIS_COLL_ALL_GATHER 2
#define IRIS_COLL_REDUCE_SCATTER 3
#define IRIS_COLL_ALL_TO_ALL 4
#define IRIS_COLL_BROADCAST 5

/*
 * Tuning knobs ([PR544]: the GEMM/comm split gemm_wgs and the GEMM tile;
 * [DOCS]: FusedConfig). A field <= 0 means "choose automatically": the
 * tuned value cached for this shape if there is one (iris_tune_gemm_wgs),
 * else the built-in default. Passing NULL means all fields automatic.
 *   block_m, block_n  GEMM output tile; supported pairs: 256x256, 256x128,
 *                     128x128, 64x64. Default 256x256.
 *   block_k           K step; 64 only. Default 64.
 *   group_m           rows of tiles per swizzle group. Default 8.
 *   gemm_wgs          workgroups that start on the GEMM queue in fused mode,
 *                     1..G-1 where G = iris_grid_size(op, cfg). Default
 *                     7/8 of G. The others start on the comm queue and
 *                     take GEMM tiles once it is empty (unless
 *                     IRIS_FLAG_NO_STEAL); in iris_ag_mm with more GEMM
 *                     tiles than G they take tiles only after every copy
 *                     unit has finished, so that they start in step. Any
 *                     value gives bit-identical results.
 *   comm_block_m      rows per comm unit (all_gather copy and the
 *                     reduce of reduce_scatter / matmul_all_reduce); must
 *                     divide block_m. Default: the largest power of two
 *                     dividing block_m that keeps a unit near 128 KiB of
 *                     shard (copy) or 32 KiB per buffer (reduce).
 *   comm_block_n      columns per reduce unit (reduce_scatter and
 *                     matmul_all_reduce), multiple of 8. Default block_n.
 *   comm_chunk        elements per flat unit (the collectives of
 *                     iris_concurrent, the peer blocks of iris_mm_ag_local),
 *                     multiple of 2048. Default 65536.
 *   mode              IRIS_MODE_FUSED (default), IRIS_MODE_SEQUENTIAL or
 *                     IRIS_MODE_TWO_STREAM.
 *   flags             IRIS_FLAG_* bits.
 */
typedef struct iris_config {
  int32_t block_m;
  int32_t block_n;
  int32_t block_k;
  int32_t group_m;
  int32_t gemm_wgs;
  int32_t comm_block_m;
  int32_t comm_block_n;
  int32_t comm_chunk;
  int32_t mode;
  int32_t flags;
} iris_config_t;

/*
 * all_gather_matmul, local share ([DOCS] all_gather_matmul):
 *   A_gathered[m][s*K_local + k] = A_shards[s][m][k]       (bit copy)
 *   C = A_gathered @ B + bias
 * C: (M, N) fp16 out. A_gathered: (M, W*K_local) fp16 out, the gathered
 * buffer the GEMM reads. A_shards: host array of W device pointers, each
 * (M, K_local) fp16, in rank order. B: (W*K_local, N) fp16. bias: N (or M).
 * In fused mode comm workgroups copy the shards while GEMM workgroups
 * compute; a GEMM tile starts on row block pm once every shard of that row
 * block has landed.
 */
int iris_ag_mm(void* C, void* A_gathered, const void* const* A_shards, int32_t W,
               const void* B, const void* bias, int64_t M, int64_t N,
               int64_t K_local, const iris_config_t* cfg, void* workspace,
               size_t workspace_bytes, void* stream);

/*
 * iris_ag_mm without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, allocation-free serving loops,
 * harnesses that forbid hipMalloc). Same arguments, results and modes as
 * iris_ag_mm; the workspace is a static device array of 1 MiB that each GPU
 * the library runs on holds until the process ends, so this entry point
 * calls no allocator. Sizes whose workspace (iris_workspace_size) exceeds
 * 1 MiB give IRIS_ERR_WORKSPACE before any HIP call (at 256x256 tiles:
 * M up to about 1.7 million rows). The first call on a device enqueues a
 * kernel that zeroes the array on `stream` ahead of the op. Every call on a
 * GPU shares that GPU's array: calls that overlap in time on one GPU (other
 * streams, other threads) race and must not be made; calls in stream order
 * are fine, since each op leaves the array zeroed for the next.
 * iris_check_device_error(NULL, stream) also reports the array's status.
 */
int iris_ag_mm_noalloc(void* C, void* A_gathered, const void* const* A_shards, int32_t W,
                       const void* B, const void* bias, int64_t M, int64_t N,
                       int64_t K_local, const iris_config_t* cfg, void* stream);

/*
 * matmul_reduce_scatter, local share for rank `rank` of W
 * ([DOCS] matmul_reduce_scatter, along N):
 *   C = A @ B + bias                                         (M, N)
 *   out[m][j] = C[m][rank*N/W + j] + sum_{p<W-1} partials[p][m][j]
 * out: (M, N/W) fp16 out. C: (M, N) fp16 out (this rank's full partial
 * product; the reduction reads its own slice back from C). partials: host
 * array of W-1 device pointers, each (M, N/W) fp16, standing in for the
 * other ranks' slices. Requires N % W == 0 and (N/W) % 8 == 0.
 */
int iris_mm_rs_local(void* out, void* C, const void* A, const void* B,
                     const void* bias, const void* const* partials, int32_t W,
                     int32_t rank, int64_t M, int64_t N, int64_t K,
                     const iris_config_t* cfg, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * matmul_all_reduce, local share ([DOCS] matmul_all_reduce):
 *   C = A @ B + bias;  out = C + sum_{p<W-1} partials[p]          (M, N)
 * partials: host array of W-1 device pointers, each (M, N) fp16.
 */
int iris_mm_ar_local(void* out, void* C, const void* A, const void* B,
                     const void* bias, const void* const* partials, int32_t W,
                     int64_t M, int64_t N, int64_t K, const iris_config_t* cfg,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * matmul_all_gather, local share ([DOCS] matmul_all_gather):
 *   out (M*W, N) = all_gather along M of every rank's A @ B + bias
 * This rank's block, rows [rank*M, (rank+1)*M), is computed here (the GEMM
 * writes it in place); the other W-1 blocks are copied from peer_blocks: a
 * host array of W-1 device pointers, each (M, N) fp16, standing in for the
 * other ranks' results, in rank order with this rank left out. The copies
 * do not depend on this rank's GEMM. A bias along M has M entries (rows of
 * this rank's block).
 */
int iris_mm_ag_local(void* out, const void* A, const void* B, const void* bias,
                     const void* const* peer_blocks, int32_t W, int32_t rank,
                     int64_t M, int64_t N, int64_t K, const iris_config_t* cfg,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Independent GEMM beside a collective ([PR544]), local share of rank
 * `rank` of W:
 *   C = A @ B + bias                                    (M, N), and
 * independently, with comm_in a host array of W device pointers (every
 * rank's buffer of n = comm_elems fp16 in rank order, this rank's own
 * included):
 *   IRIS_COLL_ALL_REDUCE      comm_out[i] = sum_w comm_in[w][i]          (n)
 *   IRIS_COLL_ALL_GATHER      comm_out[w*n + i] = comm_in[w][i]        (W*n)
 *   IRIS_COLL_REDUCE_SCATTER  comm_out[i] = sum_w comm_in[w][rank*n/W + i]
 *                                                                      (n/W)
 *   IRIS_COLL_ALL_TO_ALL      comm_out[j*n/W + i] = comm_in[j][rank*n/W + i]
 *                                                                        (n)
 *   IRIS_COLL_BROADCAST       comm_out[i] = comm_in[rank][i], rank being the
 *                             root                                       (n)
 * Sums run in fp32 in rank order and round once to fp16; the others are bit
 * copies. n % 8 == 0; for reduce_scatter and all_to_all also n % (8 W) == 0.
 * 0 <= rank < W (ignored by all_reduce and all_gather).
 */
int iris_concurrent(void* C, const void* A, const void* B, const void* bias,
                    int64_t M, int64_t N, int64_t K, int32_t collective,
                    int32_t rank, void* comm_out, const void* const* comm_in,
                    int32_t W, int64_t comm_elems, const iris_config_t* cfg,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace an op needs (0 on invalid arguments). The
 * workspace holds per-workgroup timestamps, then the queue counters (one
 * GEMM queue per XCD and the comm queue), the finished-workgroup and
 * finished-unit counters, the error and status words and the ready flags.
 * A caller passing its own must give at least this much, 256-byte aligned
 * and ZERO-FILLED before its first use; every op leaves it zeroed again (the
 * last workgroup of the launch clears what the launch used) except for the
 * status word, which only iris_check_device_error() clears, so one zero fill
 * serves any number of later ops. */
size_t iris_workspace_size(int32_t op, int64_t M, int64_t N, int64_t K, int32_t W,
                           const iris_config_t* cfg);

/* Persistent grid size G (workgroups) the fused kernel of `op` (IRIS_OP_*)
 * launches on the current device for this config: CUs times the
 * workgroups of that kernel resident per CU. Negative iris_status on error. */
int iris_grid_size(int32_t op, const iris_config_t* cfg);

/*
 * Host-side CU-split sweep ([PR544]: benchmark candidates, always including
 * the static default, cache the winner). Runs the op described by `args`
 * in fused mode once per candidate gemm_wgs (warmup + `reps` timed runs,
 * median), writes the winner to *best_gemm_wgs and the median milliseconds
 * of each candidate to ms_out[i] (may be NULL), and stores the winner in the
 * tuning cache (file named by IRIS_LOCAL_TUNE_CACHE, default
 * ~/.cache/iris_local/tune.json, one JSON object of key -> gemm_wgs; written to a temporary file then renamed;
 * a failed write is ignored; the file is read once per process, and this
 * process's later tunings update that copy). Blocks until done. Ties go to more GEMM
 * workgroups. The op's outputs hold the last candidate's results.
 * top_k > 0 (and below n_candidates): rank the candidates with
 * iris_predict_gemm_wgs first and benchmark only the top_k best predicted
 * (plus the default); ms_out of a candidate left out is -1. If the
 * predictor cannot tell the candidates apart (all predictions equal), every
 * candidate is benchmarked.
 */
typedef struct iris_op_args {
  int32_t op;             /* IRIS_OP_* */
  void* C;
  void* out;              /* A_gathered (AG), out (RS/AR/MM_AG), comm_out (concurrent) */
  const void* A;          /* A (RS/AR/MM_AG/concurrent); unused for AG */
  const void* const* srcs;/* A_shards (AG), partials (RS/AR), peer_blocks (MM_AG), comm_in */
  int32_t W;
  int32_t rank;           /* RS, MM_AG, and the concurrent collectives */
  int32_t collective;     /* IRIS_OP_CONCURRENT only */
  const void* B;
  const void* bias;
  int64_t M, N, K;        /* K is K_local for AG */
  int64_t comm_elems;     /* concurrent only */
  iris_config_t cfg;      /* gemm_wgs is overridden by each candidate */
} iris_op_args_t;

int iris_tune_gemm_wgs(const iris_op_args_t* args, const int32_t* candidates,
                       int32_t n_candidates, int32_t reps, int32_t top_k,
                       int32_t* best_gemm_wgs, float* ms_out, void* stream);

/*
 * Analytical CU split ([PR544]: predictor, a work-stealing makespan
 * simulation used to rank splits before benchmarking the top k). Replays
 * the fused schedule of the op in `args` on a grid of `grid` workgroups for
 * each candidate gemm_wgs (1 .. grid-1) with modelled durations, writes the
 * predicted milliseconds to predicted_ms[i] (may be NULL) and the best
 * candidate to *best_gemm_wgs (ties to more GEMM workgroups). Host code
 * only: no device call and no workspace; errors set iris_last_error_message.
 * params may be NULL (a rate <= 0 or an overhead, slowdown or penalty < 0
 * means its default); the defaults were measured on MI355X:
 *   gemm_tflops_per_cu      K-loop rate of one CU (256x256 tiles) with
 *                           every CU on the GEMM                    5.0
 *   tile_overhead_us        fixed cost per GEMM tile                20
 *   comm_gbps_per_cu        copy/reduce rate of one workgroup       45
 *   comm_gbps_chip          comm bandwidth of the whole chip        5200
 *   unit_overhead_us        fixed cost per comm unit                1
 *   gemm_tflops_per_cu_max  K-loop rate of one CU when few run the    5.25
 *                           GEMM (the chip's MFMA throughput is
 *                           capped by power: with n workgroups on
 *                           the GEMM queue tiles run at
 *                           min(this, gemm_tflops_per_cu * grid/n))
 *   gemm_slowdown           relative GEMM slowdown while the comm      0.10
 *                           workgroups can use the whole chip's comm
 *                           bandwidth
 *   comm_slowdown           relative comm slowdown while every         0.60
 *                           workgroup works the GEMM queue
 *   phase_penalty           relative slowdown of every tile when the   0.045
 *                           tiles of a multi-wave GEMM start with
 *                           fully spread phases (operands no longer
 *                           meet in L2)
 * The last four were fitted to measured sweeps of the bench workloads.
 */
typedef struct iris_predict_params {
  double gemm_tflops_per_cu;
  double tile_overhead_us;
  double comm_gbps_per_cu;
  double comm_gbps_chip;
  double unit_overhead_us;
  double gemm_tflops_per_cu_max;
  double gemm_slowdown;
  double comm_slowdown;
  double phase_penalty;
} iris_predict_params_t;

int iris_predict_gemm_wgs(const iris_op_args_t* args, int32_t grid, const int32_t* candidates,
                          int32_t n_candidates, const iris_predict_params_t* params,
                          float* predicted_ms, int32_t* best_gemm_wgs);

/*
 * Windows of the last op that used `workspace` (or the library's own
 * workspace for `stream` if workspace is NULL), from per-workgroup device
 * timestamps, in nanoseconds since the earliest stamp: the first start and
 * last end of any GEMM tile, and of any comm unit. In sequential mode the
 * comm window comes from the comm kernel and the GEMM window from the GEMM
 * kernel. A window with no work reads -1. Waits for `stream`. Any output may
 * be NULL.
 */
int iris_last_windows(void* workspace, void* stream, double* gemm_start_ns,
                      double* gemm_end_ns, double* comm_start_ns,
                      double* comm_end_ns);

/*
 * Shader clock (MHz) the device held during the last persistent launch that
 * used `workspace` (NULL: the library's own workspace for `stream`): the
 * shader-clock counter (s_memtime) over the constant-rate counter
 * (s_memrealtime), summed over that launch's workgroups from entry to exit.
 * Waits for `stream`. *mhz is -1 if nothing was recorded.
 */
int iris_last_clock(void* workspace, void* stream, double* mhz);

/*
 * Measurement helper (no counterpart on the pages): the dense fp16 MFMA rate
 * of the current device with no memory traffic, the achievable ceiling that
 * the GEMM's rate is compared with beside the published peak.
 * CUs x 4 workgroups of 4 waves each run `iters` trips of eight
 * v_mfma_f32_32x32x16_f16 on eight independent accumulators, operands in
 * registers: random fp16 values that change from one instruction to the
 * next if `random_operands` is non-zero (the multipliers then switch as on
 * GEMM data), else constants. One short warm-up launch, then one timed
 * launch on `stream`; waits for it. Allocates and frees two small device
 * buffers.
 *   *tflops     FLOP of the timed launch / its duration (HIP events)
 *   *clock_mhz  shader clock held, from the kernel's own counters
 * Errors: IRIS_ERR_INVALID_ARG (NULL outputs; iters outside [1, 2^22], checked
 * before any HIP call), IRIS_ERR_HIP. Outputs are -1 on error.
 */
int iris_mfma_ceiling(int32_t random_operands, int32_t iters, void* stream, double* tflops, double* clock_mhz);

/*
 * Device-side errors since the last check on `workspace` (NULL: the
 * library's own workspace for `stream` and the device's static scratch of
 * iris_ag_mm_noalloc). Waits for `stream`, then returns
 * IRIS_ERR_DEVICE_TIMEOUT (and clears the status) if a device-side wait of
 * any fused op on that workspace gave up since the last check: the outputs
 * of those ops are then not to be trusted. IRIS_OK otherwise, also when no
 * op has used the library's workspace for `stream` yet.
 */
int iris_check_device_error(void* workspace, void* stream);

/*
 * Facts about a device, and the peak rates that roofline fractions are
 * taken against. peak_fp16_tflops is the dense fp16 matrix rate at the
 * maximum engine clock: CUs x clock x 4096 FLOP per CU per clock (gfx950:
 * four matrix units per CU, each 1024 fp16 FLOP per clock; 2.5 PFLOP/s on
 * MI355X at 2.4 GHz). peak_hbm_gbps is the published HBM3E bandwidth of the
 * gfx950 parts (8 TB/s); 0 for a device this library does not run on.
 */
typedef struct iris_device_info {
  int32_t device;
  int32_t compute_units;
  int32_t clock_khz;         /* max engine clock */
  int32_t memory_clock_khz;
  int32_t lds_bytes_per_cu;
  int64_t global_mem_bytes;
  char arch[64];             /* gcnArchName, e.g. "gfx950:sramecc+:xnack-" */
  double peak_fp16_tflops;   /* dense fp16 MFMA peak at clock_khz */
  double peak_hbm_gbps;      /* published HBM bandwidth, GB/s */
} iris_device_info_t;

int iris_device_info(int32_t device, iris_device_info_t* info);

const char* iris_status_str(int32_t status);
/* Message for the last error on this thread ("" if none). */
const char* iris_last_error_message(void);
/* Frees the library's own workspaces and the stream and events of the
 * two-stream mode. */
int iris_finalize(void);

#ifdef __cplusplus
}
#endif

#endif /* IRIS_LOCAL_H */
