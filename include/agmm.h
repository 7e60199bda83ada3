/*
 * agmm.h — fused all-gather + GEMM for AMD MI355X (gfx950): the C ABI.
 *
 * Operation (pytorch/helion PR "[Benchmark] Add all gather matmul benchmark", Kraken
 * optimization comment: a = all_gather(a_shared), out = a @ b; the same comment's
 * local-tile index formula fixes the row order):
 *
 *     out[M, N] = concat(shard_0, ..., shard_{D-1})[M, K] @ B[K, N]  (+ bias[N])
 *
 * Shard d is a row-major [M/D, K] matrix holding global rows [d*M/D, (d+1)*M/D). All
 * matrices are row-major and contiguous; inputs, bias and output share one 16-bit type
 * (fp16 or bf16); products accumulate in fp32 and the result is rounded once (RNE).
 *
 * Method (ROCm/iris issue "Fused all-gather+GEMM HBM-buffer kernel for iris.ops", opening
 * summary and "New kernel"): one persistent kernel splits its workgroups into fetchers
 * and GEMM workers. Fetchers copy A tiles into a local HBM staging buffer (k_contiguous
 * or m_contiguous layout) and publish one ready flag per tile; GEMM workers wait on those
 * flags and compute each output tile as its A tiles arrive, so there is no whole-gather
 * barrier. Tiles of the local shard (`rank`) are read in place and never staged (Helion
 * thread, Kraken optimization). A baseline variant copies every staged tile first, then
 * runs the GEMM (the barrier-based baseline of the iris issue).
 *
 * On one GPU the D shards are D separate device allocations standing in for the D ranks'
 * shards; the staging copy is the all-gather's local half.
 *
 * Threading: a handle is used by one host thread at a time. Errors are returned as
 * negative codes; no C++ exception or abort crosses this interface.
 */
#ifndef AGMM_H
#define AGMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AGMM_MAX_SHARDS 64

/* ---- return codes ---- */
#define AGMM_OK 0
#define AGMM_ERR_INVALID_ARG (-1)  /* null / misaligned pointer, bad count, aliasing output */
#define AGMM_ERR_UNSUPPORTED (-2)  /* a shape or option the library does not handle */
#define AGMM_ERR_HIP (-3)          /* a HIP runtime call failed; see ag_matmul_last_hip_error */
#define AGMM_ERR_OOM (-4)          /* device allocation failed */
#define AGMM_ERR_TIMEOUT (-5)      /* a flag wait exceeded its spin limit; handle is poisoned */
#define AGMM_ERR_WRONG_DEVICE (-6) /* current HIP device differs from the handle's device */
#define AGMM_ERR_POISONED (-7)     /* an earlier run timed out; destroy and recreate */
#define AGMM_ERR_TOO_LARGE (-8)    /* ag_matmul_run_static: workspace exceeds the scratch */

/* ---- enumerations ---- */
#define AGMM_F16 0
#define AGMM_BF16 1

/* Staging-buffer layout (iris issue, "New kernel": k_contiguous and m_contiguous staged-A
 * layouts, named but not defined there). Reading used here: the unit-stride dimension of
 * the staging buffer. k_contiguous: staging is [M][K], element (m, k) at m*K + k (a straight
 * copy of the gathered rows). m_contiguous: staging is [K][M], element (m, k) at k*M + m
 * (the fetcher transposes). */
#define AGMM_K_CONTIGUOUS 0
#define AGMM_M_CONTIGUOUS 1

#define AGMM_ALGO_FUSED 0     /* fetcher + GEMM workgroups in one persistent kernel */
#define AGMM_ALGO_BASELINE 1  /* copy kernel, then stream order (the barrier), then GEMM */
/* Host stream pipeline (NVIDIA/Fuser PR #3695, the AG+GEMM host program: A's rows cut into S
 * chunks along each shard, and for chunk i, on stream i % streams (stream 0 being the
 * caller's), the chunk's all-gather, a wait for it, then the chunk's GEMM; the caller's
 * stream then waits for every other stream).
 * Chunk i holds rows [i*M_s/S, (i+1)*M_s/S) of every shard; here the chunk's gather is the
 * copy kernel over its staged units and its GEMM the GEMM-only kernel over its m-tiles, so
 * one chunk's copy overlaps another chunk's GEMM without flags. Staging is [M][K]. */
#define AGMM_ALGO_PIPELINED 2

/* Problem and tuning description. Fields marked "0 = auto" are chosen by create. */
typedef struct agmm_desc {
  int32_t D;             /* number of shards, 1..AGMM_MAX_SHARDS */
  int32_t rank;          /* index of the local shard, 0..D-1 */
  int64_t M, N, K;       /* gathered rows (M = D * M_shard), columns, inner dimension */
  int32_t dtype;         /* AGMM_F16 or AGMM_BF16 for shards, B, bias and out */
  int32_t layout;        /* AGMM_K_CONTIGUOUS or AGMM_M_CONTIGUOUS (fused algorithm) */
  int32_t algo;          /* AGMM_ALGO_FUSED, AGMM_ALGO_BASELINE or AGMM_ALGO_PIPELINED */
  int32_t direct_local;  /* 1: local-shard tiles read in place; 0: every tile staged */
  int32_t has_bias;      /* 1: run() takes a bias[N] pointer; 0: bias must be NULL */
  int32_t debug;         /* 1: record per-workgroup trace; fill the staging buffer with a
                            quiet NaN before every run (so a read of unwritten staging shows
                            in the output); run() synchronizes and reports
                            a flag-wait timeout as AGMM_ERR_TIMEOUT */
  int32_t block_m;       /* output tile edge: 64, 128 or 256 (tile is square); 0 = auto: the
                            largest with at least 3/4 of a tile per CU; fused, 128 instead
                            of 64 when 64-row tiles would leave fewer than 32 CUs for the
                            fetchers and 128-row tiles still give a quarter of the CUs one */
  int32_t k_per_flag;    /* K-tiles covered by one ready flag; 0 = auto: 512 columns when
                            K >= 4096 or in the fused 128-row case above, else 1024; fused
                            with K >= 4096, 256-row tiles and every tile in one round beside
                            32 spare workgroups, 256 */
  int32_t num_fetch_wgs; /* fetcher workgroups (fused); 0 = auto: 32, or one per fetch unit
                            when all tiles fit in one round with fewer than 32 workgroups
                            to spare */
  int32_t num_wgs;       /* workgroups in the persistent grid; 0 = one per compute unit */
  int32_t trace_cap;     /* debug trace records per workgroup; 0 = auto */
  uint32_t spin_limit;   /* flag polls before a wait gives up; 0 = auto (several seconds) */
  int32_t debug_skip_unit; /* test knob (any mode): fetch unit whose flag is never
                              published, so the waits on it time out; -1 = none */
  int32_t tail_split;    /* 1: when the tiles leave a last round at most half full, its
                            tiles are split along K into pieces (fp32 partial sums, added
                            in piece order by the piece that finishes last) so every
                            workgroup has work; 0 (default): never split. Measured on the
                            16384x3584x8192 workload the dynamic tile queues already even
                            out most of that round and the split does not pay. */
  int32_t gather_a;      /* 1: a run also returns the gathered A, concat(shards) as [M, K]
                            row-major, in a caller buffer that serves as the staging buffer
                            (ag_matmul_run_gather; ag_matmul_run is then refused). The
                            fetch also copies the local shard's tiles, which the GEMM still
                            reads in place. k_contiguous only (UNSUPPORTED otherwise). */
  int32_t pipeline_chunks; /* AGMM_ALGO_PIPELINED: chunks S per shard; 0 = auto (4). Lowered
                              to the largest S with M/D a multiple of S * block_m (1 when
                              M/D is not a multiple of block_m) */
  /* Stress knobs for the fused fetch (tests of the flag protocol; results must not change):
   * before copying unit u a fetcher sleeps hash(u, seed) % debug_fetch_delay back-off steps
   * (s_sleep 2, about 128 clocks each; 0 = no delay), and with debug_fetch_reverse = 1 the
   * n-th unit claimed is unit num_units - 1 - n of the fetch order (the units the first
   * tiles need come last). */
  int32_t debug_fetch_delay;
  uint32_t debug_fetch_seed;
  int32_t debug_fetch_reverse;
  /* Where the fused algorithm's fetchers run. 1: as a kernel of their own, launched on a
   * stream of the handle's beside the persistent GEMM grid, which then has no fetchers: one
   * fetch workgroup shares each CU with a GEMM workgroup, so every CU computes from the
   * start (the caller's stream orders the fetch kernel after the work before the run and
   * waits for it before the work after). UNSUPPORTED when a fetch workgroup does not fit
   * on a CU beside a GEMM workgroup. -1: fetcher workgroups inside the persistent grid.
   * 0 = auto: inside the grid. num_fetch_wgs then counts the fetch kernel's workgroups
   * (0 = auto: one per CU, at most one per unit). */
  int32_t fetch_kernel;
} agmm_desc;

/* Configuration resolved by create (read back with ag_matmul_get_config). */
typedef struct agmm_config {
  int32_t block_m, block_n, block_k, k_per_flag;
  int32_t T_m, T_n, G;          /* m-tiles, n-tiles, k-groups (one flag per m-tile x k-group) */
  int32_t num_units;            /* (m-tile, k-group) units the fetch copies: the staged ones,
                                   then, with gather_a and direct_local, the local shard's */
  int32_t num_tiles;            /* output tiles */
  int32_t num_fetch_wgs;        /* F */
  int32_t num_wgs;              /* W, fused grid (fetchers included) */
  int32_t num_copy_wgs;         /* baseline copy-kernel grid */
  int32_t trace_cap;
  uint32_t epoch;               /* runs enqueued through the handle's run entry points (0
                                   before the first); a replay of a captured graph is not
                                   counted here. The kernels count runs on the device. */
  int64_t staging_elems;        /* 16-bit elements in the handle's staging buffer (0 with
                                   gather_a: the caller's buffer is the staging) */
  int64_t workspace_bytes;      /* device bytes the handle owns */
  int32_t device;               /* HIP device the handle was created on */
  int32_t num_cus;
  int32_t split_tiles;          /* tail tiles split along K (the last ones, t_m * T_n + t_n) */
  int32_t split_pieces;         /* pieces per split tile (0 when none is split) */
  int32_t num_items;            /* queue entries: num_tiles + split_tiles * (split_pieces - 1) */
  int32_t row_wait;             /* fused: 1 when every fetch unit has a fetcher of its own (the
                                   whole fetch is one pass); a tile then waits at its start for
                                   all of its k-groups and its K loop never polls. 0: the K loop
                                   waits for each staged k-group as it reaches it */
  int32_t pipeline_chunks;      /* AGMM_ALGO_PIPELINED: chunks S actually used (0 otherwise) */
  int32_t pipeline_streams;     /* AGMM_ALGO_PIPELINED: streams the chunks rotate over, min(S, 4):
                                   the caller's, and pipeline_streams - 1 of the handle's */
  int32_t fetch_kernel;         /* fused: 1 when the num_fetch_wgs fetchers run as a kernel of
                                   their own beside the num_wgs GEMM workgroups; 0 when they are
                                   workgroups of the persistent grid (num_wgs includes them) */
} agmm_config;

typedef struct agmm_handle agmm_handle;

/* Fills `desc` with defaults: D=1, rank=0, fp16, k_contiguous, fused, direct_local=1, no
 * bias, no debug, every tunable auto, debug_skip_unit=-1. */
void ag_matmul_desc_init(agmm_desc* desc);

/*
 * Creates a handle for one problem shape on the current HIP device: validates `desc`,
 * chooses the tile configuration, and sets up the workspace (staging buffer of M*K elements
 * unless gather_a, flags[T_m*G] uint32, schedule tables, counters, optional trace), zeroing
 * the flags and counters and uploading the tables. This is the preamble of the iris issue
 * ("API / config changes": ..._preamble), done once so that run() allocates nothing.
 *   workspace: NULL: the library allocates the workspace (hipMalloc) and frees it in
 *              destroy. Otherwise caller-owned device memory of at least workspace_bytes
 *              bytes, 256-byte aligned, which must hold ag_matmul_workspace_bytes(desc)
 *              bytes; the caller keeps it alive and untouched until destroy has returned,
 *              and frees it afterwards. One workspace serves one handle at a time.
 * Every handle also owns 16 bytes of pinned host memory (hipHostMalloc) into which its
 * kernels copy a flag-wait timeout (see ag_matmul_run).
 * AGMM_ALGO_PIPELINED handles also create their HIP streams (up to 3, default priority,
 * non-blocking) and events here; fused handles with fetch_kernel = 1 one stream (default
 * priority, non-blocking) and two events, after checking that a fetch workgroup fits on a
 * CU beside a GEMM workgroup (UNSUPPORTED otherwise).
 * Returns AGMM_OK and *out_handle, or INVALID_ARG (also: a misaligned or too small
 * workspace) / UNSUPPORTED / OOM / HIP.
 * Shape rules: M % D == 0; N % 8 == 0 and K % 8 == 0 (16-byte rows); m_contiguous also
 * needs M % 8 == 0. M, N, K may be zero (run() then only writes what exists: K == 0 gives
 * out = bias or 0). M < 2^23, N and K < 2^22, and at most 2^24 output tiles (UNSUPPORTED
 * otherwise).
 */
int ag_matmul_create(const agmm_desc* desc, void* workspace, size_t workspace_bytes,
                     agmm_handle** out_handle);

/*
 * Enqueues one run on `hip_stream` (a hipStream_t; NULL = the null stream) and returns
 * without synchronizing (except in debug mode).
 *   shards: host array of D device pointers, shard d = [M/D, K] row-major;
 *   B:      device [K, N] row-major;  bias: device [N] or NULL (must match has_bias);
 *   out:    device [M, N] row-major, must not overlap any input.
 * Every device pointer must be 16-byte aligned. The caller keeps all buffers alive until
 * the stream work completes. One run may be in flight per handle; successive runs on one
 * stream are safe; concurrent runs of one handle on different streams are undefined.
 * With fetch_kernel = 1 the run records an event on hip_stream, makes the handle's stream
 * wait for it, launches the fetch kernel there and the GEMM grid on hip_stream, then makes
 * hip_stream wait for the handle's stream: work enqueued on hip_stream afterwards sees the
 * whole run, as without the fetch kernel.
 * Graph capture: the run's kernels take its epoch (the value its flags and split counters
 * must reach) from a run counter in the workspace, which the last workgroup of every run
 * advances. A run may therefore be captured into a HIP graph, and the graph replayed any
 * number of times, interleaved with eager runs of the same handle on the same stream. A
 * pipelined run's chunk streams join the capture through its events. Two kinds of run
 * return UNSUPPORTED on a capturing stream and enqueue nothing: a debug run, which
 * synchronizes the stream, and a fetch_kernel = 1 run, whose GEMM grid waits on flags that
 * only the fetch kernel running beside it sets (a graph may run the two one after the
 * other).
 * Returns AGMM_OK, INVALID_ARG (also for a gather_a handle), WRONG_DEVICE, POISONED, HIP,
 * UNSUPPORTED (capture, above), or TIMEOUT. A flag wait that exceeds the spin limit makes
 * every workgroup of the launch stop early (the output is then incomplete); the launch's last
 * workgroup copies the status words into the handle's pinned host word. In debug mode run()
 * synchronizes and returns TIMEOUT for that run itself. Otherwise run() does not synchronize:
 * the first later call on the handle (run, or ag_matmul_sync_status, which waits for the
 * device) that finds the word set returns TIMEOUT and poisons the handle; calls after that
 * return POISONED. The same holds for the GEMM + all-reduce entry points.
 */
int ag_matmul_run(agmm_handle* h, const void* const* shards, const void* B, const void* bias,
                  void* out, void* hip_stream);

/*
 * The run of a gather_a handle: as ag_matmul_run, and it also writes the all-gathered A
 * (Helion thread, Kraken optimization comment: the op returns a = all_gather(a_shared) with
 * out = a @ b):
 *   a_gathered: device [M, K] row-major, 16-byte aligned, must not overlap any other
 *               buffer; row m = row m - d*M/D of shard d. It is the run's staging buffer:
 *               its contents are undefined until the stream work completes.
 * Returns AGMM_OK, or INVALID_ARG (also for a handle without gather_a), WRONG_DEVICE,
 * POISONED, HIP, UNSUPPORTED (graph capture, as for ag_matmul_run) or (debug) TIMEOUT.
 */
int ag_matmul_run_gather(agmm_handle* h, const void* const* shards, const void* B,
                         const void* bias, void* out, void* a_gathered, void* hip_stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): create + run + destroy of a handle for
 * `desc` in one call that allocates nothing. Its workspace is a fixed per-device scratch
 * array of the library (80 MiB, held by each device the library has run this on until the
 * process ends; its address is looked up once per device); the caller still passes inputs
 * and outputs exactly as for ag_matmul_run, on the current device.
 *   desc: as for ag_matmul_create; algo FUSED or BASELINE; debug, gather_a, tail_split and
 *         the fetch stress knobs must be 0, and fetch_kernel must not be 1 (a fetch kernel
 *         needs a stream of the handle's): UNSUPPORTED otherwise. The workspace create
 *         would use for it, ag_matmul_workspace_bytes(desc) on this device, must fit the
 *         scratch, else TOO_LARGE and nothing is enqueued: a staging buffer of up to
 *         64 MiB, e.g. 4096 x 8192 16-bit elements of A.
 * Enqueues on `hip_stream`: a fill kernel that clears the scratch's flags and counters,
 * kernels that write the schedule tables (skipped when this device's previous call had the
 * same desc, unless a call on this device has ever been captured), then the run's kernels.
 * Nothing is synchronized, and no host memory has to outlive the call. Every call starts from
 * cleared flags, so it may be captured into a HIP graph and the graph replayed any number of
 * times; each replay rewrites the tables it uses. Every call on one device shares that
 * device's scratch: calls whose stream work overlaps (other streams, other host threads) race
 * on it and their outputs are undefined; calls on one stream are ordered and safe. A flag-wait
 * timeout (a fetch unit never published, which normal runs do not produce) ends the launch
 * early with an incomplete output and is not reported by this entry point.
 * Returns AGMM_OK, INVALID_ARG, UNSUPPORTED, TOO_LARGE, WRONG_DEVICE or HIP.
 */
int ag_matmul_run_static(const agmm_desc* desc, const void* const* shards, const void* B,
                         const void* bias, void* out, void* hip_stream);

/* ---- GEMM + all-reduce, atomics variant: one rank's share ----
 * The mirror op of the all-gather (ROCm/iris PR "Let's make Iris' All-reduce the best!": a
 * persistent GEMM whose ranks accumulate into each other's results with atomic adds). Rank
 * r of D holds A_r = A[:, K_r] and B_r = B[K_r, :] (K_r its slice of the inner dimension);
 * the op leaves C = sum_r A_r @ B_r = A @ B in every rank's fp32 result buffer.
 *
 * ag_gemm_ar_create: a handle for rank `rank` of `D` (1 <= D <= AGMM_MAX_SHARDS), output
 *   [M, N], local inner dimension K_local (the same shape rules as ag_matmul_create, with
 *   K = K_local), 16-bit type `dtype`, block_m 0 (auto), 64, 128 or 256. Destroy it with
 *   ag_matmul_destroy. ag_matmul_run and ag_matmul_run_gather refuse it.
 * ag_gemm_ar_run: enqueues this rank's share on `hip_stream`: A_local @ B_local computed in
 *   fp32 and added, element by element, into each of the D buffers C[0..D-1] (fp32 [M, N]
 *   row-major, device, 16-byte aligned, disjoint from each other and from the inputs), rank
 *   + 1's first. The caller zeroes the buffers before the first rank adds into them; once
 *   all D ranks' shares have run, each holds C. Additions from concurrent shares are
 *   atomic; their order, and so the last bits of C, then depend on timing.
 *     A_local: device [M, K_local] row-major; B_local: device [K_local, N] row-major.
 * ag_gemm_ar_finalize: out[m][n] = RNE(C[m][n] + bias[n]) in the handle's 16-bit type (bias
 *   [N] 16-bit, or NULL); out [M, N] row-major, not overlapping C.
 * Return codes as for ag_matmul_run. */
int ag_gemm_ar_create(int D, int rank, int64_t M, int64_t N, int64_t K_local, int dtype,
                      int block_m, agmm_handle** out_handle);
int ag_gemm_ar_run(agmm_handle* h, const void* A_local, const void* B_local, float* const* C,
                   void* hip_stream);
int ag_gemm_ar_finalize(agmm_handle* h, const float* C, const void* bias, void* out,
                        void* hip_stream);

/* GEMM + all-reduce with a ready flag per tile (ROCm/iris PR "Let's make Iris' All-reduce
 * the best!", the one-shot variant with per-tile locks): every rank's share in one launch.
 * Rank r's workgroups store their partial tile A_r @ B_r (fp32) into a partial buffer of
 * the handle's and publish the tile's flag for r (release); the tile's reducer waits for
 * the D flags (acquire) and writes out = RNE(sum of the D partials in rank order + bias).
 * The result is deterministic: it does not depend on timing.
 *
 * ag_gemm_ar_flags_create: D ranks (1 <= D <= AGMM_MAX_SHARDS), output [M, N], inner
 *   dimension K_local per rank (shape rules as ag_matmul_create with K = K_local), 16-bit
 *   `dtype`, block_m 0 (auto), 64, 128 or 256. Allocates D * M * N * 4 bytes of partial
 *   tiles besides the usual workspace; AGMM_ERR_OOM if that fails. Destroy it with
 *   ag_matmul_destroy; the other run entry points refuse it.
 * ag_gemm_ar_flags_run: enqueues the op on `hip_stream`. A_parts[r]: device [M, K_local]
 *   row-major; B_parts[r]: device [K_local, N] row-major (r < D); bias [N] 16-bit or NULL;
 *   out [M, N] 16-bit row-major, not overlapping any input. All 16-byte aligned. Runs of
 *   one handle on several streams at once race on its partial buffer and flags. It may be
 *   captured into a HIP graph (its epoch is counted on the device, as for ag_matmul_run).
 * Return codes as for ag_matmul_run. */
int ag_gemm_ar_flags_create(int D, int64_t M, int64_t N, int64_t K_local, int dtype,
                            int block_m, agmm_handle** out_handle);
int ag_gemm_ar_flags_run(agmm_handle* h, const void* const* A_parts, const void* const* B_parts,
                         const void* bias, void* out, void* hip_stream);

/* Host only (no device is touched): the configuration (into cfg, unless NULL) and the claim
 * order of the items that ag_gemm_ar_flags_create would build for these arguments on a
 * device of num_cus compute units. items NULL: *count is set to the number of items.
 * Otherwise *count must be that number and items receives them: (r << 24) | tile for rank
 * r's partial tile, (1 << 30) | tile for the tile's reduction, tile = t_m * T_n + t_n. */
int ag_gemm_ar_flags_plan(int D, int64_t M, int64_t N, int64_t K_local, int dtype, int block_m,
                          int num_cus, agmm_config* cfg, uint32_t* items, int64_t* count);

/* Synchronizes the handle's device and frees its workspace (and a pipelined handle's
 * streams and events). NULL-safe. */
int ag_matmul_destroy(agmm_handle* h);

/* Device bytes create would allocate for `desc` (after resolving auto fields), or a
 * negative error code. Pure host computation; touches no device. */
int64_t ag_matmul_workspace_bytes(const agmm_desc* desc);

/* Static text for a return code. */
const char* ag_matmul_strerror(int code);

/* Last hipError_t seen by this library in the calling thread (0 if none). */
int ag_matmul_last_hip_error(void);

/* Copies the resolved configuration. */
int ag_matmul_get_config(const agmm_handle* h, agmm_config* cfg);

/* Waits for the handle's device (hipDeviceSynchronize), then reports whether a launch of the
 * handle recorded a flag-wait timeout: AGMM_OK if none, TIMEOUT the first time one is found
 * (the handle is then poisoned), POISONED afterwards; or WRONG_DEVICE / HIP. */
int ag_matmul_sync_status(agmm_handle* h);

/* ---- debug / bookkeeping access (synchronizes the handle's device) ---- */
#define AGMM_Q_FLAGS 1        /* uint32[T_m * G] ready flags */
#define AGMM_Q_STAGING 2      /* uint16[staging_elems] staging buffer */
#define AGMM_Q_TRACE 3        /* agmm_trace_rec[num_wgs * trace_cap] */
#define AGMM_Q_TRACE_COUNT 4  /* uint32[num_wgs] records written per workgroup */
#define AGMM_Q_STATUS 5       /* uint32[4]: {status, workgroup, flag index, value seen} */
#define AGMM_Q_UNITS 6        /* uint32[2 * num_units]: (m-tile, k-group) in fetch order */
#define AGMM_Q_MTILES 7       /* uint32[T_m]: m-tile in GEMM order, bit 31 = read in place */
#define AGMM_Q_QUEUES 8       /* uint32[18 + num_items]: 9 queue offsets, 9 queue lengths (8
                                 per-XCD queues, then the tail queue of split-tile pieces),
                                 then the entries queue by queue: bits 0-23 tile id q
                                 (position of its m-tile in GEMM order * T_n + n-tile), bits
                                 24-27 piece, bits 28-31 pieces - 1 (0 = not split) */
#define AGMM_Q_PARTIALS 9     /* float[split_tiles * split_pieces * block_m * block_n]: the
                                 split tiles' fp32 partial sums of the last run, slot
                                 (tile, piece); inside a slot, element i of accumulator group
                                 (fm, fn, g) of thread tid at ((fm*FN + fn)*4 + g)*1024 +
                                 tid*4 + i (FN = block_n / 64, 256 threads) */
#define AGMM_Q_CHUNK_SIZES 10 /* AGMM_ALGO_PIPELINED: uint32[2 * pipeline_chunks], per chunk
                                 (staged units, m-tiles) */
#define AGMM_Q_CHUNK_UNITS 11 /* uint32[2 * num_units]: (m-tile, k-group), chunk by chunk, each
                                 chunk's units in fetch order */
#define AGMM_Q_CHUNK_MTILES 12 /* uint32[T_m]: m-tiles chunk by chunk, each chunk's in GEMM
                                  order, bit 31 = read in place */

/* Trace events (debug). One record per fetched unit, per computed tile and per flag wait
 * of wave 0, after the per-workgroup event ids of the iris issue (wg_fetch, wg_gemm,
 * wg_gemm_wait). Timestamps are the GPU's constant 100 MHz real-time counter. */
#define AGMM_EV_FETCH 1      /* id = unit index, a = m-tile, b = k-group */
#define AGMM_EV_GEMM 2       /* id = queue entry (tile id and piece, as in AGMM_Q_QUEUES),
                                a = m-tile, b = n-tile */
#define AGMM_EV_GEMM_WAIT 3  /* id = flag index, a = value seen, b = polls */

typedef struct agmm_trace_rec {
  uint32_t event, id, a, b;
  uint64_t t0, t1;
} agmm_trace_rec;

/* Copies `bytes` bytes of the queried buffer into host memory `dst` (bytes must equal the
 * buffer's size). Synchronizes the device first. */
int ag_matmul_debug_query(agmm_handle* h, int what, void* dst, size_t bytes);

/* Host only, for tests of the planner: what create would decide for `desc` on a device with
 * `num_cus` compute units, computed without touching any device. what = 0: the resolved
 * agmm_config (epoch, device and workspace fields as create sets them before allocating);
 * otherwise one of AGMM_Q_UNITS, AGMM_Q_MTILES, AGMM_Q_QUEUES, AGMM_Q_CHUNK_SIZES,
 * AGMM_Q_CHUNK_UNITS, AGMM_Q_CHUNK_MTILES, laid out as ag_matmul_debug_query returns them.
 * `bytes` must equal the size of the result. Returns AGMM_OK, INVALID_ARG or UNSUPPORTED. */
int ag_matmul_plan_query(const agmm_desc* desc, int num_cus, int what, void* dst, size_t bytes);

/* Fills the staging buffer with a 16-bit pattern (a NaN pattern exposes reads of unwritten
 * staging) on `hip_stream`. */
int ag_matmul_debug_fill_staging(agmm_handle* h, uint16_t pattern, void* hip_stream);

/* Test knob for the run count (mod 2^32) that the kernels keep on the device: enqueues on
 * `hip_stream` fill kernels that put the handle's flags, split counters and run counter
 * where `runs` runs would have left them. Every flag is set to `runs` (staged units' flags
 * equal the run count, and the per-tile flag variant stores the epoch), and every split
 * counter to runs * split_pieces. The next run then has epoch runs + 1, so runs near 2^32
 * test the wrap-around. Plain, baseline and per-tile flag all-reduce handles; INVALID_ARG
 * for pipelined and atomics all-reduce handles. Returns AGMM_OK, INVALID_ARG, POISONED,
 * WRONG_DEVICE or HIP. */
int ag_matmul_debug_set_runs(agmm_handle* h, uint32_t runs, void* hip_stream);

/* Measurement of the barrier baseline's two phases on their own: for a handle with
 * algo = AGMM_ALGO_BASELINE (and no gather_a), enqueues only the staging copy
 * (AGMM_PART_COPY: every staged unit of A into the staging buffer, [M][K]) or only the GEMM
 * over the staging buffer as it stands (AGMM_PART_GEMM), with the arguments of
 * ag_matmul_run. A GEMM part's output is the op's only once a copy part has run on the same
 * inputs. Returns the codes of ag_matmul_run; INVALID_ARG for another kind of handle or part. */
#define AGMM_PART_COPY 1
#define AGMM_PART_GEMM 2
int ag_matmul_debug_run_part(agmm_handle* h, int part, const void* const* shards, const void* B,
                             const void* bias, void* out, void* hip_stream);

/* Measurement of the MFMA ceiling (no memory traffic): enqueues `grid` workgroups of 256
 * threads, each wave running iters x 16 v_mfma_f32_32x32x16 (dtype AGMM_F16 or AGMM_BF16) on
 * register operands, i.e. grid * 4 * iters * 16 * 32768 FLOP, the operands pseudo-random
 * 16-bit values (random signs and mantissas, like real data); vary = 1 rotates them through
 * four register sets, 0 reuses one set. sink: device float[grid * 256], written. iters > 0, a
 * multiple of 4.
 * Returns AGMM_OK, INVALID_ARG or HIP. */
int ag_matmul_debug_mfma_loop(int dtype, int vary, int grid, int iters, float* sink,
                              void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* AGMM_H */
