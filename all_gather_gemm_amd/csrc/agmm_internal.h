// Internal interface between the C-ABI host code and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "agmm.h"

namespace agmm {

constexpr int kThreads = 256;  // 4 wave64s per workgroup
constexpr int kBlockK = 32;    // K-tile depth of the GEMM worker (every tile family)

// Output tiles are handed out from kQueues queues, one per XCD (workgroup w is placed on
// XCD w % 8 by the dispatcher); a workgroup drains its own queue, then steals from the
// others.
constexpr int kQueues = 8;
// A ninth queue, taken from only when the XCD queues are empty, holds the pieces of the
// tiles split along K to fill the last round (the tail); its index is kTailQueue.
constexpr int kTailQueue = kQueues;
constexpr int kQueueSlots = kQueues + 1;

// Queue entry: bits 0-23 tile id (position of its m-tile in GEMM order * T_n + n-tile),
// bits 24-27 piece, bits 28-31 pieces - 1 (0: the tile is not split).
constexpr uint32_t kItemTileMask = 0x00ffffffu;
// GEMM + all-reduce with per-tile flags: an item with this bit reduces its tile (else bits
// 24..29 name the rank whose partial tile it computes)
constexpr uint32_t kArReduceItem = 1u << 30;
constexpr int kMaxSplit = 4;

// Counter words in the workspace (uint32). Each queue counter has its own 128-byte line.
enum : int {
  CTR_DONE = 0,         // workgroups that finished; the last one resets the queue counters
  CTR_RUNS = 1,         // runs the workspace has finished (mod 2^32): the last workgroup of
                        // run e stores e, so the next run's kernels read their epoch here
  CTR_STATUS = 2,       // 0 = ok, 1 = a flag wait timed out (sticky until the host clears it)
  CTR_STATUS_WG = 3,    // workgroup that timed out
  CTR_STATUS_FLAG = 4,  // flag index it waited on
  CTR_STATUS_SEEN = 5,  // flag value it last saw
  CTR_HOST_LO = 6,      // device address of the handle's host-visible status mirror
  CTR_HOST_HI = 7,      // (uint32[4], pinned host memory), low and high words; 0 = none
  CTR_DBG_DELAY = 8,    // fetch stress knobs, written at create: max back-off steps before
  CTR_DBG_SEED = 9,     // a unit's copy (0 = none), the seed of the per-unit delay hash,
  CTR_DBG_REVERSE = 10, // and 1 = claim units in reverse fetch order
  CTR_FDONE = 32,       // fetch-kernel workgroups that finished (own 128-byte line)
  CTR_FETCH = 64,       // next fetch unit to claim (own 128-byte line)
  CTR_Q = 96,           // queue x counter at CTR_Q + x * CTR_QSTRIDE
  CTR_QSTRIDE = 32,
  CTR_WORDS = CTR_Q + kQueueSlots * CTR_QSTRIDE
};

// Everything a launch needs, passed by value as the kernel argument.
struct KParams {
  const uint16_t* shards[AGMM_MAX_SHARDS];
  const uint16_t* B;
  const uint16_t* bias;     // nullptr: no bias
  uint16_t* out;
  uint16_t* staging;
  uint32_t* flags;          // [T_m * G]
  uint32_t* ctr;            // [CTR_WORDS]
  const uint32_t* units;    // [2 * num_units]: (m-tile, k-group) in fetch order
  const uint32_t* mtiles;   // [T_m]: m-tile in GEMM order; bit 31 set = read in place
  const uint32_t* qtiles;   // [num_items]: queue entries, queue by queue
  int32_t qoff[kQueueSlots], qlen[kQueueSlots];
  float* partials;          // split tiles: [split tile][piece][BM*BN] fp32 partial sums
  uint32_t* split_cnt;      // [split tiles]: pieces finished, S per run (epoch-valued)
  int32_t split_base;       // tile (t_m * T_n + t_n) of the first split tile
  agmm_trace_rec* trace;    // [gridDim.x * trace_cap] (debug)
  uint32_t* trace_count;    // [gridDim.x] (debug)
  int64_t M, N, K, M_s;
  int32_t D, rank, T_m, T_n, G, kpf;
  int32_t num_units, num_tiles, F;
  int32_t staged_kmajor;    // 1: staging is [M][K]; 0: staging is [K][M]
  int32_t row_wait;         // fused: tiles wait at their start for all of their k-groups
  uint32_t reserved;        // (unused: a run's epoch comes from ctr[CTR_RUNS] on the device)
  int32_t debug, trace_cap;
  uint32_t spin_limit;
  int32_t skip_unit;
  // GEMM + all-reduce (atomics): this rank's partial tiles are added into the ar_D result
  // buffers (fp32 [M][N]) instead of being stored
  int32_t ar_D, ar_rank;
  // The two all-reduce variants use one table, so that the struct, and with it every
  // kernel's argument block, keeps its size: the atomics variant's result buffers, or the
  // per-tile flag variant's B slices (rank r's [K][N], K its inner dimension; its A slice
  // is shards[r], [M][K]).
  union {
    float* ar_out[AGMM_MAX_SHARDS];
    const uint16_t* ar_B[AGMM_MAX_SHARDS];
  };
};
// Every kernel of the library takes this struct by value, and its size fixes the kernel
// argument block (1312 bytes plus the runtime's hidden arguments, 1568 in all). The block
// is kept at the size every kernel has been run and profiled with; a new per-launch table
// goes into the workspace instead of growing the struct.
static_assert(sizeof(KParams) == 1312, "kernel argument block size");

// Launchers (defined in agmm_kernels.hip). block_m selects the tile family.
hipError_t launch_fused(const KParams& p, int dtype, int block_m, int grid, hipStream_t s);
hipError_t launch_gemm_only(const KParams& p, int dtype, int block_m, int grid, hipStream_t s);
hipError_t launch_copy(const KParams& p, int block_m, int grid, hipStream_t s);
// The fetch kernel (fused grid without fetchers beside it, on another stream): grid
// workgroups claim and publish the units of p.units. layout_k: k_contiguous staging.
hipError_t launch_fetch(const KParams& p, int block_m, bool layout_k, int grid, hipStream_t s);
// Whether a fetch-kernel workgroup fits on a CU beside a fused GEMM workgroup of this tile
// family (registers per SIMD and LDS per CU, from the kernels' own attributes).
hipError_t fetch_fits_beside(int dtype, int block_m, bool layout_k, bool* fits);
// The GEMM-only persistent kernel whose tiles are added (fp32 atomics) into p.ar_out[].
hipError_t launch_gemm_ar(const KParams& p, int dtype, int block_m, int grid, hipStream_t s);
// GEMM + all-reduce with per-tile flags, every rank's share in one launch: items in
// p.qtiles (queue 0), partial tiles in p.partials, flags in p.flags ([D][tiles]).
hipError_t launch_ar_flags(const KParams& p, int dtype, int block_m, int grid, hipStream_t s);
// out[m][n] = RNE(C[m][n] + bias[n]) for the 16-bit type; N % 4 == 0.
hipError_t launch_ar_finalize(const float* C, const uint16_t* bias, uint16_t* out, int64_t M,
                              int64_t N, int dtype, hipStream_t s);
hipError_t launch_fill16(uint16_t* dst, int64_t n, uint16_t v, hipStream_t s);
// Measurement: grid workgroups of 4 waves, each running iters x 16 32x32x16 MFMAs on
// pseudo-random register operands (vary: rotating through 4 sets; else one set); writes
// grid * 256 floats to sink. iters a positive multiple of 4.
hipError_t launch_mfma_loop(int dtype, bool vary, int grid, int iters, float* sink, hipStream_t s);
hipError_t launch_fill32(uint32_t* dst, int64_t n, uint32_t v, hipStream_t s);
// Resident workgroups per CU for the fused kernel of this family (occupancy query).
hipError_t fused_occupancy(int dtype, int block_m, int* per_cu);
// dst[0 .. n) = src[0 .. n) (host words) by kernels that take the words as arguments, so
// nothing on the host has to outlive the call and no copy engine or allocation is used.
hipError_t launch_upload32(uint32_t* dst, const uint32_t* src, int64_t n, hipStream_t s);

// Size of the per-device scratch array of ag_matmul_run_static (agmm_static.hip): enough
// for a 64 MiB staging buffer (e.g. 4096 x 8192 16-bit elements) and its tables.
constexpr size_t kScratchBytes = (size_t)80 << 20;
// The scratch array's device address on `device`, which must be the current device; the
// address is looked up once per device (hipGetSymbolAddress) and then kept.
hipError_t scratch_region(int device, void** ptr);

}  // namespace agmm
