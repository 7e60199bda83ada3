// gfx950 kernels for the fused all-gather + GEMM.
//
// One persistent kernel (ROCm/iris issue "Fused all-gather+GEMM HBM-buffer kernel for
// iris.ops", opening summary): workgroups [0, F) start as fetchers, copying A units
// (m-tile x k-group) from the shard allocations into the staging buffer and publishing one
// ready flag per unit; then every workgroup takes output tiles from a shared queue and
// computes them, waiting on a unit's flag only before its first K-tile is loaded. Local-
// shard m-tiles are read in place (pytorch/helion PR "[Benchmark] Add all gather matmul
// benchmark", Kraken optimization) and the source choice is made once per tile, outside
// the K loop (the same thread explains why a per-iteration choice defeats prefetching).
//
// GEMM worker: square output tiles BMxBM (256, 128 or 64), 4 wave64s in a 2x2 layout,
// v_mfma_f32_32x32x16_{f16,bf16} with fp32 accumulators, K-tiles of 32 in four LDS stages.
// Operand slices go global->LDS by buffer loads that write LDS directly, three K-tiles
// ahead of use, so no registers hold data in flight; each operand keeps the layout it has
// in memory (K-contiguous slices are read as 16-byte MFMA operands, MN-contiguous ones --
// B, and A staged m_contiguous -- through the transposing ds_read_b64_tr_b16). One
// barrier per K-tile; the output tile goes through LDS for 16-byte coalesced stores.
//
// Flag protocol: fetcher workgroups claim units from one counter; a unit's flag holds the
// run's epoch once the unit is in staging. The epoch is counted on the device: run e reads
// e - 1 from the workspace's run counter at its start and its last workgroup stores e, so
// runs count up in stream order however they were enqueued (also as replays of a captured
// graph). Flags and split counters grow by a fixed amount per run, and every comparison
// with the epoch is an equality, so the uint32 counts may wrap. Producer = every wave waits until its stores
// are acknowledged (they then sit in this XCD's L2: the vector L1 writes through),
// workgroup barrier, then one agent-scope release add of 1 by thread 0, whose L2 write-back
// publishes the whole workgroup's stores. Consumer =
// wave 0 of the GEMM workgroup: relaxed agent-scope polls with s_sleep backoff (the
// busy-wait back-off suggested in ROCm/iris PR "Let's make Iris' All-reduce the best!"),
// then one agent-scope acquire fence for every flag it has seen complete; the other waves
// request that data only after a later workgroup barrier. Every
// wait is bounded by a spin limit; a timeout is recorded in the status word, the waiting
// tile finishes on whatever staging holds (so every barrier is still met), and all
// workgroups stop taking tiles, so the grid always drains.
#include <type_traits>

#include "agmm_internal.h"

namespace agmm {
namespace {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef __bf16 b8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int DT>
struct Num;

template <>
struct Num<AGMM_F16> {
  __device__ static inline f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8_t, a),
                                                  __builtin_bit_cast(h8_t, b), c, 0, 0, 0);
  }
  __device__ static inline uint32_t to_bits(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
  }
  __device__ static inline float from_bits(uint32_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
  }
};

template <>
struct Num<AGMM_BF16> {
  __device__ static inline f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(b8_t, a),
                                                   __builtin_bit_cast(b8_t, b), c, 0, 0, 0);
  }
  __device__ static inline uint32_t to_bits(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
  }
  __device__ static inline float from_bits(uint32_t h) {
    return __builtin_bit_cast(float, (h & 0xffffu) << 16);
  }
};

// Tile family: square BMxBM output tile (BM = 256, 128, 64), BK = 32, NS LDS stages.
// A stage holds the A and B slices of one K-tile, 4*BM 16-byte chunks each, in the layout
// their source has in global memory, so both are copied global->LDS by buffer loads that
// write LDS directly (no registers, no VALU):
//  - a K-contiguous slice (A from a shard or k_contiguous staging) as [row][4 chunks], the
//    chunk index XORed with g(row) = (row>>2) & 3; an MFMA operand is one 16-byte read per
//    lane. The LDS serves a 16-byte read in passes of 16 lanes over 256 bytes (64 banks):
//    the 16 rows of a pass then fill 16 distinct 16-byte slots (row%4 picks the 64-byte
//    quarter, (row>>2)%4 the slot in it). Measured with SQ_LDS_BANK_CONFLICT: no conflict,
//    where the earlier g(row) = (row>>1 ^ row>>3) & 3 cost 4 cycles per read;
//  - an MN-contiguous slice (B, or A from m_contiguous staging) as [k][MN/8 chunks], the
//    chunk index XORed with f(k) = 4*(k%4) (4*((k>>1)%2) when a row has 8 chunks); an MFMA
//    operand is two transposing 8-byte reads (ds_read_b64_tr_b16) per lane.
// Checked on the CPU against the instruction's lane mapping (measured on the hardware):
// every MFMA lane receives its elements; each DMA instruction fills 1 KiB of LDS linearly.
// The transposing reads of the MN-contiguous slices show no bank conflicts in the counters.
template <int BM_>
struct Tile {
  static constexpr int BM = BM_, BN = BM_, BK = kBlockK, NKK = BK / 16;
  static_assert(BK == 32, "the LDS layouts below assume 32-deep K-tiles");
  static constexpr int A_CH = BM * 4, B_CH = BN * 4;     // 16-byte chunks per stage
  static constexpr int STAGE = A_CH + B_CH;
  static constexpr int ADMA = A_CH / 256, BDMA = B_CH / 256;  // DMA instructions per wave
  static constexpr int DMA_PER_TILE = ADMA + BDMA;
  static constexpr int WTM = BM / 2, WTN = BN / 2;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  // LDS stages, i.e. K-tiles in flight + 1. Four at every tile size: deeper pipelines for
  // the small tiles (8 or 16 stages at BM = 64, the same 128 KiB as BM = 256) measured
  // slower, the extra requests only lengthen the memory queues.
  static constexpr int NS = 4;
  static_assert(NS >= 4 && NS * STAGE <= 8192, "stages fit in 128 KiB");
  static_assert(STAGE * 16 >= (BM / 4) * BN * 2, "an output quarter fits in a stage");
  // requests in flight per wave: at most NS - 2 K-tiles and one A slice (counter range 63)
  static_assert((NS - 2) * DMA_PER_TILE + ADMA <= 63, "DMA requests within the counter");
};

__device__ inline int g_row(int m) { return (m >> 2) & 3; }
template <int RC>
__device__ inline int f_row(int k) { return RC >= 16 ? 4 * (k & 3) : 4 * ((k >> 1) & 1); }

__device__ inline u32x4 ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ inline void st16(uint16_t* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Row i of the transpose of an 8x8 block of 16-bit values held as 8 rows v[0..7] of four
// dwords: element j of the result is element i of v[j]. v_perm_b32 picks two 16-bit halves
// from two dwords per instruction (selector 0x05040100: low halves, 0x07060302: high).
__device__ inline u32x4 transpose_row(const u32x4 (&v)[8], int i) {
  const int w = i >> 1;
  const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
  u32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q) o[q] = __builtin_amdgcn_perm(v[2 * q + 1][w], v[2 * q][w], sel);
  return o;
}

// Buffer resource over [base, base + bytes): accesses at byte offsets at or past `bytes`
// read zero and touch no memory. The word 0x00020000 is the gfx9-family raw-buffer
// configuration.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
// Callers pass workgroup-uniform values; readfirstlane states that, so the descriptor
// lives in SGPRs as the buffer instructions require.
__device__ inline uint32_t uniform32(uint32_t x) {
  // the builtin returns a signed int: go back to 32 unsigned bits before any widening
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)x);
}
__device__ inline rsrc_t make_rsrc(const uint16_t* base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0x7fffffffll ? 0x7fffffffll : bytes);
  const uint64_t a = (uint64_t)(size_t)base;
  const uint64_t au = (uint64_t)uniform32((uint32_t)a) | ((uint64_t)uniform32((uint32_t)(a >> 32)) << 32);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(au), (short)0,
                                           (int)uniform32((uint32_t)n), 0x00020000);
}
constexpr uint32_t kOob = 0x80000000u;  // an offset past every resource range used here

// 16-byte buffer load / store; out-of-range offsets read zero / write nothing.
__device__ inline u32x4 bload16(rsrc_t rs, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0));
}
__device__ inline void bstore16(rsrc_t rs, uint32_t off, u32x4 v) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v), rs, (int)off, 0, 0);
}

typedef __attribute__((address_space(3))) void lds_void;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
// LDS pointers kept in the LDS address space, so that every access through them is a ds_*
// instruction (a generic pointer makes the compiler emit flat accesses, which are slower
// and count against both the vector-memory and the LDS wait counters)
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((address_space(3))) const char lds_cchar;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;

// 16 bytes per lane from rs at voff into LDS at byte address m0 + 16 * lane (m0 is
// wave-uniform): buffer_load_dwordx4 ... lds, with the LDS base in M0. Written as inline
// asm so that the compiler adds no waits of its own for it (it cannot tell which stage a
// DMA in flight targets across the K loop's back edge and would drain every request); the
// K loop waits for exactly the requests it needs with wait_vmcnt.
__device__ inline void dma16(rsrc_t rs, uint32_t m0, uint32_t voff) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rs), "{m0}"(m0)
               : "memory");
}

// K-contiguous operand (rows x 32 K values per stage): element (r, k) at base[r*ld + k].
// Wave w fills 1 KiB blocks b = w*NDMA + j of the slice: 16 rows x 4 chunks; lane i takes
// row 16b + i/4, stored chunk slot i%4, i.e. source chunk (i%4) ^ g(row).
template <int MN>
struct KMajorDma {
  static constexpr int NDMA = MN * 4 / 256;
  uint32_t voff[NDMA];
  int kc8[NDMA];  // first K column of the lane's chunk, relative to the stage's K offset
  __device__ inline void init(int64_t ld, int wave, int lane) {
#pragma unroll
    for (int j = 0; j < NDMA; ++j) {
      const int b = wave * NDMA + j, row = 16 * b + lane / 4, c = (lane & 3) ^ g_row(row);
      kc8[j] = 8 * c;
      voff[j] = (uint32_t)((row * ld + 8 * c) * 2);
    }
  }
  // DMA j of this wave; rs covers the operand from column k0 onwards, k_rem = K - k0
  // (columns at or past K would read the next row: those lanes load from past the range
  // instead, i.e. zeros); region = LDS byte address of the slice, wave wave-uniform.
  __device__ inline void issue(int j, rsrc_t rs, uint32_t region, uint32_t wave,
                               int64_t k_rem) const {
    dma16(rs, region + (wave * NDMA + j) * 1024u, kc8[j] < k_rem ? voff[j] : kOob);
  }
  // MFMA operand for rows rbase..rbase+31, K sub-step kk: lane l holds row rbase + l%32,
  // K values 16*kk + 8*(l/32) .. +7.
  __device__ static inline u32x4 frag(const lds_u32x4* region, int rbase, int kk, int lane) {
    const int row = rbase + (lane & 31), c = 2 * kk + (lane >> 5);
    return region[row * 4 + (c ^ g_row(row))];
  }
};

// MN-contiguous operand (32 K rows x MN per stage): element (r, k) at base[k*ld + r].
// Block b covers chunks 64b .. 64b+63 of the [k][MN/8] slice; lane i stores chunk
// q = 64b + i: row k = q / RC, slot q % RC, source chunk (q % RC) ^ f(k).
template <int MN>
struct MNMajorDma {
  static constexpr int RC = MN / 8;   // chunks per row
  static constexpr int NDMA = MN * 4 / 256;
  static constexpr int ROWB = MN * 2; // bytes per LDS row
  uint32_t voff[NDMA];
  __device__ inline void init(int64_t ld, int wave, int lane) {
#pragma unroll
    for (int j = 0; j < NDMA; ++j) {
      const int q = (wave * NDMA + j) * 64 + lane, k = q / RC, c = (q % RC) ^ f_row<RC>(k);
      voff[j] = (uint32_t)((k * ld + 8 * c) * 2);
    }
  }
  // DMA j of this wave. Rows at or past K lie past the range (zeros); columns past the
  // last valid one read neighbouring data that only reaches outputs that are never stored.
  __device__ inline void issue(int j, rsrc_t rs, uint32_t region, uint32_t wave, int64_t) const {
    dma16(rs, region + (wave * NDMA + j) * 1024u, voff[j]);
  }
  // Byte offset, inside a stage slice, of this lane's half-0 transposing read for the
  // operand block whose 32 MN positions start at mbase (K sub-step 0). The read for
  // sub-step kk, half h is at +(16*kk + 4*h) * ROWB: f(k) depends only on the lane.
  __device__ static inline int lane_off(int mbase, int lane) {
    const int gidx = lane >> 4, s = lane & 15;
    const int kl = 8 * (gidx >> 1) + (s >> 2);
    const int mn = mbase + 16 * (gidx & 1) + 4 * (s & 3);
    return kl * ROWB + (((mn >> 3) ^ f_row<RC>(kl)) * 16) + (mn & 7) * 2;
  }
  __device__ static inline u32x4 frag(const lds_u32x4* region, int off, int kk) {
    lds_cchar* p = reinterpret_cast<lds_cchar*>(region) + off + 16 * kk * ROWB;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * ROWB));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return u32x4{l2[0], l2[1], h2[0], h2[1]};
  }
};

struct Tracer {
  agmm_trace_rec* base;
  uint32_t n, cap;
  bool on;
  __device__ inline uint64_t now() const { return on ? __builtin_amdgcn_s_memrealtime() : 0; }
  __device__ inline void rec(uint32_t ev, uint32_t id, uint32_t a, uint32_t b, uint64_t t0) {
    if (on && threadIdx.x == 0) {
      if (n < cap) {
        agmm_trace_rec r;
        r.event = ev;
        r.id = id;
        r.a = a;
        r.b = b;
        r.t0 = t0;
        r.t1 = __builtin_amdgcn_s_memrealtime();
        base[n] = r;
      }
      ++n;
    }
  }
};

__device__ inline bool aborted(const KParams& p) {
  return __hip_atomic_load(p.ctr + CTR_STATUS, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
}

// Called by the last workgroup of a launch (every other workgroup has counted itself done,
// so no wait of this launch is still running): a recorded flag-wait timeout is copied into
// the handle's pinned host word (CTR_HOST_*), which the host reads at the next run without
// synchronizing. Nothing is written while the status is clear.
__device__ inline void mirror_status(const KParams& p) {
  const uint32_t st = __hip_atomic_load(p.ctr + CTR_STATUS, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t hp = (uint64_t)p.ctr[CTR_HOST_LO] | ((uint64_t)p.ctr[CTR_HOST_HI] << 32);
  if (st == 0 || hp == 0) return;
  uint32_t* h = reinterpret_cast<uint32_t*>(hp);
  for (int i = 1; i < 4; ++i)
    __hip_atomic_store(h + i,
                       __hip_atomic_load(p.ctr + CTR_STATUS + i, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  __hip_atomic_store(h, st, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Thread 0's first claim of a workgroup: the next queue entry into *next, and this run's
// epoch into *epoch, one more than the runs the workspace has finished. The two loads are in
// flight together. The run's last workgroup stores the epoch only after every workgroup has
// counted itself done, so every workgroup reads the previous run's count.
__device__ inline int grab(const KParams& p);
__device__ inline void first_claim(const KParams& p, int* next, uint32_t* epoch) {
  const uint32_t done = __hip_atomic_load(p.ctr + CTR_RUNS, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
  *next = grab(p);
  *epoch = done + 1u;
}

// Waits (every lane of the calling wave) until flags[idx] == target. No acquire: the caller
// issues one for every flag it has seen complete.
__device__ inline void poll_flag(const KParams& p, int64_t idx, uint32_t target, Tracer& tr) {
  uint32_t* f = p.flags + idx;
  const uint64_t t0 = tr.now();
  uint32_t polls = 0;
  uint32_t v = __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  int backoff = 1;
  while (v != target) {
    ++polls;
    if (polls >= p.spin_limit) {
      if ((threadIdx.x & 63) == 0 &&
          atomicCAS(p.ctr + CTR_STATUS, 0u, 1u) == 0u) {
        __hip_atomic_store(p.ctr + CTR_STATUS_WG, (uint32_t)blockIdx.x, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(p.ctr + CTR_STATUS_FLAG, (uint32_t)idx, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(p.ctr + CTR_STATUS_SEEN, v, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
      break;
    }
    if ((polls & 31) == 0 && aborted(p)) break;
    for (int i = 0; i < backoff; ++i) __builtin_amdgcn_s_sleep(2);
    if (backoff < 16) backoff <<= 1;
    v = __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  tr.rec(AGMM_EV_GEMM_WAIT, (uint32_t)idx, v, polls, t0);
}

// B is the MFMA's first operand, so each lane ends up holding 4 consecutive columns of one
// output row.
template <class T, int DT>
__device__ inline void mfmas(f32x16 (&acc)[T::FM][T::FN], const u32x4 (&a)[T::FM],
                             const u32x4 (&b)[T::FN]) {
#pragma unroll
  for (int fm = 0; fm < T::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < T::FN; ++fn) acc[fm][fn] = Num<DT>::mfma(b[fn], a[fm], acc[fm][fn]);
}

// 24 wait states: covers the longest MFMA result latency before an accumulator is read
// by the inline-asm reads below (whose AGPR operands the hazard checks may not track).
__device__ inline void mfma_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

// One accumulator element, copied out of its AGPR where it is used. Left to itself the
// register allocator moves every accumulator into VGPRs at the end of the K loop, which
// does not fit and spills.
__device__ inline float acc_read(const f32x16& v, int i) {
  float x;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(x) : "a"(v[i]));
  return x;
}

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt in bits 3:0 and 15:14).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for the K loop. __syncthreads() would also wait for every LDS DMA in
// flight (its release fence counts them as pending LDS writes) and drain the prefetch; the
// loop instead waits for exactly the DMA it needs (wait_vmcnt before this) and for its own
// LDS reads, then meets at the hardware barrier. The empty asm and scheduling fences keep
// the compiler from moving memory operations across it.
__device__ inline void kloop_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt((63 & 15) | ((63 >> 4) << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// The NS LDS stages, contiguous: stage i and its LDS byte address (uniform) are arithmetic
// on stage 0's, so they cost no registers and need no table.
template <class T>
struct Stages {
  lds_u32x4* base;
  uint32_t off0;
  __device__ inline lds_u32x4* s(int i) const { return base + i * T::STAGE; }
  __device__ inline uint32_t off(int i) const { return off0 + (uint32_t)(i * T::STAGE * 16); }
};

// Calls f(integral_constant<int, I>) for I = 0 .. N-1, in order.
template <int I, int N, class Fn>
__device__ __attribute__((always_inline)) inline void static_for(Fn&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// s_waitcnt vmcnt(a * PER), a <= A_MAX a run-time value: the largest allowed count not above
// it (a chain of uniform compares; the count has to be an immediate).
template <int PER, int A_MAX>
__device__ inline void wait_vmcnt_times(int a) {
  if constexpr (A_MAX <= 0) {
    wait_vmcnt<0>();
  } else {
    if (a >= A_MAX)
      wait_vmcnt<A_MAX * PER>();
    else
      wait_vmcnt_times<PER, A_MAX - 1>(a);
  }
}

// Issue slot of item i of n spread over the m MFMAs of a half step: item i goes after MFMA
// slot(i) (shift 0) or half a spacing later (shift 1), so that DMA requests and fragment
// reads interleave with the MFMAs instead of queueing behind each other.
__host__ __device__ constexpr int spread(int i, int n, int m, int shift) {
  return n <= 0 ? 0 : ((2 * i + shift) * m / (2 * n) < m ? (2 * i + shift) * m / (2 * n) : m - 1);
}

// One output tile. A_KMAJOR: the A source is K-contiguous (local shard or k_contiguous
// staging); otherwise it is the m_contiguous staging buffer. WAIT: fused mode, staged
// k-groups are waited for before their first K-tile is requested.
//
// Pipeline over K-tiles t (stage t % 4): DMA requests run three K-tiles ahead. Step t:
// read sub-step 1 fragments of t, run sub-step 0 MFMAs; wait for this wave's DMA of t+1
// and meet at the barrier (after it, t+1 is in LDS for every wave and no wave reads stage
// t any more); request t+4 into stage t % 4; read sub-step 0 fragments of t+1 and run
// sub-step 1 MFMAs of t. One barrier per K-tile; fragments double buffered.
__device__ inline int grab(const KParams& p);

// next_tile: thread 0 stores the workgroup's next tile index there once this tile's K loop
// is done, so the queue atomic's round trip overlaps the epilogue while no tile is claimed
// long before it can start (claiming at the start of a tile lets the first workgroups to
// arrive take two tiles each and starve the rest when tiles and workgroups are few).
// piece / pieces: a split tile's piece covers K-tiles [piece * KT / pieces, (piece + 1) * KT /
// pieces); its fp32 partial sums go to a workspace slot and the piece that finishes the tile
// last adds all of them in piece order (so the sum does not depend on which piece ends
// last) and runs the epilogue. is_last: an LDS word for that decision.
//
template <class T, int DT, bool A_KMAJOR, bool WAIT, bool ROW, int EPI = 0>
__device__ __attribute__((always_inline)) void gemm_tile(const KParams& p, int t_m, int t_n,
                                                         int piece, int pieces, bool staged,
                                                         const Stages<T>& st, u32x2* bias_lds,
                                                         int tid_in, Tracer& tr, int* next_tile,
                                                         int* is_last, uint32_t epoch,
                                                         int src = 0) {
  constexpr int BM = T::BM, BN = T::BN, BK = T::BK;
  // this piece's K-tiles [kt_lo, kt_lo + KT)
  const int KT_all = (int)((p.K + BK - 1) / BK);
  const int kt_lo = piece * KT_all / pieces;
  const int KT = (piece + 1) * KT_all / pieces - kt_lo;
  const int64_t fbase = (int64_t)t_m * p.G;
  bool waits = WAIT && staged;
  const int kpf = p.kpf;
  const uint32_t target = epoch;  // a published unit's flag
  // Consumer side of the flags. An agent-scope acquire invalidates the XCD's L2 (which all
  // workgroups on that XCD rely on for operand reuse) and drains the wave's DMA requests in
  // flight, so acquires are few: only wave 0 polls and acquires, and each acquire also
  // takes every later k-group of the tile that is published already (once the fetchers are
  // ahead, that is all of them). The other waves issue their requests for a k-group only
  // after a workgroup barrier that wave 0 reaches after its acquire has completed, and they
  // read through the same L1 and L2. ready_to: k-groups below it are acquired.
  const bool wave0 = __builtin_amdgcn_readfirstlane(tid_in >> 6) == 0;
  const int g_end = (kt_lo + KT + kpf - 1) / kpf;  // one past this piece's last k-group
  int ready_to = kt_lo / kpf;
  // First k-group at or after g0 whose flag is not published yet (g_end if none). The
  // flags are read up to 64 at a time, one per lane, so a run of published k-groups costs
  // one memory round trip rather than one per group.
  auto unpublished_from = [&](int g0) -> int {
    for (int base = g0; base < g_end; base += 64) {
      const int g = base + (tid_in & 63);
      uint32_t v = target;
      if (g < g_end)
        v = __hip_atomic_load(p.flags + fbase + g, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint64_t late = __builtin_amdgcn_ballot_w64(v != target);
      if (late) return base + (int)__builtin_ctzll(late);
    }
    return g_end;
  };
  // wave 0: wait for k-groups ready_to .. g_need, take the published ones after them, acquire
  auto acquire_groups = [&](int g_need) {
    int g = unpublished_from(ready_to);
    while (g <= g_need) {  // a needed k-group is not published yet: wait for it
      poll_flag(p, fbase + g, target, tr);
      g = unpublished_from(g + 1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    ready_to = g;
  };
  if constexpr (WAIT) {
    if (waits) {
      // every wave requests the first NS K-tiles before the K loop's first barrier: wave 0
      // acquires their k-groups first (ROW: all of the tile's k-groups, so the K loop never
      // waits), this barrier orders the requests after it
      if (wave0 && KT > 0)
        acquire_groups(ROW ? g_end - 1 : (kt_lo + min(KT - 1, T::NS - 1)) / kpf);
      __syncthreads();
      // only wave 0 waits for the rest; the other waves never poll and need no flag state
      waits = wave0 && ready_to < g_end;
    }
  }
  // The thread index through an empty asm: everything derived from it below (lane offsets,
  // swizzles) is then computed per tile instead of being kept live across the whole tile
  // loop, where the fetch above needs the registers.
  int tid = tid_in;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)t_m * BM, n0 = (int64_t)t_n * BN;
  const int rows_valid = (int)min((int64_t)BM, p.M - m0);
  const int cols_valid = (int)min((int64_t)BN, p.N - n0);
  // A source, chosen once per tile: base pointer, row stride, and the bytes from base to
  // the end of the buffer it lies in (the buffer-resource range).
  const uint16_t* abase;
  int64_t lda, a_bytes;
  if (!staged) {
    abase = p.shards[EPI == 2 ? src : p.rank] + (m0 - (int64_t)p.rank * p.M_s) * p.K;
    lda = p.K;
    a_bytes = (p.M_s * p.K - (m0 - (int64_t)p.rank * p.M_s) * p.K) * 2;
  } else if (A_KMAJOR) {
    abase = p.staging + m0 * p.K;
    lda = p.K;
    a_bytes = (p.M - m0) * p.K * 2;
  } else {
    abase = p.staging + m0;
    lda = p.M;
    a_bytes = (p.K * p.M - m0) * 2;
  }
  // step of the A base per K-tile: BK columns (K-major) or BK rows (m_contiguous)
  const int64_t a_step = A_KMAJOR ? (int64_t)BK : (int64_t)BK * lda;
  const uint16_t* bbase = (EPI == 2 ? p.ar_B[src] : p.B) + n0;
  int64_t b_bytes = (p.K * p.N - n0) * 2;
  const int64_t b_step = (int64_t)BK * p.N;
  // the operand bases start at K-tile kt_lo
  abase += kt_lo * a_step;
  a_bytes -= kt_lo * a_step * 2;
  bbase += kt_lo * b_step;
  b_bytes -= kt_lo * b_step * 2;

  using ADma = typename std::conditional<A_KMAJOR, KMajorDma<BM>, MNMajorDma<BM>>::type;
  using BDma = MNMajorDma<BN>;
  ADma ad;
  BDma bd;
  ad.init(lda, wave, lane);
  bd.init(p.N, wave, lane);

  // fragment addressing (fixed per tile)
  int aoff[T::FM], boff[T::FN];
#pragma unroll
  for (int fm = 0; fm < T::FM; ++fm)
    aoff[fm] = A_KMAJOR ? 0 : MNMajorDma<BM>::lane_off(wm * T::WTM + fm * 32, lane);
#pragma unroll
  for (int fn = 0; fn < T::FN; ++fn) boff[fn] = BDma::lane_off(wn * T::WTN + fn * 32, lane);

  f32x16 acc[T::FM][T::FN];
#pragma unroll
  for (int fm = 0; fm < T::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < T::FN; ++fn) acc[fm][fn] = (f32x16)(0.0f);

  // This tile's bias slice to LDS (read after the K loop's barriers).
  // (zeros without a bias: the epilogue then has no branch, which would otherwise make the
  // compiler move every accumulator out of the AGPRs at once and spill)
  if (tid < BN / 4)
    bias_lds[tid] = (p.bias && n0 + tid * 4 < p.N)
                        ? *reinterpret_cast<const u32x2*>(p.bias + n0 + tid * 4)
                        : u32x2{0u, 0u};

  // Request K-tile t: the flag wait (fused mode, first K-tile of a staged k-group) and the
  // buffer resources; the DMA instructions themselves are issued one by one, between MFMAs.
  struct Req {
    rsrc_t ra, rb;
    int64_t k_rem;
  };
  // Fused mode: make the staged k-groups of K-tiles up to hi (of this piece) available.
  // Called once per block of NS K-tiles, before the block that requests them (their
  // requests follow a K-loop barrier), so the polling stays outside the MFMA stream; only
  // wave 0 acts, and only when the block reaches a k-group it has not acquired yet.
  auto wait_range = [&](int hi) {
    if (!waits || !wave0) return;
    const int g_need = (kt_lo + hi) / kpf;
    if (g_need >= ready_to) acquire_groups(g_need);
  };
  auto resources = [&](int t) -> Req {
    const int64_t ka = t * a_step, kb = t * b_step;
    return Req{make_rsrc(abase + ka, a_bytes - ka * 2), make_rsrc(bbase + kb, b_bytes - kb * 2),
               p.K - (int64_t)(kt_lo + t) * BK};
  };
  const uint32_t wave_u = uniform32((uint32_t)wave);
  auto issue = [&](int d, const Req& r, uint32_t stage_off) {
    if (d < T::ADMA)
      ad.issue(d, r.ra, stage_off, wave_u, r.k_rem);
    else
      bd.issue(d - T::ADMA, r.rb, stage_off + T::A_CH * 16, wave_u, 0);
  };
  auto request = [&](int t, uint32_t stage_off) {
    const Req r = resources(t);
#pragma unroll
    for (int d = 0; d < T::DMA_PER_TILE; ++d) issue(d, r, stage_off);
  };
  // Fragment read number i of a half step: A operands first, then B.
  auto read_one = [&](int i, const lds_u32x4* stage, int kk, u32x4 (&a)[T::FM], u32x4 (&b)[T::FN]) {
    if (i < T::FM) {
      if constexpr (A_KMAJOR)
        a[i] = KMajorDma<BM>::frag(stage, wm * T::WTM + i * 32, kk, lane);
      else
        a[i] = MNMajorDma<BM>::frag(stage, aoff[i], kk);
    } else {
      b[i - T::FM] = BDma::frag(stage + T::A_CH, boff[i - T::FM], kk);
    }
  };
  constexpr int NM = T::FM * T::FN, NR = T::FM + T::FN, ND = T::DMA_PER_TILE;

  u32x4 fa[2][T::FM], fb[2][T::FN];

  // One K-tile step with compile-time stage index S (= t % NS). FULL: t + NS < KT, so every
  // request below exists. The DMA of a K-tile is issued in two halves one step apart: its
  // A slice in part 2 of step t - NS (the step that frees the stage), its B slice in part 1
  // of step t - NS + 1, so the texture path and the LDS see a steady stream of requests
  // over the whole step instead of a burst after each barrier.
  constexpr int NS = T::NS;
  auto step = [&](auto s_tag, auto full_tag, int t) __attribute__((always_inline)) {
    constexpr int S = decltype(s_tag)::value;
    constexpr bool FULL = decltype(full_tag)::value;
    const lds_u32x4* cur = st.s(S);
    const lds_u32x4* nxt = st.s((S + 1) % NS);
    // part 1: sub-step 0 MFMAs of t; sub-step 1 fragments of t and the B slice of
    // t + NS - 1 (into the stage of t - 1, free since the last barrier) in between
    const bool do_req1 = FULL || t + NS - 1 < KT;
    const Req rq1 = resources(t + NS - 1);  // plain arithmetic, also past the last K-tile
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      const int fm = i / T::FN, fn = i % T::FN;
      acc[fm][fn] = Num<DT>::mfma(fb[0][fn], fa[0][fm], acc[fm][fn]);
#pragma unroll
      for (int r = 0; r < NR; ++r)
        if (spread(r, NR, NM, 0) == i) read_one(r, cur, 1, fa[1], fb[1]);
      if (do_req1) {
#pragma unroll
        for (int d = 0; d < T::BDMA; ++d)
          if (spread(d, T::BDMA, NM, 1) == i)
            issue(T::ADMA + d, rq1, st.off((S + NS - 1) % NS));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // requests issued after the last one of t + 1, which this wave may leave in flight:
    // those of t + 2 .. t + NS - 1 that exist
    if constexpr (FULL)
      wait_vmcnt<(NS - 2) * ND>();
    else
      wait_vmcnt_times<ND, NS - 2>(min(KT - 1, t + NS - 1) - (t + 1));
    kloop_barrier();
    // part 2: sub-step 1 MFMAs of t; the A slice of t + NS into stage S and sub-step 0
    // fragments of t + 1 in between
    const bool do_req = FULL || t + NS < KT;
    const bool do_read = FULL || t + 1 < KT;
    const Req rq = resources(t + NS);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      const int fm = i / T::FN, fn = i % T::FN;
      acc[fm][fn] = Num<DT>::mfma(fb[1][fn], fa[1][fm], acc[fm][fn]);
      if (do_req) {
#pragma unroll
        for (int d = 0; d < T::ADMA; ++d)
          if (spread(d, T::ADMA, NM, 0) == i) issue(d, rq, st.off(S));
      }
      if (do_read) {
#pragma unroll
        for (int r = 0; r < NR; ++r)
          if (spread(r, NR, NM, 1) == i) read_one(r, nxt, 0, fa[0], fb[0]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using YES = std::true_type;
  using NO = std::false_type;

  if (KT > 0) {
    // K-tiles 0 .. NS - 2 and the A slice of NS - 1 (k-groups acquired before the tile's
    // barrier); step 0 requests the B slice of NS - 1
    static_for<0, NS - 1>([&](auto j) __attribute__((always_inline)) {
      if (j < KT) request(j, st.off(j));
    });
    if (KT > NS - 1) {
      const Req r = resources(NS - 1);
#pragma unroll
      for (int d = 0; d < T::ADMA; ++d) issue(d, r, st.off(NS - 1));
    }
    // requests after the last one of K-tile 0
    if (KT - 1 >= NS - 1)
      wait_vmcnt<(NS - 2) * ND + T::ADMA>();
    else
      wait_vmcnt_times<ND, NS - 2>(KT - 1);
    kloop_barrier();
#pragma unroll
    for (int r = 0; r < NR; ++r) read_one(r, st.s(0), 0, fa[0], fb[0]);
    int t = 0;
    for (; t + 2 * NS <= KT; t += NS) {
      if constexpr (!ROW) wait_range(t + 2 * NS - 1);
      static_for<0, NS>([&](auto j) __attribute__((always_inline)) { step(j, YES{}, t + j); });
    }
    // the last NS .. 2 NS - 1 K-tiles (fewer when KT < 2 NS): at most two passes
    if constexpr (!ROW) wait_range(KT - 1);
    for (; t < KT; t += NS) {
      static_for<0, NS>([&](auto j) __attribute__((always_inline)) {
        if (t + j < KT) step(j, NO{}, t + j);
      });
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  if (tid == 0) *next_tile = grab(p);

  // Split tile: this piece's partial sums go to its slot (4-float group (fm, fn, g) of
  // thread tid at index ((fm * FN + fn) * 4 + g) * kThreads + tid, so a wave writes 1 KiB
  // runs), then the piece is counted; only the piece that completes the tile goes on.
  bool finish_split = false;  // this piece completes a split tile
  const u32x4* parts = nullptr;
  mfma_drain();
  if (pieces > 1) {
    const int64_t sidx = (int64_t)t_m * p.T_n + t_n - p.split_base;
    u32x4* slots = reinterpret_cast<u32x4*>(p.partials + sidx * pieces * (BM * BN));
    u32x4* mine = slots + (int64_t)piece * (BM * BN / 4);
#pragma unroll
    for (int fm = 0; fm < T::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < T::FN; ++fn)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          mine[((fm * T::FN + fn) * 4 + g) * kThreads + tid] =
              u32x4{__builtin_bit_cast(uint32_t, acc_read(acc[fm][fn], 4 * g + 0)),
                    __builtin_bit_cast(uint32_t, acc_read(acc[fm][fn], 4 * g + 1)),
                    __builtin_bit_cast(uint32_t, acc_read(acc[fm][fn], 4 * g + 2)),
                    __builtin_bit_cast(uint32_t, acc_read(acc[fm][fn], 4 * g + 3))};
    // Published as a fetch unit is: every wave's stores acknowledged, a barrier, one
    // agent-scope release by thread 0 (one L2 write-back, not one per wave); the piece that
    // completes the tile acquires once, in wave 0, before the barrier that lets the other
    // waves read the slots (an acquire invalidates the XCD's L2 under every tile there).
    wait_vmcnt<0>();
    __syncthreads();
    if (tid == 0) {
      const uint32_t done = __hip_atomic_fetch_add(p.split_cnt + sidx, 1u, __ATOMIC_RELEASE,
                                                   __HIP_MEMORY_SCOPE_AGENT) + 1u;
      const bool last = done == (uint32_t)pieces * epoch;  // counters grow by `pieces` per run
      if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      *is_last = last;
    }
    __syncthreads();
    if (!*is_last) return;
    parts = slots;
    finish_split = true;
  }

  // GEMM + all-reduce with atomics (ROCm/iris PR "Let's make Iris' All-reduce the best!", the
  // atomics example): this rank's partial tile is added into every rank's fp32 result,
  // starting with rank + 1's (the order that spreads a multi-GPU run over its peers).
  // The accumulator layout gives a lane 4 columns of one row and the wave 32 rows, so an
  // atomic issued from it would touch 32 cache lines; instead each wave passes its block
  // through LDS 32 rows at a time and reads it back so that one instruction's lanes cover
  // consecutive columns of one row (two 128-byte lines at WTN >= 64).
  // EPI 2 (the per-tile flag variant): the same pass through LDS, read back as 16-byte row
  // pieces and stored plainly into rank src's partial buffer p.partials + src * M * N
  // ([M][N]); the caller publishes it.
  if constexpr (EPI == 1 || EPI == 2) {
    typedef __attribute__((address_space(3))) float lds_f32;
    typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
    constexpr int RS = T::WTN + 4;                   // padded row stride (floats)
    constexpr int LPR = T::WTN < 64 ? T::WTN : 64;   // lanes per row on read-back
    constexpr int RPI = 64 / LPR;                    // rows per read-back instruction
    constexpr int CPL = T::WTN / LPR;                // read-back columns per lane and row
    constexpr int NV = 32 * T::WTN / 64;             // read-back values per lane per block
    constexpr int VG = NV < 16 ? NV : 16;            // values held per group
    static_assert(kThreads / 64 * 32 * RS * 4 <= T::NS * T::STAGE * 16, "blocks fit the stages");
    static_assert(NV % VG == 0, "whole groups");
    wait_vmcnt<0>();
    __syncthreads();  // every wave is done with the stages
    lds_f32* blk = reinterpret_cast<lds_f32*>(st.s(0)) + wave * (32 * RS);
    const int rl = lane / LPR, cl = lane % LPR;
#pragma unroll
    for (int fm = 0; fm < T::FM; ++fm) {
#pragma unroll
      for (int fn = 0; fn < T::FN; ++fn)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 v;
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j] = acc_read(acc[fm][fn], 4 * g + j);
          *reinterpret_cast<lds_f32x4*>(blk + (lane & 31) * RS + fn * 32 + g * 8 + (lane >> 5) * 4) = v;
        }
      __syncthreads();
      const int tr0 = wm * T::WTM + fm * 32;  // tile row of the block's first row
      const int tc0 = wn * T::WTN;            // tile column of its first column
      if constexpr (EPI == 2) {
        // plain stores: a lane takes 4 consecutive columns of one row (16-byte LDS reads
        // and global stores; N, and so cols_valid, is a multiple of 8)
        constexpr int L4 = T::WTN / 4;  // lanes per row
        constexpr int R4 = 64 / L4;     // rows per instruction
        const int rl4 = lane / L4, c4 = (lane % L4) * 4;
        float* dst = p.partials + (int64_t)src * p.M * p.N;
#pragma unroll
        for (int i = 0; i < 32 / R4; ++i) {
          const int r = i * R4 + rl4, tr = tr0 + r, tc = tc0 + c4;
          const f32x4 v = *reinterpret_cast<lds_f32x4*>(blk + r * RS + c4);
          if (tr < rows_valid && tc < cols_valid)
            *reinterpret_cast<f32x4*>(dst + (m0 + tr) * p.N + n0 + tc) = v;
        }
      } else {
#pragma unroll
        for (int v0 = 0; v0 < NV; v0 += VG) {
          float x[VG];
#pragma unroll
          for (int k = 0; k < VG; ++k) {
            const int v = v0 + k;
            x[k] = blk[((v / CPL) * RPI + rl) * RS + (v % CPL) * LPR + cl];
          }
          for (int i = 0; i < p.ar_D; ++i) {
            float* dst = p.ar_out[(p.ar_rank + 1 + i) % p.ar_D];
#pragma unroll
            for (int k = 0; k < VG; ++k) {
              const int v = v0 + k;
              const int tr = tr0 + (v / CPL) * RPI + rl, tc = tc0 + (v % CPL) * LPR + cl;
              if (tr < rows_valid && tc < cols_valid)
                __hip_atomic_fetch_add(dst + (m0 + tr) * p.N + n0 + tc, x[k], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
          }
        }
      }
      __syncthreads();  // the block is read before the next one overwrites it
    }
    return;
  }

  // Epilogue through LDS (all stages are free: every DMA has landed and the last barrier
  // is behind every wave): each lane adds the bias in fp32, rounds once (RNE) and writes 4
  // consecutive outputs (8 bytes) of one row into the output tile, whose row quarter
  // q = r / (BM/4) lives in stage q; then every thread copies 16-byte row chunks to global
  // memory, a wave's lanes covering whole rows. 8-byte unit u of row r sits at unit
  // u ^ (r & XM), so the 32 rows written by one instruction and the chunks of a row read
  // back spread over the banks.
  wait_vmcnt<0>();
  __syncthreads();
  constexpr int ROW_U = BN / 4;  // 8-byte units per tile row
  constexpr int XM = (ROW_U < 32 ? ROW_U : 32) - 1;
  constexpr int QR = BM / 4;     // rows per quarter
  // (stages are contiguous: quarter q starts q stages after stage 0)
  auto unit_ptr = [&](int r, int u) -> lds_u32* {
    return reinterpret_cast<lds_u32*>(st.s(0)) + (r / QR) * (T::STAGE * 4) +
           ((r % QR) * ROW_U + u) * 2;
  };
  // The accumulators to LDS; SPLIT: plus the other pieces' partial sums, added in piece
  // order (reads past the last piece are out of the slots' range and return zeros, so
  // the code has no branch). Two copies, chosen once per tile.
  auto to_lds = [&](auto split_tag) {
    constexpr bool SPLIT = decltype(split_tag)::value;
    const rsrc_t prs = make_rsrc(reinterpret_cast<const uint16_t*>(parts),
                                 SPLIT ? (int64_t)pieces * BM * BN * 4 : 0);
    // this lane's bias pairs, read from LDS in one batch (one wait instead of one per group)
    u32x2 bias_r[T::FN][4];
#pragma unroll
    for (int fn = 0; fn < T::FN; ++fn)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        bias_r[fn][g] = bias_lds[(wn * T::WTN + fn * 32 + g * 8 + (lane >> 5) * 4) >> 2];
#pragma unroll
    for (int fm = 0; fm < T::FM; ++fm) {
      const int ml = wm * T::WTM + fm * 32 + (lane & 31);
#pragma unroll
      for (int fn = 0; fn < T::FN; ++fn) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int nl = wn * T::WTN + fn * 32 + g * 8 + (lane >> 5) * 4;
          float x0 = acc_read(acc[fm][fn], 4 * g + 0), x1 = acc_read(acc[fm][fn], 4 * g + 1);
          float x2 = acc_read(acc[fm][fn], 4 * g + 2), x3 = acc_read(acc[fm][fn], 4 * g + 3);
          if constexpr (SPLIT) {
            const uint32_t e = (uint32_t)(((fm * T::FN + fn) * 4 + g) * kThreads + tid) * 16u;
            float y0 = 0.f, y1 = 0.f, y2 = 0.f, y3 = 0.f;
            // The loaded vectors pass through an empty asm that takes them whole: when only
            // some lanes of a 16-byte buffer load are read, the optimizer narrows it to
            // dword loads and reads the same dword for every element.
            u32x4 lv[kMaxSplit];
#pragma unroll
            for (int sp = 0; sp < kMaxSplit; ++sp)
              lv[sp] = bload16(prs, (uint32_t)sp * (BM * BN * 4) + e);
#pragma unroll
            for (int sp = 0; sp < kMaxSplit; ++sp) asm volatile("" : "+v"(lv[sp]));
#pragma unroll
            for (int sp = 0; sp < kMaxSplit; ++sp) {
              const f32x4 lf = __builtin_bit_cast(f32x4, lv[sp]);
              const bool own = sp == piece;
              const float v0 = own ? x0 : lf.x;
              const float v1 = own ? x1 : lf.y;
              const float v2 = own ? x2 : lf.z;
              const float v3 = own ? x3 : lf.w;
              if (sp == 0) {
                y0 = v0, y1 = v1, y2 = v2, y3 = v3;
              } else {
                y0 += v0, y1 += v1, y2 += v2, y3 += v3;
              }
            }
            x0 = y0, x1 = y1, x2 = y2, x3 = y3;
          }
          const u32x2 bb = bias_r[fn][g];
          x0 += Num<DT>::from_bits(bb[0] & 0xffffu);
          x1 += Num<DT>::from_bits(bb[0] >> 16);
          x2 += Num<DT>::from_bits(bb[1] & 0xffffu);
          x3 += Num<DT>::from_bits(bb[1] >> 16);
          u32x2 o;
          o[0] = Num<DT>::to_bits(x0) | (Num<DT>::to_bits(x1) << 16);
          o[1] = Num<DT>::to_bits(x2) | (Num<DT>::to_bits(x3) << 16);
          *reinterpret_cast<lds_u32x2*>(unit_ptr(ml, (nl >> 2) ^ (ml & XM))) = o;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  if (finish_split)
    to_lds(std::true_type{});
  else
    to_lds(std::false_type{});
  __syncthreads();
  // The tile to global memory: each thread's chunks c = tid + i * kThreads, read from LDS
  // in batches of CB before their stores; chunks outside the output (ragged tiles) go to an
  // out-of-range offset, so the stores need no branch.
  constexpr int ROW_C = BN / 8;  // 16-byte chunks per row
  constexpr int CPT = BM * ROW_C / kThreads, CB = CPT < 8 ? CPT : 8;
  static_assert(CPT % CB == 0, "chunk batches");
  const rsrc_t ors = make_rsrc(p.out + m0 * p.N + n0, (p.M - m0) * p.N * 2 - n0 * 2);
#pragma unroll
  for (int i0 = 0; i0 < CPT; i0 += CB) {
    u32x4 v[CB];
    uint32_t off[CB];
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      const int c = tid + (i0 + j) * kThreads, r = c / ROW_C, ch = c % ROW_C;
      const int sw = r & XM;
      v[j] = *reinterpret_cast<const lds_u32x4*>(unit_ptr(r, ((2 * ch) ^ sw) & ~1));
      if (sw & 1) v[j] = u32x4{v[j][2], v[j][3], v[j][0], v[j][1]};
      off[j] = (r < rows_valid && ch * 8 < cols_valid) ? (uint32_t)((r * p.N + ch * 8) * 2) : kOob;
    }
#pragma unroll
    for (int j = 0; j < CB; ++j) bstore16(ors, off[j], v[j]);
  }
  __syncthreads();  // the tile area is the next tile's stages
}

// Global row m of the gathered A; `shards` is the workgroup's LDS copy of the pointers.
__device__ inline const uint16_t* arow(const KParams& p, const uint16_t* const* shards,
                                       int64_t m) {
  const uint32_t d = (uint32_t)m / (uint32_t)p.M_s;
  return shards[d] + (m - (int64_t)d * p.M_s) * p.K;
}

// Copies the shard pointer table into LDS (threads 0..D-1), so per-row lookups index LDS.
__device__ inline void load_shard_table(const KParams& p, const uint16_t** table, int tid) {
  if (tid < p.D) table[tid] = p.shards[tid];
  __syncthreads();
}

// A fetcher workgroup copies far below its share of the HBM bandwidth, so the copies run as
// a two-batch software pipeline: the loads of batch n + 1 are issued before the stores of
// batch n, so neither waits for the other (a wait for loads also waits for every store
// issued before them: the vector memory counter retires in order). A batch is BATCH
// 16-byte loads per thread (kCopyBatch: 64 KiB per workgroup); at most three batches of
// requests are in flight, within the counter's range of 63. More requests in flight do not
// make the fused run faster: with 24 loads per batch the fetchers finish sooner, but their
// denser traffic slows the GEMM workgroups beside them by more (8 per batch ran as fast as
// 16). The
// fetch kernel that runs beside the GEMM kernel takes kSmallCopyBatch, so that its data
// registers (two batches) fit in what a GEMM wave leaves of a SIMD's register file
// (8 for the m_contiguous copy, whole 8x8 blocks; 4 for the k_contiguous one, whose GEMM
// waves take 16 registers more and which also keeps an offset per load).
constexpr int kCopyBatch = 16;
template <bool LAYOUT_K>
constexpr int kSmallCopyBatch = LAYOUT_K ? 4 : 8;

// Source row pointers of one unit: rows m_beg .. m_beg + R - 1 of the gathered A. A unit
// inside one shard (the usual case) needs no per-row shard lookup.
struct UnitRows {
  const uint16_t* base;  // row m_beg when the unit lies in one shard, else nullptr
  __device__ inline UnitRows(const KParams& p, const uint16_t* const* shards, int64_t m_beg,
                             int R) {
    const int64_t d0 = m_beg / p.M_s, d1 = (m_beg + R - 1) / p.M_s;
    base = d0 == d1 ? shards[d0] + (m_beg - d0 * p.M_s) * p.K : nullptr;
  }
  __device__ inline const uint16_t* row(const KParams& p, const uint16_t* const* shards,
                                        int64_t m_beg, int r) const {
    return base ? base + (int64_t)r * p.K : arow(p, shards, m_beg + r);
  }
};


// Copy unit (t_m, g) into k_contiguous staging: 16-byte loads, then 16-byte stores. Chunk
// c = r * CR + cc of the unit goes to thread c % 256; the (r, cc) of successive chunks of a
// thread advance by fixed steps, so the loop does no division. When the unit lies in one
// shard (the usual case) the loads and stores are range-checked buffer accesses: a lane
// past the unit reads zero and its store is dropped, so every thread runs the same number
// of batches and the pipeline has no per-lane branch.
template <int BM, int BATCH = kCopyBatch>
__device__ void copy_unit_kmajor(const KParams& p, const uint16_t* const* shards, int t_m, int g,
                                 int KG, int tid, int row0, int nrows) {
  const int64_t m_beg = (int64_t)t_m * BM + row0;
  const int R = (int)min((int64_t)nrows, p.M - m_beg);
  const int64_t k_beg = (int64_t)g * KG;
  const int CR = (int)(min((int64_t)KG, p.K - k_beg) / 8);
  if (CR <= 0 || R <= 0) return;
  const UnitRows rows(p, shards, m_beg, R);
  const int dr = kThreads / CR, dc = kThreads - dr * CR;  // step of (r, cc) per chunk
  int r = tid / CR, cc = tid - (tid / CR) * CR;
  const int64_t span = (int64_t)R * p.K * 2;  // bytes of the unit's row range
  if (rows.base && span <= 0x7fffffffll) {
    const rsrc_t src = make_rsrc(rows.base, span);
    const rsrc_t dst = make_rsrc(p.staging + m_beg * p.K, span);
    const int batches = (R * CR + kThreads * BATCH - 1) / (kThreads * BATCH);
    u32x4 va[BATCH], vb[BATCH];
    uint32_t oa[BATCH], ob[BATCH];
    auto load = [&](u32x4 (&v)[BATCH], uint32_t (&o)[BATCH]) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < BATCH; ++i) {
        o[i] = r < R ? (uint32_t)(((int64_t)r * p.K + k_beg + cc * 8) * 2) : kOob;
        v[i] = bload16(src, o[i]);
        r += dr;
        cc += dc;
        if (cc >= CR) {
          cc -= CR;
          ++r;
        }
      }
    };
    auto store = [&](const u32x4 (&v)[BATCH], const uint32_t (&o)[BATCH]) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < BATCH; ++i) bstore16(dst, o[i], v[i]);
    };
    load(va, oa);
    for (int n = 0; n < batches; n += 2) {
      load(vb, ob);  // past the last batch: all out of range
      store(va, oa);
      if (n + 2 < batches) load(va, oa);
      store(vb, ob);
    }
    return;
  }
  uint16_t* const dst0 = p.staging + m_beg * p.K + k_beg;
  for (; r < R;) {
    const u32x4 v = ld16(rows.row(p, shards, m_beg, r) + k_beg + cc * 8);
    st16(dst0 + (int64_t)r * p.K + cc * 8, v);
    r += dr;
    cc += dc;
    if (cc >= CR) {
      cc -= CR;
      ++r;
    }
  }
}

// Copy unit (t_m, g) into m_contiguous staging: each thread transposes 8x8 blocks (8 rows x
// 8 K values), NB per batch. Block (kb, mb) is numbered b with kb = (b / (8 NBM)) * 8 +
// b % 8 and mb = (b / 8) % NBM, so 8 consecutive lanes read 128 contiguous bytes of one row;
// a thread's blocks b, b + 256, ... advance (kb, mb) by fixed steps (no division). Same
// buffer-access fast path and pipeline as the k_contiguous copy.
template <int BM, int BATCH = kCopyBatch>
__device__ void copy_unit_mmajor(const KParams& p, const uint16_t* const* shards, int t_m, int g,
                                 int KG, int tid, int row0, int nrows) {
  static_assert(BATCH % 8 == 0, "whole 8x8 blocks per batch");
  constexpr int NB = BATCH / 8;  // blocks per thread and batch
  const int64_t m_beg = (int64_t)t_m * BM + row0;
  const int R = (int)min((int64_t)nrows, p.M - m_beg);    // multiple of 8
  const int64_t k_beg = (int64_t)g * KG;
  const int NBK = (int)(min((int64_t)KG, p.K - k_beg) / 8);
  const int NBM = R / 8;
  if (NBK <= 0 || NBM <= 0) return;
  const UnitRows rows(p, shards, m_beg, R);
  // t = b / 8 = kbh * NBM + mb; a thread's t advances by 32 per block
  const int dkh = (kThreads / 8) / NBM, dmb = (kThreads / 8) - dkh * NBM;
  const int t0 = tid >> 3, lo = tid & 7;
  int kbh = t0 / NBM, mb = t0 - (t0 / NBM) * NBM;
  const int64_t sspan = (int64_t)R * p.K * 2, dspan = (int64_t)NBK * 8 * p.M * 2;
  if (rows.base && sspan <= 0x7fffffffll && dspan <= 0x7fffffffll) {
    const rsrc_t src = make_rsrc(rows.base, sspan);
    const rsrc_t dst = make_rsrc(p.staging + k_beg * p.M + m_beg, dspan - m_beg * 2);
    const int tt = ((NBK + 7) / 8) * NBM;  // values of t
    const int batches = (tt + (kThreads / 8) * NB - 1) / ((kThreads / 8) * NB);
    u32x4 va[NB][8], vb[NB][8];
    uint32_t da[NB], db[NB];
    auto load = [&](u32x4 (&v)[NB][8], uint32_t (&d)[NB]) __attribute__((always_inline)) {
#pragma unroll
      for (int q = 0; q < NB; ++q) {
        const int kb = kbh * 8 + lo;
        const bool ok = kb < NBK;  // also false for every t past the unit
        const uint32_t soff = (uint32_t)((((int64_t)mb * 8) * p.K + k_beg + kb * 8) * 2);
        d[q] = ok ? (uint32_t)(((int64_t)kb * 8 * p.M + mb * 8) * 2) : kOob;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          v[q][j] = bload16(src, ok ? soff + (uint32_t)(j * p.K * 2) : kOob);
        kbh += dkh;
        mb += dmb;
        if (mb >= NBM) {
          mb -= NBM;
          ++kbh;
        }
      }
    };
    auto store = [&](const u32x4 (&v)[NB][8], const uint32_t (&d)[NB]) __attribute__((always_inline)) {
#pragma unroll
      for (int q = 0; q < NB; ++q)
#pragma unroll
        for (int i = 0; i < 8; ++i)
          bstore16(dst, d[q] == kOob ? kOob : d[q] + (uint32_t)(i * p.M * 2),
                   transpose_row(v[q], i));
    };
    load(va, da);
    for (int n = 0; n < batches; n += 2) {
      load(vb, db);  // past the last batch: all out of range
      store(va, da);
      if (n + 2 < batches) load(va, da);
      store(vb, db);
    }
    return;
  }
  while (kbh * 8 < NBK) {
    const int kb = kbh * 8 + lo;
    if (kb < NBK) {
      u32x4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        v[j] = ld16(rows.row(p, shards, m_beg, mb * 8 + j) + k_beg + kb * 8);
      uint16_t* dst = p.staging + (k_beg + kb * 8) * p.M + m_beg + mb * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) st16(dst + (int64_t)i * p.M, transpose_row(v, i));
    }
    kbh += dkh;
    mb += dmb;
    if (mb >= NBM) {
      mb -= NBM;
      ++kbh;
    }
  }
}

// Baseline copy: units f, f+F, f+2F, ... of the fetch order, whole units, no flags.
template <class T>
__device__ void copy_units(const KParams& p, const uint16_t* const* shards, int f, int F, int tid) {
  const int KG = p.kpf * T::BK;
  for (int u = f; u < p.num_units; u += F) {
    const int t_m = (int)p.units[2 * u], g = (int)p.units[2 * u + 1];
    copy_unit_kmajor<T::BM>(p, shards, t_m, g, KG, tid, 0, T::BM);
  }
}

// Fused mode: copy unit u into staging, then publish it: each wave waits for its stores,
// a workgroup barrier, and thread 0 adds 1 to the unit's flag with one agent-scope release
// (a single L2 write-back for the workgroup instead of one per wave: a write-back flushes
// the XCD's whole L2, which the GEMM workgroups beside this one are using).
template <class T, bool LAYOUT_K, int BATCH = kCopyBatch>
__device__ __attribute__((always_inline)) void fetch_unit(const KParams& p,
                                                          const uint16_t* const* shards, int u,
                                                          int tid, Tracer& tr) {
  const int KG = p.kpf * T::BK;
  const uint64_t t0 = tr.now();
  const int t_m = (int)p.units[2 * u], g = (int)p.units[2 * u + 1];
  // stress knob: a per-unit delay from a hash of (unit, seed), so that units complete out of
  // their fetch order (every wave sleeps the same count: the value is workgroup-uniform)
  const uint32_t max_delay = uniform32(p.ctr[CTR_DBG_DELAY]);
  if (max_delay) {
    uint32_t h = (uint32_t)u * 0x9E3779B1u ^ uniform32(p.ctr[CTR_DBG_SEED]);
    h ^= h >> 15;
    h *= 0x2C1B3C6Du;
    h ^= h >> 12;
    for (uint32_t i = h % max_delay; i > 0; --i) __builtin_amdgcn_s_sleep(2);
  }
  if constexpr (LAYOUT_K)
    copy_unit_kmajor<T::BM, BATCH>(p, shards, t_m, g, KG, tid, 0, T::BM);
  else
    copy_unit_mmajor<T::BM, BATCH>(p, shards, t_m, g, KG, tid, 0, T::BM);
  wait_vmcnt<0>();
  __syncthreads();
  if (tid == 0) {
    if (u != p.skip_unit)
      __hip_atomic_fetch_add(p.flags + (int64_t)t_m * p.G + g, 1u, __ATOMIC_RELEASE,
                             __HIP_MEMORY_SCOPE_AGENT);
    tr.rec(AGMM_EV_FETCH, (uint32_t)u, (uint32_t)t_m, (uint32_t)g, t0);
  }
}

// Claims the next fetch unit for the workgroup (>= p.num_units: none left). slot: an LDS
// word; the caller's next claim comes after a barrier (fetch_unit has one).
__device__ inline int claim_unit(const KParams& p, int* slot, int tid) {
  if (tid == 0) {
    int u = aborted(p) ? p.num_units
                       : (int)min((uint32_t)p.num_units, atomicAdd(p.ctr + CTR_FETCH, 1u));
    // stress knob: the n-th claim takes unit num_units - 1 - n (still each unit once)
    if (u < p.num_units && p.ctr[CTR_DBG_REVERSE]) u = p.num_units - 1 - u;
    *slot = u;
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(*slot);
}

// Next queue entry for this workgroup, or -1: its XCD's queue first, then the other XCD
// queues, then the tail queue of split-tile pieces.
__device__ inline int grab(const KParams& p) {
  if (aborted(p)) return -1;
  const int x0 = (int)(blockIdx.x % kQueues);
  for (int s = 0; s < kQueueSlots; ++s) {
    const int x = s < kQueues ? (x0 + s) % kQueues : kTailQueue;
    uint32_t* c = p.ctr + CTR_Q + x * CTR_QSTRIDE;
    const uint32_t len = (uint32_t)p.qlen[x];
    if (len == 0) continue;
    // Always the read-modify-write: a plain load of another XCD's queue counter can return a
    // stale "exhausted" value and send the workgroup away while tiles are left.
    const uint32_t i = atomicAdd(c, 1u);
    if (i < len) return (int)p.qtiles[p.qoff[x] + (int)i];
  }
  return -1;
}

// FUSED: fetchers + flag waits; LAYOUT_K: staging is k_contiguous (staged and in-place
// tiles then share one K-major tile routine), else m_contiguous. ROW (fused): a tile waits
// at its start for all of its k-groups and its K loop has no waits (used when every fetch
// unit has a fetcher of its own, so the whole fetch is one pass); otherwise the K loop
// waits for each k-group as it gets there.
template <int BM, int DT, bool FUSED, bool LAYOUT_K, bool ROW, int EPI = 0>
__global__ __launch_bounds__(kThreads) void agmm_persistent(KParams p) {
  using T = Tile<BM>;
  // the stages, contiguous: a stage's base is then arithmetic on the first one's address,
  // also where the stage index is only known at run time (the epilogue)
  __shared__ u32x4 lds_stages[T::NS * T::STAGE];
  __shared__ u32x2 s_bias[T::BN / 4];
  const Stages<T> st{(lds_u32x4*)lds_stages, (uint32_t)(size_t)(lds_void*)lds_stages};
  __shared__ int s_next, s_last, s_claim;
  __shared__ uint32_t s_epoch;
  __shared__ const uint16_t* s_shards[AGMM_MAX_SHARDS];
  const int tid = threadIdx.x, wg = blockIdx.x;
  Tracer tr{p.debug ? p.trace + (size_t)wg * p.trace_cap : nullptr, 0u, (uint32_t)p.trace_cap,
            p.debug != 0};

  if constexpr (FUSED) {
    load_shard_table(p, s_shards, tid);
    if (wg < p.F) {  // fetcher: claim units until none is left, then compute like the rest
      for (;;) {
        const int u = claim_unit(p, &s_claim, tid);
        if (u >= p.num_units) break;
        fetch_unit<T, LAYOUT_K>(p, s_shards, u, tid, tr);
      }
    }
  }

  if (tid == 0) first_claim(p, &s_next, &s_epoch);
  __syncthreads();
  int q = __builtin_amdgcn_readfirstlane(s_next);  // uniform: tile addressing in SGPRs
  const uint32_t epoch = uniform32(s_epoch);
  while (q >= 0) {
    __syncthreads();  // everyone has read s_next
    const int tile = (int)((uint32_t)q & kItemTileMask);
    const int piece = ((uint32_t)q >> 24) & 15, pieces = (int)((uint32_t)q >> 28) + 1;
    const int pos = tile / p.T_n, t_n = tile - pos * p.T_n;
    const uint32_t e = p.mtiles[pos];
    const int t_m = (int)(e & 0x7fffffffu);
    const bool staged = (e >> 31) == 0u;
    const uint64_t t0 = tr.now();
    if constexpr (!FUSED) {
      gemm_tile<T, DT, true, false, false, EPI>(p, t_m, t_n, piece, pieces, staged, st, s_bias, tid, tr, &s_next, &s_last, epoch);
    } else if constexpr (LAYOUT_K) {
      gemm_tile<T, DT, true, true, ROW>(p, t_m, t_n, piece, pieces, staged, st, s_bias, tid, tr, &s_next, &s_last, epoch);
    } else {
      if (!staged)
        gemm_tile<T, DT, true, true, ROW>(p, t_m, t_n, piece, pieces, staged, st, s_bias, tid, tr, &s_next, &s_last, epoch);
      else
        gemm_tile<T, DT, false, true, ROW>(p, t_m, t_n, piece, pieces, staged, st, s_bias, tid, tr, &s_next, &s_last, epoch);
    }
    tr.rec(AGMM_EV_GEMM, (uint32_t)q, (uint32_t)t_m, (uint32_t)t_n, t0);
    __syncthreads();
    q = __builtin_amdgcn_readfirstlane(s_next);
  }

  if (tid == 0) {
    if (p.debug) p.trace_count[wg] = tr.n;
    const uint32_t old = atomicAdd(p.ctr + CTR_DONE, 1u);
    if (old == gridDim.x - 1) {  // last workgroup out resets the queues for the next run
      for (int x = 0; x < kQueueSlots; ++x)
        __hip_atomic_store(p.ctr + CTR_Q + x * CTR_QSTRIDE, 0u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      // the unit counter only when this grid held the fetchers (a fetch kernel running
      // beside it resets its own, and may still be claiming units nobody waits for)
      if (p.F > 0)
        __hip_atomic_store(p.ctr + CTR_FETCH, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(p.ctr + CTR_RUNS, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(p.ctr + CTR_DONE, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      mirror_status(p);
    }
  }
}

// GEMM + all-reduce with per-tile flags (ROCm/iris PR "Let's make Iris' All-reduce the
// best!", its one-shot variant with a ready flag per tile), every rank's share in one
// launch. Items, in the order of p.qtiles (queue 0 only): producer (r << 24 | tile)
// computes rank r's partial tile A_r @ B_r into p.partials + r * M * N and publishes flag
// r * tiles + tile with the run's epoch; reducer (kArReduceItem | tile) waits for the D flags
// of its tile and writes RNE(sum over r in rank order + bias). A reducer comes after its
// tile's D producers in the claim order, and producers never wait, so every wait ends.

template <class T, int DT>
__device__ __attribute__((always_inline)) void reduce_tile(const KParams& p, int t_m, int t_n,
                                                           int tile, int tid, Tracer& tr,
                                                           uint32_t epoch) {
  constexpr int BM = T::BM, BN = T::BN;
  const int64_t tiles = (int64_t)p.T_m * p.T_n;
  if (__builtin_amdgcn_readfirstlane(tid >> 6) == 0) {
    for (int r = 0; r < p.ar_D; ++r) poll_flag(p, r * tiles + tile, epoch, tr);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  const int64_t m0 = (int64_t)t_m * BM, n0 = (int64_t)t_n * BN, MN = p.M * p.N;
  const int rows = (int)min((int64_t)BM, p.M - m0), cols = (int)min((int64_t)BN, p.N - n0);
  // four consecutive columns per thread and step (N and so cols are multiples of 8: a group
  // is wholly inside or outside); up to 8 ranks' loads in flight before their adds
  for (int e = tid * 4; e < BM * BN; e += kThreads * 4) {
    const int row = e / BN, col = e % BN;
    if (row >= rows || col >= cols) continue;
    const float* src = p.partials + (m0 + row) * p.N + n0 + col;
    f32x4 acc = *reinterpret_cast<const f32x4*>(src);
    for (int r0 = 1; r0 < p.ar_D; r0 += 8) {
      f32x4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (r0 + j < p.ar_D) v[j] = *reinterpret_cast<const f32x4*>(src + (r0 + j) * MN);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (r0 + j < p.ar_D) acc += v[j];
    }
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float x = acc[j];
      if (p.bias) x += Num<DT>::from_bits(p.bias[n0 + col + j]);
      o[j] = Num<DT>::to_bits(x);
    }
    *reinterpret_cast<u32x2*>(p.out + (m0 + row) * p.N + n0 + col) =
        u32x2{o[0] | (o[1] << 16), o[2] | (o[3] << 16)};
  }
}

template <int BM, int DT>
__global__ __launch_bounds__(kThreads) void agmm_ar_flags(KParams p) {
  using T = Tile<BM>;
  __shared__ u32x4 lds_stages[T::NS * T::STAGE];
  __shared__ u32x2 s_bias[T::BN / 4];
  const Stages<T> st{(lds_u32x4*)lds_stages, (uint32_t)(size_t)(lds_void*)lds_stages};
  __shared__ int s_next, s_last;
  __shared__ uint32_t s_epoch;
  const int tid = threadIdx.x;
  Tracer tr{nullptr, 0u, 0u, false};
  const int64_t tiles = (int64_t)p.T_m * p.T_n;
  if (tid == 0) first_claim(p, &s_next, &s_epoch);
  __syncthreads();
  int q = __builtin_amdgcn_readfirstlane(s_next);
  const uint32_t epoch = uniform32(s_epoch);
  while (q >= 0) {
    __syncthreads();  // everyone has read s_next
    const int tile = (int)((uint32_t)q & kItemTileMask);
    const int t_m = tile / p.T_n, t_n = tile - t_m * p.T_n;
    if (((uint32_t)q & kArReduceItem) == 0u) {
      const int r = (int)(((uint32_t)q >> 24) & 63u);
      gemm_tile<T, DT, true, false, false, 2>(p, t_m, t_n, 0, 1, false, st, s_bias, tid, tr,
                                              &s_next, &s_last, epoch, r);
      wait_vmcnt<0>();  // this thread's stores of the partial tile are done
      __syncthreads();
      if (tid == 0)
        __hip_atomic_store(p.flags + r * tiles + tile, epoch, __ATOMIC_RELEASE,
                           __HIP_MEMORY_SCOPE_AGENT);
    } else {
      reduce_tile<T, DT>(p, t_m, t_n, tile, tid, tr, epoch);
      if (tid == 0) s_next = grab(p);
    }
    __syncthreads();
    q = __builtin_amdgcn_readfirstlane(s_next);
  }
  if (tid == 0) {
    const uint32_t old = atomicAdd(p.ctr + CTR_DONE, 1u);
    if (old == gridDim.x - 1) {  // last workgroup out resets the queues for the next run
      for (int x = 0; x < kQueueSlots; ++x)
        __hip_atomic_store(p.ctr + CTR_Q + x * CTR_QSTRIDE, 0u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(p.ctr + CTR_RUNS, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(p.ctr + CTR_DONE, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      mirror_status(p);
    }
  }
}

// Baseline copy: every staged unit into k_contiguous staging, no flags.
template <int BM>
__global__ __launch_bounds__(kThreads) void agmm_copy(KParams p) {
  __shared__ const uint16_t* s_shards[AGMM_MAX_SHARDS];
  load_shard_table(p, s_shards, threadIdx.x);
  copy_units<Tile<BM>>(p, s_shards, blockIdx.x, gridDim.x, threadIdx.x);
}

// Up to kUploadWords words per launch, carried in the kernel argument (kept well under the
// size of the other kernels' argument block).
constexpr int kUploadWords = 256;
struct UploadWords {
  uint32_t n;
  uint32_t w[kUploadWords];
};

// The fetch as a kernel of its own, run on a second stream beside a fused GEMM grid that has
// no fetchers (p.F == 0): its workgroups claim units from the same counter and publish them
// exactly as in-kernel fetchers do. It needs no LDS beyond the claim slot and the shard
// table, and few enough VGPRs per lane that one of its workgroups fits on a CU beside a
// GEMM workgroup (which holds 424 or 440 of a SIMD's 512 registers per lane and 129 KiB of
// the 160 KiB of LDS): the fetch then runs on every CU while every CU computes. Trace
// records (debug) go to p.trace / p.trace_count, which the host offsets past the GEMM
// grid's. The last workgroup out resets the unit counter for the next run.
template <int BM, bool LAYOUT_K>
__device__ __attribute__((always_inline)) void fetch_kernel_body(const KParams& p) {
  using T = Tile<BM>;
  __shared__ int s_claim;
  __shared__ const uint16_t* s_shards[AGMM_MAX_SHARDS];
  const int tid = threadIdx.x;
  Tracer tr{p.debug ? p.trace + (size_t)blockIdx.x * p.trace_cap : nullptr, 0u,
            (uint32_t)p.trace_cap, p.debug != 0};
  load_shard_table(p, s_shards, tid);
  for (;;) {
    const int u = claim_unit(p, &s_claim, tid);
    if (u >= p.num_units) break;
    fetch_unit<T, LAYOUT_K, kSmallCopyBatch<LAYOUT_K>>(p, s_shards, u, tid, tr);
  }
  if (tid == 0) {
    if (p.debug) p.trace_count[blockIdx.x] = tr.n;
    const uint32_t old = atomicAdd(p.ctr + CTR_FDONE, 1u);
    if (old == gridDim.x - 1) {
      __hip_atomic_store(p.ctr + CTR_FETCH, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(p.ctr + CTR_FDONE, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}
// The VGPR cap of each instance is 512 minus the allocation of the GEMM waves it runs beside.
// m_contiguous staging: beside GEMM waves of 424 registers
template <int BM>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_num_vgpr(88)))
void agmm_fetch_m(KParams p) { fetch_kernel_body<BM, false>(p); }
// k_contiguous staging: beside GEMM waves of 440 registers
template <int BM>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_num_vgpr(72)))
void agmm_fetch_k(KParams p) { fetch_kernel_body<BM, true>(p); }

__global__ __launch_bounds__(kUploadWords) void upload32_kernel(uint32_t* dst, UploadWords p) {
  const uint32_t i = threadIdx.x;
  if (i < p.n) dst[i] = p.w[i];
}

// Measurement only: the MFMA rate this GPU sustains with operands held in registers (no
// memory traffic in the loop). Every wave runs 16 independent 32x32x16 accumulators on
// pseudo-random 16-bit operands (random signs and mantissas, like real data); with VARY they
// rotate through four register sets, otherwise one set is reused. One float per thread is
// written so the loop is not removed.
template <int DT, bool VARY>
__global__ __launch_bounds__(256) void mfma_loop_kernel(float* sink, int iters) {
  u32x4 av[4], bv[4];
  uint32_t h = threadIdx.x * 2654435761u + blockIdx.x * 40503u + 12345u;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t x[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        h ^= h << 13;
        h ^= h >> 17;
        h ^= h << 5;
        // a finite 16-bit value in [-1, 1): random mantissa and sign, small exponent
        x[j] = Num<DT>::to_bits(((int)(h & 0xffffu) - 32768) * (1.0f / 32768.0f));
      }
      av[r][i] = x[0] | (x[1] << 16);
      bv[r][i] = (x[0] ^ 0x5a5au) | ((x[1] ^ 0x3c3cu) << 16);
    }
  f32x16 acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = (f32x16)(0.0f);
  for (int it = 0; it < iters; it += 4) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int j = 0; j < 16; ++j)
        acc[j] = Num<DT>::mfma(VARY ? av[(r + j) & 3] : av[0], VARY ? bv[(3 * r + j) & 3] : bv[0],
                               acc[j]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j)
#pragma unroll
    for (int k = 0; k < 16; ++k) s += acc[j][k];
  sink[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ void fill16_kernel(uint16_t* dst, int64_t n, uint16_t v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = v;
}

__global__ void fill32_kernel(uint32_t* dst, int64_t n, uint32_t v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = v;
}

template <int BM, int DT, bool FUSED, bool LAYOUT_K, bool ROW>
hipError_t launch_t(const KParams& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL((agmm_persistent<BM, DT, FUSED, LAYOUT_K, ROW>), dim3(grid), dim3(kThreads),
                     0, s, p);
  return hipGetLastError();
}

template <int BM, bool FUSED, bool LAYOUT_K>
hipError_t launch_dt(const KParams& p, int dtype, int grid, hipStream_t s) {
  if constexpr (FUSED) {
    if (p.row_wait)
      return dtype == AGMM_BF16 ? launch_t<BM, AGMM_BF16, true, LAYOUT_K, true>(p, grid, s)
                                : launch_t<BM, AGMM_F16, true, LAYOUT_K, true>(p, grid, s);
  }
  return dtype == AGMM_BF16 ? launch_t<BM, AGMM_BF16, FUSED, LAYOUT_K, false>(p, grid, s)
                            : launch_t<BM, AGMM_F16, FUSED, LAYOUT_K, false>(p, grid, s);
}

// The gemm-only kernel reads k_contiguous staging only.
template <bool FUSED>
hipError_t launch_any(const KParams& p, int dtype, int block_m, int grid, hipStream_t s) {
  const bool lk = !FUSED || p.staged_kmajor;
  switch (block_m) {
    case 256:
      return lk ? launch_dt<256, FUSED, true>(p, dtype, grid, s)
                : launch_dt<256, FUSED, !FUSED>(p, dtype, grid, s);
    case 128:
      return lk ? launch_dt<128, FUSED, true>(p, dtype, grid, s)
                : launch_dt<128, FUSED, !FUSED>(p, dtype, grid, s);
    case 64:
      return lk ? launch_dt<64, FUSED, true>(p, dtype, grid, s)
                : launch_dt<64, FUSED, !FUSED>(p, dtype, grid, s);
    default:
      return hipErrorInvalidValue;
  }
}

// The occupancy of the heaviest of the fused variants.
template <int BM, int DT>
hipError_t occ_t(int* per_cu) {
  const void* ks[4] = {reinterpret_cast<const void*>(&agmm_persistent<BM, DT, true, true, false>),
                       reinterpret_cast<const void*>(&agmm_persistent<BM, DT, true, false, false>),
                       reinterpret_cast<const void*>(&agmm_persistent<BM, DT, true, true, true>),
                       reinterpret_cast<const void*>(&agmm_persistent<BM, DT, true, false, true>)};
  int lo = 1 << 30;
  for (const void* k : ks) {
    int n = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k, kThreads, 0);
    if (e != hipSuccess) return e;
    lo = n < lo ? n : lo;
  }
  *per_cu = lo;
  return hipSuccess;
}

// out[m][n] = RNE(C[m][n] + bias[n]): four consecutive outputs per thread and step.
template <int DT>
__global__ __launch_bounds__(256) void ar_finalize(const float* C, const uint16_t* bias,
                                                   uint16_t* out, int64_t M, int64_t N) {
  const int64_t groups = M * N / 4;
  for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < groups;
       q += (int64_t)gridDim.x * 256) {
    const int64_t e = q * 4, n = e % N;
    const f32x4 v = *reinterpret_cast<const f32x4*>(C + e);
    float x[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (bias) x[j] += Num<DT>::from_bits(bias[n + j]);
      o[j] = Num<DT>::to_bits(x[j]);
    }
    *reinterpret_cast<u32x2*>(out + e) = u32x2{o[0] | (o[1] << 16), o[2] | (o[3] << 16)};
  }
}

}  // namespace

hipError_t launch_gemm_ar(const KParams& p, int dtype, int block_m, int grid, hipStream_t s) {
  const bool bf = dtype == AGMM_BF16;
  switch (block_m) {
#define AGMM_AR_CASE(B)                                                                          \
  case B:                                                                                        \
    if (bf)                                                                                      \
      hipLaunchKernelGGL((agmm_persistent<B, AGMM_BF16, false, true, false, 1>), dim3(grid),     \
                         dim3(kThreads), 0, s, p);                                               \
    else                                                                                         \
      hipLaunchKernelGGL((agmm_persistent<B, AGMM_F16, false, true, false, 1>), dim3(grid),      \
                         dim3(kThreads), 0, s, p);                                               \
    break;
    AGMM_AR_CASE(256)
    AGMM_AR_CASE(128)
    AGMM_AR_CASE(64)
#undef AGMM_AR_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_ar_flags(const KParams& p, int dtype, int block_m, int grid, hipStream_t s) {
  const bool bf = dtype == AGMM_BF16;
  switch (block_m) {
#define AGMM_ARF_CASE(B)                                                                    \
  case B:                                                                                   \
    if (bf)                                                                                 \
      hipLaunchKernelGGL((agmm_ar_flags<B, AGMM_BF16>), dim3(grid), dim3(kThreads), 0, s, p); \
    else                                                                                    \
      hipLaunchKernelGGL((agmm_ar_flags<B, AGMM_F16>), dim3(grid), dim3(kThreads), 0, s, p);  \
    break;
    AGMM_ARF_CASE(256)
    AGMM_ARF_CASE(128)
    AGMM_ARF_CASE(64)
#undef AGMM_ARF_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_ar_finalize(const float* C, const uint16_t* bias, uint16_t* out, int64_t M,
                              int64_t N, int dtype, hipStream_t s) {
  const int64_t groups = M * N / 4;
  if (groups <= 0) return hipSuccess;
  const int blocks = (int)min((int64_t)2048, (groups + 255) / 256);
  if (dtype == AGMM_BF16)
    hipLaunchKernelGGL(ar_finalize<AGMM_BF16>, dim3(blocks), dim3(256), 0, s, C, bias, out, M, N);
  else
    hipLaunchKernelGGL(ar_finalize<AGMM_F16>, dim3(blocks), dim3(256), 0, s, C, bias, out, M, N);
  return hipGetLastError();
}

hipError_t launch_fused(const KParams& p, int dtype, int block_m, int grid, hipStream_t s) {
  return launch_any<true>(p, dtype, block_m, grid, s);
}

hipError_t launch_gemm_only(const KParams& p, int dtype, int block_m, int grid, hipStream_t s) {
  return launch_any<false>(p, dtype, block_m, grid, s);
}

hipError_t launch_copy(const KParams& p, int block_m, int grid, hipStream_t s) {
  switch (block_m) {
    case 256: hipLaunchKernelGGL(agmm_copy<256>, dim3(grid), dim3(kThreads), 0, s, p); break;
    case 128: hipLaunchKernelGGL(agmm_copy<128>, dim3(grid), dim3(kThreads), 0, s, p); break;
    case 64: hipLaunchKernelGGL(agmm_copy<64>, dim3(grid), dim3(kThreads), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_fetch(const KParams& p, int block_m, bool layout_k, int grid, hipStream_t s) {
  switch (block_m) {
    case 256:
      if (layout_k) hipLaunchKernelGGL(agmm_fetch_k<256>, dim3(grid), dim3(kThreads), 0, s, p);
      else hipLaunchKernelGGL(agmm_fetch_m<256>, dim3(grid), dim3(kThreads), 0, s, p);
      break;
    case 128:
      if (layout_k) hipLaunchKernelGGL(agmm_fetch_k<128>, dim3(grid), dim3(kThreads), 0, s, p);
      else hipLaunchKernelGGL(agmm_fetch_m<128>, dim3(grid), dim3(kThreads), 0, s, p);
      break;
    case 64:
      if (layout_k) hipLaunchKernelGGL(agmm_fetch_k<64>, dim3(grid), dim3(kThreads), 0, s, p);
      else hipLaunchKernelGGL(agmm_fetch_m<64>, dim3(grid), dim3(kThreads), 0, s, p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

namespace {
// Registers per lane a wave is given (the allocation granule is 8) and static LDS bytes.
hipError_t footprint(const void* k, int* regs, int* lds) {
  hipFuncAttributes a;
  const hipError_t e = hipFuncGetAttributes(&a, k);
  if (e != hipSuccess) return e;
  *regs = (a.numRegs + 7) & ~7;
  *lds = (int)a.sharedSizeBytes;
  return hipSuccess;
}

// (the grid beside a fetch kernel waits for each k-group in its K loop: ROW = false)
template <int BM, int DT, bool LK>
hipError_t fits_t(bool* fits) {
  int fr = 0, fl = 0, r = 0, l = 0;
  const void* fk = LK ? reinterpret_cast<const void*>(&agmm_fetch_k<BM>)
                      : reinterpret_cast<const void*>(&agmm_fetch_m<BM>);
  hipError_t e = footprint(fk, &fr, &fl);
  if (e != hipSuccess) return e;
  e = footprint(reinterpret_cast<const void*>(&agmm_persistent<BM, DT, true, LK, false>), &r, &l);
  if (e != hipSuccess) return e;
  // a SIMD holds 512 registers per lane; a CU 160 KiB of LDS
  *fits = r + fr <= 512 && l + fl <= 160 * 1024;
  return hipSuccess;
}

template <int BM>
hipError_t fits_dt(int dtype, bool layout_k, bool* fits) {
  if (dtype == AGMM_BF16)
    return layout_k ? fits_t<BM, AGMM_BF16, true>(fits) : fits_t<BM, AGMM_BF16, false>(fits);
  return layout_k ? fits_t<BM, AGMM_F16, true>(fits) : fits_t<BM, AGMM_F16, false>(fits);
}
}  // namespace

hipError_t fetch_fits_beside(int dtype, int block_m, bool layout_k, bool* fits) {
  switch (block_m) {
    case 256: return fits_dt<256>(dtype, layout_k, fits);
    case 128: return fits_dt<128>(dtype, layout_k, fits);
    case 64: return fits_dt<64>(dtype, layout_k, fits);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_upload32(uint32_t* dst, const uint32_t* src, int64_t n, hipStream_t s) {
  for (int64_t o = 0; o < n; o += kUploadWords) {
    UploadWords p;
    p.n = (uint32_t)(n - o < kUploadWords ? n - o : kUploadWords);
    for (uint32_t i = 0; i < kUploadWords; ++i) p.w[i] = i < p.n ? src[o + i] : 0u;
    hipLaunchKernelGGL(upload32_kernel, dim3(1), dim3(kUploadWords), 0, s, dst + o, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_mfma_loop(int dtype, bool vary, int grid, int iters, float* sink,
                            hipStream_t s) {
  if (grid <= 0 || iters <= 0 || (iters & 3)) return hipErrorInvalidValue;
  if (dtype == AGMM_BF16) {
    if (vary) hipLaunchKernelGGL((mfma_loop_kernel<AGMM_BF16, true>), dim3(grid), dim3(256), 0, s, sink, iters);
    else hipLaunchKernelGGL((mfma_loop_kernel<AGMM_BF16, false>), dim3(grid), dim3(256), 0, s, sink, iters);
  } else {
    if (vary) hipLaunchKernelGGL((mfma_loop_kernel<AGMM_F16, true>), dim3(grid), dim3(256), 0, s, sink, iters);
    else hipLaunchKernelGGL((mfma_loop_kernel<AGMM_F16, false>), dim3(grid), dim3(256), 0, s, sink, iters);
  }
  return hipGetLastError();
}

hipError_t launch_fill16(uint16_t* dst, int64_t n, uint16_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = min((int64_t)1024, (n + 255) / 256);
  hipLaunchKernelGGL(fill16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, dst, n, v);
  return hipGetLastError();
}

hipError_t launch_fill32(uint32_t* dst, int64_t n, uint32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = min((int64_t)1024, (n + 255) / 256);
  hipLaunchKernelGGL(fill32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, dst, n, v);
  return hipGetLastError();
}

hipError_t fused_occupancy(int dtype, int block_m, int* per_cu) {
  const bool bf = dtype == AGMM_BF16;
  switch (block_m) {
    case 256: return bf ? occ_t<256, AGMM_BF16>(per_cu) : occ_t<256, AGMM_F16>(per_cu);
    case 128: return bf ? occ_t<128, AGMM_BF16>(per_cu) : occ_t<128, AGMM_F16>(per_cu);
    case 64: return bf ? occ_t<64, AGMM_BF16>(per_cu) : occ_t<64, AGMM_F16>(per_cu);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace agmm
