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
// GEMM worker: square output tiles BMxBM with BK = 16384/BM (256x256x64, 128x128x128,
// 64x64x256), 4 wave64s in a 2x2 layout, v_mfma_f32_32x32x16_{f16,bf16} with fp32
// accumulators, two LDS stages of 64 KiB (global loads for K-tile k+1 are in flight while
// K-tile k is multiplied). LDS holds each operand as 16-byte chunks of 8 consecutive K
// values ([K/8][MN] chunks, XOR-swizzled), the form the MFMA operands are read in; a
// K-contiguous source is copied chunk for chunk, an MN-contiguous source (B, and A staged
// m_contiguous) is transposed 8x8 in registers on its way into LDS.
//
// Flag protocol: producer = every thread's agent-scope release fence (L2 write-back),
// workgroup barrier, one agent-scope release store of the run's epoch. Consumer = relaxed
// agent-scope polls with s_sleep backoff (the busy-wait back-off suggested in ROCm/iris PR
// "Let's make Iris' All-reduce the best!"), then one agent-scope acquire fence. Every
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

// Tile family: square BMxBM output tile, BK = 16384/BM so that each operand's stage holds
// 2048 16-byte chunks: 8 K-major chunks or one 8x8 MN-major block per thread.
//
// LDS layout of an operand stage: chunk (row r, K-chunk kc) -- 8 consecutive K values of
// row r -- sits at kc * RS + phys(r), with the chunk-row stride RS = MN + 8 (8 chunks of
// padding) and phys(r) = r ^ ((r>>3 ^ r>>6) & 7). The padding makes the K-chunk term
// additive (each MFMA sub-step reads at a fixed offset from one base per lane); the XOR
// spreads 8x8 transposed blocks. Checked exhaustively: MFMA operand reads, K-major stores
// (8 rows x 8 K-chunks per wave instruction) and MN-major stores (16 blocks) hit distinct
// 16-byte bank groups whether a 128-bit LDS access is served 8 or 16 lanes at a time.
template <int BM_>
struct Tile {
  static constexpr int BM = BM_, BN = BM_, BK = 16384 / BM_;
  static constexpr int KC = BK / 8;            // 16-byte K-chunks per row
  static constexpr int RSA = BM + 8, RSB = BN + 8;
  static constexpr int A_CH = KC * RSA;        // chunks per stage, A
  static constexpr int B_CH = KC * RSB;        // chunks per stage, B
  static constexpr int STAGE = A_CH + B_CH;
  static constexpr int WTM = BM / 2, WTN = BN / 2;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static_assert(2 * STAGE * 16 >= BM * BN * 2, "epilogue tile fits in the stages");
};

__device__ inline int phys(int r) { return r ^ (((r >> 3) ^ (r >> 6)) & 7); }

__device__ inline u32x4 ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

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
__device__ inline void st16(uint16_t* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Buffer resource over [base, base + bytes): loads at byte offsets at or past `bytes`
// return zero, so a tile that runs past the end of its operand reads zeros without a
// branch per load. The word 0x00020000 is the gfx9-family raw-buffer configuration.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ inline rsrc_t make_rsrc(const uint16_t* base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0xffffffffll ? 0xffffffffll : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), (short)0,
                                           (int)(uint32_t)n, 0x00020000);
}
__device__ inline u32x4 bload(rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}

// K-contiguous operand tile (MN rows x BK), element (r, k) at base[r*ld + k]. Chunk
// c = i*256 + tid is row (c / (8*KC))*8 + c % 8, K-chunk (c / 8) % KC: a wave instruction
// covers 8 rows x 8 K-chunks (whole 128-byte row segments). A thread's K-chunk is the same
// for every i and its row advances by 256/KC per i, so its byte offset is off0 + i*rstride.
template <class T, int MN>
struct KMajor {
  static constexpr int PER = MN * T::KC / kThreads;
  static constexpr int RPI = kThreads / T::KC;  // rows per i
  typedef u32x4 Regs[PER];
  uint32_t off0, rstride;
  __device__ static inline int row0(int tid) { return (tid / (8 * T::KC)) * 8 + tid % 8; }
  __device__ static inline int kchunk(int tid) { return (tid / 8) % T::KC; }
  __device__ inline void init(int64_t ld, int tid) {
    off0 = (uint32_t)((row0(tid) * ld + kchunk(tid) * 8) * 2);
    rstride = (uint32_t)(RPI * ld * 2);
  }
  // rs covers the operand from column k0 onwards; k_rem = K - k0. Columns at or past K
  // would read the next row, so the last K-tile of a ragged K is masked explicitly.
  __device__ inline void load(rsrc_t rs, int64_t k_rem, int tid, Regs& v) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) v[i] = bload(rs, off0 + i * rstride);
    if (k_rem < T::BK && kchunk(tid) * 8 >= k_rem) {
#pragma unroll
      for (int i = 0; i < PER; ++i) v[i] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ inline void store(u32x4* region, int tid, const Regs& v) const {
    constexpr int RS = MN + 8;
    u32x4* base = region + kchunk(tid) * RS;
    const int r0 = row0(tid);
#pragma unroll
    for (int i = 0; i < PER; ++i) base[phys(r0 + i * RPI)] = v[i];
  }
};

// MN-contiguous operand tile (BK x MN), element (r, k) at base[k*ld + r]. Each thread moves
// one 8x8 block: 8 rows of 8 MN-consecutive values in, 8 chunks of 8 K-consecutive out.
// Rows at or past K lie past the operand's end (zeros); columns past the last valid one
// read neighbouring data that only reaches output columns that are never stored.
template <class T, int MN>
struct MNMajor {
  static constexpr int NBM = MN / 8;
  static_assert(NBM * T::KC == kThreads, "one 8x8 block per thread");
  typedef u32x4 Regs[8];
  uint32_t off0, ld2;
  __device__ inline void init(int64_t ld, int tid) {
    const int nb = tid % NBM, kb = tid / NBM;
    ld2 = (uint32_t)(ld * 2);
    off0 = (uint32_t)((kb * 8 * ld + nb * 8) * 2);
  }
  __device__ inline void load(rsrc_t rs, int64_t /*k_rem*/, int /*tid*/, Regs& v) const {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = bload(rs, off0 + j * ld2);
  }
  __device__ inline void store(u32x4* region, int tid, const Regs& v) const {
    constexpr int RS = MN + 8;
    const int nb = tid % NBM, kb = tid / NBM;
    u32x4* base = region + kb * RS;
#pragma unroll
    for (int i = 0; i < 8; ++i) base[phys(nb * 8 + i)] = transpose_row(v, i);
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

// Waits (every lane of the calling wave) until flags[idx] == epoch, then acquires.
__device__ inline void wait_flag(const KParams& p, int64_t idx, Tracer& tr) {
  uint32_t* f = p.flags + idx;
  const uint64_t t0 = tr.now();
  uint32_t polls = 0;
  uint32_t v = __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  int backoff = 1;
  while (v != p.epoch) {
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
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  tr.rec(AGMM_EV_GEMM_WAIT, (uint32_t)idx, v, polls, t0);
}

// MFMA operand fragments of sub-step kk (16 K values): lane l holds row (l % 32) of each
// 32-row block, K values 8*(l / 32) .. +7.
template <class T>
__device__ inline void read_frags(const u32x4* As, const u32x4* Bs, int kk, u32x4 (&a)[T::FM],
                                  u32x4 (&b)[T::FN], int lane, int wm, int wn) {
  // lane-dependent part (K-chunk parity and row), then the sub-step as a constant offset
  const u32x4* pa = As + (lane >> 5) * T::RSA + 2 * kk * T::RSA;
  const u32x4* pb = Bs + (lane >> 5) * T::RSB + 2 * kk * T::RSB;
#pragma unroll
  for (int fm = 0; fm < T::FM; ++fm) a[fm] = pa[phys(wm * T::WTM + fm * 32 + (lane & 31))];
#pragma unroll
  for (int fn = 0; fn < T::FN; ++fn) b[fn] = pb[phys(wn * T::WTN + fn * 32 + (lane & 31))];
}

// B is the MFMA's first operand, so each lane ends up holding 4 consecutive columns of one
// output row (8-byte stores in the epilogue).
template <class T, int DT>
__device__ inline void mfmas(f32x16 (&acc)[T::FM][T::FN], const u32x4 (&a)[T::FM],
                             const u32x4 (&b)[T::FN]) {
#pragma unroll
  for (int fm = 0; fm < T::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < T::FN; ++fn) acc[fm][fn] = Num<DT>::mfma(b[fn], a[fm], acc[fm][fn]);
}

// One output tile. A_KMAJOR: the A source is K-contiguous (local shard or k_contiguous
// staging); otherwise it is the m_contiguous staging buffer. WAIT: fused mode, staged
// k-groups are waited for before their first K-tile is loaded.
//
// Pipeline (K-tile t): at the top of step t the global loads of K-tile t+1 are issued into
// registers; K-tile t is multiplied out of LDS stage t & 1 with the fragments of sub-step
// kk+1 read while sub-step kk's MFMAs run; during the last sub-step the registers are
// written (transposed where needed) into the other stage. One barrier per K-tile.
template <class T, int DT, bool A_KMAJOR, bool WAIT>
__device__ void gemm_tile(const KParams& p, int t_m, int t_n, bool staged, u32x4* lds,
                          u32x2* bias_lds, int tid, Tracer& tr) {
  constexpr int BM = T::BM, BN = T::BN, BK = T::BK, NKK = BK / 16;
  const int lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)t_m * BM, n0 = (int64_t)t_n * BN;
  const int rows_valid = (int)min((int64_t)BM, p.M - m0);
  const int cols_valid = (int)min((int64_t)BN, p.N - n0);
  // A source, chosen once per tile: base pointer, row stride, and the bytes from base to
  // the end of the buffer it lies in (the buffer-resource range).
  const uint16_t* abase;
  int64_t lda, a_bytes;
  if (!staged) {
    abase = p.shards[p.rank] + (m0 - (int64_t)p.rank * p.M_s) * p.K;
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
  const uint16_t* bbase = p.B + n0;
  const int64_t b_bytes = (p.K * p.N - n0) * 2;
  const int64_t b_step = (int64_t)BK * p.N;

  f32x16 acc[T::FM][T::FN];
#pragma unroll
  for (int fm = 0; fm < T::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < T::FN; ++fn) acc[fm][fn] = (f32x16)(0.0f);

  using ALoad = typename std::conditional<A_KMAJOR, KMajor<T, BM>, MNMajor<T, BM>>::type;
  using BLoad = MNMajor<T, BN>;
  ALoad al;
  BLoad bl;
  al.init(lda, tid);
  bl.init(p.N, tid);
  typename ALoad::Regs ga;
  typename BLoad::Regs gb;
  u32x4 fa[2][T::FM], fb[2][T::FN];

  const int KT = (int)((p.K + BK - 1) / BK);
  const int64_t fbase = (int64_t)t_m * p.G;
  const bool waits = WAIT && staged;

  // This tile's bias slice to LDS (read after the K loop's barriers).
  if (p.bias && tid < BN / 4)
    bias_lds[tid] = (n0 + tid * 4 < p.N) ? *reinterpret_cast<const u32x2*>(p.bias + n0 + tid * 4)
                                         : u32x2{0u, 0u};

  // Issue the global loads of K-tile t, after its k-group's flag.
  auto issue = [&](int t) {
    if (waits && t % p.kpf == 0) wait_flag(p, fbase + t / p.kpf, tr);
    const int64_t ka = t * a_step, kb = t * b_step;
    al.load(make_rsrc(abase + ka, a_bytes - ka * 2), p.K - (int64_t)t * BK, tid, ga);
    bl.load(make_rsrc(bbase + kb, b_bytes - kb * 2), 0, tid, gb);
  };

  if (KT > 0) {
    issue(0);
    al.store(lds, tid, ga);
    bl.store(lds + T::A_CH, tid, gb);
    __syncthreads();
    read_frags<T>(lds, lds + T::A_CH, 0, fa[0], fb[0], lane, wm, wn);
    for (int kt = 0; kt < KT; ++kt) {
      const int cur = kt & 1;
      const u32x4* As = lds + cur * T::STAGE;
      const u32x4* Bs = As + T::A_CH;
      u32x4* An = lds + (cur ^ 1) * T::STAGE;
      u32x4* Bn = An + T::A_CH;
      const bool has1 = kt + 1 < KT;
      if (has1) issue(kt + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        if (kk + 1 < NKK)
          read_frags<T>(As, Bs, kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1], lane, wm, wn);
        if (kk == NKK - 1 && has1) {
          al.store(An, tid, ga);
          bl.store(Bn, tid, gb);
        }
        mfmas<T, DT>(acc, fa[kk & 1], fb[kk & 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
      __syncthreads();
      if (has1) read_frags<T>(An, Bn, 0, fa[0], fb[0], lane, wm, wn);
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // Epilogue through LDS (the operand stages are free after the last barrier): each lane
  // adds the bias in fp32, rounds once (RNE) and writes 4 consecutive outputs (8 bytes) of
  // one row into a [BM][BN] 16-bit tile; then every thread copies 16-byte row chunks to
  // global memory, a wave's lanes covering whole rows. 8-byte unit u of row r sits at unit
  // u ^ (r & XM), so the 32 rows written by one instruction and the chunks of a row read
  // back spread over the banks (XM keeps the unit inside its row for narrow tiles).
  __syncthreads();  // the bias slice is visible even when the K loop ran no barrier (K == 0)
  uint32_t* otile = reinterpret_cast<uint32_t*>(lds);
  constexpr int ROW_U = BN / 4;  // 8-byte units per tile row
  constexpr int XM = (ROW_U < 32 ? ROW_U : 32) - 1;
#pragma unroll
  for (int fm = 0; fm < T::FM; ++fm) {
    const int ml = wm * T::WTM + fm * 32 + (lane & 31);
#pragma unroll
    for (int fn = 0; fn < T::FN; ++fn) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int nl = wn * T::WTN + fn * 32 + g * 8 + (lane >> 5) * 4;
        float x0 = acc[fm][fn][4 * g + 0], x1 = acc[fm][fn][4 * g + 1];
        float x2 = acc[fm][fn][4 * g + 2], x3 = acc[fm][fn][4 * g + 3];
        if (p.bias) {
          const u32x2 bb = bias_lds[nl >> 2];
          x0 += Num<DT>::from_bits(bb[0] & 0xffffu);
          x1 += Num<DT>::from_bits(bb[0] >> 16);
          x2 += Num<DT>::from_bits(bb[1] & 0xffffu);
          x3 += Num<DT>::from_bits(bb[1] >> 16);
        }
        u32x2 o;
        o[0] = Num<DT>::to_bits(x0) | (Num<DT>::to_bits(x1) << 16);
        o[1] = Num<DT>::to_bits(x2) | (Num<DT>::to_bits(x3) << 16);
        const int u = (nl >> 2) ^ (ml & XM);
        *reinterpret_cast<u32x2*>(otile + (ml * ROW_U + u) * 2) = o;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __syncthreads();
  constexpr int ROW_C = BN / 8;  // 16-byte chunks per row
#pragma unroll 4
  for (int c = tid; c < BM * ROW_C; c += kThreads) {
    const int r = c / ROW_C, ch = c % ROW_C;
    const int s = r & XM;
    u32x4 v = *reinterpret_cast<const u32x4*>(otile + (r * ROW_U + (((2 * ch) ^ s) & ~1)) * 2);
    if (s & 1) v = u32x4{v[2], v[3], v[0], v[1]};
    if (r < rows_valid && ch * 8 < cols_valid)
      *reinterpret_cast<u32x4*>(p.out + (m0 + r) * p.N + n0 + ch * 8) = v;
  }
  __syncthreads();  // the tile area is the next tile's stage 0
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

// Copy unit (t_m, g) into k_contiguous staging: 16-byte loads and stores, 8 in flight.
template <int BM>
__device__ void copy_unit_kmajor(const KParams& p, const uint16_t* const* shards, int t_m, int g,
                                 int KG, int tid) {
  const int64_t m_beg = (int64_t)t_m * BM;
  const int R = (int)min((int64_t)BM, p.M - m_beg);
  const int64_t k_beg = (int64_t)g * KG;
  const int CR = (int)(min((int64_t)KG, p.K - k_beg) / 8);
  const int total = R * CR;
  for (int base = 0; base < total; base += kThreads * 8) {
    u32x4 v[8];
    int64_t dst[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = base + i * kThreads + tid;
      if (c < total) {
        const int r = c / CR, cc = c - r * CR;
        const int64_t m = m_beg + r;
        v[i] = ld16(arow(p, shards, m) + k_beg + cc * 8);
        dst[i] = m * p.K + k_beg + cc * 8;
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = base + i * kThreads + tid;
      if (c < total) st16(p.staging + dst[i], v[i]);
    }
  }
}

// Copy unit (t_m, g) into m_contiguous staging: each thread transposes 8x8 blocks. Lanes
// are ordered so that 8 lanes read 128 contiguous bytes of one row and 8 lanes write 128
// contiguous bytes of one staging row.
template <int BM>
__device__ void copy_unit_mmajor(const KParams& p, const uint16_t* const* shards, int t_m, int g,
                                 int KG, int tid) {
  const int64_t m_beg = (int64_t)t_m * BM;
  const int R = (int)min((int64_t)BM, p.M - m_beg);       // multiple of 8
  const int64_t k_beg = (int64_t)g * KG;
  const int NBK = (int)(min((int64_t)KG, p.K - k_beg) / 8);
  const int NBM = R / 8;
  const int total = ((NBK + 7) & ~7) * NBM;
  for (int b = tid; b < total; b += kThreads) {
    const int kb = (b / (8 * NBM)) * 8 + (b & 7);
    const int mb = (b >> 3) % NBM;
    if (kb >= NBK) continue;
    u32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = ld16(arow(p, shards, m_beg + mb * 8 + j) + k_beg + kb * 8);
    uint16_t* dst = p.staging + (k_beg + kb * 8) * p.M + m_beg + mb * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) st16(dst + (int64_t)i * p.M, transpose_row(v, i));
  }
}

// Units f, f+F, f+2F, ... of the fetch order. publish: fused mode, set each unit's flag.
template <class T>
__device__ void fetch_loop(const KParams& p, const uint16_t* const* shards, int f, int F,
                           bool publish, Tracer& tr, int tid) {
  const int KG = p.kpf * T::BK;
  for (int u = f; u < p.num_units; u += F) {
    const int t_m = (int)p.units[2 * u], g = (int)p.units[2 * u + 1];
    const uint64_t t0 = tr.now();
    if (p.staged_kmajor)
      copy_unit_kmajor<T::BM>(p, shards, t_m, g, KG, tid);
    else
      copy_unit_mmajor<T::BM>(p, shards, t_m, g, KG, tid);
    if (publish) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      __syncthreads();
      if (tid == 0 && u != p.skip_unit)
        __hip_atomic_store(p.flags + (int64_t)t_m * p.G + g, p.epoch, __ATOMIC_RELEASE,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    tr.rec(AGMM_EV_FETCH, (uint32_t)u, (uint32_t)t_m, (uint32_t)g, t0);
  }
}

// Next tile for this workgroup, or -1: its XCD's queue first, then the other queues.
__device__ inline int grab(const KParams& p) {
  if (aborted(p)) return -1;
  const int x0 = (int)(blockIdx.x % kQueues);
  for (int s = 0; s < kQueues; ++s) {
    const int x = (x0 + s) % kQueues;
    uint32_t* c = p.ctr + CTR_Q + x * CTR_QSTRIDE;
    const uint32_t len = (uint32_t)p.qlen[x];
    if (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= len) continue;
    const uint32_t i = atomicAdd(c, 1u);
    if (i < len) return (int)p.qtiles[p.qoff[x] + (int)i];
  }
  return -1;
}

template <int BM, int DT, bool FUSED>
__global__ __launch_bounds__(kThreads) void agmm_persistent(KParams p) {
  using T = Tile<BM>;
  __shared__ u32x4 lds[2 * T::STAGE];
  __shared__ u32x2 s_bias[T::BN / 4];
  __shared__ int s_next;
  __shared__ const uint16_t* s_shards[AGMM_MAX_SHARDS];
  const int tid = threadIdx.x, wg = blockIdx.x;
  Tracer tr{p.debug ? p.trace + (size_t)wg * p.trace_cap : nullptr, 0u, (uint32_t)p.trace_cap,
            p.debug != 0};

  if (FUSED && wg < p.F) {
    load_shard_table(p, s_shards, tid);
    fetch_loop<T>(p, s_shards, wg, p.F, true, tr, tid);
  }

  int nxt = -1;
  if (tid == 0) s_next = grab(p);
  __syncthreads();
  int q = s_next;
  while (q >= 0) {
    __syncthreads();  // everyone has read s_next
    if (tid == 0) nxt = grab(p);  // next tile's index travels while this one computes
    const int pos = q / p.T_n, t_n = q - pos * p.T_n;
    const uint32_t e = p.mtiles[pos];
    const int t_m = (int)(e & 0x7fffffffu);
    const bool staged = (e >> 31) == 0u;
    const uint64_t t0 = tr.now();
    if constexpr (!FUSED) {
      gemm_tile<T, DT, true, false>(p, t_m, t_n, staged, lds, s_bias, tid, tr);
    } else {
      if (!staged || p.staged_kmajor)
        gemm_tile<T, DT, true, true>(p, t_m, t_n, staged, lds, s_bias, tid, tr);
      else
        gemm_tile<T, DT, false, true>(p, t_m, t_n, staged, lds, s_bias, tid, tr);
    }
    tr.rec(AGMM_EV_GEMM, (uint32_t)q, (uint32_t)t_m, (uint32_t)t_n, t0);
    if (tid == 0) s_next = nxt;
    __syncthreads();
    q = s_next;
  }

  if (tid == 0) {
    if (p.debug) p.trace_count[wg] = tr.n;
    const uint32_t old = atomicAdd(p.ctr + CTR_DONE, 1u);
    if (old == gridDim.x - 1) {  // last workgroup out resets the queues for the next run
      for (int x = 0; x < kQueues; ++x)
        __hip_atomic_store(p.ctr + CTR_Q + x * CTR_QSTRIDE, 0u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(p.ctr + CTR_DONE, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Baseline copy: every staged unit into k_contiguous staging, no flags.
template <int BM>
__global__ __launch_bounds__(kThreads) void agmm_copy(KParams p) {
  __shared__ const uint16_t* s_shards[AGMM_MAX_SHARDS];
  Tracer tr{nullptr, 0u, 0u, false};
  load_shard_table(p, s_shards, threadIdx.x);
  fetch_loop<Tile<BM>>(p, s_shards, blockIdx.x, gridDim.x, false, tr, threadIdx.x);
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

template <int BM, int DT, bool FUSED>
hipError_t launch_t(const KParams& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL((agmm_persistent<BM, DT, FUSED>), dim3(grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

template <bool FUSED>
hipError_t launch_any(const KParams& p, int dtype, int block_m, int grid, hipStream_t s) {
  const bool bf = dtype == AGMM_BF16;
  switch (block_m) {
    case 256:
      return bf ? launch_t<256, AGMM_BF16, FUSED>(p, grid, s) : launch_t<256, AGMM_F16, FUSED>(p, grid, s);
    case 128:
      return bf ? launch_t<128, AGMM_BF16, FUSED>(p, grid, s) : launch_t<128, AGMM_F16, FUSED>(p, grid, s);
    case 64:
      return bf ? launch_t<64, AGMM_BF16, FUSED>(p, grid, s) : launch_t<64, AGMM_F16, FUSED>(p, grid, s);
    default:
      return hipErrorInvalidValue;
  }
}

template <int BM, int DT>
hipError_t occ_t(int* per_cu) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(
      per_cu, reinterpret_cast<const void*>(&agmm_persistent<BM, DT, true>), kThreads, 0);
}

}  // namespace

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
