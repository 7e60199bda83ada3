// Host side of the C ABI declared in include/agmm.h: validation, tile-configuration
// choice, schedule tables, workspace, launch.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <vector>

#include "agmm_internal.h"

using agmm::KParams;

// One chunk of the host stream pipeline: its slices of the chunk tables (units in 2-word
// records, m-tiles, queue entries) and its queue offsets / lengths inside its entries.
struct PipeChunk {
  int32_t u_off, u_len, m_off, m_len, q_off, q_len;
  int32_t qoff[agmm::kQueueSlots], qlen[agmm::kQueueSlots];
};
// The nvFuser host program's stream rotation: chunk i runs on stream i % streams, stream 0
// being the caller's own; the other streams are the handle's.
constexpr int kPipeStreams = 4;

struct agmm_handle {
  agmm_desc desc;
  agmm_config cfg;
  int64_t M_s;
  char* ws;                 // one device allocation (or the caller's workspace), carved below
  bool own_ws;              // ws was allocated by create (freed by destroy)
  uint32_t* host_status;    // pinned host mirror of the status words {status, wg, flag, seen}
  uint16_t* staging;
  uint32_t* flags;
  uint32_t* ctr;
  uint32_t* units;
  uint32_t* mtiles;
  agmm_trace_rec* trace;
  uint32_t* trace_count;
  int64_t flags_n;
  int64_t split_base;
  int64_t trace_wgs;        // workgroups the trace buffer has room for
  uint32_t* qtiles;
  uint32_t* split_cnt;
  float* partials;
  std::vector<uint32_t> h_units, h_mtiles, h_qtiles;
  int32_t qoff[agmm::kQueueSlots], qlen[agmm::kQueueSlots];
  bool poisoned;
  // AGMM_ALGO_PIPELINED
  std::vector<PipeChunk> chunks;
  uint32_t *c_units, *c_mtiles, *c_qtiles, *c_ctr;
  hipStream_t pstreams[kPipeStreams - 1];  // streams 1 .. of the rotation
  hipEvent_t ev_start, ev_done[kPipeStreams - 1];
  int n_pstreams, n_events;  // created so far (destroy releases these)
  // fetch kernel (cfg.fetch_kernel): its stream, and the events that order it after the work
  // before a run on the caller's stream (ev_fin) and that stream after it (ev_fout)
  hipStream_t fstream;
  hipEvent_t ev_fin, ev_fout;
  bool has_fstream, has_fev;
  // GEMM + all-reduce handles (ag_gemm_ar_create): ranks and this rank; 0 otherwise
  int32_t ar_D, ar_rank;
  // ag_gemm_ar_flags_create: every rank's share in one launch. A second device allocation
  // holds the partial tiles [D][M][N] fp32, the flags [D][tiles] and the item list.
  bool ar_flags_mode;
  char* ar_ws;
  float* ar_partials;
  uint32_t* ar_flags;
  uint32_t* ar_items;
  int64_t ar_flags_n, ar_items_n;
};

namespace {

thread_local int g_last_hip = 0;

// Byte offsets inside a tile are 32-bit and a buffer resource spans at most 2^31 - 1 bytes:
// 256 rows of an N- or K-element stride (output rows, K-major operand rows) must stay below
// 2^31 bytes, so N and K stay below 2^22; M only strides the m_contiguous staging, 32 rows
// of it per K-tile, so M may reach 2^23.
constexpr int64_t kMaxDim = (int64_t)1 << 23;
constexpr int64_t kMaxDimNK = (int64_t)1 << 22;
constexpr int64_t kMaxCount = (int64_t)1 << 31;
constexpr uint32_t kDefaultSpinLimit = 1u << 22;  // ~ several seconds of backed-off polls
constexpr int kDefaultTraceCap = 512;
constexpr uint16_t kNanF16 = 0x7E00, kNanBF16 = 0x7FC0;  // quiet NaNs: debug staging poison
constexpr int kTraceWgsAuto = 2048;
constexpr int kDefaultFetchWgs = 32;  // the iris issue's tuned num_fetch_sms default
constexpr int kDefaultChunks = 4;     // AGMM_ALGO_PIPELINED: chunks per shard
constexpr int kMaxChunks = 64;

#define AGMM_HIP(x)                      \
  do {                                   \
    hipError_t e_ = (x);                 \
    if (e_ != hipSuccess) {              \
      g_last_hip = (int)e_;              \
      return AGMM_ERR_HIP;               \
    }                                    \
  } while (0)

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t align256(int64_t x) { return (x + 255) & ~(int64_t)255; }

int validate_desc(const agmm_desc* d) {
  if (!d) return AGMM_ERR_INVALID_ARG;
  if (d->D < 1 || d->D > AGMM_MAX_SHARDS) return AGMM_ERR_INVALID_ARG;
  if (d->rank < 0 || d->rank >= d->D) return AGMM_ERR_INVALID_ARG;
  if (d->M < 0 || d->N < 0 || d->K < 0) return AGMM_ERR_INVALID_ARG;
  if (d->M >= kMaxDim || d->N >= kMaxDimNK || d->K >= kMaxDimNK) return AGMM_ERR_UNSUPPORTED;
  if (d->M % d->D != 0) return AGMM_ERR_INVALID_ARG;
  if (d->dtype != AGMM_F16 && d->dtype != AGMM_BF16) return AGMM_ERR_INVALID_ARG;
  if (d->layout != AGMM_K_CONTIGUOUS && d->layout != AGMM_M_CONTIGUOUS) return AGMM_ERR_INVALID_ARG;
  if (d->algo != AGMM_ALGO_FUSED && d->algo != AGMM_ALGO_BASELINE && d->algo != AGMM_ALGO_PIPELINED)
    return AGMM_ERR_INVALID_ARG;
  if (d->pipeline_chunks < 0 || d->pipeline_chunks > kMaxChunks) return AGMM_ERR_INVALID_ARG;
  if ((d->direct_local | d->has_bias | d->debug) & ~1) return AGMM_ERR_INVALID_ARG;
  if (d->block_m != 0 && d->block_m != 64 && d->block_m != 128 && d->block_m != 256)
    return AGMM_ERR_INVALID_ARG;
  if (d->k_per_flag < 0 || d->num_fetch_wgs < 0 || d->num_wgs < 0 || d->trace_cap < 0)
    return AGMM_ERR_INVALID_ARG;
  if (d->debug_skip_unit < -1) return AGMM_ERR_INVALID_ARG;
  if (d->tail_split != 0 && d->tail_split != 1) return AGMM_ERR_INVALID_ARG;
  if (d->gather_a != 0 && d->gather_a != 1) return AGMM_ERR_INVALID_ARG;
  if (d->debug_fetch_delay < 0 || (d->debug_fetch_reverse & ~1)) return AGMM_ERR_INVALID_ARG;
  if (d->fetch_kernel < -1 || d->fetch_kernel > 1) return AGMM_ERR_INVALID_ARG;
  if (d->gather_a && d->layout != AGMM_K_CONTIGUOUS) return AGMM_ERR_UNSUPPORTED;
  if (d->N % 8 != 0 || d->K % 8 != 0) return AGMM_ERR_UNSUPPORTED;
  if (d->layout == AGMM_M_CONTIGUOUS && d->algo == AGMM_ALGO_FUSED && d->M % 8 != 0)
    return AGMM_ERR_UNSUPPORTED;
  return AGMM_OK;
}

bool is_direct(const agmm_desc& d, int64_t M_s, int bm, int64_t t) {
  if (!d.direct_local) return false;
  const int64_t lo = t * bm, hi = std::min(d.M, (t + 1) * bm);
  return (int64_t)d.rank * M_s <= lo && hi <= (int64_t)(d.rank + 1) * M_s;
}

// Everything create decides, computed on the host only.
struct Plan {
  agmm_config cfg;
  int64_t M_s;
  std::vector<uint32_t> units, mtiles, qtiles;
  int32_t qoff[agmm::kQueueSlots], qlen[agmm::kQueueSlots];
  int64_t flags_n, trace_wgs, split_base;
  int64_t off_staging, off_flags, off_ctr, off_split, off_units, off_mtiles, off_qtiles,
      off_partials, off_trace, off_tcount, total;
  // AGMM_ALGO_PIPELINED: chunk tables, and one counter block per chunk
  std::vector<PipeChunk> chunks;
  std::vector<uint32_t> c_units, c_mtiles, c_qtiles;
  int64_t off_c_ctr, off_c_units, off_c_mtiles, off_c_qtiles;
};

// Tile queues (one per XCD): GEMM-order m-tiles are taken in super-rows of kSuperRows; a
// super-row's tiles are listed in column blocks of kColBlock n-tiles (so the 32 CUs of an
// XCD share 4 A row-blocks and 8 B column-blocks in L2), and super-rows are dealt to the
// queues round-robin. Tile id q = (position of its m-tile in GEMM order) * T_n + n-tile.
constexpr int kSuperRows = 4;
constexpr int kColBlock = 8;

// Split tiles (tiles t_m * T_n + t_n >= split_base, when S >= 2) stay out of the XCD queues;
// their pieces, S per tile in tile order, form the tail queue.
void make_queues(int64_t T_m, int64_t T_n, const std::vector<uint32_t>& mtiles, int S,
                 Plan* pl) {
  std::vector<std::vector<uint32_t>> qs(agmm::kQueueSlots);
  std::vector<int64_t> pos_of(S >= 2 ? T_m : 0);  // split tiles only: m-tile -> position
  if (S >= 2)
    for (int64_t pos = 0; pos < T_m; ++pos) pos_of[mtiles[pos] & 0x7fffffffu] = pos;
  auto split = [&](int64_t pos, int64_t n) {
    return S >= 2 && (int64_t)(mtiles[pos] & 0x7fffffffu) * T_n + n >= pl->split_base;
  };
  for (int64_t s0 = 0, j = 0; s0 < T_m; s0 += kSuperRows, ++j) {
    const int64_t s1 = std::min(T_m, s0 + kSuperRows);
    auto& q = qs[j % agmm::kQueues];
    for (int64_t nb = 0; nb < T_n; nb += kColBlock)
      for (int64_t pos = s0; pos < s1; ++pos)
        for (int64_t n = nb; n < std::min(T_n, nb + kColBlock); ++n)
          if (!split(pos, n)) q.push_back((uint32_t)(pos * T_n + n));
  }
  if (S >= 2)
    for (int64_t c = pl->split_base; c < T_m * T_n; ++c) {
      const uint32_t q = (uint32_t)(pos_of[c / T_n] * T_n + c % T_n);
      for (int piece = 0; piece < S; ++piece)
        qs[agmm::kTailQueue].push_back(q | ((uint32_t)piece << 24) | ((uint32_t)(S - 1) << 28));
    }
  pl->qtiles.clear();
  for (int x = 0; x < agmm::kQueueSlots; ++x) {
    pl->qoff[x] = (int32_t)pl->qtiles.size();
    pl->qlen[x] = (int32_t)qs[x].size();
    pl->qtiles.insert(pl->qtiles.end(), qs[x].begin(), qs[x].end());
  }
}

int make_plan(const agmm_desc& d, int num_cus, Plan* pl) {
  agmm_config& c = pl->cfg;
  memset(&c, 0, sizeof(c));
  const int64_t M_s = d.M / d.D;
  pl->M_s = M_s;
  c.num_cus = num_cus;

  // Tile family: the largest square tile that still gives most CUs a tile.
  int bm = d.block_m;
  bool fused_128 = false;
  if (bm == 0) {
    bm = 64;
    for (int cand : {256, 128}) {
      if (cdiv(d.M, cand) * cdiv(d.N, cand) * 4 >= (int64_t)num_cus * 3) {
        bm = cand;
        break;
      }
    }
    // Fused, with 64-row tiles taking the whole grid: the fetchers' own tiles would start
    // only after their units. 128-row tiles (a quarter as many, and at this size about as
    // long, their K steps being dominated by fixed costs) leave the fetchers CUs of their
    // own. Measured at 1024^3 with 8 shards: 5% faster than the baseline instead of 5% slower.
    const bool staged = d.D > 1 || !d.direct_local;
    const int64_t t64 = cdiv(d.M, 64) * cdiv(d.N, 64), t128 = cdiv(d.M, 128) * cdiv(d.N, 128);
    if (bm == 64 && d.algo == AGMM_ALGO_FUSED && staged && t64 + kDefaultFetchWgs > num_cus &&
        t128 * 4 >= num_cus) {
      bm = 128;
      fused_128 = true;
    }
  }
  c.block_m = c.block_n = bm;
  c.block_k = agmm::kBlockK;
  const int64_t T_m = cdiv(d.M, bm), T_n = cdiv(d.N, bm);
  // k-group: 1024 K columns (the pages' default), or 512 once K >= 4096. Measured on one
  // MI355X: tiles of a one-round grid start as soon as the first k-group of their m-tile
  // arrives, and a smaller first group arrives sooner; with short K, finer groups catch up
  // with the fetch front and cost more acquires than they save.
  // The 128-row fused case above takes 512 columns too: twice the units, so twice the
  // fetchers, each done in half the time. A long-K grid of 256-row tiles that runs in one
  // round beside the default fetchers (4096x3584x8192 with 4 or 8 shards) takes 256: its
  // tiles then start on half the first k-group (1-3% faster there). One-round grids of
  // 128-row tiles keep 512 (1024x3584x8192 with 2 to 8 shards: 2-5% faster than with 256,
  // whose twice as many k-groups cost the short tiles more acquires than they save).
  int kg_cols = (d.K >= 4096 || fused_128) ? 512 : 1024;
  const int64_t W_cap = std::min<int64_t>(d.num_wgs ? d.num_wgs : num_cus, num_cus);
  if (d.algo == AGMM_ALGO_FUSED && d.K >= 4096 && bm == 256 &&
      T_m * T_n + kDefaultFetchWgs <= W_cap)
    kg_cols = 256;
  c.k_per_flag = d.k_per_flag ? d.k_per_flag : std::max(1, kg_cols / c.block_k);
  const int64_t KG = (int64_t)c.k_per_flag * c.block_k;
  const int64_t G = d.K > 0 ? cdiv(d.K, KG) : 0;
  if (T_m * T_n >= kMaxCount || T_m * G >= kMaxCount) return AGMM_ERR_UNSUPPORTED;
  // queue entries carry the tile id in 24 bits
  if (T_m * T_n > (int64_t)agmm::kItemTileMask + 1) return AGMM_ERR_UNSUPPORTED;
  c.T_m = (int32_t)T_m;
  c.T_n = (int32_t)T_n;
  c.G = (int32_t)G;
  c.num_tiles = (int32_t)(T_m * T_n);

  // GEMM order of m-tiles: in-place (local-shard) tiles first, then the others by shard in
  // rank-rotated order (rank+1, rank+2, ...), ascending within a shard.
  std::vector<int64_t> direct, other;
  for (int64_t t = 0; t < T_m; ++t) (is_direct(d, M_s, bm, t) ? direct : other).push_back(t);
  std::stable_sort(other.begin(), other.end(), [&](int64_t a, int64_t b) {
    const int64_t ka = ((a * bm) / M_s - d.rank + d.D) % d.D;
    const int64_t kb = ((b * bm) / M_s - d.rank + d.D) % d.D;
    return ka < kb;
  });
  pl->mtiles.clear();
  for (int64_t t : direct) pl->mtiles.push_back((uint32_t)t | 0x80000000u);
  for (int64_t t : other) pl->mtiles.push_back((uint32_t)t);

  // gather_a: the local shard's m-tiles are fetched too (after every staged one; no tile
  // waits for them), so that the staging buffer ends up holding all of A.
  const int64_t n_units = ((int64_t)other.size() + (d.gather_a ? (int64_t)direct.size() : 0)) * G;
  if (n_units >= kMaxCount) return AGMM_ERR_UNSUPPORTED;
  c.num_units = (int32_t)n_units;

  // Tail split: with Wg GEMM workgroups, num_tiles % Wg tiles are left for a last round. When
  // that round would be at most half full, the last tiles (by t_m * T_n + t_n) are cut along
  // K into S pieces (at least 16 K-tiles each) so the round has about Wg pieces.
  const int64_t W_base = std::min<int64_t>(d.num_wgs ? d.num_wgs : num_cus, num_cus);
  const int64_t Wg = std::min<int64_t>(W_base, c.num_tiles);
  const int64_t KT = cdiv(d.K, c.block_k);
  int S = 0;
  int64_t tail = 0;
  if (d.tail_split == 1 && Wg > 0 && c.num_tiles > Wg && c.num_tiles <= (int64_t)agmm::kItemTileMask) {
    tail = c.num_tiles % Wg;
    if (tail > 0) {
      S = (int)std::min<int64_t>({(int64_t)agmm::kMaxSplit, Wg / tail, KT / 16});
      if (S < 2) S = 0;
    }
    if (S == 0) tail = 0;
  }
  c.split_tiles = (int32_t)tail;
  c.split_pieces = S;
  c.num_items = (int32_t)(c.num_tiles + tail * (S > 0 ? S - 1 : 0));
  pl->split_base = c.num_tiles - tail;

  // Grid: one workgroup per CU (a 128 KiB LDS footprint allows one), fetchers first.
  // Fetchers: the default count, unless every tile runs in the first round and fewer
  // workgroups than that are left over: then every fetcher would hold back a tile for the
  // whole fetch, and one fetcher per unit finishes the fetch in one pass instead.
  int F = 0;
  int64_t W = W_base;
  c.fetch_kernel = (d.algo == AGMM_ALGO_FUSED && n_units > 0 && d.fetch_kernel == 1) ? 1 : 0;
  if (c.fetch_kernel) {
    // Fetch kernel beside the grid: F of its workgroups (one per CU by default, none idle),
    // and every grid workgroup computes. Its units arrive over the GEMM's first K steps, so
    // the K loop waits for each staged k-group as it reaches it.
    F = (int)std::min<int64_t>(d.num_fetch_wgs ? d.num_fetch_wgs : num_cus, n_units);
    W = std::max<int64_t>(1, std::min<int64_t>(W_base, c.num_items));
    c.num_fetch_wgs = F;
    c.num_wgs = (int32_t)W;
    c.row_wait = 0;
  } else {
    if (n_units > 0) {
      F = d.num_fetch_wgs ? d.num_fetch_wgs : kDefaultFetchWgs;
      if (!d.num_fetch_wgs && c.num_items <= W_base && W_base - c.num_items < kDefaultFetchWgs)
        F = (int)std::min<int64_t>(n_units, W_base);
    }
    F = (int)std::min<int64_t>(F, n_units);
    W = std::min<int64_t>(W, (int64_t)F + c.num_items);  // every workgroup resident, none idle
    F = (int)std::min<int64_t>(F, W);
    if (c.num_tiles > 0 && W < 1) W = 1;
    c.num_fetch_wgs = F;
    c.num_wgs = (int32_t)W;
    // Every unit has a fetcher of its own: the fetch is one pass, so tiles wait for their
    // whole row at their start and run a K loop without polls (measured faster than
    // per-k-group waits in that case, and slower when fetchers take several units each).
    c.row_wait = (n_units > 0 && F >= n_units) ? 1 : 0;
  }
  c.num_copy_wgs = (int32_t)std::min<int64_t>(n_units, 4LL * num_cus);

  make_queues(T_m, T_n, pl->mtiles, S, pl);

  // Fetch order follows the order in which the tile queues reach the m-tiles, modelled as
  // the W workgroups draining the 8 per-XCD queues evenly (stealing included): entry i of
  // queue x is the k-th in the order (i, x) over existing entries, reached in round k / W.
  // An m-tile's window is the first round that reaches one of its tiles (tail-queue pieces
  // count as after every round). Staged m-tiles are fetched window by window, in GEMM order
  // inside a window, and inside a window k-group by k-group, so the first k-groups of every
  // m-tile a round starts on come first.
  std::vector<int64_t> first_round(T_m, INT64_MAX);
  int32_t longest = 0;
  for (int x = 0; x < agmm::kQueues; ++x) longest = std::max(longest, pl->qlen[x]);
  for (int64_t i = 0, k = 0; i < longest; ++i)
    for (int x = 0; x < agmm::kQueues; ++x) {
      if (i >= pl->qlen[x]) continue;
      const uint32_t q = pl->qtiles[pl->qoff[x] + i] & agmm::kItemTileMask;
      const int64_t pos = (int64_t)q / T_n;
      first_round[pos] = std::min<int64_t>(first_round[pos], k / std::max<int64_t>(1, W));
      ++k;
    }
  std::vector<std::pair<int64_t, int64_t>> staged_pos;  // (window, GEMM position)
  for (int64_t pos = 0; pos < T_m; ++pos)
    if (!(pl->mtiles[pos] >> 31)) staged_pos.push_back({first_round[pos], pos});
  std::stable_sort(staged_pos.begin(), staged_pos.end(),
                   [](const std::pair<int64_t, int64_t>& a, const std::pair<int64_t, int64_t>& b) {
                     return a.first < b.first;
                   });
  pl->units.clear();
  for (size_t ws = 0; ws < staged_pos.size();) {
    size_t we = ws;
    while (we < staged_pos.size() && staged_pos[we].first == staged_pos[ws].first) ++we;
    for (int64_t g = 0; g < G; ++g)
      for (size_t i = ws; i < we; ++i) {
        pl->units.push_back(pl->mtiles[staged_pos[i].second] & 0x7fffffffu);
        pl->units.push_back((uint32_t)g);
      }
    ws = we;
  }
  if (d.gather_a)
    for (int64_t g = 0; g < G; ++g)
      for (int64_t t : direct) {
        pl->units.push_back((uint32_t)t);
        pl->units.push_back((uint32_t)g);
      }

  // Host stream pipeline: S chunks, chunk i = rows [i*M_s/S, (i+1)*M_s/S) of every shard,
  // each chunk's tables the global ones filtered to its m-tiles (fetch and GEMM order kept).
  pl->chunks.clear();
  pl->c_units.clear();
  pl->c_mtiles.clear();
  pl->c_qtiles.clear();
  if (d.algo == AGMM_ALGO_PIPELINED) {
    int S = d.pipeline_chunks ? d.pipeline_chunks : kDefaultChunks;
    if (M_s == 0 || M_s % bm != 0) S = 1;
    while (S > 1 && M_s % ((int64_t)S * bm) != 0) --S;
    const int64_t rows = S > 1 ? M_s / S : 1;
    auto chunk_of = [&](uint32_t t) { return S == 1 ? 0 : (int)((((int64_t)t * bm) % M_s) / rows); };
    for (int i = 0; i < S; ++i) {
      PipeChunk ch;
      memset(&ch, 0, sizeof(ch));
      ch.u_off = (int32_t)(pl->c_units.size() / 2);
      for (size_t k = 0; k < pl->units.size(); k += 2)
        if (chunk_of(pl->units[k]) == i) {
          pl->c_units.push_back(pl->units[k]);
          pl->c_units.push_back(pl->units[k + 1]);
        }
      ch.u_len = (int32_t)(pl->c_units.size() / 2) - ch.u_off;
      std::vector<uint32_t> mt;
      for (uint32_t e : pl->mtiles)
        if (chunk_of(e & 0x7fffffffu) == i) mt.push_back(e);
      ch.m_off = (int32_t)pl->c_mtiles.size();
      ch.m_len = (int32_t)mt.size();
      pl->c_mtiles.insert(pl->c_mtiles.end(), mt.begin(), mt.end());
      Plan q;
      q.split_base = 0;
      make_queues((int64_t)mt.size(), T_n, mt, 0, &q);
      ch.q_off = (int32_t)pl->c_qtiles.size();
      ch.q_len = (int32_t)q.qtiles.size();
      memcpy(ch.qoff, q.qoff, sizeof(ch.qoff));
      memcpy(ch.qlen, q.qlen, sizeof(ch.qlen));
      pl->c_qtiles.insert(pl->c_qtiles.end(), q.qtiles.begin(), q.qtiles.end());
      pl->chunks.push_back(ch);
    }
    c.pipeline_chunks = S;
    c.pipeline_streams = std::min(S, kPipeStreams);
  }

  c.trace_cap = d.debug ? (d.trace_cap ? d.trace_cap : kDefaultTraceCap) : 0;
  // debug trace: the grid's workgroups, then the fetch kernel's
  pl->trace_wgs = d.debug ? std::max<int64_t>(W, 1) + (c.fetch_kernel ? F : 0) : 0;
  c.staging_elems = (n_units > 0 && !d.gather_a) ? d.M * d.K : 0;
  pl->flags_n = std::max<int64_t>(1, T_m * G);

  int64_t off = 0;
  pl->off_staging = off; off = align256(off + c.staging_elems * 2);
  pl->off_flags = off;   off = align256(off + pl->flags_n * 4);
  pl->off_ctr = off;     off = align256(off + agmm::CTR_WORDS * 4);
  pl->off_split = off;   off = align256(off + std::max<int64_t>(1, tail) * 4);
  pl->off_units = off;   off = align256(off + std::max<int64_t>(1, n_units) * 8);
  pl->off_mtiles = off;  off = align256(off + std::max<int64_t>(1, T_m) * 4);
  pl->off_qtiles = off;  off = align256(off + std::max<int64_t>(1, c.num_items) * 4);
  pl->off_partials = off; off = align256(off + tail * S * (int64_t)bm * bm * 4);
  pl->off_trace = off;   off = align256(off + pl->trace_wgs * c.trace_cap * (int64_t)sizeof(agmm_trace_rec));
  pl->off_tcount = off;  off = align256(off + std::max<int64_t>(1, pl->trace_wgs) * 4);
  pl->off_c_ctr = off;   off = align256(off + (int64_t)pl->chunks.size() * agmm::CTR_WORDS * 4);
  pl->off_c_units = off; off = align256(off + (int64_t)pl->c_units.size() * 4);
  pl->off_c_mtiles = off; off = align256(off + (int64_t)pl->c_mtiles.size() * 4);
  pl->off_c_qtiles = off; off = align256(off + (int64_t)pl->c_qtiles.size() * 4);
  pl->total = off;
  c.workspace_bytes = off;
  return AGMM_OK;
}

// The handle's host-side state from a plan (no device work).
void init_handle(agmm_handle* h, const agmm_desc& desc, const Plan& pl, int dev) {
  h->desc = desc;
  h->cfg = pl.cfg;
  h->cfg.device = dev;
  h->M_s = pl.M_s;
  h->flags_n = pl.flags_n;
  h->trace_wgs = pl.trace_wgs;
  h->h_units = pl.units;
  h->h_mtiles = pl.mtiles;
  h->h_qtiles = pl.qtiles;
  memcpy(h->qoff, pl.qoff, sizeof(h->qoff));
  memcpy(h->qlen, pl.qlen, sizeof(h->qlen));
  h->poisoned = false;
  h->chunks = pl.chunks;
}

// Points the handle's buffers into its workspace h->ws, at the plan's offsets.
void carve_workspace(agmm_handle* h, const Plan& pl) {
  h->staging = reinterpret_cast<uint16_t*>(h->ws + pl.off_staging);
  h->flags = reinterpret_cast<uint32_t*>(h->ws + pl.off_flags);
  h->ctr = reinterpret_cast<uint32_t*>(h->ws + pl.off_ctr);
  h->units = reinterpret_cast<uint32_t*>(h->ws + pl.off_units);
  h->mtiles = reinterpret_cast<uint32_t*>(h->ws + pl.off_mtiles);
  h->qtiles = reinterpret_cast<uint32_t*>(h->ws + pl.off_qtiles);
  h->split_cnt = reinterpret_cast<uint32_t*>(h->ws + pl.off_split);
  h->partials = reinterpret_cast<float*>(h->ws + pl.off_partials);
  h->split_base = pl.split_base;
  h->trace = pl.trace_wgs ? reinterpret_cast<agmm_trace_rec*>(h->ws + pl.off_trace) : nullptr;
  h->trace_count = reinterpret_cast<uint32_t*>(h->ws + pl.off_tcount);
  h->c_ctr = reinterpret_cast<uint32_t*>(h->ws + pl.off_c_ctr);
  h->c_units = reinterpret_cast<uint32_t*>(h->ws + pl.off_c_units);
  h->c_mtiles = reinterpret_cast<uint32_t*>(h->ws + pl.off_c_mtiles);
  h->c_qtiles = reinterpret_cast<uint32_t*>(h->ws + pl.off_c_qtiles);
}

bool overlaps(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
  if (!a || !b || abytes <= 0 || bbytes <= 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

bool misaligned(const void* p) { return ((uintptr_t)p & 15u) != 0; }

// A flag-wait timeout of an earlier launch, copied to the handle's pinned host word by that
// launch's last workgroup: poisons the handle. Reads the word without synchronizing, so a
// launch still running is seen by a later call (or by ag_matmul_sync_status).
bool timed_out(agmm_handle* h) {
  if (!h->host_status || __atomic_load_n(&h->host_status[0], __ATOMIC_ACQUIRE) == 0) return false;
  h->poisoned = true;
  return true;
}

// Runs that a captured graph could not replay refuse a capturing stream: a debug run
// synchronizes the stream, and a fetch-kernel run's GEMM grid waits on flags that only the
// fetch kernel beside it sets, which a graph may run after it instead. (The kernels count
// runs on the device, so a fused run itself replays correctly, and a pipelined run's chunk
// streams join the capture through its events.)
int refuse_capture(hipStream_t s) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  AGMM_HIP(hipStreamIsCapturing(s, &cs));
  return cs == hipStreamCaptureStatusNone ? AGMM_OK : AGMM_ERR_UNSUPPORTED;
}

// Destroys the pipeline's streams and events created so far (errors ignored: teardown).
void release_streams(agmm_handle* h) {
  for (int j = 0; j < h->n_pstreams; ++j) (void)hipStreamDestroy(h->pstreams[j]);
  if (h->n_events > 0) (void)hipEventDestroy(h->ev_start);
  for (int j = 0; j + 1 < h->n_events; ++j) (void)hipEventDestroy(h->ev_done[j]);
  h->n_pstreams = 0;
  h->n_events = 0;
  if (h->has_fstream) (void)hipStreamDestroy(h->fstream);
  if (h->has_fev) {
    (void)hipEventDestroy(h->ev_fin);
    (void)hipEventDestroy(h->ev_fout);
  }
  h->has_fstream = h->has_fev = false;
}

}  // namespace

extern "C" {

void ag_matmul_desc_init(agmm_desc* d) {
  if (!d) return;
  memset(d, 0, sizeof(*d));
  d->D = 1;
  d->dtype = AGMM_F16;
  d->layout = AGMM_K_CONTIGUOUS;
  d->algo = AGMM_ALGO_FUSED;
  d->direct_local = 1;
  d->debug_skip_unit = -1;
}

const char* ag_matmul_strerror(int code) {
  switch (code) {
    case AGMM_OK: return "ok";
    case AGMM_ERR_INVALID_ARG: return "invalid argument";
    case AGMM_ERR_UNSUPPORTED: return "unsupported shape or option";
    case AGMM_ERR_HIP: return "HIP runtime error";
    case AGMM_ERR_OOM: return "device out of memory";
    case AGMM_ERR_TIMEOUT: return "flag wait timed out";
    case AGMM_ERR_WRONG_DEVICE: return "current device differs from the handle's device";
    case AGMM_ERR_POISONED: return "handle poisoned by an earlier timeout";
    case AGMM_ERR_TOO_LARGE: return "workspace larger than the static scratch";
    default: return "unknown error code";
  }
}

int ag_matmul_last_hip_error(void) { return g_last_hip; }

int64_t ag_matmul_workspace_bytes(const agmm_desc* desc) {
  const int rc = validate_desc(desc);
  if (rc != AGMM_OK) return rc;
  Plan pl;
  // The CU count only shapes the grid; take the MI355X's 256 when no device is asked.
  const int prc = make_plan(*desc, 256, &pl);
  if (prc != AGMM_OK) return prc;
  return pl.total;
}

int ag_matmul_create(const agmm_desc* desc, void* workspace, size_t workspace_bytes,
                     agmm_handle** out_handle) {
  if (!out_handle) return AGMM_ERR_INVALID_ARG;
  *out_handle = nullptr;
  if (workspace && ((uintptr_t)workspace & 255u) != 0) return AGMM_ERR_INVALID_ARG;
  int rc = validate_desc(desc);
  if (rc != AGMM_OK) return rc;
  int dev = 0;
  AGMM_HIP(hipGetDevice(&dev));
  int num_cus = 0;
  AGMM_HIP(hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, dev));
  Plan pl;
  rc = make_plan(*desc, num_cus, &pl);
  if (rc != AGMM_OK) return rc;
  int per_cu = 0;
  AGMM_HIP(agmm::fused_occupancy(desc->dtype, pl.cfg.block_m, &per_cu));
  if (per_cu < 1) return AGMM_ERR_UNSUPPORTED;
  if (pl.cfg.fetch_kernel) {
    bool fits = false;
    AGMM_HIP(agmm::fetch_fits_beside(desc->dtype, pl.cfg.block_m,
                                     desc->layout == AGMM_K_CONTIGUOUS, &fits));
    if (!fits) return AGMM_ERR_UNSUPPORTED;
  }

  agmm_handle* h = new (std::nothrow) agmm_handle();
  if (!h) return AGMM_ERR_OOM;
  init_handle(h, *desc, pl, dev);
  h->n_pstreams = 0;
  h->n_events = 0;
  h->has_fstream = h->has_fev = false;
  if (workspace && workspace_bytes < (size_t)pl.total) {
    delete h;
    return AGMM_ERR_INVALID_ARG;
  }
  hipError_t e = hipHostMalloc(reinterpret_cast<void**>(&h->host_status), 4 * sizeof(uint32_t),
                               hipHostMallocCoherent);
  if (e != hipSuccess) {
    g_last_hip = (int)e;
    (void)hipGetLastError();
    delete h;
    return e == hipErrorOutOfMemory ? AGMM_ERR_OOM : AGMM_ERR_HIP;
  }
  memset(h->host_status, 0, 4 * sizeof(uint32_t));
  h->own_ws = workspace == nullptr;
  if (h->own_ws) {
    e = hipMalloc(reinterpret_cast<void**>(&h->ws), (size_t)pl.total);
  } else {
    h->ws = static_cast<char*>(workspace);
    e = hipSuccess;
  }
  if (e != hipSuccess) {
    g_last_hip = (int)e;
    (void)hipGetLastError();
    (void)hipHostFree(h->host_status);
    delete h;
    return e == hipErrorOutOfMemory ? AGMM_ERR_OOM : AGMM_ERR_HIP;
  }
  carve_workspace(h, pl);

  auto fail = [&](hipError_t err) {
    g_last_hip = (int)err;
    release_streams(h);
    if (h->own_ws) (void)hipFree(h->ws);
    (void)hipHostFree(h->host_status);
    delete h;
    return AGMM_ERR_HIP;
  };
  // Flags, counters (queues, split tiles) and trace counts start at zero; the schedule
  // tables are uploaded once.
  if ((e = hipMemset(h->ws + pl.off_flags, 0, (size_t)(pl.off_units - pl.off_flags))) != hipSuccess)
    return fail(e);
  {
    // the kernels copy a recorded timeout to the host word through its device address
    void* dptr = nullptr;
    if ((e = hipHostGetDevicePointer(&dptr, h->host_status, 0)) != hipSuccess) return fail(e);
    const uint32_t words[5] = {(uint32_t)(uintptr_t)dptr,
                               (uint32_t)((uint64_t)(uintptr_t)dptr >> 32),
                               (uint32_t)desc->debug_fetch_delay, desc->debug_fetch_seed,
                               (uint32_t)desc->debug_fetch_reverse};
    static_assert(agmm::CTR_HOST_HI == agmm::CTR_HOST_LO + 1 &&
                      agmm::CTR_DBG_DELAY == agmm::CTR_HOST_LO + 2 &&
                      agmm::CTR_DBG_SEED == agmm::CTR_HOST_LO + 3 &&
                      agmm::CTR_DBG_REVERSE == agmm::CTR_HOST_LO + 4,
                  "the words written together are contiguous");
    if ((e = hipMemcpy(h->ctr + agmm::CTR_HOST_LO, words, sizeof(words), hipMemcpyHostToDevice)) !=
        hipSuccess)
      return fail(e);
  }
  if (pl.trace_wgs &&
      (e = hipMemset(h->ws + pl.off_trace, 0, (size_t)(pl.total - pl.off_trace))) != hipSuccess)
    return fail(e);
  if (!pl.units.empty() &&
      (e = hipMemcpy(h->units, pl.units.data(), pl.units.size() * 4, hipMemcpyHostToDevice)) != hipSuccess)
    return fail(e);
  if (!pl.mtiles.empty() &&
      (e = hipMemcpy(h->mtiles, pl.mtiles.data(), pl.mtiles.size() * 4, hipMemcpyHostToDevice)) != hipSuccess)
    return fail(e);
  if (!pl.qtiles.empty() &&
      (e = hipMemcpy(h->qtiles, pl.qtiles.data(), pl.qtiles.size() * 4, hipMemcpyHostToDevice)) != hipSuccess)
    return fail(e);
  if (!pl.chunks.empty()) {
    if ((e = hipMemset(h->c_ctr, 0, pl.chunks.size() * agmm::CTR_WORDS * 4)) != hipSuccess)
      return fail(e);
    const std::vector<uint32_t>* tabs[3] = {&pl.c_units, &pl.c_mtiles, &pl.c_qtiles};
    uint32_t* dsts[3] = {h->c_units, h->c_mtiles, h->c_qtiles};
    for (int k = 0; k < 3; ++k)
      if (!tabs[k]->empty() &&
          (e = hipMemcpy(dsts[k], tabs[k]->data(), tabs[k]->size() * 4, hipMemcpyHostToDevice)) !=
              hipSuccess)
        return fail(e);
    // default-priority streams that do not synchronize with the null stream (stream 0 of
    // the rotation is the caller's)
    for (int j = 1; j < pl.cfg.pipeline_streams; ++j) {
      if ((e = hipStreamCreateWithFlags(&h->pstreams[j - 1], hipStreamNonBlocking)) != hipSuccess)
        return fail(e);
      ++h->n_pstreams;
    }
    if ((e = hipEventCreateWithFlags(&h->ev_start, hipEventDisableTiming)) != hipSuccess)
      return fail(e);
    ++h->n_events;
    for (int j = 1; j < pl.cfg.pipeline_streams; ++j) {
      if ((e = hipEventCreateWithFlags(&h->ev_done[j - 1], hipEventDisableTiming)) != hipSuccess)
        return fail(e);
      ++h->n_events;
    }
  }
  if (pl.cfg.fetch_kernel) {
    // a default-priority stream that does not synchronize with the null stream
    if ((e = hipStreamCreateWithFlags(&h->fstream, hipStreamNonBlocking)) != hipSuccess)
      return fail(e);
    h->has_fstream = true;
    if ((e = hipEventCreateWithFlags(&h->ev_fin, hipEventDisableTiming)) != hipSuccess)
      return fail(e);
    if ((e = hipEventCreateWithFlags(&h->ev_fout, hipEventDisableTiming)) != hipSuccess) {
      (void)hipEventDestroy(h->ev_fin);
      return fail(e);
    }
    h->has_fev = true;
  }
  if ((e = hipDeviceSynchronize()) != hipSuccess) return fail(e);
  *out_handle = h;
  return AGMM_OK;
}

int ag_matmul_destroy(agmm_handle* h) {
  if (!h) return AGMM_OK;
  int rc = AGMM_OK;
  int cur = 0;
  if (hipGetDevice(&cur) == hipSuccess && cur != h->cfg.device) (void)hipSetDevice(h->cfg.device);
  hipError_t e = hipDeviceSynchronize();
  release_streams(h);
  if (e == hipSuccess && h->own_ws) e = hipFree(h->ws);
  if (e == hipSuccess && h->ar_ws) e = hipFree(h->ar_ws);
  if (e == hipSuccess) e = hipHostFree(h->host_status);
  if (e != hipSuccess) {
    g_last_hip = (int)e;
    rc = AGMM_ERR_HIP;
  }
  if (cur != h->cfg.device) (void)hipSetDevice(cur);
  delete h;
  return rc;
}

int ag_matmul_get_config(const agmm_handle* h, agmm_config* cfg) {
  if (!h || !cfg) return AGMM_ERR_INVALID_ARG;
  *cfg = h->cfg;
  return AGMM_OK;
}

int ag_matmul_sync_status(agmm_handle* h) {
  if (!h) return AGMM_ERR_INVALID_ARG;
  int cur = 0;
  AGMM_HIP(hipGetDevice(&cur));
  if (cur != h->cfg.device) return AGMM_ERR_WRONG_DEVICE;
  AGMM_HIP(hipDeviceSynchronize());
  if (h->poisoned) return AGMM_ERR_POISONED;
  return timed_out(h) ? AGMM_ERR_TIMEOUT : AGMM_OK;
}

}  // extern "C"

namespace {

// The launch parameters of a handle's run: its tables and counters, the given buffers.
KParams run_params(agmm_handle* h, const void* const* shards, const void* B, const void* bias,
                   void* out, uint16_t* staging) {
  const agmm_desc& d = h->desc;
  const agmm_config& c = h->cfg;
  KParams p;
  memset(&p, 0, sizeof(p));
  for (int i = 0; i < d.D; ++i) p.shards[i] = static_cast<const uint16_t*>(shards[i]);
  p.B = static_cast<const uint16_t*>(B);
  p.bias = static_cast<const uint16_t*>(bias);
  p.out = static_cast<uint16_t*>(out);
  p.staging = staging;
  p.flags = h->flags;
  p.ctr = h->ctr;
  p.units = h->units;
  p.mtiles = h->mtiles;
  p.qtiles = h->qtiles;
  for (int x = 0; x < agmm::kQueueSlots; ++x) {
    p.qoff[x] = h->qoff[x];
    p.qlen[x] = h->qlen[x];
  }
  p.partials = h->partials;
  p.split_cnt = h->split_cnt;
  p.split_base = (int32_t)h->split_base;
  p.trace = h->trace;
  p.trace_count = h->trace_count;
  p.M = d.M;
  p.N = d.N;
  p.K = d.K;
  p.M_s = h->M_s;
  p.D = d.D;
  p.rank = d.rank;
  p.T_m = c.T_m;
  p.T_n = c.T_n;
  p.G = c.G;
  p.kpf = c.k_per_flag;
  p.num_units = c.num_units;
  p.num_tiles = c.num_tiles;
  p.debug = d.debug;
  p.trace_cap = c.trace_cap;
  p.spin_limit = d.spin_limit ? d.spin_limit : kDefaultSpinLimit;
  p.skip_unit = d.debug_skip_unit;
  return p;
}

// GEMM + all-reduce with per-tile flags, the claim order: tile by tile, its D producers
// (r << 24 | tile); tile t's reducer (kArReduceItem | t) follows the producers of tile
// t + lag, lag = the tiles whose producers one round of the grid covers, so that a reducer
// mostly finds its flags set. Every reducer comes after its tile's producers.
std::vector<uint32_t> ar_flag_items(int D, int64_t tiles, int64_t num_cus) {
  const int64_t lag = (std::max<int64_t>(1, num_cus) + D - 1) / D;
  std::vector<uint32_t> items;
  items.reserve((size_t)(tiles * (D + 1)));
  for (int64_t t = 0; t < tiles; ++t) {
    for (int r = 0; r < D; ++r) items.push_back(((uint32_t)r << 24) | (uint32_t)t);
    if (t >= lag) items.push_back(agmm::kArReduceItem | (uint32_t)(t - lag));
  }
  for (int64_t t = std::max<int64_t>(0, tiles - lag); t < tiles; ++t)
    items.push_back(agmm::kArReduceItem | (uint32_t)t);
  return items;
}

// The planner descriptor of one rank's share: a one-shard GEMM over K_local, read in place.
agmm_desc ar_share_desc(int64_t M, int64_t N, int64_t K_local, int dtype, int block_m) {
  agmm_desc d;
  ag_matmul_desc_init(&d);
  d.M = M;
  d.N = N;
  d.K = K_local;
  d.dtype = dtype;
  d.algo = AGMM_ALGO_BASELINE;
  d.block_m = block_m;
  return d;
}

// gather: called as ag_matmul_run_gather; a_gathered is then the caller's [M, K] buffer,
// which serves as the staging buffer (NULL allowed only when it has no bytes).
// part (AGMM_ALGO_BASELINE only): 0 = the whole run, AGMM_PART_COPY = only its staging copy,
// AGMM_PART_GEMM = only its GEMM.
int run_impl(agmm_handle* h, const void* const* shards, const void* B, const void* bias,
             void* out, bool gather, void* a_gathered, void* hip_stream, int part = 0) {
  if (!h || h->ar_D) return AGMM_ERR_INVALID_ARG;
  if (h->poisoned) return AGMM_ERR_POISONED;
  if (timed_out(h)) return AGMM_ERR_TIMEOUT;
  const agmm_desc& d = h->desc;
  const agmm_config& c = h->cfg;
  int cur = 0;
  AGMM_HIP(hipGetDevice(&cur));
  if (cur != c.device) return AGMM_ERR_WRONG_DEVICE;

  const int64_t esz = 2;
  const int64_t shard_bytes = h->M_s * d.K * esz;
  const int64_t b_bytes = d.K * d.N * esz;
  const int64_t out_bytes = d.M * d.N * esz;
  const int64_t bias_bytes = d.has_bias ? d.N * esz : 0;
  if (!shards) return AGMM_ERR_INVALID_ARG;
  if ((bias != nullptr) != (d.has_bias != 0)) return AGMM_ERR_INVALID_ARG;
  for (int i = 0; i < d.D; ++i) {
    if (shard_bytes > 0 && !shards[i]) return AGMM_ERR_INVALID_ARG;
    if (misaligned(shards[i])) return AGMM_ERR_INVALID_ARG;
  }
  if ((b_bytes > 0 && !B) || misaligned(B)) return AGMM_ERR_INVALID_ARG;
  if ((out_bytes > 0 && !out) || misaligned(out)) return AGMM_ERR_INVALID_ARG;
  if (misaligned(bias)) return AGMM_ERR_INVALID_ARG;
  for (int i = 0; i < d.D; ++i)
    if (overlaps(out, out_bytes, shards[i], shard_bytes)) return AGMM_ERR_INVALID_ARG;
  if (overlaps(out, out_bytes, B, b_bytes) || overlaps(out, out_bytes, bias, bias_bytes))
    return AGMM_ERR_INVALID_ARG;
  if (gather != (d.gather_a != 0)) return AGMM_ERR_INVALID_ARG;
  if (d.gather_a) {
    const int64_t a_bytes = d.M * d.K * esz;
    if ((a_bytes > 0 && !a_gathered) || misaligned(a_gathered)) return AGMM_ERR_INVALID_ARG;
    if (overlaps(a_gathered, a_bytes, out, out_bytes) || overlaps(a_gathered, a_bytes, B, b_bytes) ||
        overlaps(a_gathered, a_bytes, bias, bias_bytes))
      return AGMM_ERR_INVALID_ARG;
    for (int i = 0; i < d.D; ++i)
      if (overlaps(a_gathered, a_bytes, shards[i], shard_bytes)) return AGMM_ERR_INVALID_ARG;
  }
  // M == 0 or N == 0: no output tile; only a gathered A (N == 0) may have rows to copy
  if (c.num_tiles == 0 && c.num_units == 0) return AGMM_OK;

  hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
  if (c.fetch_kernel || d.debug) {
    const int rc = refuse_capture(s);
    if (rc != AGMM_OK) return rc;
  }
  ++h->cfg.epoch;  // runs enqueued through the handle (the kernels count their own)

  KParams p = run_params(h, shards, B, bias, out,
                          d.gather_a ? static_cast<uint16_t*>(a_gathered) : h->staging);
  // debug: the staging buffer holds a quiet NaN everywhere before the run, so a tile that
  // read a staged unit before it was written would put NaN into the output
  if (d.debug && c.staging_elems > 0)
    AGMM_HIP(agmm::launch_fill16(h->staging, c.staging_elems,
                                 d.dtype == AGMM_BF16 ? kNanBF16 : kNanF16, s));

  if (d.algo == AGMM_ALGO_FUSED && c.fetch_kernel) {
    // The fetch kernel on the handle's stream, after the caller's stream reaches this point;
    // the GEMM grid (no fetchers) on the caller's stream; the caller's stream then waits for
    // the fetch kernel, so the run ends when both have.
    p.F = 0;
    p.staged_kmajor = d.layout == AGMM_K_CONTIGUOUS ? 1 : 0;
    p.row_wait = c.row_wait;
    KParams q = p;
    if (p.trace) q.trace = p.trace + (size_t)c.num_wgs * c.trace_cap;
    q.trace_count = p.trace_count + c.num_wgs;
    AGMM_HIP(hipEventRecord(h->ev_fin, s));
    AGMM_HIP(hipStreamWaitEvent(h->fstream, h->ev_fin, 0));
    AGMM_HIP(agmm::launch_fetch(q, c.block_m, p.staged_kmajor != 0, c.num_fetch_wgs, h->fstream));
    AGMM_HIP(agmm::launch_fused(p, d.dtype, c.block_m, c.num_wgs, s));
    AGMM_HIP(hipEventRecord(h->ev_fout, h->fstream));
    AGMM_HIP(hipStreamWaitEvent(s, h->ev_fout, 0));
  } else if (d.algo == AGMM_ALGO_FUSED) {
    p.F = c.num_fetch_wgs;
    p.staged_kmajor = d.layout == AGMM_K_CONTIGUOUS ? 1 : 0;
    p.row_wait = c.row_wait;
    AGMM_HIP(agmm::launch_fused(p, d.dtype, c.block_m, c.num_wgs, s));
  } else if (d.algo == AGMM_ALGO_PIPELINED) {
    p.F = 0;
    p.staged_kmajor = 1;  // chunks gather into plain [M][K] rows
    p.debug = 0;
    p.trace_cap = 0;
    const int ns = c.pipeline_streams;
    if (ns > 1) {
      AGMM_HIP(hipEventRecord(h->ev_start, s));
      for (int j = 1; j < ns; ++j) AGMM_HIP(hipStreamWaitEvent(h->pstreams[j - 1], h->ev_start, 0));
    }
    for (size_t i = 0; i < h->chunks.size(); ++i) {
      const PipeChunk& ch = h->chunks[i];
      hipStream_t sj = i % ns == 0 ? s : h->pstreams[i % ns - 1];
      KParams q = p;
      q.units = h->c_units + 2 * (int64_t)ch.u_off;
      q.num_units = ch.u_len;
      q.mtiles = h->c_mtiles + ch.m_off;
      q.T_m = ch.m_len;
      q.qtiles = h->c_qtiles + ch.q_off;
      memcpy(q.qoff, ch.qoff, sizeof(q.qoff));
      memcpy(q.qlen, ch.qlen, sizeof(q.qlen));
      q.ctr = h->c_ctr + (int64_t)i * agmm::CTR_WORDS;
      q.num_tiles = ch.m_len * c.T_n;
      // the chunk's gather, then (same stream) the chunk's GEMM
      if (ch.u_len > 0)
        AGMM_HIP(agmm::launch_copy(q, c.block_m, (int)std::min<int64_t>(ch.u_len, 4LL * c.num_cus), sj));
      const int grid = (int)std::min<int64_t>(std::min<int64_t>(c.num_cus, ch.q_len),
                                              d.num_wgs ? d.num_wgs : c.num_cus);
      if (grid > 0) AGMM_HIP(agmm::launch_gemm_only(q, d.dtype, c.block_m, grid, sj));
    }
    for (int j = 1; j < ns; ++j) {
      AGMM_HIP(hipEventRecord(h->ev_done[j - 1], h->pstreams[j - 1]));
      AGMM_HIP(hipStreamWaitEvent(s, h->ev_done[j - 1], 0));
    }
  } else {
    p.F = 0;
    p.staged_kmajor = 1;  // the baseline gathers into plain [M][K] rows
    // debug: the GEMM kernel records its tiles in the trace like the fused kernel does
    if (c.num_units > 0 && part != AGMM_PART_GEMM)
      AGMM_HIP(agmm::launch_copy(p, c.block_m, c.num_copy_wgs, s));
    const int grid = (int)std::min<int64_t>(std::min(c.num_cus, c.num_items),
                                            d.num_wgs ? d.num_wgs : c.num_cus);
    if (grid > 0 && part != AGMM_PART_COPY)
      AGMM_HIP(agmm::launch_gemm_only(p, d.dtype, c.block_m, grid, s));
  }

  if (d.debug) {
    AGMM_HIP(hipStreamSynchronize(s));
    uint32_t status = 0;
    AGMM_HIP(hipMemcpy(&status, h->ctr + agmm::CTR_STATUS, 4, hipMemcpyDeviceToHost));
    if (status != 0) {
      h->poisoned = true;
      return AGMM_ERR_TIMEOUT;
    }
  }
  return AGMM_OK;
}

}  // namespace

extern "C" {

int ag_matmul_run(agmm_handle* h, const void* const* shards, const void* B, const void* bias,
                  void* out, void* hip_stream) {
  return run_impl(h, shards, B, bias, out, false, nullptr, hip_stream);
}

int ag_matmul_run_gather(agmm_handle* h, const void* const* shards, const void* B,
                         const void* bias, void* out, void* a_gathered, void* hip_stream) {
  return run_impl(h, shards, B, bias, out, true, a_gathered, hip_stream);
}

int ag_matmul_debug_run_part(agmm_handle* h, int part, const void* const* shards, const void* B,
                             const void* bias, void* out, void* hip_stream) {
  if (!h || h->desc.algo != AGMM_ALGO_BASELINE || h->desc.gather_a) return AGMM_ERR_INVALID_ARG;
  if (part != AGMM_PART_COPY && part != AGMM_PART_GEMM) return AGMM_ERR_INVALID_ARG;
  return run_impl(h, shards, B, bias, out, false, nullptr, hip_stream, part);
}

int ag_gemm_ar_create(int D, int rank, int64_t M, int64_t N, int64_t K_local, int dtype,
                      int block_m, agmm_handle** out_handle) {
  if (!out_handle) return AGMM_ERR_INVALID_ARG;
  *out_handle = nullptr;
  if (D < 1 || D > AGMM_MAX_SHARDS || rank < 0 || rank >= D) return AGMM_ERR_INVALID_ARG;
  // one rank's share is a plain GEMM over its K columns: the planner's one-shard,
  // read-in-place case (no fetch units, no staging), run by the atomic-epilogue kernel
  agmm_desc d = ar_share_desc(M, N, K_local, dtype, block_m);
  const int rc = ag_matmul_create(&d, nullptr, 0, out_handle);
  if (rc != AGMM_OK) return rc;
  (*out_handle)->ar_D = D;
  (*out_handle)->ar_rank = rank;
  return AGMM_OK;
}

int ag_gemm_ar_run(agmm_handle* h, const void* A_local, const void* B_local, float* const* C,
                   void* hip_stream) {
  if (!h || !h->ar_D || h->ar_flags_mode || !C) return AGMM_ERR_INVALID_ARG;
  if (h->poisoned) return AGMM_ERR_POISONED;
  if (timed_out(h)) return AGMM_ERR_TIMEOUT;
  const agmm_desc& d = h->desc;
  const agmm_config& c = h->cfg;
  int cur = 0;
  AGMM_HIP(hipGetDevice(&cur));
  if (cur != c.device) return AGMM_ERR_WRONG_DEVICE;
  const int64_t a_bytes = d.M * d.K * 2, b_bytes = d.K * d.N * 2, c_bytes = d.M * d.N * 4;
  if ((a_bytes > 0 && !A_local) || misaligned(A_local)) return AGMM_ERR_INVALID_ARG;
  if ((b_bytes > 0 && !B_local) || misaligned(B_local)) return AGMM_ERR_INVALID_ARG;
  for (int r = 0; r < h->ar_D; ++r) {
    if ((c_bytes > 0 && !C[r]) || misaligned(C[r])) return AGMM_ERR_INVALID_ARG;
    if (overlaps(C[r], c_bytes, A_local, a_bytes) || overlaps(C[r], c_bytes, B_local, b_bytes))
      return AGMM_ERR_INVALID_ARG;
    for (int q = 0; q < r; ++q)
      if (overlaps(C[r], c_bytes, C[q], c_bytes)) return AGMM_ERR_INVALID_ARG;
  }
  if (c.num_tiles == 0) return AGMM_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
  ++h->cfg.epoch;
  const void* shards[1] = {A_local};
  KParams p = run_params(h, shards, B_local, nullptr, nullptr, h->staging);
  p.F = 0;
  p.staged_kmajor = 1;
  p.debug = 0;
  p.trace_cap = 0;
  p.ar_D = h->ar_D;
  p.ar_rank = h->ar_rank;
  for (int r = 0; r < h->ar_D; ++r) p.ar_out[r] = C[r];
  const int grid = (int)std::min<int64_t>(c.num_cus, c.num_items);
  AGMM_HIP(agmm::launch_gemm_ar(p, d.dtype, c.block_m, grid, s));
  return AGMM_OK;
}

int ag_gemm_ar_finalize(agmm_handle* h, const float* C, const void* bias, void* out,
                        void* hip_stream) {
  if (!h || !h->ar_D || h->ar_flags_mode) return AGMM_ERR_INVALID_ARG;
  const agmm_desc& d = h->desc;
  int cur = 0;
  AGMM_HIP(hipGetDevice(&cur));
  if (cur != h->cfg.device) return AGMM_ERR_WRONG_DEVICE;
  const int64_t c_bytes = d.M * d.N * 4, o_bytes = d.M * d.N * 2;
  if ((c_bytes > 0 && (!C || !out)) || misaligned(C) || misaligned(out) || misaligned(bias))
    return AGMM_ERR_INVALID_ARG;
  if (overlaps(out, o_bytes, C, c_bytes) || overlaps(out, o_bytes, bias, d.N * 2))
    return AGMM_ERR_INVALID_ARG;
  AGMM_HIP(agmm::launch_ar_finalize(C, static_cast<const uint16_t*>(bias),
                                    static_cast<uint16_t*>(out), d.M, d.N, d.dtype,
                                    reinterpret_cast<hipStream_t>(hip_stream)));
  return AGMM_OK;
}

int ag_gemm_ar_flags_create(int D, int64_t M, int64_t N, int64_t K_local, int dtype,
                            int block_m, agmm_handle** out_handle) {
  if (!out_handle) return AGMM_ERR_INVALID_ARG;
  *out_handle = nullptr;
  if (D < 1 || D > AGMM_MAX_SHARDS) return AGMM_ERR_INVALID_ARG;
  agmm_handle* h = nullptr;
  int rc = ag_gemm_ar_create(D, 0, M, N, K_local, dtype, block_m, &h);
  if (rc != AGMM_OK) return rc;
  const agmm_config& c = h->cfg;
  const std::vector<uint32_t> items = ar_flag_items(D, (int64_t)c.T_m * c.T_n, c.num_cus);
  const int64_t tiles = (int64_t)c.T_m * c.T_n;
  h->ar_flags_mode = true;
  h->ar_items_n = (int64_t)items.size();
  h->ar_flags_n = D * tiles;
  const int64_t part_b = align256((int64_t)D * M * N * 4);
  const int64_t flag_b = align256(h->ar_flags_n * 4), item_b = align256(h->ar_items_n * 4);
  if (part_b + flag_b + item_b > 0) {
    if (hipMalloc(&h->ar_ws, (size_t)(part_b + flag_b + item_b)) != hipSuccess) {
      (void)hipGetLastError();
      ag_matmul_destroy(h);
      return AGMM_ERR_OOM;
    }
    h->ar_partials = reinterpret_cast<float*>(h->ar_ws);
    h->ar_flags = reinterpret_cast<uint32_t*>(h->ar_ws + part_b);
    h->ar_items = reinterpret_cast<uint32_t*>(h->ar_ws + part_b + flag_b);
    hipError_t e = hipMemset(h->ar_flags, 0, (size_t)flag_b);
    if (e == hipSuccess && !items.empty())
      e = hipMemcpy(h->ar_items, items.data(), items.size() * 4, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      g_last_hip = (int)e;
      ag_matmul_destroy(h);
      return AGMM_ERR_HIP;
    }
  }
  *out_handle = h;
  return AGMM_OK;
}

int ag_gemm_ar_flags_run(agmm_handle* h, const void* const* A_parts, const void* const* B_parts,
                         const void* bias, void* out, void* hip_stream) {
  if (!h || !h->ar_flags_mode || !A_parts || !B_parts) return AGMM_ERR_INVALID_ARG;
  if (h->poisoned) return AGMM_ERR_POISONED;
  if (timed_out(h)) return AGMM_ERR_TIMEOUT;
  const agmm_desc& d = h->desc;
  const agmm_config& c = h->cfg;
  int cur = 0;
  AGMM_HIP(hipGetDevice(&cur));
  if (cur != c.device) return AGMM_ERR_WRONG_DEVICE;
  const int D = h->ar_D;
  const int64_t a_bytes = d.M * d.K * 2, b_bytes = d.K * d.N * 2, o_bytes = d.M * d.N * 2;
  if ((o_bytes > 0 && !out) || misaligned(out) || misaligned(bias)) return AGMM_ERR_INVALID_ARG;
  if (overlaps(out, o_bytes, bias, d.N * 2)) return AGMM_ERR_INVALID_ARG;
  for (int r = 0; r < D; ++r) {
    if ((a_bytes > 0 && !A_parts[r]) || misaligned(A_parts[r])) return AGMM_ERR_INVALID_ARG;
    if ((b_bytes > 0 && !B_parts[r]) || misaligned(B_parts[r])) return AGMM_ERR_INVALID_ARG;
    if (overlaps(out, o_bytes, A_parts[r], a_bytes) || overlaps(out, o_bytes, B_parts[r], b_bytes))
      return AGMM_ERR_INVALID_ARG;
  }
  if (c.num_tiles == 0) return AGMM_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
  ++h->cfg.epoch;
  KParams p = run_params(h, A_parts, nullptr, bias, out, h->staging);
  for (int r = 0; r < D; ++r) {
    p.shards[r] = static_cast<const uint16_t*>(A_parts[r]);
    p.ar_B[r] = static_cast<const uint16_t*>(B_parts[r]);
  }
  p.F = 0;
  p.staged_kmajor = 1;
  p.debug = 0;
  p.trace_cap = 0;
  p.ar_D = D;
  p.partials = h->ar_partials;
  p.flags = h->ar_flags;
  p.qtiles = h->ar_items;
  for (int x = 0; x < agmm::kQueueSlots; ++x) p.qoff[x] = p.qlen[x] = 0;
  p.qlen[0] = (int32_t)h->ar_items_n;
  const int grid = (int)std::min<int64_t>(c.num_cus, h->ar_items_n);
  AGMM_HIP(agmm::launch_ar_flags(p, d.dtype, c.block_m, grid, s));
  return AGMM_OK;
}

int ag_matmul_debug_query(agmm_handle* h, int what, void* dst, size_t bytes) {
  if (!h || !dst) return AGMM_ERR_INVALID_ARG;
  const agmm_config& c = h->cfg;
  const void* src = nullptr;
  size_t n = 0;
  std::vector<uint32_t> status;
  switch (what) {
    case AGMM_Q_FLAGS: src = h->flags; n = (size_t)c.T_m * c.G * 4; break;
    case AGMM_Q_STAGING: src = h->staging; n = (size_t)c.staging_elems * 2; break;
    case AGMM_Q_TRACE: src = h->trace; n = (size_t)h->trace_wgs * c.trace_cap * sizeof(agmm_trace_rec); break;
    case AGMM_Q_TRACE_COUNT: src = h->trace_count; n = (size_t)h->trace_wgs * 4; break;
    case AGMM_Q_STATUS: src = h->ctr + agmm::CTR_STATUS; n = 16; break;
    case AGMM_Q_PARTIALS:
      src = h->partials;
      n = (size_t)c.split_tiles * c.split_pieces * c.block_m * c.block_n * 4;
      break;
    case AGMM_Q_UNITS:
      if (bytes != h->h_units.size() * 4) return AGMM_ERR_INVALID_ARG;
      if (bytes) memcpy(dst, h->h_units.data(), bytes);
      return AGMM_OK;
    case AGMM_Q_MTILES:
      if (bytes != h->h_mtiles.size() * 4) return AGMM_ERR_INVALID_ARG;
      if (bytes) memcpy(dst, h->h_mtiles.data(), bytes);
      return AGMM_OK;
    case AGMM_Q_QUEUES: {
      const size_t n = (2 * agmm::kQueueSlots + h->h_qtiles.size()) * 4;
      if (bytes != n) return AGMM_ERR_INVALID_ARG;
      uint32_t* o = static_cast<uint32_t*>(dst);
      for (int x = 0; x < agmm::kQueueSlots; ++x) {
        o[x] = (uint32_t)h->qoff[x];
        o[agmm::kQueueSlots + x] = (uint32_t)h->qlen[x];
      }
      if (!h->h_qtiles.empty())
        memcpy(o + 2 * agmm::kQueueSlots, h->h_qtiles.data(), h->h_qtiles.size() * 4);
      return AGMM_OK;
    }
    case AGMM_Q_CHUNK_SIZES: {
      if (bytes != h->chunks.size() * 8) return AGMM_ERR_INVALID_ARG;
      uint32_t* o = static_cast<uint32_t*>(dst);
      for (size_t i = 0; i < h->chunks.size(); ++i) {
        o[2 * i] = (uint32_t)h->chunks[i].u_len;
        o[2 * i + 1] = (uint32_t)h->chunks[i].m_len;
      }
      return AGMM_OK;
    }
    case AGMM_Q_CHUNK_UNITS:
      src = h->c_units;
      for (const PipeChunk& ch : h->chunks) n += (size_t)ch.u_len * 8;
      break;
    case AGMM_Q_CHUNK_MTILES:
      src = h->c_mtiles;
      for (const PipeChunk& ch : h->chunks) n += (size_t)ch.m_len * 4;
      break;
    default: return AGMM_ERR_INVALID_ARG;
  }
  if (bytes != n) return AGMM_ERR_INVALID_ARG;
  int cur = 0;
  AGMM_HIP(hipGetDevice(&cur));
  if (cur != c.device) return AGMM_ERR_WRONG_DEVICE;
  AGMM_HIP(hipDeviceSynchronize());
  if (n) AGMM_HIP(hipMemcpy(dst, src, n, hipMemcpyDeviceToHost));
  return AGMM_OK;
}

int ag_matmul_plan_query(const agmm_desc* desc, int num_cus, int what, void* dst, size_t bytes) {
  if (!dst || num_cus < 1) return AGMM_ERR_INVALID_ARG;
  int rc = validate_desc(desc);
  if (rc != AGMM_OK) return rc;
  Plan pl;
  rc = make_plan(*desc, num_cus, &pl);
  if (rc != AGMM_OK) return rc;
  auto put = [&](const void* src, size_t n) {
    if (bytes != n) return AGMM_ERR_INVALID_ARG;
    if (n) memcpy(dst, src, n);
    return AGMM_OK;
  };
  switch (what) {
    case 0: return put(&pl.cfg, sizeof(agmm_config));
    case AGMM_Q_UNITS: return put(pl.units.data(), pl.units.size() * 4);
    case AGMM_Q_MTILES: return put(pl.mtiles.data(), pl.mtiles.size() * 4);
    case AGMM_Q_QUEUES: {
      std::vector<uint32_t> v(2 * agmm::kQueueSlots);
      for (int x = 0; x < agmm::kQueueSlots; ++x) {
        v[x] = (uint32_t)pl.qoff[x];
        v[agmm::kQueueSlots + x] = (uint32_t)pl.qlen[x];
      }
      v.insert(v.end(), pl.qtiles.begin(), pl.qtiles.end());
      return put(v.data(), v.size() * 4);
    }
    case AGMM_Q_CHUNK_SIZES: {
      std::vector<uint32_t> v;
      for (const PipeChunk& ch : pl.chunks) {
        v.push_back((uint32_t)ch.u_len);
        v.push_back((uint32_t)ch.m_len);
      }
      return put(v.data(), v.size() * 4);
    }
    case AGMM_Q_CHUNK_UNITS: return put(pl.c_units.data(), pl.c_units.size() * 4);
    case AGMM_Q_CHUNK_MTILES: return put(pl.c_mtiles.data(), pl.c_mtiles.size() * 4);
    default: return AGMM_ERR_INVALID_ARG;
  }
}

int ag_gemm_ar_flags_plan(int D, int64_t M, int64_t N, int64_t K_local, int dtype, int block_m,
                          int num_cus, agmm_config* cfg, uint32_t* items, int64_t* count) {
  if (!count || num_cus < 1 || D < 1 || D > AGMM_MAX_SHARDS) return AGMM_ERR_INVALID_ARG;
  const agmm_desc d = ar_share_desc(M, N, K_local, dtype, block_m);
  int rc = validate_desc(&d);
  if (rc != AGMM_OK) return rc;
  Plan pl;
  rc = make_plan(d, num_cus, &pl);
  if (rc != AGMM_OK) return rc;
  const std::vector<uint32_t> v = ar_flag_items(D, (int64_t)pl.cfg.T_m * pl.cfg.T_n, num_cus);
  if (cfg) *cfg = pl.cfg;
  if (items) {
    if (*count != (int64_t)v.size()) return AGMM_ERR_INVALID_ARG;
    if (!v.empty()) memcpy(items, v.data(), v.size() * 4);
  }
  *count = (int64_t)v.size();
  return AGMM_OK;
}

namespace {

// The tables that the current device's scratch holds, by the (descriptor, CU count) they
// were planned for, so that repeated calls with one shape upload them once.
struct StaticTables {
  bool valid;
  agmm_desc desc;
  int num_cus;
  // A run was captured on this device: its graph rewrites the tables whenever it replays, so
  // from then on every run uploads its own tables instead of trusting the cache.
  bool captured;
};
std::mutex g_static_mu;
StaticTables g_static_tables[64];

bool same_desc(const agmm_desc& a, const agmm_desc& b) { return memcmp(&a, &b, sizeof(a)) == 0; }

}  // namespace

int ag_matmul_run_static(const agmm_desc* desc, const void* const* shards, const void* B,
                         const void* bias, void* out, void* hip_stream) {
  int rc = validate_desc(desc);
  if (rc != AGMM_OK) return rc;
  // (a fetch kernel would need a stream of its own, which this entry point cannot create)
  if (desc->algo == AGMM_ALGO_PIPELINED || desc->gather_a || desc->debug || desc->tail_split ||
      desc->debug_fetch_delay || desc->debug_fetch_reverse || desc->fetch_kernel == 1)
    return AGMM_ERR_UNSUPPORTED;
  int dev = 0;
  AGMM_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64) return AGMM_ERR_WRONG_DEVICE;
  int num_cus = 0;
  AGMM_HIP(hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, dev));
  Plan pl;
  rc = make_plan(*desc, num_cus, &pl);
  if (rc != AGMM_OK) return rc;
  if (pl.total > (int64_t)agmm::kScratchBytes) return AGMM_ERR_TOO_LARGE;
  int per_cu = 0;
  AGMM_HIP(agmm::fused_occupancy(desc->dtype, pl.cfg.block_m, &per_cu));
  if (per_cu < 1) return AGMM_ERR_UNSUPPORTED;
  void* base = nullptr;
  AGMM_HIP(agmm::scratch_region(dev, &base));

  // A handle on the host stack, its workspace the scratch; it allocates nothing (the
  // vectors are host memory) and it has no host status word.
  agmm_handle h{};
  init_handle(&h, *desc, pl, dev);
  h.ws = static_cast<char*>(base);
  h.own_ws = false;
  h.host_status = nullptr;
  carve_workspace(&h, pl);
  hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
  // Flags, counters (the run counter too) and split counters start at zero: one fill kernel
  // (not a memset, which a captured graph would record as a memset node). The run is then
  // epoch 1.
  AGMM_HIP(agmm::launch_fill32(reinterpret_cast<uint32_t*>(h.ws + pl.off_flags),
                               (pl.off_units - pl.off_flags) / 4, 0u, s));
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  AGMM_HIP(hipStreamIsCapturing(s, &cs));
  {
    std::lock_guard<std::mutex> lock(g_static_mu);
    StaticTables& t = g_static_tables[dev];
    if (cs != hipStreamCaptureStatusNone) t.captured = true;
    if (t.captured || !(t.valid && t.num_cus == num_cus && same_desc(t.desc, *desc))) {
      t.valid = false;
      AGMM_HIP(agmm::launch_upload32(h.units, pl.units.data(), (int64_t)pl.units.size(), s));
      AGMM_HIP(agmm::launch_upload32(h.mtiles, pl.mtiles.data(), (int64_t)pl.mtiles.size(), s));
      AGMM_HIP(agmm::launch_upload32(h.qtiles, pl.qtiles.data(), (int64_t)pl.qtiles.size(), s));
      t.valid = true;
      t.desc = *desc;
      t.num_cus = num_cus;
    }
  }
  return run_impl(&h, shards, B, bias, out, false, nullptr, hip_stream);
}

int ag_matmul_debug_mfma_loop(int dtype, int vary, int grid, int iters, float* sink,
                              void* hip_stream) {
  if (dtype != AGMM_F16 && dtype != AGMM_BF16) return AGMM_ERR_INVALID_ARG;
  if (!sink || grid <= 0 || iters <= 0 || (iters & 3) || (vary & ~1)) return AGMM_ERR_INVALID_ARG;
  AGMM_HIP(agmm::launch_mfma_loop(dtype, vary != 0, grid, iters, sink,
                                  reinterpret_cast<hipStream_t>(hip_stream)));
  return AGMM_OK;
}

int ag_matmul_debug_set_runs(agmm_handle* h, uint32_t runs, void* hip_stream) {
  if (!h || h->desc.algo == AGMM_ALGO_PIPELINED || (h->ar_D && !h->ar_flags_mode))
    return AGMM_ERR_INVALID_ARG;
  if (h->poisoned) return AGMM_ERR_POISONED;
  int cur = 0;
  AGMM_HIP(hipGetDevice(&cur));
  if (cur != h->cfg.device) return AGMM_ERR_WRONG_DEVICE;
  hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
  // the state `runs` runs leave: every flag at the last run's epoch (the per-tile flag
  // variant stores it, the fetch adds one per run), every split counter at pieces per run,
  // and the run counter
  if (h->ar_flags_mode) {
    AGMM_HIP(agmm::launch_fill32(h->ar_flags, h->ar_flags_n, runs, s));
  } else {
    AGMM_HIP(agmm::launch_fill32(h->flags, h->flags_n, runs, s));
    AGMM_HIP(agmm::launch_fill32(h->split_cnt, h->cfg.split_tiles,
                                 runs * (uint32_t)h->cfg.split_pieces, s));
  }
  AGMM_HIP(agmm::launch_fill32(h->ctr + agmm::CTR_RUNS, 1, runs, s));
  return AGMM_OK;
}

int ag_matmul_debug_fill_staging(agmm_handle* h, uint16_t pattern, void* hip_stream) {
  if (!h) return AGMM_ERR_INVALID_ARG;
  int cur = 0;
  AGMM_HIP(hipGetDevice(&cur));
  if (cur != h->cfg.device) return AGMM_ERR_WRONG_DEVICE;
  AGMM_HIP(agmm::launch_fill16(h->staging, h->cfg.staging_elems, pattern,
                               reinterpret_cast<hipStream_t>(hip_stream)));
  return AGMM_OK;
}

}  // extern "C"
