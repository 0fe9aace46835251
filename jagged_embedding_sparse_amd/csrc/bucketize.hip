// Indexed permute + ranged dispatch: balanced batch -> shard-major buffers.
//
// "FreeScale: distributed training for sequence recommendation models",
// section 4.2: the indexed-permute kernel applies the partition to the
// gathered IDs and the ranged-dispatch kernel lays them out per destination
// for the ID AllToAll; section 3.2 defines the batch-major and shard-major
// forms. One GPU produces every virtual rank's send buffers at once.
//
// The shard-major order (shard d, source rank r, table t, balanced sample q,
// token j) is a stable counting sort by d of the items enumerated in (r, t,
// q, j) order. Each (rank, table) segment is cut into chunks of 512 tokens,
// one per wave; a tile is four consecutive chunks of one rank (several tables
// share a tile when their segments are short), numbered in (r, t, chunk)
// order, so an item's output position is its shard's base, plus the shard's
// count in all earlier tiles, plus its stable rank inside its tile:
//   k_lens, k_bal, k_tiles (or k_prep1)   balanced offsets, per-sample
//              shifts, tile descriptors (short dependent-load chains)
//   k_hist     per-tile shard histograms -> rows of a tiles x shards matrix;
//              each item's 32-bit key, batch-major
//   k_colsum, k_colscan   exclusive column scans of that matrix in place,
//              with coalesced row loads (lanes = shards)
//   k_scatter  per tile: shard bases from the totals, the keys back, stable
//              ranks (LDS lane masks), sort by shard in LDS, one contiguous
//              run per shard; extra workgroups of the same launch write the
//              shard offsets and splits[d][r] (differences of the scanned
//              matrix at rank boundaries, transposed through LDS).
// Consecutive tiles run on the same XCD (workgroups are dealt to the 8 XCDs
// round-robin), so the short runs that neighbouring tiles of one segment
// write next to each other meet in one L2. No device-scope atomics.
#include "common.hpp"
#include "colscan.hpp"
#include "divu32.hpp"

namespace fs {
namespace {

constexpr int kThreads = 256;  // 4 waves
// items per lane: 8 keeps the tile kernels' register counts low enough (42
// and 78) to share SIMDs with the update kernels of the other stream
constexpr int kRounds = 8;
constexpr int kWaveItems = kWave * kRounds;
constexpr int kTile = kThreads * kRounds;  // 2048 tokens per tile

struct TableRows {
  int64_t rows[FS_MAX_TABLES];
  int64_t row_base[FS_MAX_TABLES];
  int64_t block[FS_MAX_TABLES];  // ceil(rows / W)
  DivU32 div[FS_MAX_TABLES];     // division by block
};

constexpr uint32_t kDropKey = 0xFFFFFFFFu;  // item key of a dropped ID (keys < 2^32 - 1)

constexpr int kTileWaves = kThreads / kWave;
// one-launch column scan up to this many tile rows: the scan stops at the
// tiles in use, which several tables leave well below the launch bound
constexpr int32_t kColOneRowsUsed = 1536;

// A tile: one chunk of at most kWaveItems tokens per wave, all of one rank.
struct TileDesc {
  int64_t bm_lo[kTileWaves];  // each chunk's first batch-major token
  int32_t n[kTileWaves];      // each chunk's tokens (0: the wave has none)
  int32_t t[kTileWaves];      // each chunk's table
  int32_t q0[kTileWaves];     // the sample of each chunk's first token, or -1: unknown
  int32_t q_lo, q_hi;         // the rank's balanced samples
};

// ---------------------------------------------------------------- prep
// Three launches, each with short chains of dependent loads (the index path
// runs beside the bandwidth-bound update of another stream, where every
// dependent round trip to memory waits in deep queues); batches of up to
// 2048 samples take one workgroup for all three (k_prep1):
//   k_lens   one thread per balanced sample: its length and first token
//            under perm, validation of perm and the sample offsets, per
//            workgroup sums and flags
//   k_bal    one thread per balanced sample: bal_offsets and shift from the
//            workgroup sums and a workgroup scan
//   k_tiles  one workgroup: rank offsets validated, the tile table
// Invalid input (offsets not rising from 0 to n_tok, a perm entry out of
// range, rank offsets not rising from 0 to n, or lengths under perm not
// summing to n_tok) flags FS_EF_SHAPE and leaves zero tiles, so nothing is
// written past the outputs.
constexpr int kPrepThreads = 256;
constexpr int kPrepRanks = (FS_MAX_RANKS + 1) / kPrepThreads;  // ranks per thread (+ W)
constexpr int kMaxLenBlocks = FS_MAX_SAMPLES / kPrepThreads + 1;

__global__ void __launch_bounds__(kPrepThreads)
k_lens(const int64_t* __restrict__ so, int32_t n, int64_t n_tok, const int32_t* __restrict__ perm,
       int32_t* __restrict__ lens, int32_t* __restrict__ begs, int64_t* __restrict__ bsum,
       int32_t* __restrict__ flags) {
  __shared__ int64_t tmp64[17];
  const int32_t q = blockIdx.x * kPrepThreads + threadIdx.x;
  bool bad = false;
  int64_t len = 0;
  if (q < n) {
    const int32_t p = perm[q];
    const bool pin = p >= 0 && p < n;
    bad |= !pin;
    const int64_t b0 = pin ? so[p] : 0, b1 = pin ? so[p + 1] : 0;
    len = b1 - b0;
    lens[q] = (int32_t)len;  // offsets fit 32 bits (T * n_tok < 2^31)
    begs[q] = (int32_t)b0;
  }
  if (q <= n) {
    const int64_t v = so[q];
    if ((q == 0 && v != 0) || (q == n && v != n_tok) || (q < n && so[q + 1] < v)) bad = true;
  }
  int64_t tot;
  (void)block_excl_scan<int64_t>(len, tmp64, &tot);
  const int any = __syncthreads_or(bad ? 1 : 0);
  if (threadIdx.x == 0) {
    bsum[blockIdx.x] = tot;
    flags[blockIdx.x] = any;
  }
}

__global__ void __launch_bounds__(kPrepThreads)
k_bal(int32_t n, const int32_t* __restrict__ lens, const int32_t* __restrict__ begs,
      const int64_t* __restrict__ bsum, int64_t* __restrict__ bal, int64_t* __restrict__ shift) {
  __shared__ int64_t tmp64[17];
  __shared__ int64_t base_s;
  const int32_t q = blockIdx.x * kPrepThreads + threadIdx.x;
  const int32_t len = q < n ? lens[q] : 0;
  const int32_t beg = q < n ? begs[q] : 0;
  if (threadIdx.x < kWave) {  // sums of the earlier workgroups (at most 65)
    int64_t x = 0;
    for (int32_t k = threadIdx.x; k < (int32_t)blockIdx.x; k += kWave) x += bsum[k];
    x = wave_sum(x);
    if (threadIdx.x == 0) base_s = x;
  }
  int64_t tot;
  const int64_t ex = block_excl_scan<int64_t>(len, tmp64, &tot);  // barriers publish base_s
  if (q < n) {
    const int64_t b = base_s + ex;
    bal[q] = b;
    shift[q] = (int64_t)beg - b;
  }
}

// The tile table (one workgroup): rank offsets validated, ranks' token
// ranges from bal, tiles per rank and their descriptors. `part` is this
// thread's share of the token count and `bad` the result of its input checks; bal
// holds the balanced offsets of samples 0..n-1 (bal[n] is written here).
// With a copy of bal[0..n] in LDS (bal_lds), each chunk's first sample is
// found here by an LDS search and stored, so the tile kernels need not
// search bal in memory.
__device__ __forceinline__ void tile_table(int32_t n, int64_t n_tok, bool bad, int64_t part,
                                           const int32_t* __restrict__ ro, int32_t W, int32_t T,
                                           int64_t* __restrict__ bal, const int64_t* bal_lds,
                                           int32_t* __restrict__ tile_pref,
                                           TileDesc* __restrict__ tiles, int32_t* __restrict__ err) {
  __shared__ int64_t tmp64[17];
  __shared__ int32_t tmp32[17];
  __shared__ int64_t s_A[FS_MAX_RANKS], s_m[FS_MAX_RANKS];
  __shared__ int32_t s_pref[FS_MAX_RANKS + 1], s_q[FS_MAX_RANKS + 1];
  int32_t ro_v[kPrepRanks + 1];
#pragma unroll
  for (int k = 0; k <= kPrepRanks; ++k) {
    const int32_t r = threadIdx.x * kPrepRanks + k;
    ro_v[k] = r <= W ? ro[r] : n;
    if (r <= W && ((r == 0 && ro_v[k] != 0) || (r == W && ro_v[k] != n))) bad = true;
    if (k > 0 && r <= W && ro_v[k] < ro_v[k - 1]) bad = true;
    if (r <= W && (ro_v[k] < 0 || ro_v[k] > n)) bad = true;
  }
  int64_t total;
  (void)block_excl_scan<int64_t>(part, tmp64, &total);
  const bool ok = !__syncthreads_or(bad ? 1 : 0) && total == n_tok;
  if (threadIdx.x == 0) {
    bal[n] = ok ? total : 0;
    if (!ok && err) atomicOr(err, FS_EF_SHAPE);
  }
  // rank r's T segments of m_r tokens make T * ceil(m_r / kWaveItems)
  // chunks, t-major, and ceil(chunks / 4) tiles (bal[n] is read only through
  // ranks that end at n, where it equals total)
  int64_t A[kPrepRanks], m[kPrepRanks];
  int32_t c[kPrepRanks];
  int32_t mine = 0;
#pragma unroll
  for (int k = 0; k < kPrepRanks; ++k) {
    const int32_t r = threadIdx.x * kPrepRanks + k;
    A[k] = 0;
    m[k] = 0;
    c[k] = 0;
    if (ok && r < W) {
      A[k] = ro_v[k] < n ? bal[ro_v[k]] : total;
      m[k] = (ro_v[k + 1] < n ? bal[ro_v[k + 1]] : total) - A[k];
      c[k] = (int32_t)cdiv((int64_t)T * cdiv(m[k], kWaveItems), kTileWaves);
    }
    mine += c[k];
  }
  int32_t ttot;
  int32_t pref = block_excl_scan<int32_t>(mine, tmp32, &ttot);
  if (threadIdx.x == 0) {
    tile_pref[W] = ttot;
    s_pref[W] = ttot;
  }
#pragma unroll
  for (int k = 0; k < kPrepRanks; ++k) {
    const int32_t r = threadIdx.x * kPrepRanks + k;
    if (r < W) {
      tile_pref[r] = pref;
      s_pref[r] = pref;
      s_A[r] = A[k];
      s_m[r] = m[k];
      s_q[r] = ro_v[k];
      if (r == W - 1) s_q[W] = ro_v[k + 1];
    }
    pref += c[k];
  }
  __syncthreads();
  // the tile table, all threads over all tiles: tile u belongs to the last
  // rank r with s_pref[r] <= u (ranks without tokens share their first tile)
  for (int32_t u = threadIdx.x; u < ttot; u += kPrepThreads) {
    int32_t a = 0, b = W;  // s_pref[0] = 0 <= u < ttot = s_pref[W]
    while (b - a > 1) {
      const int32_t mid = (a + b) >> 1;
      if (s_pref[mid] <= u) a = mid; else b = mid;
    }
    // rank a owns tile u (it has tokens): chunk c of the rank is chunk
    // c % cpt of table c / cpt
    const int32_t cpt = (int32_t)cdiv(s_m[a], kWaveItems);
    const int32_t i = u - s_pref[a];
    TileDesc d;
#pragma unroll
    for (int w = 0; w < kTileWaves; ++w) {
      const int32_t ch = i * kTileWaves + w;
      const int32_t t = ch / cpt, kk = ch % cpt;
      const bool on = t < T;
      d.bm_lo[w] = s_A[a] + (on ? (int64_t)kk * kWaveItems : 0);
      d.n[w] = on ? (int32_t)min((int64_t)kWaveItems, s_m[a] - (int64_t)kk * kWaveItems) : 0;
      d.t[w] = on ? t : 0;
      d.q0[w] = -1;
      if (bal_lds && on) {
        // the last sample q in [q_lo, q_hi) with bal[q] <= the chunk's first token
        int32_t lo = s_q[a], hi = s_q[a + 1];  // bal[lo] <= first < bal[hi]
        while (hi - lo > 1) {
          const int32_t mid = (lo + hi) >> 1;
          if (bal_lds[mid] <= d.bm_lo[w]) lo = mid; else hi = mid;
        }
        d.q0[w] = lo;
      }
    }
    d.q_lo = s_q[a];
    d.q_hi = s_q[a + 1];
    tiles[u] = d;
  }
}

__global__ void __launch_bounds__(kPrepThreads)
k_tiles(int32_t n, int64_t n_tok, int32_t n_len_blocks, const int64_t* __restrict__ bsum,
        const int32_t* __restrict__ flags, const int32_t* __restrict__ ro, int32_t W, int32_t T,
        int64_t* __restrict__ bal, int32_t* __restrict__ tile_pref,
        TileDesc* __restrict__ tiles, int32_t* __restrict__ err) {
  bool bad = false;
  int64_t part = 0;
  for (int32_t k = threadIdx.x; k < n_len_blocks; k += kPrepThreads) {
    bad |= flags[k] != 0;
    part += bsum[k];
  }
  tile_table(n, n_tok, bad, part, ro, W, T, bal, nullptr, tile_pref, tiles, err);
}

// Batches of at most kPrepThreads * P samples: the three prep steps in one
// workgroup (each launch on the index path waits for wave slots beside the
// update, so two fewer launches save more than the one workgroup costs).
// Thread i owns samples iP .. iP + P - 1: their lengths and first tokens under
// perm (all loads in flight), then bal and shift from one workgroup scan.
template <int P>
__global__ void __launch_bounds__(kPrepThreads)
k_prep1(const int64_t* __restrict__ so, int32_t n, int64_t n_tok,
        const int32_t* __restrict__ perm, const int32_t* __restrict__ ro, int32_t W, int32_t T,
        int64_t* __restrict__ bal, int64_t* __restrict__ shift, int32_t* __restrict__ tile_pref,
        TileDesc* __restrict__ tiles, int32_t* __restrict__ err) {
  __shared__ int64_t tmp[17];
  __shared__ int64_t s_bal[kPrepThreads * P + 1];
  const int32_t q0 = threadIdx.x * P;
  bool bad = false;
  int32_t pv[P];
#pragma unroll
  for (int k = 0; k < P; ++k) pv[k] = q0 + k < n ? perm[q0 + k] : 0;
  int64_t beg[P], len[P];
#pragma unroll
  for (int k = 0; k < P; ++k) {
    const bool on = q0 + k < n;
    const bool pin = pv[k] >= 0 && pv[k] < n;
    bad |= on && !pin;
    beg[k] = (on && pin) ? so[pv[k]] : 0;
    len[k] = (on && pin) ? so[pv[k] + 1] - beg[k] : 0;
  }
  // the sample offsets rise from 0 to n_tok: this thread checks so[q0 .. q0 + P]
  int64_t sv[P + 1];
#pragma unroll
  for (int k = 0; k <= P; ++k) sv[k] = q0 + k <= n ? so[q0 + k] : 0;
#pragma unroll
  for (int k = 0; k <= P; ++k) {
    const int32_t q = q0 + k;
    if (q <= n && ((q == 0 && sv[k] != 0) || (q == n && sv[k] != n_tok))) bad = true;
    if (k < P && q < n && sv[k + 1] < sv[k]) bad = true;
  }
  int64_t local = 0;
#pragma unroll
  for (int k = 0; k < P; ++k) local += len[k];
  int64_t tot;
  int64_t b = block_excl_scan<int64_t>(local, tmp, &tot);
#pragma unroll
  for (int k = 0; k < P; ++k) {
    if (q0 + k < n) {
      bal[q0 + k] = b;
      shift[q0 + k] = beg[k] - b;
      s_bal[q0 + k] = b;
    }
    b += len[k];
  }
  if (threadIdx.x == kPrepThreads - 1) s_bal[n] = b;  // the last thread's b is the total
  __syncthreads();  // bal of every sample visible to the workgroup
  tile_table(n, n_tok, bad, local, ro, W, T, bal, s_bal, tile_pref, tiles, err);
}

// ---------------------------------------------------------------- tiles
// One wave's chunk of a tile.
struct TileInfo {
  int32_t t;
  int64_t bm_lo, bm_hi;  // the chunk's batch-major token range (table t)
  int32_t q_lo, q_hi;    // the rank's balanced samples
  int32_t q0;            // the sample of the chunk's first token, or -1
};

__device__ __forceinline__ bool tile_info(int32_t tile, int w, const int32_t* tile_pref,
                                          int32_t W, const TileDesc* tiles, TileInfo& ti) {
  if (tile >= tile_pref[W]) return false;
  const TileDesc& d = tiles[tile];
  ti.t = d.t[w];
  ti.bm_lo = d.bm_lo[w];
  ti.bm_hi = d.bm_lo[w] + d.n[w];
  ti.q_lo = d.q_lo;
  ti.q_hi = d.q_hi;
  ti.q0 = d.q0[w];
  return true;
}

// Loads one wave's kRounds rounds of 64 consecutive tokens of its chunk
// (table t, batch-major positions bm) and returns, per round and lane, the
// item's key and bin (shard, -1 for a dropped ID, `sentinel` past the
// chunk's end).
//
// The wave finds the balanced sample of its first token with one cooperative
// search, then loads a window of 64 samples: their end offsets and shifts
// from batch-major to original token index. A lane finds its token's sample
// in the window by binary lifting over the window with shuffles; the window
// restarts at a round's first sample only when the round reaches past it, and
// a lane whose token still lies past the window (only possible with runs of
// empty samples) walks forward on its own. All the ID loads are independent.
struct Window {
  int32_t qa;     // first sample of the window
  int64_t bnd;    // this lane: end offset of sample qa + lane (INT64_MAX past q_hi)
  int64_t shift;  // this lane: shift[qa + lane]
};

__device__ __forceinline__ Window load_window(int32_t qa, int32_t q_hi, const int64_t* bal,
                                              const int64_t* shift) {
  Window win;
  win.qa = qa;
  const int32_t q = qa + lane();
  win.bnd = INT64_MAX;
  win.shift = 0;
  if (q < q_hi) {
    win.bnd = bal[q + 1];
    win.shift = shift[q];
  }
  return win;
}

__device__ __forceinline__ void wave_items(const TileInfo& ti, const int64_t* ids,
                                           const int64_t* shift, const int64_t* bal,
                                           int64_t n_tok, const TableRows& tr, int32_t sentinel,
                                           uint32_t (&key)[kRounds], int32_t (&bin)[kRounds]) {
  const int64_t first = ti.bm_lo;
#pragma unroll
  for (int i = 0; i < kRounds; ++i) {
    key[i] = 0;
    bin[i] = sentinel;
  }
  if (first >= ti.bm_hi) return;
  // sample of the first token: one past the last q in (q_lo, q_hi) with
  // bal[q] <= first (stored in the tile table when it was known there)
  const int32_t qa = ti.q0 >= 0 ? ti.q0
                                : (int32_t)wave_partition_point(
                                      ti.q_lo + 1, ti.q_hi,
                                      [&](int64_t q) { return bal[q] <= first; }) - 1;
  Window win = load_window(qa, ti.q_hi, bal, shift);
  const int t = ti.t;
  const int64_t rows = tr.rows[t], rbase = tr.row_base[t];
  const DivU32 div = tr.div[t];
  int64_t tok[kRounds];
  bool valid[kRounds];
#pragma unroll
  for (int i = 0; i < kRounds; ++i) {
    const int64_t rb = first + i * kWave;  // the round's first token
    if (rb < ti.bm_hi && __shfl(win.bnd, kWave - 1, kWave) <= rb + kWave - 1) {
      // the round reaches past the window: restart it at the round's first
      // sample (64 tokens then span at most the window, unless samples are
      // empty)
      const int kf = popc(__ballot(win.bnd <= rb));
      if (kf > 0) win = load_window(win.qa + kf, ti.q_hi, bal, shift);
    }
    const int64_t bm = rb + lane();
    valid[i] = bm < ti.bm_hi;
    int pos = 0;  // window samples ending at or before bm (binary lifting)
#pragma unroll
    for (int step = kWave / 2; step >= 1; step >>= 1) {
      const int64_t v = __shfl(win.bnd, pos + step - 1, kWave);
      if (v <= bm) pos += step;
    }
    const int64_t last = __shfl(win.bnd, kWave - 1, kWave);
    if (pos == kWave - 1 && last <= bm) pos = kWave;
    int64_t sh = __shfl(win.shift, pos < kWave ? pos : 0, kWave);
    if (valid[i] && pos >= kWave) {  // past the window: walk (rare)
      int32_t q = win.qa + kWave - 1;
      while (q + 1 < ti.q_hi && bal[q + 1] <= bm) ++q;
      sh = shift[q];
    }
    tok[i] = bm + sh;
  }
#pragma unroll
  for (int i = 0; i < kRounds; ++i) {
    if (!valid[i]) continue;
    // read once (streaming load: keeps the sample tables in the caches)
    const int64_t id = __builtin_nontemporal_load(ids + (int64_t)t * n_tok + tok[i]);
    const bool in = id >= 0 && id < rows;
    key[i] = (uint32_t)(rbase + id);
    bin[i] = in ? (int32_t)divu32((uint32_t)id, div) : -1;
  }
}

// ---------------------------------------------------------------- histogram
// One row of the tiles x shards count matrix per tile (zeros for unused
// tiles); column W counts dropped IDs. Also stores every item's 32-bit key
// (kDropKey for a dropped ID) at ikey[t * n_tok + bm], so the scatter reads
// its tile's items back coalesced instead of walking the samples again.
__global__ void __launch_bounds__(kThreads)
k_hist(const int64_t* __restrict__ ids, int64_t n_tok, const int64_t* __restrict__ shift,
       const int64_t* __restrict__ bal, const int32_t* __restrict__ tile_pref,
       const TileDesc* __restrict__ tiles, TableRows tr, int32_t W, int32_t T, int32_t nbits,
       uint32_t* __restrict__ counts, int32_t ld, uint32_t* __restrict__ ikey,
       int32_t* __restrict__ err) {
  __shared__ uint32_t h[FS_MAX_RANKS + 1];
  const int32_t tile = xcd_tile(blockIdx.x, gridDim.x);
  for (int b = threadIdx.x; b <= W; b += kThreads) h[b] = 0;
  __syncthreads();
  TileInfo ti;
  // the wave index made provably uniform: the chunk's fields load into scalar registers
  if (tile_info(tile, __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), tile_pref, W, tiles,
                ti)) {
    const int32_t sentinel = (1 << nbits) - 1;  // > W: lanes without an item
    uint32_t key[kRounds];
    int32_t bin[kRounds];
    wave_items(ti, ids, shift, bal, n_tok, tr, sentinel, key, bin);
    uint32_t* out = ikey + (int64_t)ti.t * n_tok + ti.bm_lo + lane();
    bool dropped_any = false;
#pragma unroll
    for (int i = 0; i < kRounds; ++i) {
      const int32_t b = bin[i];
      if (b == sentinel) continue;
      dropped_any |= b < 0;
      atomicAdd(&h[b < 0 ? W : b], 1u);
      out[i * kWave] = b < 0 ? kDropKey : key[i];
    }
    flag_err(err, dropped_any, FS_EF_ID_RANGE);
  }
  __syncthreads();
  for (int b = threadIdx.x; b <= W; b += kThreads) counts[(int64_t)tile * ld + b] = h[b];
}

// ---------------------------------------------------------------- scatter
// LDS of one workgroup, sized for nb = W + 1 bins at launch (the bins in use,
// not the call limit, so more workgroups fit on a CU): per-wave shard counts,
// each shard's output position and start in the sorted tile, then a staging
// area that holds, in turn, the per-wave lane-mask tables of the ranking and
// the tile's items sorted by shard -- or, for a splits workgroup, a 64 x 64
// transpose.
struct ScatterLds {
  uint16_t* cnt;    // [4][nbp]
  uint32_t* run;    // [nbp]
  uint32_t* tbin;   // [nbp]
  uint64_t* peers;  // [4][nb]  (staging)
  uint32_t* skey;   // [kTile]  (staging)
  int32_t* sbm;     // [kTile]  (staging)
  uint16_t* sbin;   // [kTile]  (staging)
  int32_t* tr;      // [64][65] (staging)
};

__host__ __device__ __forceinline__ size_t scatter_lds_bytes(int32_t nb, ScatterLds* l,
                                                              char* base) {
  const size_t nbp = align_up((size_t)nb, 8);
  const size_t nw = kThreads / kWave;
  size_t off = 0;
  const size_t o_cnt = off;
  off += align_up(nw * nbp * sizeof(uint16_t), 16);
  const size_t o_run = off;
  off += nbp * sizeof(uint32_t);
  const size_t o_tbin = off;
  off += nbp * sizeof(uint32_t);
  const size_t o_stage = off;
  const size_t peers = nw * (size_t)nb * sizeof(uint64_t);
  const size_t items = (size_t)kTile * (sizeof(uint32_t) + sizeof(int32_t) + sizeof(uint16_t));
  const size_t trans = (size_t)kWave * (kWave + 1) * sizeof(int32_t);
  size_t stage = peers > items ? peers : items;
  stage = stage > trans ? stage : trans;
  off += stage;
  if (l) {
    l->cnt = (uint16_t*)(base + o_cnt);
    l->run = (uint32_t*)(base + o_run);
    l->tbin = (uint32_t*)(base + o_tbin);
    l->peers = (uint64_t*)(base + o_stage);
    l->skey = (uint32_t*)(base + o_stage);
    l->sbm = (int32_t*)(base + o_stage + kTile * sizeof(uint32_t));
    l->sbin = (uint16_t*)(base + o_stage + kTile * (sizeof(uint32_t) + sizeof(int32_t)));
    l->tr = (int32_t*)(base + o_stage);
  }
  return off;
}

constexpr int kBinPer = (FS_MAX_RANKS + 1 + kThreads - 1) / kThreads;

// base[b] = exclusive scan of the bin totals (start of bin b in the output)
__device__ __forceinline__ void bin_bases(const uint32_t* tot, int32_t W, int64_t* tmp,
                                          int64_t (&base)[kBinPer]) {
  uint32_t v[kBinPer];
  int64_t local = 0;
#pragma unroll
  for (int k = 0; k < kBinPer; ++k) {
    const int b = threadIdx.x * kBinPer + k;
    v[k] = b <= W ? tot[b] : 0u;
    local += v[k];
  }
  int64_t all;
  int64_t x = block_excl_scan<int64_t>(local, tmp, &all);
#pragma unroll
  for (int k = 0; k < kBinPer; ++k) {
    base[k] = x;
    x += v[k];
  }
}

// Splits workgroup (x, y): ranks [64x, 64x + 64) x shards [64y, 64y + 64) of
// splits[d][r] = (scanned count of shard d at rank r + 1's first tile) -
// (at rank r's first tile); rows past the tiles in use read the column
// totals.
// Workgroup (0, 0) also writes shard_offsets (entry W: the valid items;
// dropped IDs follow it).
__device__ __forceinline__ void splits_part(int32_t x, int32_t y, const uint32_t* counts,
                                            int32_t ld, int32_t G, const int32_t* tile_pref,
                                            const uint32_t* tot, int32_t W, int64_t* splits,
                                            int64_t* shard_offsets, int32_t* tr, int64_t* tmp) {
  const int w = threadIdx.x / kWave, l = lane();
  if (x == 0 && y == 0) {
    int64_t base[kBinPer];
    bin_bases(tot, W, tmp, base);
#pragma unroll
    for (int k = 0; k < kBinPer; ++k) {
      const int b = threadIdx.x * kBinPer + k;
      if (b <= W) shard_offsets[b] = base[k];
    }
  }
  const int32_t d = y * kWave + l;
  const int32_t used = min(G, tile_pref[W]);  // the column scan rewrote only these rows
  for (int rl = w; rl < kWave; rl += kThreads / kWave) {
    const int32_t r = x * kWave + rl;
    int32_t val = 0;  // items of one rank for one shard: fewer than 2^31
    if (r < W && d < W) {
      const int32_t a = tile_pref[r], z = tile_pref[r + 1];
      const uint32_t va = a < used ? counts[(int64_t)a * ld + d] : tot[d];
      const uint32_t vz = z < used ? counts[(int64_t)z * ld + d] : tot[d];
      val = (int32_t)(vz - va);
    }
    tr[rl * (kWave + 1) + l] = val;
  }
  __syncthreads();
  const int32_t r = x * kWave + l;
  for (int dl = w; dl < kWave; dl += kThreads / kWave) {
    const int32_t dd = y * kWave + dl;
    if (r < W && dd < W) splits[(int64_t)dd * W + r] = (int64_t)tr[l * (kWave + 1) + dl];
  }
}

// Workgroups [0, G): tiles (XCD order); [G, G + splits workgroups): splits.
__global__ void __launch_bounds__(kThreads)
k_scatter(const uint32_t* __restrict__ ikey, int64_t n_tok, const int32_t* __restrict__ tile_pref,
          const TileDesc* __restrict__ tiles, TableRows tr, int32_t W, int32_t T, int32_t nbits,
          const uint32_t* __restrict__ offs, int32_t ld, int32_t G,
          const uint32_t* __restrict__ tot, int64_t* __restrict__ splits,
          int64_t* __restrict__ shard_offsets, int64_t* __restrict__ shard_keys,
          int32_t* __restrict__ shard_bm) {
  extern __shared__ __align__(16) char lds_dyn[];
  __shared__ int64_t tmp[17];
  constexpr int kPer = kBinPer;
  ScatterLds L;
  (void)scatter_lds_bytes(W + 1, &L, lds_dyn);
  const int32_t nbp = (int32_t)align_up((size_t)W + 1, 8);
  if ((int32_t)blockIdx.x >= G) {
    const int32_t sb = blockIdx.x - G, nx = (int32_t)cdiv(W, kWave);
    splits_part(sb % nx, sb / nx, offs, ld, G, tile_pref, tot, W, splits, shard_offsets, L.tr,
                tmp);
    return;
  }
  const int32_t tile = xcd_tile(blockIdx.x, G);
  const int32_t w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // provably uniform
  TileInfo ti;
  if (!tile_info(tile, w, tile_pref, W, tiles, ti)) return;  // uniform per workgroup
  const int32_t nb = W + 1;
  {
    int64_t base[kBinPer];
    bin_bases(tot, W, tmp, base);
#pragma unroll
    for (int k = 0; k < kBinPer; ++k) {
      const int b = threadIdx.x * kBinPer + k;
      if (b < nb) L.run[b] = (uint32_t)(base[k] + offs[(int64_t)tile * ld + b]);
    }
  }
  uint16_t* cnt_w = L.cnt + w * nbp;
  uint64_t* peers_w = L.peers + (int64_t)w * nb;
  for (int b = lane(); b < nb; b += kWave) {
    cnt_w[b] = 0;
    peers_w[b] = 0;
  }
  const int32_t sentinel = (1 << nbits) - 1;  // > W: lanes without an item
  const int t = ti.t;
  const uint32_t rbase = (uint32_t)tr.row_base[t];
  const DivU32 div = tr.div[t];
  const int64_t first = ti.bm_lo;
  const uint32_t* in = ikey + (int64_t)t * n_tok + first + lane();
  uint32_t key[kRounds];
  int32_t bin[kRounds];
#pragma unroll
  for (int i = 0; i < kRounds; ++i) {
    const bool valid = first + i * kWave + lane() < ti.bm_hi;
    key[i] = valid ? __builtin_nontemporal_load(in + i * kWave) : 0u;  // last read
    bin[i] = !valid ? sentinel : key[i] == kDropKey ? W : (int32_t)divu32(key[i] - rbase, div);
  }
  // stable rank of each item among the wave's items of its shard
  const uint64_t lt = lanemask_lt();
  int32_t rk[kRounds];
#pragma unroll
  for (int i = 0; i < kRounds; ++i) {
    const int32_t b = bin[i];
    const bool on = b != sentinel;
    const uint64_t peers = lds_peers(peers_w, (uint32_t)(on ? b : 0), on);
    const uint32_t before = cnt_w[on ? b : 0];
    rk[i] = (int32_t)before + popc(peers & lt);
    if (on && (peers & lt) == 0) cnt_w[b] = (uint16_t)(before + (uint32_t)popc(peers));
  }
  __syncthreads();
  // per shard: exclusive prefix over the waves, then the shards' starts in the tile
  int m;  // the tile's items
  {
    uint32_t tb[kPer];
    int64_t local = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int b = threadIdx.x * kPer + k;
      uint32_t r = 0;
      if (b < nb) {
#pragma unroll
        for (int x = 0; x < kThreads / kWave; ++x) {
          const uint32_t c = L.cnt[x * nbp + b];
          L.cnt[x * nbp + b] = (uint16_t)r;
          r += c;
        }
      }
      tb[k] = r;
      local += r;
    }
    int64_t all;
    int64_t r0 = block_excl_scan<int64_t>(local, tmp, &all);
    m = (int)all;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int b = threadIdx.x * kPer + k;
      if (b < nb) L.tbin[b] = (uint32_t)r0;
      r0 += tb[k];
    }
  }
  __syncthreads();  // also ends every wave's use of the mask tables
#pragma unroll
  for (int i = 0; i < kRounds; ++i) {
    const int32_t b = bin[i];
    if (b == sentinel) continue;
    const uint32_t p = L.tbin[b] + cnt_w[b] + (uint32_t)rk[i];
    L.skey[p] = key[i];
    L.sbm[p] = (int32_t)(first + i * kWave + lane());
    L.sbin[p] = (uint16_t)b;
  }
  __syncthreads();
  for (int p = threadIdx.x; p < m; p += kThreads) {
    const int b = L.sbin[p];
    const int64_t pos = (int64_t)L.run[b] + (p - (int)L.tbin[b]);
    shard_keys[pos] = (int64_t)L.skey[p];
    shard_bm[pos] = L.sbm[p];
  }
}

// tiles the launches cover: sum_r ceil(T * ceil(m_r / 512) / 4) with
// sum_r m_r = n_tok is at most (T * n_tok + W * (511 T + 1536)) / 2048,
// rounded up to a multiple of the XCD count
int32_t grid_tiles(int64_t n_tok, int32_t T, int32_t W) {
  const int64_t b = ((int64_t)T * n_tok +
                     (int64_t)W * ((kWaveItems - 1) * T + (kTileWaves - 1) * kWaveItems)) /
                    ((int64_t)kTileWaves * kWaveItems);
  return (int32_t)align_up((size_t)(b > 0 ? b : 1), kXcd);
}

}  // namespace
}  // namespace fs

using namespace fs;

extern "C" size_t fs_bucketize_workspace_size(int64_t n_tok, int32_t n, int32_t T, int32_t W) {
  const int64_t G = grid_tiles(n_tok > 0 ? n_tok : 0, T, W);
  const int64_t ld = (int64_t)align_up((size_t)W + 1, kWave);
  Carve c(nullptr);
  c.take<int64_t>((size_t)(n > 0 ? n : 1));                 // shift
  c.take<int32_t>((size_t)W + 1);                           // tile_pref
  c.take<TileDesc>((size_t)G);                              // tiles
  c.take<uint32_t>((size_t)(G * ld));                       // counts, then offsets
  c.take<uint32_t>((size_t)(cdiv(G, kColBlockRows) * ld));  // column partials
  c.take<uint32_t>((size_t)ld);                             // column totals
  c.take<uint32_t>((size_t)(T * (n_tok > 0 ? n_tok : 1)));  // item keys, batch-major
  c.take<int32_t>((size_t)(n > 0 ? n : 1));                 // lengths under perm
  c.take<int32_t>((size_t)(n > 0 ? n : 1));                 // first tokens under perm
  c.take<int64_t>((size_t)kMaxLenBlocks);                   // per-workgroup length sums
  c.take<int32_t>((size_t)kMaxLenBlocks);                   // per-workgroup input flags
  return c.used + 256;
}

extern "C" int fs_bucketize_permute(const int64_t* ids, int64_t n_tok,
                                    const int64_t* sample_offsets, int32_t n,
                                    const fs_table* tables, int32_t T, const int32_t* perm,
                                    const int32_t* rank_offsets, int32_t W, int64_t* bal_offsets,
                                    int64_t* shard_keys, int32_t* shard_bm, int64_t* splits,
                                    int64_t* shard_offsets, int32_t* err, void* ws,
                                    size_t ws_bytes, hipStream_t stream) {
  if (n < 0 || n > FS_MAX_SAMPLES || W < 1 || W > FS_MAX_RANKS || T < 1 || T > FS_MAX_TABLES ||
      n_tok < 0 || (int64_t)T * n_tok >= (int64_t)INT32_MAX)
    return FS_ERR_INVALID_ARG;
  if (!tables || !sample_offsets || !rank_offsets || !bal_offsets || !splits || !shard_offsets)
    return FS_ERR_INVALID_ARG;
  if (n > 0 && !perm) return FS_ERR_INVALID_ARG;
  if (n_tok > 0 && (!ids || !shard_keys || !shard_bm)) return FS_ERR_INVALID_ARG;
  TableRows tr;
  int64_t base = 0;
  for (int t = 0; t < T; ++t) {
    if (tables[t].rows < 1) return FS_ERR_INVALID_ARG;
    tr.rows[t] = tables[t].rows;
    tr.row_base[t] = base;
    tr.block[t] = cdiv(tables[t].rows, W);
    base += tables[t].rows;
    if (base <= (int64_t)UINT32_MAX) tr.div[t] = make_divu32((uint32_t)tr.block[t]);
  }
  if (base > (int64_t)UINT32_MAX) return FS_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < fs_bucketize_workspace_size(n_tok, n, T, W)) return FS_ERR_WORKSPACE;
  const int32_t G = grid_tiles(n_tok, T, W);
  const int32_t ld = (int32_t)align_up((size_t)W + 1, kWave);
  Carve c(ws);
  int64_t* shift = c.take<int64_t>((size_t)(n > 0 ? n : 1));
  int32_t* tile_pref = c.take<int32_t>((size_t)W + 1);
  TileDesc* tiles = c.take<TileDesc>((size_t)G);
  uint32_t* counts = c.take<uint32_t>((size_t)G * ld);
  uint32_t* part = c.take<uint32_t>((size_t)cdiv(G, kColBlockRows) * ld);
  uint32_t* tot = c.take<uint32_t>((size_t)ld);
  uint32_t* ikey = c.take<uint32_t>((size_t)(T * (n_tok > 0 ? n_tok : 1)));
  int32_t* lens = c.take<int32_t>((size_t)(n > 0 ? n : 1));
  int32_t* begs = c.take<int32_t>((size_t)(n > 0 ? n : 1));
  int64_t* bsum = c.take<int64_t>((size_t)kMaxLenBlocks);
  int32_t* flags = c.take<int32_t>((size_t)kMaxLenBlocks);
  int nbits = 1;
  while ((1 << nbits) - 1 <= W) ++nbits;  // sentinel (2^nbits - 1) > W
  const int32_t n_len_blocks = (int32_t)cdiv(n + 1, kPrepThreads);  // <= kMaxLenBlocks
  const int32_t split_blocks = (int32_t)(cdiv(W, kWave) * cdiv(W, kWave));

  if (n <= kPrepThreads * 4) {
    hipLaunchKernelGGL(k_prep1<4>, dim3(1), dim3(kPrepThreads), 0, stream, sample_offsets, n,
                       n_tok, perm, rank_offsets, W, T, bal_offsets, shift, tile_pref, tiles, err);
    FS_LAUNCH_CHECK();
  } else if (n <= kPrepThreads * 8) {
    hipLaunchKernelGGL(k_prep1<8>, dim3(1), dim3(kPrepThreads), 0, stream, sample_offsets, n,
                       n_tok, perm, rank_offsets, W, T, bal_offsets, shift, tile_pref, tiles, err);
    FS_LAUNCH_CHECK();
  } else {
    hipLaunchKernelGGL(k_lens, dim3(n_len_blocks), dim3(kPrepThreads), 0, stream,
                       sample_offsets, n, n_tok, perm, lens, begs, bsum, flags);
    FS_LAUNCH_CHECK();
    hipLaunchKernelGGL(k_bal, dim3((unsigned)cdiv(n, kPrepThreads)), dim3(kPrepThreads), 0,
                       stream, n, lens, begs, bsum, bal_offsets, shift);
    FS_LAUNCH_CHECK();
    hipLaunchKernelGGL(k_tiles, dim3(1), dim3(kPrepThreads), 0, stream, n, n_tok, n_len_blocks,
                       bsum, flags, rank_offsets, W, T, bal_offsets, tile_pref, tiles, err);
    FS_LAUNCH_CHECK();
  }
  hipLaunchKernelGGL(k_hist, dim3(G), dim3(kThreads), 0, stream, ids, n_tok, shift, bal_offsets,
                     tile_pref, tiles, tr, W, T, nbits, counts, ld, ikey, err);
  FS_LAUNCH_CHECK();
  // rows past the tiles in use (tile_pref[W], known on the device) stay zero
  int rc = launch_colscan(counts, ld, G, W + 1, part, tot, stream, tile_pref + W,
                          kColOneRowsUsed);
  if (rc) return rc;
  const size_t lds = scatter_lds_bytes(W + 1, nullptr, nullptr);
  hipLaunchKernelGGL(k_scatter, dim3((unsigned)(G + split_blocks)), dim3(kThreads), lds, stream,
                     ikey, n_tok, tile_pref, tiles, tr, W, T, nbits, counts, ld, G, tot, splits,
                     shard_offsets, shard_keys, shard_bm);
  FS_LAUNCH_CHECK();
  return FS_OK;
}
