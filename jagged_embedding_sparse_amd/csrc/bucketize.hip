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
// q, j) order. Items are cut into tiles of 4096 tokens that never straddle a
// (rank, table) segment and are numbered in (r, t, chunk) order, so an
// item's output position is its shard's base, plus the shard's count in all
// earlier tiles, plus its stable rank inside its tile:
//   k_prep     balanced offsets, per-sample shifts, tile descriptors (one
//              workgroup of 256 threads)
//   k_hist     per-tile shard histograms -> rows of a tiles x shards matrix;
//              each item's 32-bit key, batch-major
//   k_colsum, k_colscan   exclusive column scans of that matrix in place,
//              with coalesced row loads (lanes = shards)
//   k_splits   shard offsets; splits[d][r] as differences of the scanned
//              matrix at rank boundaries (transposed through LDS)
//   k_scatter  per tile: the keys back, stable ranks (LDS lane masks), sort
//              by shard in LDS, one contiguous run per shard.
// Consecutive tiles run on the same XCD (workgroups are dealt to the 8 XCDs
// round-robin), so the short runs that neighbouring tiles of one segment
// write next to each other meet in one L2. No device-scope atomics.
#include "common.hpp"
#include "colscan.hpp"
#include "divu32.hpp"

namespace fs {
namespace {

constexpr int kThreads = 256;  // 4 waves
constexpr int kRounds = 16;    // items per lane
constexpr int kWaveItems = kWave * kRounds;
constexpr int kTile = kThreads * kRounds;  // 4096 tokens per tile

struct TableRows {
  int64_t rows[FS_MAX_TABLES];
  int64_t row_base[FS_MAX_TABLES];
  int64_t block[FS_MAX_TABLES];  // ceil(rows / W)
  DivU32 div[FS_MAX_TABLES];     // division by block
};

constexpr uint32_t kDropKey = 0xFFFFFFFFu;  // item key of a dropped ID (keys < 2^32 - 1)

struct TileDesc {
  int64_t bm_lo;       // first batch-major token
  int32_t n;           // tokens (<= kTile)
  int32_t seg;         // r * T + t
  int32_t q_lo, q_hi;  // rank r's balanced samples
  int32_t pad[2];
};

// ---------------------------------------------------------------- prep
// One workgroup of 256 threads (larger ones wait for free slots while another
// stream's kernels hold the CUs). Thread i owns balanced samples
// [64 i, 64 i + 64) and ranks 4 i .. 4 i + 3.
constexpr int kPrepThreads = 256;
constexpr int kPrepPer = FS_MAX_SAMPLES / kPrepThreads;       // samples per thread
constexpr int kPrepRanks = (FS_MAX_RANKS + 1) / kPrepThreads;  // ranks per thread (+ W)
constexpr int kPrepUnroll = 8;  // offset validation: loads in flight per thread
constexpr int kPrepBatch = 16;  // samples whose loads are in flight together

// Validation, bal_offsets, shift[q] = so[perm[q]] - bal[q], the tile table.
// Invalid input (offsets not rising from 0 to n_tok, a perm entry out of
// range, rank offsets not rising from 0 to n, or lengths under perm not
// summing to n_tok) flags FS_EF_SHAPE and leaves zero tiles, so nothing is
// written past the outputs.
__global__ void __launch_bounds__(kPrepThreads)
k_prep(const int64_t* __restrict__ so, int32_t n, int64_t n_tok, const int32_t* __restrict__ perm,
       const int32_t* __restrict__ ro, int32_t W, int32_t T, int64_t* __restrict__ bal,
       int64_t* __restrict__ shift, int32_t* __restrict__ tile_pref, TileDesc* __restrict__ tiles,
       int32_t* __restrict__ err) {
  __shared__ int64_t tmp64[17];
  __shared__ int32_t tmp32[17];
  __shared__ int bad_s;
  if (threadIdx.x == 0) bad_s = 0;
  bool bad = false;
  for (int32_t s0 = threadIdx.x; s0 <= n; s0 += kPrepThreads * kPrepUnroll) {
#pragma unroll
    for (int k = 0; k < kPrepUnroll; ++k) {
      const int32_t s = s0 + k * kPrepThreads;
      if (s <= n) {
        const int64_t v = so[s];
        if ((s == 0 && v != 0) || (s == n && v != n_tok) || (s < n && so[s + 1] < v)) bad = true;
      }
    }
  }
  // lengths of the thread's balanced samples, 16 at a time (perm loads, then
  // offset loads, each batch in flight together; few registers, so that the
  // workgroup fits beside another stream's kernels)
  const int32_t q0 = threadIdx.x * kPrepPer;
  int64_t local = 0;
  for (int k0 = 0; k0 < kPrepPer; k0 += kPrepBatch) {
    int32_t pp[kPrepBatch];
#pragma unroll
    for (int k = 0; k < kPrepBatch; ++k) pp[k] = q0 + k0 + k < n ? perm[q0 + k0 + k] : -1;
#pragma unroll
    for (int k = 0; k < kPrepBatch; ++k) {
      const bool pin = pp[k] >= 0 && pp[k] < n;
      if (q0 + k0 + k < n && !pin) bad = true;
      if (pin) local += so[pp[k] + 1] - so[pp[k]];
    }
  }
  int32_t ro_v[kPrepRanks + 1];
#pragma unroll
  for (int k = 0; k <= kPrepRanks; ++k) {
    const int32_t r = threadIdx.x * kPrepRanks + k;
    ro_v[k] = r <= W ? ro[r] : n;
    if (r <= W && ((r == 0 && ro_v[k] != 0) || (r == W && ro_v[k] != n))) bad = true;
    if (k > 0 && r <= W && ro_v[k] < ro_v[k - 1]) bad = true;
  }
  __syncthreads();
  if (bad) atomicOr(&bad_s, 1);
  __syncthreads();
  bool ok = bad_s == 0;
  int64_t total;
  int64_t run = block_excl_scan<int64_t>(ok ? local : 0, tmp64, &total);
  ok = ok && total == n_tok;  // perm repeats a sample: refuse before any tile exists
  if (!ok && threadIdx.x == 0 && err) atomicOr(err, FS_EF_SHAPE);
  if (ok) {
    for (int k0 = 0; k0 < kPrepPer && q0 + k0 < n; k0 += kPrepBatch) {
      int32_t pp[kPrepBatch];
      int64_t b0[kPrepBatch], b1[kPrepBatch];
#pragma unroll
      for (int k = 0; k < kPrepBatch; ++k) pp[k] = q0 + k0 + k < n ? perm[q0 + k0 + k] : 0;
#pragma unroll
      for (int k = 0; k < kPrepBatch; ++k) {
        b0[k] = so[pp[k]];
        b1[k] = so[pp[k] + 1];
      }
#pragma unroll
      for (int k = 0; k < kPrepBatch; ++k) {
        const int32_t q = q0 + k0 + k;
        if (q < n) {
          bal[q] = run;
          shift[q] = b0[k] - run;
          run += b1[k] - b0[k];
        }
      }
    }
  }
  if (threadIdx.x == 0) bal[n] = ok ? total : 0;
  __syncthreads();  // bal visible to the workgroup

  // rank r owns T * ceil(m_r / kTile) tiles, t-major
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
      A[k] = bal[ro_v[k]];
      m[k] = bal[ro_v[k + 1]] - A[k];
      c[k] = (int32_t)cdiv(m[k], kTile);
    }
    mine += T * c[k];
  }
  int32_t ttot;
  int32_t pref = block_excl_scan<int32_t>(mine, tmp32, &ttot);
  if (threadIdx.x == 0) tile_pref[W] = ttot;
#pragma unroll
  for (int k = 0; k < kPrepRanks; ++k) {
    const int32_t r = threadIdx.x * kPrepRanks + k;
    if (r < W) tile_pref[r] = pref;
    for (int32_t t = 0; t < T; ++t)
      for (int32_t kk = 0; kk < c[k]; ++kk) {
        TileDesc d;
        d.bm_lo = A[k] + (int64_t)kk * kTile;
        d.n = (int32_t)min((int64_t)kTile, m[k] - (int64_t)kk * kTile);
        d.seg = r * T + t;
        d.q_lo = ro_v[k];
        d.q_hi = ro_v[k + 1];
        d.pad[0] = d.pad[1] = 0;
        tiles[pref + t * c[k] + kk] = d;
      }
    pref += T * c[k];
  }
}

// ---------------------------------------------------------------- tiles
struct TileInfo {
  int32_t r, t;
  int64_t bm_lo, bm_hi;  // this tile's batch-major token range
  int32_t q_lo, q_hi;    // rank r's balanced samples
};

__device__ __forceinline__ bool tile_info(int32_t tile, const int32_t* tile_pref, int32_t W,
                                          int32_t T, const TileDesc* tiles, TileInfo& ti) {
  if (tile >= tile_pref[W]) return false;
  const TileDesc d = tiles[tile];
  ti.r = d.seg / T;
  ti.t = d.seg % T;
  ti.bm_lo = d.bm_lo;
  ti.bm_hi = d.bm_lo + d.n;
  ti.q_lo = d.q_lo;
  ti.q_hi = d.q_hi;
  return true;
}

// Loads one wave's 16 rounds of 64 consecutive tokens of a tile (table t,
// batch-major positions bm) and returns, per round and lane, the item's key
// and bin (shard, -1 for a dropped ID, `sentinel` past the tile's end).
//
// The wave finds the balanced sample of its first token with one cooperative
// search, then loads a window of 64 samples: their end offsets and shifts
// from batch-major to original token index. A lane finds its token's sample
// in the window by binary lifting over the window with shuffles; the window
// restarts at each round's first sample, and a lane whose token lies past
// the window (only possible with runs of empty samples) walks forward on its
// own. All 16 ID loads are independent.
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

__device__ __forceinline__ void wave_items(const TileInfo& ti, int32_t w, const int64_t* ids,
                                           const int64_t* shift, const int64_t* bal,
                                           int64_t n_tok, const TableRows& tr, int32_t sentinel,
                                           uint32_t (&key)[kRounds], int32_t (&bin)[kRounds]) {
  const int64_t first = ti.bm_lo + (int64_t)w * kWaveItems;
#pragma unroll
  for (int i = 0; i < kRounds; ++i) {
    key[i] = 0;
    bin[i] = sentinel;
  }
  if (first >= ti.bm_hi) return;
  // sample of the first token: one past the last q in (q_lo, q_hi) with bal[q] <= first
  const int32_t qa = (int32_t)wave_partition_point(
      ti.q_lo + 1, ti.q_hi, [&](int64_t q) { return bal[q] <= first; }) - 1;
  Window win = load_window(qa, ti.q_hi, bal, shift);
  const int t = ti.t;
  const int64_t rows = tr.rows[t], rbase = tr.row_base[t];
  const DivU32 div = tr.div[t];
  int64_t tok[kRounds];
  bool valid[kRounds];
#pragma unroll
  for (int i = 0; i < kRounds; ++i) {
    const int64_t rb = first + i * kWave;  // the round's first token
    if (rb < ti.bm_hi) {
      // restart the window at the round's first sample (a round of 64
      // tokens then spans at most the window, unless samples are empty)
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
    const int64_t id = ids[(int64_t)t * n_tok + tok[i]];
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
  if (tile_info(tile, tile_pref, W, T, tiles, ti)) {
    const int32_t sentinel = (1 << nbits) - 1;  // > W: lanes without an item
    const int32_t w = threadIdx.x / kWave;
    uint32_t key[kRounds];
    int32_t bin[kRounds];
    wave_items(ti, w, ids, shift, bal, n_tok, tr, sentinel, key, bin);
    uint32_t* out = ikey + (int64_t)ti.t * n_tok + ti.bm_lo + (int64_t)w * kWaveItems + lane();
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

// ---------------------------------------------------------------- splits
// Workgroup (x, y): ranks [64x, 64x + 64) x shards [64y, 64y + 64) of
// splits[d][r] = (scanned count of shard d at rank r + 1's first tile) -
// (at rank r's first tile); rows past the matrix read the column totals.
// Workgroup (0, 0) also writes shard_offsets = exclusive scan of the totals
// (entry W: the valid items; dropped IDs follow it).
__global__ void __launch_bounds__(kThreads)
k_splits(const uint32_t* __restrict__ counts, int32_t ld, int32_t G,
         const int32_t* __restrict__ tile_pref, const uint32_t* __restrict__ tot, int32_t W,
         int64_t* __restrict__ splits, int64_t* __restrict__ shard_offsets) {
  __shared__ int64_t tr_[kWave][kWave + 1];
  __shared__ int64_t tmp[17];
  const int w = threadIdx.x / kWave, l = lane();
  if (blockIdx.x == 0 && blockIdx.y == 0) {
    constexpr int kPer = (FS_MAX_RANKS + 1 + kThreads - 1) / kThreads;
    uint32_t v[kPer];
    int64_t local = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int b = threadIdx.x * kPer + k;
      v[k] = b <= W ? tot[b] : 0u;
      local += v[k];
    }
    int64_t all;
    int64_t base = block_excl_scan<int64_t>(local, tmp, &all);
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int b = threadIdx.x * kPer + k;
      if (b <= W) shard_offsets[b] = base;
      base += v[k];
    }
  }
  const int32_t d = blockIdx.y * kWave + l;
  for (int rl = w; rl < kWave; rl += kThreads / kWave) {
    const int32_t r = blockIdx.x * kWave + rl;
    int64_t val = 0;
    if (r < W && d < W) {
      const int32_t a = tile_pref[r], z = tile_pref[r + 1];
      const uint32_t va = a < G ? counts[(int64_t)a * ld + d] : tot[d];
      const uint32_t vz = z < G ? counts[(int64_t)z * ld + d] : tot[d];
      val = (int64_t)vz - (int64_t)va;
    }
    tr_[rl][l] = val;
  }
  __syncthreads();
  const int32_t r = blockIdx.x * kWave + l;
  for (int dl = w; dl < kWave; dl += kThreads / kWave) {
    const int32_t dd = blockIdx.y * kWave + dl;
    if (r < W && dd < W) splits[(int64_t)dd * W + r] = tr_[l][dl];
  }
}

// ---------------------------------------------------------------- scatter
// Staging area of one tile: first the per-wave lane-mask tables of the
// ranking, then the tile's items sorted by shard.
union ScatterStage {
  uint64_t peers[kThreads / kWave][FS_MAX_RANKS + 1];
  struct {
    uint32_t key[kTile];
    int32_t bm[kTile];
    uint16_t bin[kTile];
  } s;
};

__global__ void __launch_bounds__(kThreads)
k_scatter(const uint32_t* __restrict__ ikey, int64_t n_tok, const int32_t* __restrict__ tile_pref,
          const TileDesc* __restrict__ tiles, TableRows tr, int32_t W, int32_t T, int32_t nbits,
          const uint32_t* __restrict__ offs, int32_t ld, const int64_t* __restrict__ shard_offsets,
          int64_t* __restrict__ shard_keys, int32_t* __restrict__ shard_bm) {
  __shared__ uint16_t cnt[kThreads / kWave][FS_MAX_RANKS + 1];
  __shared__ uint32_t run[FS_MAX_RANKS + 1];   // output position of each shard's run
  __shared__ uint32_t tbin[FS_MAX_RANKS + 1];  // start of each shard in the sorted tile
  __shared__ ScatterStage st;
  __shared__ int64_t tmp[17];
  constexpr int kPer = (FS_MAX_RANKS + 1 + kThreads - 1) / kThreads;
  const int32_t tile = xcd_tile(blockIdx.x, gridDim.x);
  TileInfo ti;
  if (!tile_info(tile, tile_pref, W, T, tiles, ti)) return;  // uniform per workgroup
  const int32_t nb = W + 1;
  const int32_t w = threadIdx.x / kWave;
  for (int b = threadIdx.x; b < nb; b += kThreads)
    run[b] = (uint32_t)(shard_offsets[b] + offs[(int64_t)tile * ld + b]);
  for (int b = lane(); b < nb; b += kWave) {
    cnt[w][b] = 0;
    st.peers[w][b] = 0;
  }
  const int32_t sentinel = (1 << nbits) - 1;  // > W: lanes without an item
  const int t = ti.t;
  const uint32_t rbase = (uint32_t)tr.row_base[t];
  const DivU32 div = tr.div[t];
  const int64_t first = ti.bm_lo + (int64_t)w * kWaveItems;
  const uint32_t* in = ikey + (int64_t)t * n_tok + first + lane();
  uint32_t key[kRounds];
  int32_t bin[kRounds];
#pragma unroll
  for (int i = 0; i < kRounds; ++i) {
    const bool valid = first + i * kWave + lane() < ti.bm_hi;
    key[i] = valid ? in[i * kWave] : 0u;
    bin[i] = !valid ? sentinel : key[i] == kDropKey ? W : (int32_t)divu32(key[i] - rbase, div);
  }
  // stable rank of each item among the wave's items of its shard
  const uint64_t lt = lanemask_lt();
  int32_t rk[kRounds];
#pragma unroll
  for (int i = 0; i < kRounds; ++i) {
    const int32_t b = bin[i];
    const bool on = b != sentinel;
    const uint64_t peers = lds_peers(st.peers[w], (uint32_t)(on ? b : 0), on);
    const uint32_t before = cnt[w][on ? b : 0];
    rk[i] = (int32_t)before + popc(peers & lt);
    if (on && (peers & lt) == 0) cnt[w][b] = (uint16_t)(before + (uint32_t)popc(peers));
  }
  __syncthreads();
  // per shard: exclusive prefix over the waves, then the shards' starts in the tile
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
          const uint32_t c = cnt[x][b];
          cnt[x][b] = (uint16_t)r;
          r += c;
        }
      }
      tb[k] = r;
      local += r;
    }
    int64_t all;
    int64_t r0 = block_excl_scan<int64_t>(local, tmp, &all);
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int b = threadIdx.x * kPer + k;
      if (b < nb) tbin[b] = (uint32_t)r0;
      r0 += tb[k];
    }
  }
  __syncthreads();  // also ends every wave's use of the mask tables
#pragma unroll
  for (int i = 0; i < kRounds; ++i) {
    const int32_t b = bin[i];
    if (b == sentinel) continue;
    const uint32_t p = tbin[b] + cnt[w][b] + (uint32_t)rk[i];
    st.s.key[p] = key[i];
    st.s.bm[p] = (int32_t)(first + i * kWave + lane());
    st.s.bin[p] = (uint16_t)b;
  }
  __syncthreads();
  const int m = (int)(ti.bm_hi - ti.bm_lo);
  for (int p = threadIdx.x; p < m; p += kThreads) {
    const int b = st.s.bin[p];
    const int64_t pos = (int64_t)run[b] + (p - (int)tbin[b]);
    shard_keys[pos] = (int64_t)st.s.key[p];
    shard_bm[pos] = st.s.bm[p];
  }
}

// tiles the launches cover: an upper bound on sum_r T * ceil(m_r / 4096),
// rounded up to a multiple of the XCD count
int32_t grid_tiles(int64_t n_tok, int32_t T, int32_t W) {
  return (int32_t)align_up((size_t)(T * (cdiv(n_tok, kTile) + W)), kXcd);
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
  int nbits = 1;
  while ((1 << nbits) - 1 <= W) ++nbits;  // sentinel (2^nbits - 1) > W
  const dim3 split_grid((unsigned)cdiv(W, kWave), (unsigned)cdiv(W, kWave));

  hipLaunchKernelGGL(k_prep, dim3(1), dim3(kPrepThreads), 0, stream, sample_offsets, n, n_tok,
                     perm, rank_offsets, W, T, bal_offsets, shift, tile_pref, tiles, err);
  FS_LAUNCH_CHECK();
  hipLaunchKernelGGL(k_hist, dim3(G), dim3(kThreads), 0, stream, ids, n_tok, shift, bal_offsets,
                     tile_pref, tiles, tr, W, T, nbits, counts, ld, ikey, err);
  FS_LAUNCH_CHECK();
  int rc = launch_colscan(counts, ld, G, W + 1, part, tot, stream);
  if (rc) return rc;
  hipLaunchKernelGGL(k_splits, split_grid, dim3(kThreads), 0, stream, counts, ld, G, tile_pref,
                     tot, W, splits, shard_offsets);
  FS_LAUNCH_CHECK();
  hipLaunchKernelGGL(k_scatter, dim3(G), dim3(kThreads), 0, stream, ikey, n_tok, tile_pref,
                     tiles, tr, W, T, nbits, counts, ld, shard_offsets, shard_keys, shard_bm);
  FS_LAUNCH_CHECK();
  return FS_OK;
}
