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
// q, j) order. Items are cut into tiles of 4096 that never straddle an (r, t)
// segment, so:
//   * every tile knows its rank and table without a search per item,
//   * splits[d][r] is a difference of the per-shard tile-count prefix sums.
// Four launches: prep (balanced offsets + tile table), per-tile histograms,
// per-shard column scans (+ splits, shard totals), stable per-tile scatter
// staged through LDS (+ shard offsets). No device-scope atomics.
#include "common.hpp"

namespace fs {
namespace {

constexpr int kThreads = 256;  // 4 waves
constexpr int kRounds = 16;    // items per lane
constexpr int kWaveItems = kWave * kRounds;
constexpr int kTile = kThreads * kRounds;  // 4096

struct TableRows {
  int64_t rows[FS_MAX_TABLES];
  int64_t row_base[FS_MAX_TABLES];
  int64_t block[FS_MAX_TABLES];  // ceil(rows / W)
};

// ---------------------------------------------------------------- prep
// bal_offsets, input validation, tile table.
__global__ void __launch_bounds__(1024)
k_prep(const int64_t* __restrict__ so, int32_t n, int64_t n_tok, const int32_t* __restrict__ perm,
       const int32_t* __restrict__ ro, int32_t W, int32_t T, int64_t* __restrict__ bal,
       int32_t* __restrict__ tile_pref, int32_t* __restrict__ err) {
  __shared__ int64_t tmp64[17];
  __shared__ int32_t tmp32[17];
  __shared__ int bad_s;
  if (threadIdx.x == 0) bad_s = 0;
  __syncthreads();
  bool bad = false;
  // validate offsets and the partition
  for (int32_t s = threadIdx.x; s <= n; s += blockDim.x) {
    int64_t v = so[s];
    if (s == 0 && v != 0) bad = true;
    if (s == n && v != n_tok) bad = true;
    if (s < n && so[s + 1] < v) bad = true;
  }
  for (int32_t q = threadIdx.x; q < n; q += blockDim.x) {
    int32_t p = perm[q];
    if (p < 0 || p >= n) bad = true;
  }
  for (int32_t r = threadIdx.x; r <= W; r += blockDim.x) {
    int32_t v = ro[r];
    if ((r == 0 && v != 0) || (r == W && v != n) || (r < W && ro[r + 1] < v)) bad = true;
  }
  if (bad) atomicOr(&bad_s, 1);
  __syncthreads();
  const bool ok = bad_s == 0;
  if (!ok && threadIdx.x == 0 && err) atomicOr(err, FS_EF_SHAPE);

  // balanced offsets: per-thread contiguous slices, then a block scan
  const int32_t per = (n + blockDim.x - 1) / blockDim.x;
  const int32_t q0 = min(n, (int32_t)threadIdx.x * per), q1 = min(n, q0 + per);
  int64_t local = 0;
  for (int32_t q = q0; q < q1; ++q) {
    int32_t s = perm[q];
    if (ok) local += so[s + 1] - so[s];
  }
  int64_t total;
  int64_t run = block_excl_scan<int64_t>(local, tmp64, &total);
  for (int32_t q = q0; q < q1; ++q) {
    bal[q] = run;
    int32_t s = perm[q];
    if (ok) run += so[s + 1] - so[s];
  }
  if (threadIdx.x == 0) bal[n] = total;
  __syncthreads();

  // tile table: rank r owns T * ceil(m_r / kTile) tiles (t-major)
  int32_t r = threadIdx.x;  // W <= 1024 = blockDim.x
  int32_t my_tiles = 0;
  if (ok && r < W) {
    int64_t m = bal[ro[r + 1]] - bal[ro[r]];
    my_tiles = (int32_t)(T * cdiv(m, kTile));
  }
  int32_t ttot;
  int32_t pref = block_excl_scan<int32_t>(my_tiles, tmp32, &ttot);
  if (r < W) tile_pref[r] = pref;
  if (threadIdx.x == 0) tile_pref[W] = ttot;
}

// ---------------------------------------------------------------- tiles
struct TileInfo {
  int32_t r, t;
  int64_t bm_lo, bm_hi;  // this tile's batch-major token range
  int32_t q_lo, q_hi;    // rank r's balanced samples
};

__device__ __forceinline__ bool tile_info(int32_t tile, const int32_t* tile_pref, int32_t W,
                                          int32_t T, const int64_t* bal, const int32_t* ro,
                                          TileInfo& ti) {
  if (tile >= tile_pref[W]) return false;
  int32_t lo = 0, hi = W;  // largest r with tile_pref[r] <= tile
  while (hi - lo > 1) {
    int32_t mid = (lo + hi) >> 1;
    if (tile_pref[mid] <= tile) lo = mid; else hi = mid;
  }
  const int32_t r = lo;
  const int32_t per_t = (tile_pref[r + 1] - tile_pref[r]) / T;
  const int32_t local = tile - tile_pref[r];
  ti.r = r;
  ti.t = local / per_t;
  const int32_t k = local % per_t;
  ti.q_lo = ro[r];
  ti.q_hi = ro[r + 1];
  const int64_t A = bal[ti.q_lo], B = bal[ti.q_hi];
  ti.bm_lo = A + (int64_t)k * kTile;
  ti.bm_hi = min(B, ti.bm_lo + kTile);
  return true;
}

// Loads one wave's 16 rounds of 64 consecutive tokens of a tile (table t,
// batch-major positions bm) and returns, per round and lane, the item's key
// and bin (shard, -1 for a dropped ID, `sentinel` past the tile's end).
//
// The wave finds the balanced sample of its first token with one cooperative
// search, then loads a window of 64 samples: their end offsets and the shift
// from batch-major to original token index (so[perm[q]] - bal[q]). A lane
// finds its token's sample in the window by binary lifting over the window
// with shuffles; the window restarts at each round's first sample, and a lane
// whose token lies past the window (only possible with runs of empty
// samples) walks forward on its own. All 16 ID loads are independent.
struct Window {
  int32_t qa;    // first sample of the window
  int64_t bnd;   // this lane: end offset of sample qa + lane (INT64_MAX past q_hi)
  int64_t shift; // this lane: so[perm[q]] - bal[q] for q = qa + lane
};

__device__ __forceinline__ Window load_window(int32_t qa, int32_t q_hi, const int64_t* bal,
                                              const int32_t* perm, const int64_t* so) {
  Window win;
  win.qa = qa;
  const int32_t q = qa + lane();
  win.bnd = INT64_MAX;
  win.shift = 0;
  if (q < q_hi) {
    win.bnd = bal[q + 1];
    win.shift = so[perm[q]] - bal[q];
  }
  return win;
}

__device__ __forceinline__ void wave_items(const TileInfo& ti, int32_t w, const int64_t* ids,
                                           const int64_t* so, const int32_t* perm,
                                           const int64_t* bal, int64_t n_tok,
                                           const TableRows& tr, int32_t sentinel,
                                           int64_t (&key)[kRounds], int32_t (&bin)[kRounds]) {
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
  Window win = load_window(qa, ti.q_hi, bal, perm, so);
  const int t = ti.t;
  const int64_t rows = tr.rows[t], rbase = tr.row_base[t], block = tr.block[t];
  int64_t tok[kRounds];
  bool valid[kRounds];
#pragma unroll
  for (int i = 0; i < kRounds; ++i) {
    const int64_t rb = first + i * kWave;  // the round's first token
    if (rb < ti.bm_hi) {
      // restart the window at the round's first sample (a round of 64
      // tokens then spans at most the window, unless samples are empty)
      const int kf = popc(__ballot(win.bnd <= rb));
      if (kf > 0) win = load_window(win.qa + kf, ti.q_hi, bal, perm, so);
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
      sh = so[perm[q]] - bal[q];
    }
    tok[i] = bm + sh;
  }
#pragma unroll
  for (int i = 0; i < kRounds; ++i) {
    if (!valid[i]) continue;
    const int64_t id = ids[(int64_t)t * n_tok + tok[i]];
    const bool in = id >= 0 && id < rows;
    key[i] = rbase + id;
    bin[i] = in ? (int32_t)(id / block) : -1;
  }
}

// ---------------------------------------------------------------- histogram
__global__ void __launch_bounds__(kThreads)
k_hist(const int64_t* __restrict__ ids, int64_t n_tok, const int64_t* __restrict__ so,
       const int32_t* __restrict__ perm, const int32_t* __restrict__ ro,
       const int64_t* __restrict__ bal, const int32_t* __restrict__ tile_pref, TableRows tr,
       int32_t W, int32_t T, int64_t tiles_cap, uint32_t* __restrict__ hist,
       int32_t* __restrict__ err) {
  __shared__ uint32_t h[FS_MAX_RANKS + 1];
  TileInfo ti;
  const int32_t tile = blockIdx.x;
  if (!tile_info(tile, tile_pref, W, T, bal, ro, ti)) return;
  for (int b = threadIdx.x; b <= W; b += kThreads) h[b] = 0;
  __syncthreads();
  const int32_t w = threadIdx.x / kWave;
  int64_t key[kRounds];
  int32_t bin[kRounds];
  wave_items(ti, w, ids, so, perm, bal, n_tok, tr, W + 1, key, bin);
  bool dropped_any = false;
  int nbits = 1;
  while ((1 << nbits) - 1 <= W + 1) ++nbits;
  const uint64_t lt = lanemask_lt();
#pragma unroll
  for (int i = 0; i < kRounds; ++i) {
    int32_t b = bin[i];
    if (b < 0) {
      b = W;
      dropped_any = true;
    }
    // one LDS add per distinct shard of the round (hot rows share a shard)
    const uint64_t peers = match_bits((uint32_t)b, nbits);
    if (b != W + 1 && (peers & lt) == 0) atomicAdd(&h[b], (uint32_t)popc(peers));
  }
  flag_err(err, dropped_any, FS_EF_ID_RANGE);
  __syncthreads();
  for (int b = threadIdx.x; b <= W; b += kThreads) hist[(int64_t)b * tiles_cap + tile] = h[b];
}

// ---------------------------------------------------------------- column scan
// One workgroup per bin b (shard d = b, or b == W for dropped items): the
// bin's tile counts become exclusive offsets within the bin, in place; the
// bin total goes to tot[b]; splits[b][r] sums rank r's tiles (the tiles of a
// rank are contiguous). The bins' global bases are formed by the scatter.
__global__ void __launch_bounds__(kThreads)
k_scan(const int32_t* __restrict__ tile_pref, int32_t W, int64_t tiles_cap,
       uint32_t* __restrict__ hist, uint32_t* __restrict__ tot, int64_t* __restrict__ splits) {
  __shared__ int64_t tmp[17];
  const int32_t b = blockIdx.x;
  const int32_t n_tiles = tile_pref[W];
  uint32_t* col = hist + (int64_t)b * tiles_cap;
  int64_t carry = 0;
  for (int32_t c0 = 0; c0 < n_tiles; c0 += kThreads) {
    const int32_t c = c0 + threadIdx.x;
    const int64_t v = c < n_tiles ? col[c] : 0;
    int64_t sum;
    const int64_t ex = block_excl_scan<int64_t>(v, tmp, &sum);
    if (c < n_tiles) col[c] = (uint32_t)(carry + ex);
    carry += sum;
  }
  __syncthreads();
  if (threadIdx.x == 0) tot[b] = (uint32_t)carry;
  if (b < W) {
    for (int32_t r = threadIdx.x; r < W; r += kThreads) {
      const int32_t a = tile_pref[r], z = tile_pref[r + 1];
      const int64_t pa = a < n_tiles ? (int64_t)col[a] : carry;
      const int64_t pz = z < n_tiles ? (int64_t)col[z] : carry;
      splits[(int64_t)b * W + r] = pz - pa;
    }
  }
}

// ---------------------------------------------------------------- scatter
// Each tile ranks its items stably per bin (ballot match inside a wave, wave
// order across waves), derives every bin's global base from the bin totals,
// sorts the tile by bin in LDS and writes each bin's run contiguously.
// Workgroup 0 also publishes the shard offsets.
__global__ void __launch_bounds__(kThreads)
k_scatter(const int64_t* __restrict__ ids, int64_t n_tok, const int64_t* __restrict__ so,
          const int32_t* __restrict__ perm, const int32_t* __restrict__ ro,
          const int64_t* __restrict__ bal, const int32_t* __restrict__ tile_pref, TableRows tr,
          int32_t W, int32_t T, int32_t nbits, int64_t tiles_cap,
          const uint32_t* __restrict__ hist, const uint32_t* __restrict__ tot,
          int64_t* __restrict__ shard_keys, int32_t* __restrict__ shard_bm,
          int64_t* __restrict__ shard_offsets) {
  __shared__ uint32_t cnt[kThreads / kWave][FS_MAX_RANKS + 1];
  __shared__ uint32_t gbase[FS_MAX_RANKS + 1];  // global start of each bin
  __shared__ uint32_t tbin[FS_MAX_RANKS + 1];   // start of each bin in the sorted tile
  __shared__ uint32_t skey[kTile];
  __shared__ int32_t sbm[kTile];
  __shared__ uint16_t sbin[kTile];
  __shared__ int64_t tmp[17];
  TileInfo ti;
  const int32_t tile = blockIdx.x;
  const bool has_tile = tile_info(tile, tile_pref, W, T, bal, ro, ti);
  if (!has_tile && tile != 0) return;
  const int32_t w = threadIdx.x / kWave;
  const int32_t nb = W + 1;
  // global bin bases: exclusive scan of the bin totals (4+ bins per thread)
  {
    constexpr int kPer = (FS_MAX_RANKS + 1 + kThreads - 1) / kThreads;
    uint32_t v[kPer];
    int64_t local = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int b = threadIdx.x * kPer + k;
      v[k] = b < nb ? tot[b] : 0u;
      local += v[k];
    }
    int64_t all;
    int64_t run = block_excl_scan<int64_t>(local, tmp, &all);
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int b = threadIdx.x * kPer + k;
      if (b < nb) {
        gbase[b] = (uint32_t)run;
        if (tile == 0) shard_offsets[b] = run;
      }
      run += v[k];
    }
  }
  if (!has_tile) return;
  const int32_t sentinel = (1 << nbits) - 1;  // > W: lanes without an item
  for (int b = lane(); b <= W; b += kWave) cnt[w][b] = 0;
  int64_t key[kRounds];
  int32_t bin[kRounds], rk[kRounds];
  wave_items(ti, w, ids, so, perm, bal, n_tok, tr, sentinel, key, bin);
  const uint64_t lt = lanemask_lt();
#pragma unroll
  for (int i = 0; i < kRounds; ++i) {
    int32_t b = bin[i];
    if (b < 0) b = W;
    bin[i] = b;
    const uint64_t peers = match_bits((uint32_t)b, nbits);
    const uint32_t before = cnt[w][b == sentinel ? 0 : b];
    rk[i] = (int32_t)before + popc(peers & lt);
    if (b != sentinel && (peers & lt) == 0) cnt[w][b] = before + (uint32_t)popc(peers);
  }
  __syncthreads();
  // per bin: exclusive prefix over the waves, then the bins' starts in the tile
  {
    constexpr int kPer = (FS_MAX_RANKS + 1 + kThreads - 1) / kThreads;
    uint32_t tot_b[kPer];
    int64_t local = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int b = threadIdx.x * kPer + k;
      uint32_t run = 0;
      if (b < nb) {
#pragma unroll
        for (int x = 0; x < kThreads / kWave; ++x) {
          const uint32_t c = cnt[x][b];
          cnt[x][b] = run;
          run += c;
        }
      }
      tot_b[k] = run;
      local += run;
    }
    int64_t all;
    int64_t run = block_excl_scan<int64_t>(local, tmp, &all);
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int b = threadIdx.x * kPer + k;
      if (b < nb) tbin[b] = (uint32_t)run;
      run += tot_b[k];
    }
  }
  __syncthreads();
  const int32_t bm_base = (int32_t)(ti.bm_lo + (int64_t)w * kWaveItems);
#pragma unroll
  for (int i = 0; i < kRounds; ++i) {
    const int32_t b = bin[i];
    if (b == sentinel) continue;
    const uint32_t p = tbin[b] + cnt[w][b] + (uint32_t)rk[i];
    skey[p] = (uint32_t)key[i];
    sbm[p] = bm_base + i * kWave + lane();
    sbin[p] = (uint16_t)b;
  }
  __syncthreads();
  const int m = (int)(ti.bm_hi - ti.bm_lo);
  for (int p = threadIdx.x; p < m; p += kThreads) {
    const int b = sbin[p];
    const int64_t pos = (int64_t)gbase[b] + hist[(int64_t)b * tiles_cap + tile] + (p - (int)tbin[b]);
    shard_keys[pos] = (int64_t)skey[p];
    shard_bm[pos] = sbm[p];
  }
}

}  // namespace
}  // namespace fs

using namespace fs;

static int64_t tiles_capacity(int64_t n_tok, int32_t T, int32_t W) {
  return (int64_t)T * (cdiv(n_tok, kTile) + W);
}

extern "C" size_t fs_bucketize_workspace_size(int64_t n_tok, int32_t n, int32_t T, int32_t W) {
  (void)n;
  Carve c(nullptr);
  c.take<int32_t>((size_t)W + 1);                                       // tile_pref
  c.take<uint32_t>((size_t)W + 1);                                      // tot
  c.take<uint32_t>((size_t)(W + 1) * (size_t)tiles_capacity(n_tok, T, W));  // hist
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
  }
  if (base > (int64_t)UINT32_MAX) return FS_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < fs_bucketize_workspace_size(n_tok, n, T, W)) return FS_ERR_WORKSPACE;
  const int64_t tiles_cap = tiles_capacity(n_tok, T, W);
  if (tiles_cap >= INT32_MAX) return FS_ERR_UNSUPPORTED;
  Carve c(ws);
  int32_t* tile_pref = c.take<int32_t>((size_t)W + 1);
  uint32_t* tot = c.take<uint32_t>((size_t)W + 1);
  uint32_t* hist = c.take<uint32_t>((size_t)(W + 1) * (size_t)tiles_cap);
  int nbits = 1;
  while ((1 << nbits) - 1 <= W) ++nbits;  // sentinel (2^nbits - 1) > W

  hipLaunchKernelGGL(k_prep, dim3(1), dim3(1024), 0, stream, sample_offsets, n, n_tok, perm,
                     rank_offsets, W, T, bal_offsets, tile_pref, err);
  FS_LAUNCH_CHECK();
  if (tiles_cap > 0) {
    hipLaunchKernelGGL(k_hist, dim3((unsigned)tiles_cap), dim3(kThreads), 0, stream, ids, n_tok,
                       sample_offsets, perm, rank_offsets, bal_offsets, tile_pref, tr, W, T,
                       tiles_cap, hist, err);
    FS_LAUNCH_CHECK();
  }
  hipLaunchKernelGGL(k_scan, dim3(W + 1), dim3(kThreads), 0, stream, tile_pref, W, tiles_cap, hist,
                     tot, splits);
  FS_LAUNCH_CHECK();
  // at least one workgroup runs: workgroup 0 writes the shard offsets
  hipLaunchKernelGGL(k_scatter, dim3((unsigned)(tiles_cap > 0 ? tiles_cap : 1)), dim3(kThreads),
                     0, stream, ids, n_tok, sample_offsets, perm, rank_offsets, bal_offsets,
                     tile_pref, tr, W, T, nbits, tiles_cap, hist, tot, shard_keys, shard_bm,
                     shard_offsets);
  FS_LAUNCH_CHECK();
  return FS_OK;
}
