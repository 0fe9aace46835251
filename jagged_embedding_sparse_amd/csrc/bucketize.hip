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
// per-shard column scans (+ splits, shard offsets), stable per-tile scatter.
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
// bal_offsets, input validation, tile table, zeroed shard totals.
__global__ void __launch_bounds__(1024)
k_prep(const int64_t* __restrict__ so, int32_t n, int64_t n_tok, const int32_t* __restrict__ perm,
       const int32_t* __restrict__ ro, int32_t W, int32_t T, int64_t* __restrict__ bal,
       int32_t* __restrict__ tile_pref, uint32_t* __restrict__ tot, int32_t* __restrict__ err) {
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
  for (int32_t b = threadIdx.x; b <= W; b += blockDim.x) tot[b] = 0;
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

// first balanced sample q in [q_lo, q_hi) whose tokens reach past bm
__device__ __forceinline__ int32_t sample_of(const int64_t* bal, int32_t q_lo, int32_t q_hi,
                                             int64_t bm) {
  int32_t lo = q_lo, hi = q_hi - 1;  // answer in [q_lo, q_hi-1]
  while (lo < hi) {
    int32_t mid = (lo + hi + 1) >> 1;
    if (bal[mid] <= bm) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Walks one wave's 1024 consecutive tokens of a tile, round by round, and
// yields (valid, key, bin, bm) per lane. The balanced sample of a lane's
// token is found by walking forward from the sample of the round's first
// token (tokens are contiguous, so a round spans few samples).
struct ItemWalker {
  const int64_t* ids;
  const int64_t* so;
  const int32_t* perm;
  const int64_t* bal;
  int64_t n_tok;
  int64_t rows, row_base, block;
  int32_t t, q_hi, nbin;
  int32_t q_cur;

  __device__ __forceinline__ void next(int64_t bm, int64_t bm_hi, bool& valid, int64_t& key,
                                       int32_t& bin) {
    valid = bm < bm_hi;
    int32_t q = q_cur;
    if (valid)
      while (q + 1 < q_hi && bal[q + 1] <= bm) ++q;
    // the next round starts at or after the last valid lane's sample
    q_cur = __shfl(q, kWave - 1, kWave);
    key = 0;
    bin = nbin;  // sentinel: not counted
    if (valid) {
      const int32_t s = perm[q];
      const int64_t tok = so[s] + (bm - bal[q]);
      const int64_t id = ids[(int64_t)t * n_tok + tok];
      const bool in = id >= 0 && id < rows;
      key = row_base + id;
      bin = in ? (int32_t)(id / block) : -1;  // -1 marks a dropped ID
    }
  }
};

__device__ __forceinline__ ItemWalker make_walker(const TileInfo& ti, int32_t w,
                                                  const int64_t* ids, const int64_t* so,
                                                  const int32_t* perm, const int64_t* bal,
                                                  int64_t n_tok, const TableRows& tr,
                                                  int32_t nbin) {
  ItemWalker it;
  it.ids = ids;
  it.so = so;
  it.perm = perm;
  it.bal = bal;
  it.n_tok = n_tok;
  it.t = ti.t;
  it.rows = tr.rows[ti.t];
  it.row_base = tr.row_base[ti.t];
  it.block = tr.block[ti.t];
  it.q_hi = ti.q_hi;
  it.nbin = nbin;
  const int64_t first = ti.bm_lo + (int64_t)w * kWaveItems;
  it.q_cur = sample_of(bal, ti.q_lo, ti.q_hi, min(first, ti.bm_hi - 1));
  return it;
}

// ---------------------------------------------------------------- histogram
__global__ void __launch_bounds__(kThreads)
k_hist(const int64_t* __restrict__ ids, int64_t n_tok, const int64_t* __restrict__ so,
       const int32_t* __restrict__ perm, const int32_t* __restrict__ ro,
       const int64_t* __restrict__ bal, const int32_t* __restrict__ tile_pref, TableRows tr,
       int32_t W, int32_t T, int64_t tiles_cap, uint32_t* __restrict__ hist,
       uint32_t* __restrict__ tot, int32_t* __restrict__ err) {
  __shared__ uint32_t h[FS_MAX_RANKS + 1];
  TileInfo ti;
  const int32_t tile = blockIdx.x;
  if (!tile_info(tile, tile_pref, W, T, bal, ro, ti)) return;
  for (int b = threadIdx.x; b <= W; b += kThreads) h[b] = 0;
  __syncthreads();
  const int32_t w = threadIdx.x / kWave;
  ItemWalker it = make_walker(ti, w, ids, so, perm, bal, n_tok, tr, W + 1);
  bool dropped_any = false;
  for (int i = 0; i < kRounds; ++i) {
    const int64_t bm = ti.bm_lo + (int64_t)w * kWaveItems + i * kWave + lane();
    bool valid;
    int64_t key;
    int32_t bin;
    it.next(bm, ti.bm_hi, valid, key, bin);
    if (valid) {
      if (bin < 0) {
        bin = W;
        dropped_any = true;
      }
      atomicAdd(&h[bin], 1u);
    }
  }
  flag_err(err, dropped_any, FS_EF_ID_RANGE);
  __syncthreads();
  for (int b = threadIdx.x; b <= W; b += kThreads) {
    uint32_t c = h[b];
    hist[(int64_t)b * tiles_cap + tile] = c;
    if (c) atomicAdd(&tot[b], c);
  }
}

// ---------------------------------------------------------------- column scan
// One workgroup per bin b (shard d = b, or b == W for dropped items): the
// bin's base is the sum of the lower bins' totals; its tiles' counts become
// exclusive output offsets in place; splits[b][r] sums rank r's tiles.
__global__ void __launch_bounds__(kThreads)
k_scan(const int32_t* __restrict__ tile_pref, int32_t W, int64_t tiles_cap,
       uint32_t* __restrict__ hist, const uint32_t* __restrict__ tot,
       int64_t* __restrict__ splits, int64_t* __restrict__ shard_offsets) {
  __shared__ int64_t tmp[17];
  const int32_t b = blockIdx.x;
  int64_t lower = 0;
  for (int32_t x = threadIdx.x; x < b; x += kThreads) lower += tot[x];
  int64_t base;
  (void)block_excl_scan<int64_t>(lower, tmp, &base);
  const int32_t n_tiles = tile_pref[W];
  uint32_t* col = hist + (int64_t)b * tiles_cap;
  int64_t carry = base;
  for (int32_t c0 = 0; c0 < n_tiles; c0 += kThreads) {
    const int32_t c = c0 + threadIdx.x;
    const int64_t v = c < n_tiles ? col[c] : 0;
    int64_t sum;
    const int64_t ex = block_excl_scan<int64_t>(v, tmp, &sum);
    if (c < n_tiles) col[c] = (uint32_t)(carry + ex);
    carry += sum;
  }
  __syncthreads();
  if (threadIdx.x == 0) shard_offsets[b] = base;
  if (b < W) {
    const int64_t end = carry;  // base + column total
    for (int32_t r = threadIdx.x; r < W; r += kThreads) {
      const int32_t a = tile_pref[r], z = tile_pref[r + 1];
      const int64_t pa = a < n_tiles ? (int64_t)col[a] : end;
      const int64_t pz = z < n_tiles ? (int64_t)col[z] : end;
      splits[(int64_t)b * W + r] = pz - pa;
    }
  }
}

// ---------------------------------------------------------------- scatter
__global__ void __launch_bounds__(kThreads)
k_scatter(const int64_t* __restrict__ ids, int64_t n_tok, const int64_t* __restrict__ so,
          const int32_t* __restrict__ perm, const int32_t* __restrict__ ro,
          const int64_t* __restrict__ bal, const int32_t* __restrict__ tile_pref, TableRows tr,
          int32_t W, int32_t T, int32_t nbits, int64_t tiles_cap,
          const uint32_t* __restrict__ hist, int64_t* __restrict__ shard_keys,
          int32_t* __restrict__ shard_bm) {
  __shared__ uint32_t cnt[kThreads / kWave][FS_MAX_RANKS + 1];
  TileInfo ti;
  const int32_t tile = blockIdx.x;
  if (!tile_info(tile, tile_pref, W, T, bal, ro, ti)) return;
  const int32_t w = threadIdx.x / kWave;
  const int32_t sentinel = (1 << nbits) - 1;  // > W: lanes without an item
  for (int b = lane(); b <= W; b += kWave) cnt[w][b] = 0;
  // (each wave only touches its own row until the barrier below)
  ItemWalker it = make_walker(ti, w, ids, so, perm, bal, n_tok, tr, sentinel);
  int64_t key[kRounds];
  int32_t bm32[kRounds], bin[kRounds], rk[kRounds];
  const uint64_t lt = lanemask_lt();
#pragma unroll
  for (int i = 0; i < kRounds; ++i) {
    const int64_t bm = ti.bm_lo + (int64_t)w * kWaveItems + i * kWave + lane();
    bool valid;
    int32_t b;
    it.next(bm, ti.bm_hi, valid, key[i], b);
    if (valid && b < 0) b = W;
    bin[i] = b;
    bm32[i] = (int32_t)bm;
    const uint64_t peers = match_bits((uint32_t)b, nbits);
    const uint32_t before = cnt[w][b == sentinel ? 0 : b];
    rk[i] = (int32_t)before + popc(peers & lt);
    if (b != sentinel && (peers & lt) == 0) cnt[w][b] = before + (uint32_t)popc(peers);
  }
  __syncthreads();
  // exclusive prefix over the waves of each bin
  for (int b = threadIdx.x; b <= W; b += kThreads) {
    uint32_t run = 0;
#pragma unroll
    for (int x = 0; x < kThreads / kWave; ++x) {
      uint32_t c = cnt[x][b];
      cnt[x][b] = run;
      run += c;
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kRounds; ++i) {
    const int32_t b = bin[i];
    if (b == sentinel) continue;
    const int64_t pos = (int64_t)hist[(int64_t)b * tiles_cap + tile] + cnt[w][b] + rk[i];
    shard_keys[pos] = key[i];
    shard_bm[pos] = bm32[i];
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
  if (base > (int64_t)UINT32_MAX + 1) return FS_ERR_UNSUPPORTED;
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
                     rank_offsets, W, T, bal_offsets, tile_pref, tot, err);
  FS_LAUNCH_CHECK();
  if (tiles_cap > 0) {
    hipLaunchKernelGGL(k_hist, dim3((unsigned)tiles_cap), dim3(kThreads), 0, stream, ids, n_tok,
                       sample_offsets, perm, rank_offsets, bal_offsets, tile_pref, tr, W, T,
                       tiles_cap, hist, tot, err);
    FS_LAUNCH_CHECK();
  }
  hipLaunchKernelGGL(k_scan, dim3(W + 1), dim3(kThreads), 0, stream, tile_pref, W, tiles_cap, hist,
                     tot, splits, shard_offsets);
  FS_LAUNCH_CHECK();
  if (tiles_cap > 0) {
    hipLaunchKernelGGL(k_scatter, dim3((unsigned)tiles_cap), dim3(kThreads), 0, stream, ids,
                       n_tok, sample_offsets, perm, rank_offsets, bal_offsets, tile_pref, tr, W, T,
                       nbits, tiles_cap, hist, shard_keys, shard_bm);
    FS_LAUNCH_CHECK();
  }
  return FS_OK;
}
