// Per-shard dedup into CSR + collision/exclusive split.
//
// "FreeScale: distributed training for sequence recommendation models",
// section 3.2 and Algorithm 2: the collision and exclusive index sets of
// iterations i and i+1 are computed on the shard-major (post-AllToAll) IDs.
//
//  1. LSD radix sort of (key, bm) inside every shard of the shard-major
//     items, on the shard-local key (rows of one shard of every table,
//     numbered densely: ~19 bits at 200M rows over 512 shards, so two passes
//     of up to 10-bit digits), stable; the last pass writes global keys and,
//     with several tables, moves each (table, shard) group to its place in
//     table-major order. Every pass is a stable counting sort (per-tile digit
//     histograms as rows of a tiles x digits matrix, coalesced column scans,
//     per-tile ranked scatter), so equal keys keep their shard-major order,
//     which for one key is ascending bm: the CSR's occurrence order falls out.
//  2. Head flags (key differs from its left neighbour), one scan over tiles,
//     compaction: unique keys, CSR segment starts, occurrence -> unique index,
//     and the (table, shard) group offsets, written where the group changes.
//  3. Set intersection of the new and previous unique lists, group by
//     (table, shard) group: chunks of each group's rows and the previous
//     rows in their key range staged in LDS, membership tests both ways.
#include "colscan.hpp"
#include "common.hpp"

namespace fs {
namespace {

constexpr int kThreads = 256;
constexpr int kRounds = 8;  // items per lane (register counts stay low)
constexpr int kWaveItems = kWave * kRounds;
constexpr int kTile = kThreads * kRounds;  // 2048
constexpr int kMaxDigitBits = 10;
constexpr int kMaxBins = 1 << kMaxDigitBits;  // also the count matrix's row length
// fixed cost of a radix pass, in tiles: its three dependent launches take
// about as long as streaming 400-500 tiles (measured: a pass over 432 tiles
// ~30 us, of which ~15 us is the floor of three launches)
constexpr int64_t kPassTiles = 512;

struct Groups {
  int64_t row_base[FS_MAX_TABLES + 1];
  int64_t block[FS_MAX_TABLES];
  int32_t T, W;
};

__device__ __forceinline__ int32_t group_of(uint32_t key, const Groups& g) {
  int t = 0;
  while (t + 1 < g.T && (int64_t)key >= g.row_base[t + 1]) ++t;
  // row within the table and the shard block both fit 32 bits; clamped so
  // that keys which are no row still name a group
  const uint32_t d = (uint32_t)((int64_t)key - g.row_base[t]) / (uint32_t)g.block[t];
  return t * g.W + (int32_t)min(d, (uint32_t)(g.W - 1));
}

// Valid item count of the call: shard_offsets[W] clamped to the capacity the
// host sized every buffer for (the prep kernel stores it; later kernels read
// it).
__device__ __forceinline__ int64_t n_valid_of(const int64_t* n_valid, int32_t W) {
  (void)W;
  return *n_valid;
}

// ---------------------------------------------------------------- shard-local keys
// Shard d holds rows [d*block_t, (d+1)*block_t) of every table t. Inside the
// shard a key is (t, row - d*block_t); numbered densely over the tables,
// local = shard_off[t] + row - d*block_t < shard_off[T] = sum_t block_t, it
// sorts exactly as the global key and needs far fewer bits.
struct SegKeys {
  int64_t row_base[FS_MAX_TABLES + 1];
  int64_t block[FS_MAX_TABLES];
  uint32_t shard_off[FS_MAX_TABLES + 1];
  int32_t T, W;
};

__device__ __forceinline__ int table_of_key(int64_t key, const SegKeys& k) {
  int t = 0;
  while (t + 1 < k.T && key >= k.row_base[t + 1]) ++t;
  return t;
}

// shard-local key of a global key in shard d (rows outside the shard clamp)
__device__ __forceinline__ uint32_t local_key(int64_t key, int32_t d, const SegKeys& k) {
  const int t = table_of_key(key, k);
  int64_t r = key - k.row_base[t] - (int64_t)d * k.block[t];
  r = r < 0 ? 0 : (r >= k.block[t] ? k.block[t] - 1 : r);
  return k.shard_off[t] + (uint32_t)r;
}

__device__ __forceinline__ int table_of_local(uint32_t lk, const SegKeys& k) {
  int t = 0;
  while (t + 1 < k.T && lk >= k.shard_off[t + 1]) ++t;
  return t;
}

__device__ __forceinline__ uint32_t global_key(uint32_t lk, int32_t d, const SegKeys& k) {
  const int t = table_of_local(lk, k);
  return (uint32_t)(k.row_base[t] + (int64_t)d * k.block[t] + (lk - k.shard_off[t]));
}

// A tile: items [lo, lo + n) of shard d, n <= kTile; tiles never straddle a
// shard and are numbered in position order.
struct UTile {
  int32_t lo, n, d, pad;
};

// ---------------------------------------------------------------- prep
// Segment bounds (shard_offsets clamped into [0, n_cap] and made
// non-decreasing, segment 0 from 0; with one segment: all valid items), the
// valid item count and the tile table. Thread i owns segments 5i .. 5i + 4
// (and the end bound W).
constexpr int kSegPer = (FS_MAX_RANKS + 1 + kThreads - 1) / kThreads;

__global__ void __launch_bounds__(kThreads)
k_seg_prep(const int64_t* __restrict__ so, int32_t W_so, int32_t W, int64_t n_cap,
           int64_t* __restrict__ n_valid, int32_t* __restrict__ seg_lo,
           int32_t* __restrict__ tile_first, UTile* __restrict__ tiles) {
  __shared__ int32_t wmax[kThreads / kWave];
  __shared__ int32_t tmp32[17];
  __shared__ int32_t s_lo[FS_MAX_RANKS + 1], s_first[FS_MAX_RANKS + 1];
  int32_t v[kSegPer];
  int32_t run = 0;
#pragma unroll
  for (int k = 0; k < kSegPer; ++k) {
    const int32_t d = threadIdx.x * kSegPer + k;
    // one segment (W == 1): all valid items; else shard d starts at so[d]
    int64_t x = (d > 0 && d <= W) ? so[W == 1 ? W_so : d] : 0;
    x = x < 0 ? 0 : (x > n_cap ? n_cap : x);
    run = max(run, (int32_t)x);
    v[k] = run;  // running maximum inside the thread
  }
  // exclusive maximum over the threads before this one
  int32_t inc = run;
#pragma unroll
  for (int dd = 1; dd < kWave; dd <<= 1) {
    const int32_t t = __shfl_up(inc, dd, kWave);
    if (lane() >= dd) inc = max(inc, t);
  }
  const int w = threadIdx.x / kWave;
  if (lane() == kWave - 1) wmax[w] = inc;
  __syncthreads();
  int32_t before = 0;
  for (int x = 0; x < w; ++x) before = max(before, wmax[x]);
  int32_t ex = __shfl_up(inc, 1, kWave);
  before = max(before, lane() == 0 ? 0 : ex);
  int32_t lo[kSegPer];
#pragma unroll
  for (int k = 0; k < kSegPer; ++k) lo[k] = max(before, v[k]);
#pragma unroll
  for (int k = 0; k < kSegPer; ++k) {
    const int32_t d = threadIdx.x * kSegPer + k;
    if (d <= W) {
      seg_lo[d] = lo[k];
      s_lo[d] = lo[k];
    }
    if (d == W) *n_valid = lo[k];
  }
  __syncthreads();  // s_lo visible to the workgroup
  int32_t c[kSegPer];
  int32_t mine = 0;
#pragma unroll
  for (int k = 0; k < kSegPer; ++k) {
    const int32_t d = threadIdx.x * kSegPer + k;
    c[k] = d < W ? (int32_t)cdiv(s_lo[d + 1] - lo[k], kTile) : 0;
    mine += c[k];
  }
  int32_t tt;
  int32_t pref = block_excl_scan<int32_t>(mine, tmp32, &tt);
#pragma unroll
  for (int k = 0; k < kSegPer; ++k) {
    const int32_t d = threadIdx.x * kSegPer + k;
    if (d <= W) {
      const int32_t f = d < W ? pref : tt;
      tile_first[d] = f;
      s_first[d] = f;
    }
    pref += c[k];
  }
  __syncthreads();
  // the tile table, all threads over all tiles: tile t belongs to the last
  // segment d with s_first[d] <= t (empty segments share their first tile)
  for (int32_t t = threadIdx.x; t < tt; t += kThreads) {
    int32_t a = 0, b = W;  // s_first[0] = 0 <= t < tt = s_first[W]
    while (b - a > 1) {
      const int32_t m = (a + b) >> 1;
      if (s_first[m] <= t) a = m; else b = m;
    }
    const int32_t j = t - s_first[a];
    UTile u;
    u.lo = s_lo[a] + j * kTile;
    u.n = min(kTile, s_lo[a + 1] - u.lo);
    u.d = a;
    u.pad = 0;
    tiles[t] = u;
  }
}

// ---------------------------------------------------------------- radix pass
// LSD radix sort of every shard's items by shard-local key, stable, digits of
// up to 10 bits. Per pass: k_seg_hist writes each tile's digit histogram as
// one row of the count matrix (LDS atomics; zero rows for unused tiles; the
// first pass also counts items per table); the column scans turn each
// digit's column into exclusive offsets over all tiles; k_seg_scatter takes
// its shard's digit counts as differences of the scanned rows at the shard's
// first tile and the next shard's, so positions restart at every shard,
// ranks its tile stably, sorts it in LDS and writes each digit's run
// contiguously. The last pass writes global keys, moved to their (table,
// shard) group when there are several tables. Tiles follow the XCD order.
template <typename KIn, bool kFirst>
__global__ void __launch_bounds__(kThreads)
k_seg_hist(const KIn* __restrict__ keys, const UTile* __restrict__ tiles,
           const int32_t* __restrict__ tile_first, SegKeys sk, int shift, uint32_t mask,
           uint32_t* __restrict__ hist, uint32_t* __restrict__ cnt_t) {
  __shared__ uint32_t h[kMaxBins];
  __shared__ uint32_t ht[FS_MAX_TABLES];
  const int32_t tile = xcd_tile(blockIdx.x, gridDim.x);
  const int nb = (int)mask + 1;
  for (int b = threadIdx.x; b < nb; b += kThreads) h[b] = 0;
  if (threadIdx.x < FS_MAX_TABLES) ht[threadIdx.x] = 0;
  __syncthreads();
  if (tile < tile_first[sk.W]) {
    const UTile u = tiles[tile];
    // all loads in flight (past the tile: its last item, not counted)
    uint32_t dg[kRounds];
    int tb[kRounds];
#pragma unroll
    for (int i = 0; i < kRounds; ++i) {
      const int x = i * kThreads + threadIdx.x;
      const KIn kv = keys[u.lo + (x < u.n ? x : u.n - 1)];
      uint32_t lk;
      if constexpr (kFirst) {
        lk = local_key((int64_t)kv, u.d, sk);
        tb[i] = table_of_local(lk, sk);
      } else {
        lk = (uint32_t)kv;
        tb[i] = 0;
      }
      dg[i] = (lk >> shift) & mask;
    }
#pragma unroll
    for (int i = 0; i < kRounds; ++i) {
      if (i * kThreads + (int)threadIdx.x < u.n) {
        atomicAdd(&h[dg[i]], 1u);
        if (kFirst && cnt_t) atomicAdd(&ht[tb[i]], 1u);
      }
    }
  }
  __syncthreads();
  for (int b = threadIdx.x; b < nb; b += kThreads) hist[(int64_t)tile * kMaxBins + b] = h[b];
  if (kFirst && cnt_t && threadIdx.x < FS_MAX_TABLES)
    cnt_t[(int64_t)tile * FS_MAX_TABLES + threadIdx.x] = ht[threadIdx.x];
}

// Several tables: shard d's sorted items are table-major; group (t, d) must
// move to its place in (table, shard) order. delta[t*W + d] = that place
// minus where the group starts inside the shard-sorted order.
__global__ void __launch_bounds__(kThreads)
k_seg_groups(const uint32_t* __restrict__ cnt_t, const UTile* __restrict__ tiles,
             const int32_t* __restrict__ tile_first, const int32_t* __restrict__ seg_lo,
             int32_t W, int32_t T, int32_t* __restrict__ delta) {
  __shared__ int64_t tmp[17];
  __shared__ uint32_t gsize[FS_MAX_RANKS][FS_MAX_TABLES];  // items of group (t, d), [d][t]
  for (int32_t x = threadIdx.x; x < W * FS_MAX_TABLES; x += kThreads) (&gsize[0][0])[x] = 0;
  __syncthreads();
  // every tile adds its per-table counts to its shard's row (all threads)
  const int32_t n_tiles = tile_first[W];
  for (int32_t q = threadIdx.x; q < n_tiles; q += kThreads) {
    const int32_t d = tiles[q].d;
    for (int t = 0; t < T; ++t) {
      const uint32_t c = cnt_t[(int64_t)q * FS_MAX_TABLES + t];
      if (c) atomicAdd(&gsize[d][t], c);
    }
  }
  __syncthreads();
  // per table: groups in shard order after the earlier tables; inside the
  // shard-sorted order the group follows the shard's earlier tables
  int64_t table_base = 0;
  for (int t = 0; t < T; ++t) {
    int64_t local = 0;
#pragma unroll
    for (int k = 0; k < kSegPer; ++k) {
      const int32_t d = threadIdx.x * kSegPer + k;
      local += d < W ? gsize[d][t] : 0u;
    }
    int64_t tot;
    int64_t g = table_base + block_excl_scan<int64_t>(local, tmp, &tot);
#pragma unroll
    for (int k = 0; k < kSegPer; ++k) {
      const int32_t d = threadIdx.x * kSegPer + k;
      if (d < W) {
        int64_t inside = seg_lo[d];
        for (int t2 = 0; t2 < t; ++t2) inside += gsize[d][t2];
        delta[t * W + d] = (int32_t)(g - inside);
        g += gsize[d][t];
      }
    }
    table_base += tot;
  }
}

// Staging area of one tile: first the per-wave lane-mask tables of the
// ranking, then the tile's items sorted by digit.
union RadixStage {
  uint64_t peers[kThreads / kWave][kMaxBins];
  struct {
    uint32_t key[kTile];
    int32_t val[kTile];
  } s;
};

template <typename KIn, bool kFirst, bool kLast>
__global__ void __launch_bounds__(kThreads)
k_seg_scatter(const KIn* __restrict__ keys_in, const int32_t* __restrict__ vals_in,
              const UTile* __restrict__ tiles, const int32_t* __restrict__ tile_first,
              const int32_t* __restrict__ seg_lo, SegKeys sk, int shift, uint32_t mask,
              const uint32_t* __restrict__ offs, const uint32_t* __restrict__ tot,
              const int32_t* __restrict__ delta, uint32_t* __restrict__ keys_out,
              int32_t* __restrict__ vals_out) {
  __shared__ uint16_t cnt[kThreads / kWave][kMaxBins];
  __shared__ uint32_t dig_base[kMaxBins];  // output start of each digit's run of this tile
  __shared__ uint32_t dig_tile[kMaxBins];  // start of each digit inside the LDS-sorted tile
  __shared__ RadixStage st;
  __shared__ int64_t tmp[17];
  constexpr int kPer = kMaxBins / kThreads;
  const int32_t tile = xcd_tile(blockIdx.x, gridDim.x);
  const int32_t n_tiles = tile_first[sk.W];
  if (tile >= n_tiles) return;  // uniform per workgroup
  const UTile u = tiles[tile];
  const int nb = (int)mask + 1;
  const int w = threadIdx.x / kWave;
  for (int b = lane(); b < nb; b += kWave) {
    cnt[w][b] = 0;
    st.peers[w][b] = 0;
  }
  uint32_t key[kRounds], dig[kRounds], rk[kRounds];
  int32_t val[kRounds];
  const uint32_t none = mask + 1;  // lanes without an item
#pragma unroll
  for (int i = 0; i < kRounds; ++i) {
    const int x = w * kWaveItems + i * kWave + lane();
    const bool valid = x < u.n;
    const int xc = u.lo + (valid ? x : u.n - 1);  // unconditional loads, all in flight
    // the pass's last read of its input (the histogram read it before):
    // streaming loads
    const KIn kv = __builtin_nontemporal_load(keys_in + xc);
    if constexpr (kFirst) key[i] = local_key((int64_t)kv, u.d, sk);
    else key[i] = (uint32_t)kv;
    val[i] = __builtin_nontemporal_load(vals_in + xc);
    dig[i] = valid ? ((key[i] >> shift) & mask) : none;
  }
  // stable rank of each item among the wave's items of its digit
  const uint64_t lt = lanemask_lt();
#pragma unroll
  for (int i = 0; i < kRounds; ++i) {
    const bool on = dig[i] != none;
    const uint32_t dd = on ? dig[i] : 0u;
    const uint64_t peers = lds_peers(st.peers[w], dd, on);
    const uint32_t before = cnt[w][dd];
    rk[i] = before + (uint32_t)popc(peers & lt);
    if (on && (peers & lt) == 0) cnt[w][dd] = (uint16_t)(before + (uint32_t)popc(peers));
  }
  __syncthreads();
  {
    // per digit: exclusive prefix over the waves, the digits' starts in the
    // tile, and the output bases: the shard's start, plus the shard's items
    // of smaller digits, plus the digit's items in the shard's earlier tiles
    const int32_t f = tile_first[u.d], nx = tile_first[u.d + 1];
    const uint32_t* pf = offs + (int64_t)f * kMaxBins;
    const uint32_t* pn = nx < (int32_t)gridDim.x ? offs + (int64_t)nx * kMaxBins : tot;
    const uint32_t* pt = offs + (int64_t)tile * kMaxBins;
    uint32_t tb[kPer], sc[kPer], mine[kPer];
    int64_t local = 0, slocal = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int b = threadIdx.x * kPer + k;
      uint32_t run = 0;
      sc[k] = 0;
      mine[k] = 0;
      if (b < nb) {
#pragma unroll
        for (int x = 0; x < kThreads / kWave; ++x) {
          const uint32_t c = cnt[x][b];
          cnt[x][b] = (uint16_t)run;
          run += c;
        }
        const uint32_t first = pf[b];
        sc[k] = pn[b] - first;  // the shard's items with digit b
        mine[k] = pt[b] - first;  // ... in the shard's tiles before this one
      }
      tb[k] = run;
      local += run;
      slocal += sc[k];
    }
    int64_t all;
    int64_t r0 = block_excl_scan<int64_t>(local, tmp, &all);
    int64_t ssum;
    int64_t s0 = block_excl_scan<int64_t>(slocal, tmp, &ssum);
    const int64_t base = seg_lo[u.d];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int b = threadIdx.x * kPer + k;
      if (b < nb) {
        dig_tile[b] = (uint32_t)r0;
        dig_base[b] = (uint32_t)(base + s0 + mine[k]);
      }
      r0 += tb[k];
      s0 += sc[k];
    }
  }
  __syncthreads();  // also ends every wave's use of the mask tables
#pragma unroll
  for (int i = 0; i < kRounds; ++i) {
    if (dig[i] == none) continue;
    const uint32_t p = dig_tile[dig[i]] + cnt[w][dig[i]] + rk[i];
    st.s.key[p] = key[i];
    st.s.val[p] = val[i];
  }
  __syncthreads();
  for (int p = threadIdx.x; p < u.n; p += kThreads) {
    const uint32_t k = st.s.key[p];
    const uint32_t dd = (k >> shift) & mask;
    uint32_t pos = dig_base[dd] + (uint32_t)p - dig_tile[dd];
    uint32_t kout = k;
    if constexpr (kLast) {
      kout = global_key(k, u.d, sk);
      if (sk.T > 1 && sk.W > 1) pos += (uint32_t)delta[table_of_local(k, sk) * sk.W + u.d];
    }
    keys_out[pos] = kout;
    vals_out[pos] = st.s.val[p];
  }
}

// ---------------------------------------------------------------- unique
__global__ void __launch_bounds__(kThreads)
k_heads(const uint32_t* __restrict__ sk, const int64_t* __restrict__ nvp, int32_t W,
        uint32_t* __restrict__ tile_heads) {
  __shared__ uint32_t tmp[kThreads / kWave];
  const int64_t n = n_valid_of(nvp, W);
  const int64_t t0 = (int64_t)blockIdx.x * kTile;
  if (t0 >= n) return;
  uint32_t c = 0;
  for (int i = 0; i < kRounds; ++i) {
    const int64_t x = t0 + i * kThreads + threadIdx.x;
    if (x < n) c += (x == 0 || sk[x] != sk[x - 1]);
  }
  c = wave_sum(c);
  if (lane() == 0) tmp[threadIdx.x / kWave] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t s = 0;
    for (int k = 0; k < kThreads / kWave; ++k) s += tmp[k];
    tile_heads[blockIdx.x] = s;
  }
}

__global__ void __launch_bounds__(kThreads)
k_heads_scan(const int64_t* __restrict__ nvp, int32_t W, int32_t n_groups, int32_t no_prev,
             uint32_t* __restrict__ tile_heads, int64_t* __restrict__ counts,
             int32_t* __restrict__ seg_offsets, int64_t* __restrict__ unique_offsets) {
  __shared__ int64_t tmp[17];
  const int64_t n = n_valid_of(nvp, W);
  const int64_t n_tiles = cdiv(n, kTile);
  // thread i scans a contiguous slice of the tile counts: its loads are all
  // in flight, and one workgroup scan joins the slices
  constexpr int kSlice = 16;
  int64_t carry = 0;
  for (int64_t c0 = 0; c0 < n_tiles; c0 += (int64_t)kSlice * blockDim.x) {
    const int64_t lo = c0 + (int64_t)threadIdx.x * kSlice;
    uint32_t v[kSlice];
    int64_t local = 0;
#pragma unroll
    for (int k = 0; k < kSlice; ++k) {
      v[k] = lo + k < n_tiles ? tile_heads[lo + k] : 0u;
      local += v[k];
    }
    int64_t sum;
    int64_t ex = carry + block_excl_scan<int64_t>(local, tmp, &sum);
#pragma unroll
    for (int k = 0; k < kSlice; ++k) {
      if (lo + k < n_tiles) tile_heads[lo + k] = (uint32_t)ex;
      ex += v[k];
    }
    carry += sum;
  }
  if (threadIdx.x == 0) {
    counts[0] = carry;  // U
    counts[1] = 0;
    counts[2] = no_prev ? carry : 0;  // without previous rows every row is exclusive
    counts[3] = 0;
    seg_offsets[carry] = (int32_t)n;
  }
  if (carry == 0)
    for (int32_t g = threadIdx.x; g <= n_groups; g += blockDim.x) unique_offsets[g] = 0;
}

// Striped layout: wave w of the tile owns kRounds rounds of 64 consecutive items.
// Head flags by comparing with the left neighbour (shuffle, or the previous
// round's last lane), counts by ballot; the wave prefix over the tile's
// waves comes from LDS, the tile's base (heads in earlier tiles) and U from
// the tile scan. Tile blockIdx.x, which starts at t0 < n.
__device__ __forceinline__ void compact_tile(const uint32_t* __restrict__ sk, int64_t n,
                                             const Groups& g, int64_t t0, int64_t tile_base,
                                             int64_t U, int64_t* __restrict__ unique,
                                             int32_t* __restrict__ seg_offsets,
                                             int32_t* __restrict__ occ_uid,
                                             int64_t* __restrict__ unique_offsets,
                                             uint8_t* __restrict__ cls_exclusive,
                                             uint32_t* wave_heads) {
  const int w = threadIdx.x / kWave, l = lane();
  const int64_t x0 = t0 + (int64_t)w * kWaveItems;
  uint32_t k[kRounds], prevk[kRounds];
  uint64_t hm[kRounds];
  uint32_t carry = (x0 > 0 && x0 <= n) ? sk[x0 - 1] : 0u;  // key left of the wave's first item
  uint32_t total = 0;
#pragma unroll
  for (int i = 0; i < kRounds; ++i) {
    const int64_t x = x0 + i * kWave + l;
    const bool in = x < n;
    k[i] = in ? sk[x] : 0u;
    const uint32_t up = (uint32_t)__shfl_up((int)k[i], 1, kWave);
    prevk[i] = l == 0 ? carry : up;
    carry = (uint32_t)__shfl((int)k[i], kWave - 1, kWave);
    hm[i] = __ballot(in && (x == 0 || k[i] != prevk[i]));
    total += (uint32_t)popc(hm[i]);
  }
  if (l == 0) wave_heads[w] = total;
  __syncthreads();
  uint32_t before = 0;
  for (int x = 0; x < w; ++x) before += wave_heads[x];
  const int32_t n_groups = g.T * g.W;
  int64_t base = tile_base + before;  // heads before this round
  const uint64_t le = lanemask_lt() | (1ull << l);
#pragma unroll
  for (int i = 0; i < kRounds; ++i) {
    const int64_t x = x0 + i * kWave + l;
    const int64_t uid = base + popc(hm[i] & le) - 1;
    if (x < n) {
      occ_uid[x] = (int32_t)uid;
      if ((hm[i] >> l) & 1ull) {
        unique[uid] = (int64_t)k[i];
        seg_offsets[uid] = (int32_t)x;
        if (cls_exclusive) cls_exclusive[uid] = FS_EXCLUSIVE;  // no previous rows
        // every group in (group(previous unique), group(this)] starts here
        const int32_t gi = group_of(k[i], g);
        const int32_t gp = uid == 0 ? -1 : group_of(prevk[i], g);
        for (int32_t q = gp + 1; q <= gi; ++q) unique_offsets[q] = uid;
        if (uid == U - 1)
          for (int32_t q = gi + 1; q <= n_groups; ++q) unique_offsets[q] = U;
      }
    }
    base += popc(hm[i]);
  }
}

__global__ void __launch_bounds__(kThreads)
k_compact(const uint32_t* __restrict__ sk, const int64_t* __restrict__ nvp, Groups g,
          const uint32_t* __restrict__ tile_base, const int64_t* __restrict__ counts,
          int64_t* __restrict__ unique, int32_t* __restrict__ seg_offsets,
          int32_t* __restrict__ occ_uid, int64_t* __restrict__ unique_offsets,
          uint8_t* __restrict__ cls_exclusive) {
  __shared__ uint32_t wave_heads[kThreads / kWave];
  const int64_t n = n_valid_of(nvp, g.W);
  const int64_t t0 = (int64_t)blockIdx.x * kTile;
  if (t0 >= n) return;
  compact_tile(sk, n, g, t0, tile_base[blockIdx.x], counts[0], unique, seg_offsets, occ_uid,
               unique_offsets, cls_exclusive, wave_heads);
}

// Calls of at most kScanTiles tiles: the compaction without k_heads_scan's
// launch. Every workgroup sums the tiles' head counts itself (at most
// kScanTiles values: the heads before its tile and U), and workgroup 0 writes
// what k_heads_scan writes (counts, the end of the last segment, the group
// offsets of an empty call). One launch fewer on the index path of mid-size
// batches, where each launch costs the host more than the scan costs the GPU.
constexpr int64_t kScanTiles = 512;

__global__ void __launch_bounds__(kThreads)
k_compact_scan(const uint32_t* __restrict__ sk, const int64_t* __restrict__ nvp, Groups g,
               const uint32_t* __restrict__ tile_heads, int32_t no_prev,
               int64_t* __restrict__ counts, int64_t* __restrict__ unique,
               int32_t* __restrict__ seg_offsets, int32_t* __restrict__ occ_uid,
               int64_t* __restrict__ unique_offsets, uint8_t* __restrict__ cls_exclusive) {
  __shared__ uint32_t wave_heads[kThreads / kWave];
  __shared__ int64_t tmp[17];
  const int64_t n = n_valid_of(nvp, g.W);
  const int64_t n_tiles = cdiv(n, kTile);
  int64_t before = 0, all = 0;
  for (int64_t q = threadIdx.x; q < n_tiles; q += kThreads) {
    const int64_t c = tile_heads[q];
    all += c;
    before += q < (int64_t)blockIdx.x ? c : 0;
  }
  int64_t U, base;
  block_excl_scan<int64_t>(all, tmp, &U);
  block_excl_scan<int64_t>(before, tmp, &base);
  if (blockIdx.x == 0) {
    if (threadIdx.x == 0) {
      counts[0] = U;
      counts[1] = 0;
      counts[2] = no_prev ? U : 0;  // without previous rows every row is exclusive
      counts[3] = 0;
      seg_offsets[U] = (int32_t)n;
    }
    if (U == 0)
      for (int32_t q = threadIdx.x; q <= g.T * g.W; q += kThreads) unique_offsets[q] = 0;
  }
  const int64_t t0 = (int64_t)blockIdx.x * kTile;
  if (t0 >= n) return;
  compact_tile(sk, n, g, t0, base, U, unique, seg_offsets, occ_uid, unique_offsets, cls_exclusive,
               wave_heads);
}

// ---------------------------------------------------------------- small calls
// A call of at most kSmallMax items runs in one workgroup instead of the
// ten-odd launches of the radix path. Wave w holds items w * 256 + 64 i +
// lane (four rounds) in registers; an LSD radix sort by global key with
// 8-bit digits runs in LDS: per pass, every wave counts its items' digits
// (LDS atomics), prefixes over the waves and the digits give each wave's
// first position of each digit, and the waves rank their items round by
// round (lane masks, a running count per digit) and write each to its
// sorted place, so equal keys keep their input order (ascending bm). Then
// head flags, one workgroup scan and the compaction's outputs: unique keys,
// segment starts, occurrence -> unique index, the (table, shard) group
// offsets, and the all-exclusive classes and counts (the collision split,
// when there are previous rows, follows as usual).
constexpr int kSmallThreads = 1024;
constexpr int kSmallWaves = kSmallThreads / kWave;
constexpr int kSmallRounds = 4;
constexpr int kSmallWaveItems = kWave * kSmallRounds;
constexpr int kSmallMax = kSmallThreads * kSmallRounds;  // 4096 items
constexpr int kSmallBits = 8;
constexpr int kSmallBins = 1 << kSmallBits;

__global__ void __launch_bounds__(kSmallThreads)
k_dedup_small(const int64_t* __restrict__ keys, const int32_t* __restrict__ bm,
              const int64_t* __restrict__ so, int32_t W, int64_t n_cap, Groups g, int32_t kbits,
              int32_t no_prev, int64_t* __restrict__ unique, int64_t* __restrict__ unique_offsets,
              int32_t* __restrict__ seg_offsets, int32_t* __restrict__ occ_bm,
              int32_t* __restrict__ occ_uid, uint8_t* __restrict__ cls,
              int64_t* __restrict__ counts) {
  __shared__ uint32_t s_key[kSmallMax];
  __shared__ int32_t s_val[kSmallMax];
  __shared__ uint64_t peers_tab[kSmallWaves][kSmallBins];  // lane masks of the ranking
  __shared__ uint32_t base[kSmallWaves][kSmallBins];  // counts, then each wave's next position
  __shared__ uint32_t tmp[17];
  __shared__ int32_t s_n;
  // valid items: the largest shard bound, clamped into [0, n_cap] (the
  // radix path's running maximum over the bounds ends at the same value)
  if (threadIdx.x == 0) s_n = 0;
  __syncthreads();
  if ((int32_t)threadIdx.x < W) {
    int64_t x = so[threadIdx.x + 1];
    x = x < 0 ? 0 : (x > n_cap ? n_cap : x);
    atomicMax(&s_n, (int32_t)x);
  }
  __syncthreads();
  const int32_t n = s_n;
  const int32_t n_groups = g.T * g.W;
  const int w = threadIdx.x / kWave, l = lane();
  if (n > 0) {  // uniform
    const int32_t wn = n - w * kSmallWaveItems;  // this wave's items
    uint32_t key[kSmallRounds];
    int32_t val[kSmallRounds];
    // lanes past the end load the last item again: registers written
    // unconditionally, all loads in flight
#pragma unroll
    for (int i = 0; i < kSmallRounds; ++i) {
      const int32_t x = w * kSmallWaveItems + i * kWave + l;
      const int32_t xc = x < n ? x : n - 1;
      key[i] = (uint32_t)keys[xc];
      val[i] = bm[xc];
    }
    for (int b = l; b < kSmallBins; b += kWave) peers_tab[w][b] = 0;
    const uint64_t lt = lanemask_lt();
    for (int32_t shift = 0; shift < kbits; shift += kSmallBits) {
      for (int b = l; b < kSmallBins; b += kWave) base[w][b] = 0;
      // this wave's digit counts (a wave's LDS operations complete in order)
#pragma unroll
      for (int i = 0; i < kSmallRounds; ++i)
        if (i * kWave + l < wn) atomicAdd(&base[w][(key[i] >> shift) & (kSmallBins - 1)], 1u);
      __syncthreads();
      // per digit: prefix over the waves, then over the digits
      uint32_t tot = 0;
      if (threadIdx.x < kSmallBins) {
        const int b = threadIdx.x;
#pragma unroll
        for (int x = 0; x < kSmallWaves; ++x) {
          const uint32_t c = base[x][b];
          base[x][b] = tot;
          tot += c;
        }
      }
      uint32_t all;
      const uint32_t ex =
          block_excl_scan<uint32_t>(threadIdx.x < kSmallBins ? tot : 0u, tmp, &all);
      if (threadIdx.x < kSmallBins) {
#pragma unroll
        for (int x = 0; x < kSmallWaves; ++x) base[x][threadIdx.x] += ex;
      }
      __syncthreads();
      // stable ranks in order (round by round, lanes in order), each item
      // written to its place at once; the lowest lane of each digit
      // advances the wave's next position for it
#pragma unroll
      for (int i = 0; i < kSmallRounds; ++i) {
        if (i * kWave < wn) {  // uniform per wave
          const bool on = i * kWave + l < wn;
          const uint32_t dd = on ? (key[i] >> shift) & (kSmallBins - 1) : 0u;
          const uint64_t peers = lds_peers(peers_tab[w], dd, on);
          const uint32_t at = base[w][dd];
          if (on) {
            const uint32_t p = at + (uint32_t)popc(peers & lt);
            s_key[p] = key[i];
            s_val[p] = val[i];
            if ((peers & lt) == 0) base[w][dd] = at + (uint32_t)popc(peers);
          }
        }
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < kSmallRounds; ++i) {
        // every slot is inside the stage; slots past the items are never used
        const int32_t x = w * kSmallWaveItems + i * kWave + l;
        key[i] = s_key[x];
        val[i] = s_val[x];
      }
      __syncthreads();  // the stage is rewritten by the next pass
    }
    // s_key / s_val hold the sorted items (the last pass wrote them)
    // thread t owns sorted slots kSmallRounds * t ..: head flags and their scan
    const int p0 = threadIdx.x * kSmallRounds;
    bool hd[kSmallRounds];
    uint32_t heads = 0;
#pragma unroll
    for (int k = 0; k < kSmallRounds; ++k) {
      const int p = p0 + k;
      hd[k] = p < n && (p == 0 || s_key[p - 1] != s_key[p]);
      heads += hd[k];
    }
    uint32_t U;
    uint32_t uid = block_excl_scan<uint32_t>(heads, tmp, &U);
#pragma unroll
    for (int k = 0; k < kSmallRounds; ++k) {
      const int p = p0 + k;
      if (p >= n) break;
      uid += hd[k];
      const uint32_t u = uid - 1;  // this item's unique row
      occ_bm[p] = s_val[p];
      occ_uid[p] = (int32_t)u;
      if (hd[k]) {
        const uint32_t kk = s_key[p];
        unique[u] = (int64_t)kk;
        seg_offsets[u] = p;
        if (no_prev) cls[u] = FS_EXCLUSIVE;
        // every group in (group of the previous unique key, this key's
        // group] starts here; after the last unique key the rest end at U
        const int32_t gi = group_of(kk, g);
        const int32_t gp = u == 0 ? -1 : group_of(s_key[p - 1], g);
        for (int32_t q = gp + 1; q <= gi; ++q) unique_offsets[q] = u;
        if (u == U - 1)
          for (int32_t q = gi + 1; q <= n_groups; ++q) unique_offsets[q] = U;
      }
    }
    if (threadIdx.x == 0) {
      seg_offsets[U] = n;
      counts[0] = U;
      counts[1] = 0;
      counts[2] = no_prev ? U : 0;
      counts[3] = 0;
    }
  } else {
    for (int32_t q = threadIdx.x; q <= n_groups; q += kSmallThreads) unique_offsets[q] = 0;
    if (threadIdx.x == 0) {
      seg_offsets[0] = 0;
      counts[0] = counts[1] = counts[2] = counts[3] = 0;
    }
  }
}

// ---------------------------------------------------------------- collision
// Both unique lists are ascending and split into the same (table, shard)
// groups (unique_offsets of this call and of the previous one), and a key of
// group g can only meet keys of group g, so the intersection runs per group.
// Group g's new rows are cut into chunks of kCoChunk; workgroup s of the
// group takes chunks s, s + S, .... Chunk c owns the previous rows whose keys
// lie from its first key up to the next chunk's first key (the first chunk
// from the group's start, the last one to its end), so every previous row
// is classed by exactly one chunk. Each chunk's rows, and its previous rows
// in pieces of kCoPiece, are staged in LDS as 32-bit keys (every key is
// below 2^32) and tested for membership both ways by binary search. Reads
// are one pass over both lists, plus two wave searches per chunk of a group
// with more than one chunk.
constexpr int kCoThreads = 512;
constexpr int kCoChunk = 4096;  // a typical group (a few thousand rows) is one chunk: no search
constexpr int kCoPer = kCoChunk / kCoThreads;
constexpr int kCoPiece = 4096;

__device__ __forceinline__ bool lds_has(const uint32_t* s, int n, uint32_t v) {
  int lo = 0, hi = n;  // first s[k] >= v
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (s[mid] < v) lo = mid + 1; else hi = mid;
  }
  return lo < n && s[lo] == v;
}

__global__ void __launch_bounds__(kCoThreads)
k_collide(const int64_t* __restrict__ a, const int64_t* __restrict__ a_off,
          const int64_t* __restrict__ counts_a, int64_t cap_a, const int64_t* __restrict__ b,
          const int64_t* __restrict__ b_off, const int64_t* __restrict__ counts_b, int64_t cap_b,
          int32_t S, uint8_t* __restrict__ cls, uint8_t* __restrict__ prev_cls,
          uint32_t* __restrict__ block_hits) {
  __shared__ uint32_t sa[kCoChunk], sb[kCoPiece];
  __shared__ int64_t span[2];
  __shared__ uint32_t hits[kCoThreads / kWave];
  const int32_t g = blockIdx.x / S, s0 = blockIdx.x % S;
  const int64_t na = min(counts_a[0], cap_a);
  const int64_t a_lo = min(max(a_off[g], (int64_t)0), na);
  const int64_t a_hi = min(max(a_off[g + 1], a_lo), na);
  int64_t b_lo = 0, b_hi = 0;
  if (b) {
    const int64_t nb = max((int64_t)0, min(counts_b[0], cap_b));
    b_lo = min(max(b_off[g], (int64_t)0), nb);
    b_hi = min(max(b_off[g + 1], b_lo), nb);
  }
  const int64_t nchunks = max((int64_t)1, cdiv(a_hi - a_lo, kCoChunk));
  const int w = threadIdx.x / kWave;
  uint32_t mine = 0;
  for (int64_t c = s0; c < nchunks; c += S) {
    const int64_t i0 = a_lo + c * kCoChunk, i1 = min(i0 + kCoChunk, a_hi);
    const int na_c = (int)(i1 - i0);
    if (!b) {  // no previous rows (uniform): every row exclusive
      for (int x = threadIdx.x; x < na_c; x += kCoThreads) cls[i0 + x] = FS_EXCLUSIVE;
      continue;
    }
    // this chunk's previous rows: wave 0 finds where they start, wave 1
    // where they end (the first key of the next chunk)
    if (w < 2) {
      int64_t r;
      if (w == 0) {
        const int64_t key = c == 0 ? -1 : a[i0];
        r = c == 0 ? b_lo
                   : wave_partition_point(b_lo, b_hi, [&](int64_t k) { return b[k] < key; });
      } else {
        const int64_t key = c + 1 < nchunks ? a[i1] : 0;
        r = c + 1 < nchunks
                ? wave_partition_point(b_lo, b_hi, [&](int64_t k) { return b[k] < key; })
                : b_hi;
      }
      if (lane() == 0) span[w] = r;
    }
    for (int x = threadIdx.x; x < na_c; x += kCoThreads) sa[x] = (uint32_t)a[i0 + x];
    __syncthreads();
    const int64_t j0 = span[0], j1 = span[1];
    bool found[kCoPer];
#pragma unroll
    for (int k = 0; k < kCoPer; ++k) found[k] = false;
    for (int64_t jp = j0; jp < j1; jp += kCoPiece) {
      const int nb_p = (int)min((int64_t)kCoPiece, j1 - jp);
      for (int x = threadIdx.x; x < nb_p; x += kCoThreads) sb[x] = (uint32_t)b[jp + x];
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kCoPer; ++k) {
        const int x = k * kCoThreads + threadIdx.x;
        if (x < na_c) found[k] = found[k] || lds_has(sb, nb_p, sa[x]);
      }
      for (int x = threadIdx.x; x < nb_p; x += kCoThreads)
        prev_cls[jp + x] = lds_has(sa, na_c, sb[x]) ? FS_COLLISION : FS_EXCLUSIVE;
      __syncthreads();  // sb is reused by the next piece
    }
#pragma unroll
    for (int k = 0; k < kCoPer; ++k) {
      const int x = k * kCoThreads + threadIdx.x;
      if (x < na_c) {
        cls[i0 + x] = found[k] ? FS_COLLISION : FS_EXCLUSIVE;
        mine += found[k];
      }
    }
    __syncthreads();  // sa and span are reused by the next chunk
  }
  mine = wave_sum(mine);
  if (lane() == 0) hits[w] = mine;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t sum = 0;
    for (int k = 0; k < kCoThreads / kWave; ++k) sum += hits[k];
    block_hits[blockIdx.x] = sum;
  }
}

// counts[1..3] from the per-block collision counts (one block).
__global__ void __launch_bounds__(kThreads)
k_collide_counts(const uint32_t* __restrict__ block_hits, int64_t n_blocks,
                 const int64_t* __restrict__ counts_b, int64_t cap_b,
                 int64_t* __restrict__ counts) {
  __shared__ int64_t tmp[17];
  int64_t local = 0;
  for (int64_t i = threadIdx.x; i < n_blocks; i += blockDim.x) local += block_hits[i];
  int64_t C;
  (void)block_excl_scan<int64_t>(local, tmp, &C);
  if (threadIdx.x == 0) {
    const int64_t na = counts[0];
    const int64_t nb = counts_b ? max((int64_t)0, min(counts_b[0], cap_b)) : 0;
    counts[1] = C;
    counts[2] = na - C;
    counts[3] = nb - C;
  }
}

}  // namespace
}  // namespace fs

using namespace fs;

static int key_bits(int64_t key_space) {
  int b = 1;
  while (b < 32 && ((int64_t)1 << b) < key_space) ++b;
  return b;
}

// tiles of the radix passes: sum over shards of ceil(items / kTile) <= this
static int64_t seg_tiles(int64_t cap, int32_t W) {
  return (int64_t)align_up((size_t)(cdiv(cap, kTile) + W), kXcd);
}

// Workgroups per (table, shard) group of the collision split: about four
// chunks of the group's expected rows (a fourth of its items) each
static int32_t collide_splits(int64_t cap, int32_t T, int32_t W) {
  const int64_t s = cdiv(cap, (int64_t)T * W * kCoChunk * 4);
  return (int32_t)(s < 1 ? 1 : (s > 64 ? 64 : s));
}

// The collision split of new rows (unique, unique_offsets, counts[0] = U, at
// most n_cap rows) against the previous call's rows (or none): classes of
// both sets and counts[1..3]; block_hits holds T * W * collide_splits(...)
// entries.
static int launch_collide(const int64_t* unique, const int64_t* unique_offsets, int64_t n_cap,
                          int32_t T, int32_t W, const int64_t* prev_unique,
                          const int64_t* prev_unique_offsets, const int64_t* prev_counts,
                          int64_t prev_cap, uint8_t* cls, uint8_t* prev_cls, int64_t* counts,
                          uint32_t* block_hits, hipStream_t stream) {
  const int64_t cap = n_cap > 0 ? n_cap : 1;
  const int32_t co_split = collide_splits(cap, T, W);
  const int64_t co_blocks = (int64_t)T * W * co_split;
  hipLaunchKernelGGL(k_collide, dim3((unsigned)co_blocks), dim3(kCoThreads), 0, stream, unique,
                     unique_offsets, counts, n_cap, prev_unique, prev_unique_offsets,
                     prev_counts, prev_cap, co_split, cls, prev_cls, block_hits);
  FS_LAUNCH_CHECK();
  hipLaunchKernelGGL(k_collide_counts, dim3(1), dim3(kThreads), 0, stream, block_hits, co_blocks,
                     prev_counts, prev_cap, counts);
  FS_LAUNCH_CHECK();
  return FS_OK;
}

extern "C" size_t fs_collision_split_workspace_size(int64_t n_cap, int32_t T, int32_t W) {
  const int64_t cap = n_cap > 0 ? n_cap : 1;
  const int32_t t = T > 0 ? T : 1, w = W > 0 ? W : 1;
  Carve c(nullptr);
  c.take<uint32_t>((size_t)t * w * collide_splits(cap, t, w));
  return c.used + 256;
}

extern "C" int fs_collision_split(const int64_t* unique, const int64_t* unique_offsets,
                                  int64_t n_cap, int32_t T, int32_t W,
                                  const int64_t* prev_unique, const int64_t* prev_unique_offsets,
                                  const int64_t* prev_counts, int64_t prev_cap, uint8_t* cls,
                                  uint8_t* prev_cls, int64_t* counts, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  if (n_cap < 0 || n_cap >= (int64_t)INT32_MAX || T < 1 || T > FS_MAX_TABLES || W < 1 ||
      W > FS_MAX_RANKS || !unique_offsets || !counts)
    return FS_ERR_INVALID_ARG;
  if (n_cap > 0 && (!unique || !cls)) return FS_ERR_INVALID_ARG;
  if ((prev_unique == nullptr) != (prev_counts == nullptr) ||
      (prev_unique == nullptr) != (prev_unique_offsets == nullptr))
    return FS_ERR_INVALID_ARG;
  if (prev_unique && (prev_cap < 0 || !prev_cls)) return FS_ERR_INVALID_ARG;
  if (!prev_unique) prev_cap = 0;
  if (!ws || ws_bytes < fs_collision_split_workspace_size(n_cap, T, W)) return FS_ERR_WORKSPACE;
  const int64_t cap = n_cap > 0 ? n_cap : 1;
  Carve c(ws);
  uint32_t* block_hits = c.take<uint32_t>((size_t)T * W * collide_splits(cap, T, W));
  return launch_collide(unique, unique_offsets, n_cap, T, W, prev_unique, prev_unique_offsets,
                        prev_counts, prev_cap, cls, prev_cls, counts, block_hits, stream);
}

extern "C" size_t fs_unique_workspace_size(int64_t n_cap, int64_t prev_cap, int32_t T,
                                           int32_t W) {
  (void)prev_cap;  // the collision split needs no space per previous row
  const int64_t cap = n_cap > 0 ? n_cap : 1;
  const int64_t tiles = cdiv(cap, kTile);
  const int64_t G = seg_tiles(cap, W);
  Carve c(nullptr);
  c.take<uint32_t>((size_t)cap);                // keys A
  c.take<uint32_t>((size_t)cap);                // keys B
  c.take<int32_t>((size_t)cap);                 // vals A
  c.take<int32_t>((size_t)cap);                 // vals B
  c.take<uint32_t>((size_t)(G * kMaxBins));     // tiles x digits counts, then offsets
  c.take<uint32_t>((size_t)(cdiv(G, kColBlockRows) * kMaxBins));  // column partials
  c.take<uint32_t>((size_t)kMaxBins);           // digit totals
  c.take<UTile>((size_t)G);                     // radix tiles
  c.take<uint32_t>((size_t)(G * FS_MAX_TABLES));  // items per tile and table
  c.take<int32_t>((size_t)W + 1);               // shard starts
  c.take<int32_t>((size_t)W + 1);               // first tile of each shard
  c.take<int32_t>((size_t)T * W);               // group moves (several tables)
  c.take<uint32_t>((size_t)tiles);              // heads per tile
  c.take<int64_t>(1);                           // valid item count
  c.take<uint32_t>((size_t)T * W * collide_splits(cap, T, W));  // collisions per workgroup
  return c.used + 256;
}

extern "C" int fs_unique_collision_split(const int64_t* shard_keys, const int32_t* shard_bm,
                                         const int64_t* shard_offsets, int64_t n_cap,
                                         const fs_table* tables, int32_t T, int32_t W,
                                         const int64_t* prev_unique,
                                         const int64_t* prev_unique_offsets,
                                         const int64_t* prev_counts, int64_t prev_cap,
                                         int64_t* unique,
                                         int64_t* unique_offsets, int32_t* seg_offsets,
                                         int32_t* occ_bm, int32_t* occ_uid, uint8_t* cls,
                                         uint8_t* prev_cls, int64_t* counts, void* ws,
                                         size_t ws_bytes, hipStream_t stream) {
  if (n_cap < 0 || n_cap >= (int64_t)INT32_MAX || T < 1 || T > FS_MAX_TABLES || W < 1 ||
      W > FS_MAX_RANKS || !tables || !shard_offsets || !unique_offsets || !seg_offsets ||
      !counts)
    return FS_ERR_INVALID_ARG;
  if (n_cap > 0 && (!shard_keys || !shard_bm || !unique || !occ_bm || !occ_uid || !cls))
    return FS_ERR_INVALID_ARG;
  if ((prev_unique == nullptr) != (prev_counts == nullptr) ||
      (prev_unique == nullptr) != (prev_unique_offsets == nullptr))
    return FS_ERR_INVALID_ARG;
  if (prev_unique && (prev_cap < 0 || !prev_cls)) return FS_ERR_INVALID_ARG;
  if (!prev_unique) prev_cap = 0;
  Groups g;
  g.T = T;
  g.W = W;
  int64_t base = 0;
  for (int t = 0; t < T; ++t) {
    if (tables[t].rows < 1) return FS_ERR_INVALID_ARG;
    g.row_base[t] = base;
    g.block[t] = cdiv(tables[t].rows, W);
    base += tables[t].rows;
  }
  g.row_base[T] = base;
  if (base > (int64_t)UINT32_MAX) return FS_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < fs_unique_workspace_size(n_cap, prev_cap, T, W)) return FS_ERR_WORKSPACE;

  // small calls: one workgroup sorts and compacts every item
  if (n_cap <= kSmallMax) {
    const int32_t no_prev = prev_unique == nullptr;
    hipLaunchKernelGGL(k_dedup_small, dim3(1), dim3(kSmallThreads), 0, stream, shard_keys,
                       shard_bm, shard_offsets, W, n_cap, g, key_bits(base), no_prev, unique,
                       unique_offsets, seg_offsets, occ_bm, occ_uid, cls, counts);
    FS_LAUNCH_CHECK();
    if (no_prev) return FS_OK;
    Carve cs(ws);
    const int64_t cap1 = n_cap > 0 ? n_cap : 1;
    uint32_t* block_hits = cs.take<uint32_t>((size_t)T * W * collide_splits(cap1, T, W));
    return launch_collide(unique, unique_offsets, n_cap, T, W, prev_unique, prev_unique_offsets,
                          prev_counts, prev_cap, cls, prev_cls, counts, block_hits, stream);
  }

  // Sort inside the W shards (shard-local keys: fewer bits, so often one pass
  // fewer) or over all items as one segment (local key = global key). A pass
  // costs a fixed part (three dependent launches, about as long as streaming
  // kPassTiles tiles) plus its tile count; the shard tiling adds up to one
  // partial tile per shard.
  int64_t span_w = 0, span_1 = base;
  for (int t = 0; t < T; ++t) span_w += g.block[t];
  const int64_t cap_tiles = cdiv(n_cap > 0 ? n_cap : 1, kTile);
  const int passes_w = (key_bits(span_w) + kMaxDigitBits - 1) / kMaxDigitBits;
  const int passes_1 = (key_bits(span_1) + kMaxDigitBits - 1) / kMaxDigitBits;
  const bool by_shard = W > 1 && passes_w * (cap_tiles + W + kPassTiles) <
                                     passes_1 * (cap_tiles + kPassTiles);
  const int32_t nseg = by_shard ? W : 1;
  SegKeys lk;
  lk.T = T;
  lk.W = nseg;
  uint32_t span = 0;
  for (int t = 0; t < T; ++t) {
    lk.row_base[t] = g.row_base[t];
    lk.block[t] = by_shard ? g.block[t] : tables[t].rows;
    lk.shard_off[t] = span;
    span += (uint32_t)lk.block[t];  // at most the sum of rows < 2^32
  }
  lk.row_base[T] = base;
  lk.shard_off[T] = span;

  const int64_t cap = n_cap > 0 ? n_cap : 1;
  const int64_t tiles = cdiv(cap, kTile);
  const int64_t G = seg_tiles(cap, W);
  Carve c(ws);
  uint32_t* ka = c.take<uint32_t>((size_t)cap);
  uint32_t* kb = c.take<uint32_t>((size_t)cap);
  int32_t* va = c.take<int32_t>((size_t)cap);
  int32_t* vb = c.take<int32_t>((size_t)cap);
  uint32_t* hist = c.take<uint32_t>((size_t)(G * kMaxBins));
  uint32_t* part = c.take<uint32_t>((size_t)(cdiv(G, kColBlockRows) * kMaxBins));
  uint32_t* tot = c.take<uint32_t>((size_t)kMaxBins);
  UTile* utiles = c.take<UTile>((size_t)G);
  uint32_t* cnt_t = c.take<uint32_t>((size_t)(G * FS_MAX_TABLES));
  int32_t* seg_lo = c.take<int32_t>((size_t)W + 1);
  int32_t* tile_first = c.take<int32_t>((size_t)W + 1);
  int32_t* delta = c.take<int32_t>((size_t)T * W);
  uint32_t* tile_heads = c.take<uint32_t>((size_t)tiles);
  int64_t* n_valid = c.take<int64_t>(1);
  const int32_t co_split = collide_splits(cap, T, W);
  const int64_t co_blocks = (int64_t)T * W * co_split;
  uint32_t* block_hits = c.take<uint32_t>((size_t)co_blocks);

  const int kbits = key_bits(span);
  const int passes = (kbits + kMaxDigitBits - 1) / kMaxDigitBits;
  hipLaunchKernelGGL(k_seg_prep, dim3(1), dim3(kThreads), 0, stream, shard_offsets, W, nseg,
                     n_cap, n_valid, seg_lo, tile_first, utiles);
  FS_LAUNCH_CHECK();
  uint32_t* kbuf[2] = {ka, kb};
  int32_t* vbuf[2] = {va, vb};
  const unsigned grid = (unsigned)tiles;
  const unsigned rgrid = (unsigned)G;
  int shift = 0;
  for (int p = 0; p < passes; ++p) {
    // digits as even as the passes allow: 19 bits -> 10, 9
    const int bits = (kbits - shift + (passes - p) - 1) / (passes - p);
    const uint32_t mask = (1u << bits) - 1u;
    const bool first = p == 0, last = p == passes - 1;
    uint32_t* kout = kbuf[p & 1];
    int32_t* vout = last ? occ_bm : vbuf[p & 1];
    if (first)
      hipLaunchKernelGGL((k_seg_hist<int64_t, true>), dim3(rgrid), dim3(kThreads), 0, stream,
                         shard_keys, utiles, tile_first, lk, shift, mask, hist,
                         (T > 1 && nseg > 1) ? cnt_t : (uint32_t*)nullptr);
    else
      hipLaunchKernelGGL((k_seg_hist<uint32_t, false>), dim3(rgrid), dim3(kThreads), 0, stream,
                         kbuf[(p - 1) & 1], utiles, tile_first, lk, shift, mask, hist,
                         (uint32_t*)nullptr);
    FS_LAUNCH_CHECK();
    int rc = launch_colscan(hist, kMaxBins, (int32_t)G, (int32_t)mask + 1, part, tot, stream);
    if (rc) return rc;
    if (last && T > 1 && nseg > 1) {
      hipLaunchKernelGGL(k_seg_groups, dim3(1), dim3(kThreads), 0, stream, cnt_t, utiles,
                         tile_first, seg_lo, W, T, delta);
      FS_LAUNCH_CHECK();
    }
    if (first && last)
      hipLaunchKernelGGL((k_seg_scatter<int64_t, true, true>), dim3(rgrid), dim3(kThreads), 0,
                         stream, shard_keys, shard_bm, utiles, tile_first, seg_lo, lk, shift,
                         mask, hist, tot, delta, kout, vout);
    else if (first)
      hipLaunchKernelGGL((k_seg_scatter<int64_t, true, false>), dim3(rgrid), dim3(kThreads), 0,
                         stream, shard_keys, shard_bm, utiles, tile_first, seg_lo, lk, shift,
                         mask, hist, tot, delta, kout, vout);
    else if (last)
      hipLaunchKernelGGL((k_seg_scatter<uint32_t, false, true>), dim3(rgrid), dim3(kThreads), 0,
                         stream, kbuf[(p - 1) & 1], vbuf[(p - 1) & 1], utiles, tile_first,
                         seg_lo, lk, shift, mask, hist, tot, delta, kout, vout);
    else
      hipLaunchKernelGGL((k_seg_scatter<uint32_t, false, false>), dim3(rgrid), dim3(kThreads), 0,
                         stream, kbuf[(p - 1) & 1], vbuf[(p - 1) & 1], utiles, tile_first,
                         seg_lo, lk, shift, mask, hist, tot, delta, kout, vout);
    FS_LAUNCH_CHECK();
    shift += bits;
  }
  const uint32_t* sk = kbuf[(passes - 1) & 1];
  hipLaunchKernelGGL(k_heads, dim3(grid), dim3(kThreads), 0, stream, sk, n_valid, W,
                     tile_heads);
  FS_LAUNCH_CHECK();
  // without previous rows the classes and counts come from the compaction
  // (every row exclusive) and the collision kernels are not launched
  const int32_t no_prev = prev_unique == nullptr;
  if ((int64_t)grid <= kScanTiles) {
    hipLaunchKernelGGL(k_compact_scan, dim3(grid), dim3(kThreads), 0, stream, sk, n_valid, g,
                       tile_heads, no_prev, counts, unique, seg_offsets, occ_uid, unique_offsets,
                       no_prev ? cls : (uint8_t*)nullptr);
    FS_LAUNCH_CHECK();
  } else {
    hipLaunchKernelGGL(k_heads_scan, dim3(1), dim3(kThreads), 0, stream, n_valid, W, T * W,
                       no_prev, tile_heads, counts, seg_offsets, unique_offsets);
    FS_LAUNCH_CHECK();
    hipLaunchKernelGGL(k_compact, dim3(grid), dim3(kThreads), 0, stream, sk, n_valid, g,
                       tile_heads, counts, unique, seg_offsets, occ_uid, unique_offsets,
                       no_prev ? cls : (uint8_t*)nullptr);
    FS_LAUNCH_CHECK();
  }
  if (no_prev) return FS_OK;
  return launch_collide(unique, unique_offsets, n_cap, T, W, prev_unique, prev_unique_offsets,
                        prev_counts, prev_cap, cls, prev_cls, counts, block_hits, stream);
}
