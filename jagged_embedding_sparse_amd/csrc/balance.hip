// Sequence load balancing: FBS and VBS partition functions.
//
// "FreeScale: distributed training for sequence recommendation models",
// section 4.1 (Partitioning Algorithms): both sort the global batch by UIH
// length; FBS deals the sorted samples to ranks zig-zag, VBS cuts them into W
// contiguous segments of about equal weight L^alpha. Inside the load-balancing
// protocol of section 3.1 (Algorithm 1) every rank computes the same P from
// the gathered lengths, so one GPU computing it is exactly what each rank does.
//
// Sort: the batch is small (n <= 16384) and every key (length, index) is
// distinct, so the sorted position of sample s is the number of keys below
// its own. Workgroup (x, y) takes samples 64x .. 64x + 63 and slice y of Q
// slices of the comparands, one lane per sample and a quarter slice per
// wave, and stores the slice's count; a second launch sums the Q counts of
// each sample and places it. O(n^2 / 64) wave instructions over about 512
// workgroups, no atomics, stable by construction. Batches of at most 1024
// samples take one workgroup for the whole partition (k_balance_small).
#include "common.hpp"

namespace fs {
namespace {

// 4 waves, a quarter of the comparand slice each. Workgroups of the index path stay at 256
// threads: a larger one needs that many free wave slots on one CU at once,
// which it does not get while bandwidth-bound kernels of another stream keep
// refilling every slot they free.
constexpr int kRankThreads = 256;
constexpr int kMaxSlices = 16;

__device__ __forceinline__ uint32_t clamp_len(int32_t L) {
  return (uint32_t)(L < 0 ? 0 : (L > FS_MAX_UIH ? FS_MAX_UIH : L));
}

__device__ __forceinline__ uint64_t sort_key(int32_t L, int32_t s) {
  return ((uint64_t)clamp_len(L) << 32) | (uint32_t)s;
}

__device__ __forceinline__ int64_t isqrt64(int64_t x) {
  if (x <= 0) return 0;
  int64_t r = (int64_t)sqrt((double)x);
  while (r * r > x) --r;
  while ((r + 1) * (r + 1) <= x) ++r;
  return r;
}

// round(L^(num/den)) for den in {1, 2}, exact (half-integer powers are
// integers or irrational, so there is no tie to break).
__device__ __forceinline__ int64_t vbs_weight(int64_t L, int num, int den) {
  if (den == 2 && (num & 1) == 0) {
    num >>= 1;
    den = 1;
  }
  int64_t p = 1;
  for (int k = 0; k < num; ++k) p *= L;
  if (den == 1) return p;
  return (isqrt64(4 * p) + 1) / 2;
}

// FBS deal. Sorted position p goes to rank (round even ? p%W : W-1-p%W)
// with round = p/W, as that rank's round-th sample; rank r's first slot is
// r*F plus the ranks before it that got a sample in the final partial round.
__device__ __forceinline__ int32_t fbs_rank_start(int32_t r, int32_t n, int32_t W) {
  int32_t F = n / W, Rm = n % W;
  int32_t extra = (F % 2 == 0) ? min(r, Rm) : max(0, r - (W - Rm));
  return r * F + extra;
}

// comparand slices per sample block: about 512 workgroups in all
inline int32_t rank_slices(int32_t n) {
  const int32_t xb = (int32_t)cdiv(n > 0 ? n : 1, kWave);
  const int32_t q = 512 / xb;
  return q < 1 ? 1 : (q > kMaxSlices ? kMaxSlices : q);
}

// cnt[y * n + s] = keys below sample s's among comparand slice y.
__global__ void __launch_bounds__(kRankThreads)
k_rank_part(const int32_t* __restrict__ len, int32_t n, int32_t* __restrict__ cnt,
            int32_t* __restrict__ err) {
  __shared__ int32_t part[kRankThreads / kWave][kWave];
  const int w = threadIdx.x / kWave, l = lane();
  const int nw = kRankThreads / kWave;
  const int32_t s = blockIdx.x * kWave + l;
  const bool valid = s < n;
  const int32_t Ls = valid ? len[s] : 0;
  if (blockIdx.y == 0 && w == 0)
    flag_err(err, valid && (Ls < 0 || Ls > FS_MAX_UIH), FS_EF_LEN_RANGE);
  const uint64_t mine = sort_key(Ls, s);
  // slice y of the comparands, a quarter per wave, in whole 64-key loads
  // broadcast lane by lane with readlane (uniform operands for the compares)
  const int32_t q = gridDim.y;
  const int32_t chunk = (int32_t)cdiv(cdiv(n, (int64_t)q * nw), kWave) * kWave;
  const int32_t c0 = min(n, ((int32_t)blockIdx.y * nw + w) * chunk), c1 = min(n, c0 + chunk);
  int32_t below = 0;
  for (int32_t cb = c0; cb < c1; cb += kWave) {
    const int32_t c = cb + l;
    const int32_t Lc = c < c1 ? len[c] : 0;
    const int32_t m = min(kWave, c1 - cb);
#pragma unroll 16
    for (int j = 0; j < kWave; ++j) {
      const int32_t Lj = __builtin_amdgcn_readlane(Lc, j);
      below += (j < m) && sort_key(Lj, cb + j) < mine;
    }
  }
  part[w][l] = below;
  __syncthreads();
  if (w == 0 && valid) {
    int32_t p = 0;
    for (int k = 0; k < nw; ++k) p += part[k][l];
    cnt[(int64_t)blockIdx.y * n + s] = p;
  }
}

// Sorted position p of sample s = its Q counts summed; FBS deals p to its
// rank, VBS stores s at p with its weight. With FBS, the first workgroup also
// writes rank_offsets (also for an empty batch).
template <bool kFbs>
__global__ void __launch_bounds__(kRankThreads)
k_place(const int32_t* __restrict__ len, int32_t n, int32_t W, int32_t q,
        const int32_t* __restrict__ cnt, int32_t* __restrict__ perm,
        int32_t* __restrict__ rank_offsets, int64_t* __restrict__ wsorted, int anum, int aden) {
  const int32_t s = blockIdx.x * kRankThreads + threadIdx.x;
  if (s < n) {
    // the q slice counts, all loads in flight at once
    int32_t v[kMaxSlices];
#pragma unroll
    for (int32_t y = 0; y < kMaxSlices; ++y) v[y] = y < q ? cnt[(int64_t)y * n + s] : 0;
    int32_t p = 0;
#pragma unroll
    for (int32_t y = 0; y < kMaxSlices; ++y) p += v[y];
    if (kFbs) {
      int32_t round = p / W, off = p % W;
      int32_t r = (round % 2 == 0) ? off : (W - 1 - off);
      perm[fbs_rank_start(r, n, W) + round] = s;
    } else {
      perm[p] = s;
      wsorted[p] = vbs_weight(clamp_len(len[s]), anum, aden);
    }
  }
  if (kFbs && blockIdx.x == 0)
    for (int32_t r = threadIdx.x; r <= W; r += kRankThreads)
      rank_offsets[r] = r == W ? n : fbs_rank_start(r, n, W);
}

// VBS cuts. With S_k the weight of the first k sorted samples (S_0 = 0,
// S_n = T), rank r starts at the first k with W*S_k >= r*T. S does not
// decrease, so the ranks starting at k+1 are exactly those with
// W*S_k < r*T <= W*S_{k+1}: the thread that holds sample k writes them, and
// the weight at every cut, without a search.
constexpr int kCutThreads = 256;
constexpr int kCutBatch = 16;

// The cuts over the sorted weights wsorted[0 .. n) (global memory or LDS), by
// a workgroup of NT threads; tmp (17) and scut (W + 1) are LDS scratch.
template <int NT>
__device__ __forceinline__ void vbs_cut_body(const int64_t* wsorted, int32_t n, int32_t W,
                                             int32_t* __restrict__ rank_offsets,
                                             int64_t* __restrict__ rank_weight, int64_t* tmp,
                                             int64_t* scut) {
  const int32_t per = (n + NT - 1) / NT;
  const int32_t k0 = min(n, (int32_t)threadIdx.x * per), k1 = min(n, k0 + per);
  // a thread's weights in batches of kCutBatch independent loads (one
  // memory round trip per batch, not per sample)
  int64_t local = 0;
  for (int32_t kb = k0; kb < k1; kb += kCutBatch) {
    int64_t v[kCutBatch];
#pragma unroll
    for (int i = 0; i < kCutBatch; ++i) v[i] = kb + i < k1 ? wsorted[kb + i] : 0;
#pragma unroll
    for (int i = 0; i < kCutBatch; ++i) local += v[i];
  }
  int64_t T;
  int64_t run = block_excl_scan<int64_t>(local, tmp, &T);
  if (T == 0) {  // no samples: every rank starts at 0, the last ends at n
    for (int32_t r = threadIdx.x; r <= W; r += NT) {
      rank_offsets[r] = r == W ? n : 0;
      if (rank_weight && r < W) rank_weight[r] = 0;
    }
    return;
  }
  if (threadIdx.x == 0) {
    rank_offsets[0] = 0;
    rank_offsets[W] = n;
    scut[0] = 0;
    scut[W] = T;
  }
  for (int32_t kb = k0; kb < k1; kb += kCutBatch) {
    int64_t v[kCutBatch];
#pragma unroll
    for (int i = 0; i < kCutBatch; ++i) v[i] = kb + i < k1 ? wsorted[kb + i] : 0;
    for (int i = 0; i < kCutBatch && kb + i < k1; ++i) {
      const int32_t k = kb + i;
      const int64_t s1 = run + v[i];  // S_{k+1}; run = S_k
      // ranks r in [1, W-1] with r > W*S_k / T and r <= W*S_{k+1} / T
      const int64_t r_lo = (int64_t)W * run / T + 1;
      const int64_t r_hi = min((int64_t)W * s1 / T, (int64_t)W - 1);
      for (int64_t r = r_lo; r <= r_hi; ++r) {
        rank_offsets[r] = k + 1;
        scut[r] = s1;
      }
      run = s1;
    }
  }
  __syncthreads();
  if (rank_weight)
    for (int32_t r = threadIdx.x; r < W; r += NT) rank_weight[r] = scut[r + 1] - scut[r];
}

__global__ void __launch_bounds__(kCutThreads)
k_vbs_cut(const int64_t* __restrict__ wsorted, int32_t n, int32_t W,
          int32_t* __restrict__ rank_offsets, int64_t* __restrict__ rank_weight) {
  __shared__ int64_t tmp[17];
  __shared__ int64_t scut[FS_MAX_RANKS + 1];  // S at each rank's first sample
  vbs_cut_body<kCutThreads>(wsorted, n, W, rank_offsets, rank_weight, tmp, scut);
}

// Batches of at most kBalSmallMax samples: one workgroup sorts, deals or
// cuts, in one launch instead of two (FBS) or three (VBS), since for such
// batches the launches cost more than the work. The keys go to LDS; each
// thread ranks its kBalSmallPer samples (the keys below each, counted in one
// pass over the keys), then places them as k_place does; VBS keeps the
// sorted weights in LDS and cuts them as k_vbs_cut does. 256 threads, like
// every workgroup of the index path.
constexpr int kBalSmallMax = 1024;
constexpr int kBalSmallPer = kBalSmallMax / kCutThreads;

template <bool kFbs>
__global__ void __launch_bounds__(kCutThreads)
k_balance_small(const int32_t* __restrict__ len, int32_t n, int32_t W, int anum, int aden,
                int32_t* __restrict__ perm, int32_t* __restrict__ rank_offsets,
                int64_t* __restrict__ rank_weight, int32_t* __restrict__ err) {
  __shared__ uint64_t keys[kBalSmallMax];
  __shared__ int64_t wsorted[kFbs ? 1 : kBalSmallMax];
  __shared__ int64_t tmp[17];
  __shared__ int64_t scut[kFbs ? 1 : FS_MAX_RANKS + 1];
  for (int32_t b = 0; b < n; b += kCutThreads) {  // uniform trip count: flag_err votes
    const int32_t s = b + (int32_t)threadIdx.x;
    const bool valid = s < n;
    const int32_t L = valid ? len[s] : 0;
    flag_err(err, valid && (L < 0 || L > FS_MAX_UIH), FS_EF_LEN_RANGE);
    if (valid) keys[s] = sort_key(L, s);
  }
  __syncthreads();
  uint64_t mine[kBalSmallPer];
  int32_t pos[kBalSmallPer];
#pragma unroll
  for (int i = 0; i < kBalSmallPer; ++i) {
    const int32_t s = (int32_t)threadIdx.x + i * kCutThreads;
    mine[i] = s < n ? keys[s] : ~0ull;
    pos[i] = 0;
  }
  for (int32_t c = 0; c < n; ++c) {
    const uint64_t kc = keys[c];
#pragma unroll
    for (int i = 0; i < kBalSmallPer; ++i) pos[i] += kc < mine[i];
  }
#pragma unroll
  for (int i = 0; i < kBalSmallPer; ++i) {
    const int32_t s = (int32_t)threadIdx.x + i * kCutThreads;
    if (s >= n) continue;
    const int32_t p = pos[i];
    if constexpr (kFbs) {
      const int32_t round = p / W, off = p % W;
      const int32_t r = (round % 2 == 0) ? off : (W - 1 - off);
      perm[fbs_rank_start(r, n, W) + round] = s;
    } else {
      perm[p] = s;
      wsorted[p] = vbs_weight((int64_t)(mine[i] >> 32), anum, aden);  // the clamped length
    }
  }
  if constexpr (kFbs) {
    for (int32_t r = threadIdx.x; r <= W; r += kCutThreads)
      rank_offsets[r] = r == W ? n : fbs_rank_start(r, n, W);
  } else {
    __syncthreads();
    vbs_cut_body<kCutThreads>(wsorted, n, W, rank_offsets, rank_weight, tmp, scut);
  }
}

// VBS cuts with per-rank shares s_r of the weight (the AutoTune mechanism of
// section 4.1 and Figure 4 moves them): with Q_r = s_0 + ... + s_{r-1} and
// Q = Q_W, rank r starts at the first k with Q*S_k >= Q_r*T; equal shares
// give k_vbs_cut's cuts. The products reach 2^96 (Q < 2^50, T < 2^47), so
// they are taken in 128 bits. Shares outside [1, 2^40] are clamped and flag
// FS_EF_SHAPE. Each thread walks its samples in order with a pointer to the
// next rank to place, found once by binary search over the Q_r in LDS.
typedef unsigned __int128 u128;
constexpr int64_t kShareMax = (int64_t)1 << 40;

__device__ __forceinline__ int64_t clamp_share(int64_t x) {
  return x < 1 ? 1 : (x > kShareMax ? kShareMax : x);
}

__global__ void __launch_bounds__(kCutThreads)
k_vbs_cut_shares(const int64_t* __restrict__ wsorted, int32_t n, int32_t W,
                 const int64_t* __restrict__ shares, int32_t* __restrict__ rank_offsets,
                 int64_t* __restrict__ rank_weight, int32_t* __restrict__ err) {
  __shared__ int64_t tmp[17];
  __shared__ int64_t sQ[FS_MAX_RANKS + 1];    // Q_r
  __shared__ int64_t scut[FS_MAX_RANKS + 1];  // S at each rank's first sample
  // prefix of the shares: a few ranks per thread
  const int32_t pw = (W + kCutThreads - 1) / kCutThreads;
  const int32_t q0 = min(W, (int32_t)threadIdx.x * pw), q1 = min(W, q0 + pw);
  int64_t qloc = 0;
  bool bad = false;
  for (int32_t r = q0; r < q1; ++r) {
    const int64_t x = shares[r];
    bad |= x != clamp_share(x);
    qloc += clamp_share(x);
  }
  flag_err(err, bad, FS_EF_SHAPE);
  int64_t Q;
  int64_t qrun = block_excl_scan<int64_t>(qloc, tmp, &Q);
  for (int32_t r = q0; r < q1; ++r) {
    sQ[r] = qrun;
    qrun += clamp_share(shares[r]);
  }
  if (threadIdx.x == 0) sQ[W] = Q;
  // weight prefix, as in k_vbs_cut
  const int32_t per = (n + kCutThreads - 1) / kCutThreads;
  const int32_t k0 = min(n, (int32_t)threadIdx.x * per), k1 = min(n, k0 + per);
  int64_t local = 0;
  for (int32_t kb = k0; kb < k1; kb += kCutBatch) {
    int64_t v[kCutBatch];
#pragma unroll
    for (int i = 0; i < kCutBatch; ++i) v[i] = kb + i < k1 ? wsorted[kb + i] : 0;
#pragma unroll
    for (int i = 0; i < kCutBatch; ++i) local += v[i];
  }
  int64_t T;
  int64_t run = block_excl_scan<int64_t>(local, tmp, &T);  // its barriers publish sQ
  if (T == 0) {  // no weight: every rank starts at 0, the last ends at n
    for (int32_t r = threadIdx.x; r <= W; r += kCutThreads) {
      rank_offsets[r] = r == W ? n : 0;
      if (rank_weight && r < W) rank_weight[r] = 0;
    }
    return;
  }
  if (threadIdx.x == 0) {
    rank_offsets[0] = 0;
    rank_offsets[W] = n;
    scut[0] = 0;
    scut[W] = T;
  }
  const u128 uQ = (u128)(uint64_t)Q, uT = (u128)(uint64_t)T;
  // the first rank r >= 1 whose cut lies beyond S_{k0}: Q_r*T > Q*S_{k0}
  int32_t lo = 1, hi = W;
  const u128 a0 = uQ * (uint64_t)run;
  while (lo < hi) {
    const int32_t mid = (lo + hi) >> 1;
    if ((u128)(uint64_t)sQ[mid] * uT > a0) hi = mid;
    else lo = mid + 1;
  }
  int32_t r = lo;
  for (int32_t kb = k0; kb < k1; kb += kCutBatch) {
    int64_t v[kCutBatch];
#pragma unroll
    for (int i = 0; i < kCutBatch; ++i) v[i] = kb + i < k1 ? wsorted[kb + i] : 0;
    for (int i = 0; i < kCutBatch && kb + i < k1; ++i) {
      const int64_t s1 = run + v[i];  // S_{k+1}
      const u128 b1 = uQ * (uint64_t)s1;
      // ranks with Q*S_k < Q_r*T <= Q*S_{k+1} start at k + 1
      while (r < W && (u128)(uint64_t)sQ[r] * uT <= b1) {
        rank_offsets[r] = kb + i + 1;
        scut[r] = s1;
        ++r;
      }
      run = s1;
    }
  }
  __syncthreads();
  if (rank_weight)
    for (int32_t q = threadIdx.x; q < W; q += kCutThreads) rank_weight[q] = scut[q + 1] - scut[q];
}

int check_common(const int32_t* uih_len, int32_t n, int32_t W, const int32_t* perm,
                 const int32_t* rank_offsets) {
  if (n < 0 || n > FS_MAX_SAMPLES || W < 1 || W > FS_MAX_RANKS) return FS_ERR_INVALID_ARG;
  if (!rank_offsets || (n > 0 && (!uih_len || !perm))) return FS_ERR_INVALID_ARG;
  return FS_OK;
}

}  // namespace
}  // namespace fs

using namespace fs;

// Per-slice count entries of a call with n samples: n * rank_slices(n), which
// drops where the slice count steps down; the query takes the largest over
// every n' <= n (the last n' of each sample-block count), so that a workspace
// sized for n serves every smaller call. Past 512 blocks one slice remains
// and the product only grows.
static size_t max_slice_counts(int32_t n) {
  const int32_t m = n > 0 ? n : 1;
  size_t best = (size_t)m * (size_t)rank_slices(m);
  const int64_t xb_end = cdiv(m, kWave) < 513 ? cdiv(m, kWave) : 513;
  for (int64_t xb = 1; xb <= xb_end; ++xb) {
    const int32_t k = (int32_t)(xb * kWave < m ? xb * kWave : m);
    const size_t v = (size_t)k * (size_t)rank_slices(k);
    best = v > best ? v : best;
  }
  return best;
}

extern "C" size_t fs_balance_workspace_size(int32_t n, int32_t W) {
  (void)W;
  const size_t m = (size_t)(n > 0 ? n : 1);
  Carve c(nullptr);
  c.take<int64_t>(m);                        // sorted weights
  c.take<int32_t>(max_slice_counts(n));      // per-slice counts
  return c.used + 256;
}

namespace {
// both partitions: per-slice counts, then placement
template <bool kFbs>
int launch_sort(const int32_t* uih_len, int32_t n, int32_t W, int32_t* perm,
                int32_t* rank_offsets, int64_t* wsorted, int anum, int aden, int32_t* cnt,
                int32_t* err, hipStream_t stream) {
  const int32_t q = rank_slices(n);
  if (n > 0) {
    hipLaunchKernelGGL(k_rank_part, dim3((unsigned)cdiv(n, kWave), (unsigned)q),
                       dim3(kRankThreads), 0, stream, uih_len, n, cnt, err);
    FS_LAUNCH_CHECK();
  }
  if (n > 0 || kFbs) {
    const int blocks = n > 0 ? (int)cdiv(n, kRankThreads) : 1;
    hipLaunchKernelGGL(k_place<kFbs>, dim3(blocks), dim3(kRankThreads), 0, stream, uih_len, n, W,
                       q, cnt, perm, rank_offsets, wsorted, anum, aden);
    FS_LAUNCH_CHECK();
  }
  return FS_OK;
}
}  // namespace

extern "C" int fs_balance_fbs(const int32_t* uih_len, int32_t n, int32_t W, int32_t* perm,
                              int32_t* rank_offsets, int32_t* err, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  int rc = check_common(uih_len, n, W, perm, rank_offsets);
  if (rc) return rc;
  if (!ws || ws_bytes < fs_balance_workspace_size(n, W)) return FS_ERR_WORKSPACE;
  if (n <= kBalSmallMax) {
    hipLaunchKernelGGL(k_balance_small<true>, dim3(1), dim3(kCutThreads), 0, stream, uih_len, n,
                       W, 0, 1, perm, rank_offsets, (int64_t*)nullptr, err);
    FS_LAUNCH_CHECK();
    return FS_OK;
  }
  Carve c(ws);
  c.take<int64_t>((size_t)(n > 0 ? n : 1));
  int32_t* cnt = c.take<int32_t>((size_t)(n > 0 ? n : 1) * (size_t)rank_slices(n));
  return launch_sort<true>(uih_len, n, W, perm, rank_offsets, nullptr, 0, 1, cnt, err, stream);
}

extern "C" int fs_balance_vbs(const int32_t* uih_len, int32_t n, int32_t W, int32_t alpha_num,
                              int32_t alpha_den, int32_t* perm, int32_t* rank_offsets,
                              int64_t* rank_weight, int32_t* err, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  int rc = check_common(uih_len, n, W, perm, rank_offsets);
  if (rc) return rc;
  bool ok = (alpha_den == 1 && alpha_num >= 0 && alpha_num <= 2) ||
            (alpha_den == 2 && alpha_num >= 0 && alpha_num <= 4);
  if (!ok) return FS_ERR_UNSUPPORTED;
  if (ws_bytes < fs_balance_workspace_size(n, W) || !ws) return FS_ERR_WORKSPACE;
  if (n <= kBalSmallMax) {
    hipLaunchKernelGGL(k_balance_small<false>, dim3(1), dim3(kCutThreads), 0, stream, uih_len,
                       n, W, alpha_num, alpha_den, perm, rank_offsets, rank_weight, err);
    FS_LAUNCH_CHECK();
    return FS_OK;
  }
  Carve c(ws);
  int64_t* wsorted = c.take<int64_t>((size_t)(n > 0 ? n : 1));
  int32_t* cnt = c.take<int32_t>((size_t)(n > 0 ? n : 1) * (size_t)rank_slices(n));
  rc = launch_sort<false>(uih_len, n, W, perm, rank_offsets, wsorted, alpha_num, alpha_den, cnt,
                          err, stream);
  if (rc) return rc;
  hipLaunchKernelGGL(k_vbs_cut, dim3(1), dim3(kCutThreads), 0, stream, wsorted, n, W,
                     rank_offsets, rank_weight);
  FS_LAUNCH_CHECK();
  return FS_OK;
}

extern "C" int fs_balance_vbs_shares(const int32_t* uih_len, int32_t n, int32_t W,
                                     int32_t alpha_num, int32_t alpha_den, const int64_t* shares,
                                     int32_t* perm, int32_t* rank_offsets, int64_t* rank_weight,
                                     int32_t* err, void* ws, size_t ws_bytes, hipStream_t stream) {
  int rc = check_common(uih_len, n, W, perm, rank_offsets);
  if (rc) return rc;
  if (!shares) return FS_ERR_INVALID_ARG;
  bool ok = (alpha_den == 1 && alpha_num >= 0 && alpha_num <= 2) ||
            (alpha_den == 2 && alpha_num >= 0 && alpha_num <= 4);
  if (!ok) return FS_ERR_UNSUPPORTED;
  if (ws_bytes < fs_balance_workspace_size(n, W) || !ws) return FS_ERR_WORKSPACE;
  Carve c(ws);
  int64_t* wsorted = c.take<int64_t>((size_t)(n > 0 ? n : 1));
  int32_t* cnt = c.take<int32_t>((size_t)(n > 0 ? n : 1) * (size_t)rank_slices(n));
  rc = launch_sort<false>(uih_len, n, W, perm, rank_offsets, wsorted, alpha_num, alpha_den, cnt,
                          err, stream);
  if (rc) return rc;
  hipLaunchKernelGGL(k_vbs_cut_shares, dim3(1), dim3(kCutThreads), 0, stream, wsorted, n, W,
                     shares, rank_offsets, rank_weight, err);
  FS_LAUNCH_CHECK();
  return FS_OK;
}
