// VBS AutoTune: per-rank time of a partition and the share update.
//
// "FreeScale: distributed training for sequence recommendation models",
// section 4.1: the VBS weights L^alpha need not match a rank's real
// execution time, so an autotune mechanism (the AutoTune module of
// Figure 4) raises or lowers each rank's local batch size by how its time
// compares with the global average; section 3.1's Algorithm 1 takes that
// runtime information as its input R. Here the local batch sizes are moved
// through per-rank shares of the weight, which fs_balance_vbs_shares cuts by.
//
// k_rank_cost    modelled time per rank: the sum over its samples of
//                c2 L^2 + c1 L + c0 (attention-like plus linear work), one
//                wave per rank
// k_vbs_autotune one step on the shares from per-rank times (measured or
//                modelled), one workgroup, all integer: the decisions compare
//                W t_r tol_den with (sum t)(tol_den +- tol_num) in 128 bits
#include "common.hpp"

namespace fs {
namespace {

typedef __int128 i128;
constexpr int64_t kShareMax = (int64_t)1 << 40;
constexpr int64_t kTimeMax = (int64_t)1 << 52;
constexpr int kCostThreads = 256;
constexpr int kTuneThreads = 1024;  // one rank per thread: W <= FS_MAX_RANKS

__global__ void __launch_bounds__(kCostThreads)
k_rank_cost(const int32_t* __restrict__ uih_len, int32_t n, const int32_t* __restrict__ perm,
            const int32_t* __restrict__ rank_offsets, int32_t W, int64_t c2, int64_t c1,
            int64_t c0, int64_t* __restrict__ cost) {
  const int32_t r = blockIdx.x * (kCostThreads / kWave) + threadIdx.x / kWave;
  if (r >= W) return;
  // offsets outside [0, n] or decreasing are clipped (the rank then counts
  // fewer samples); sample indices outside [0, n) count nothing
  const int32_t a = min(max(rank_offsets[r], 0), n);
  const int32_t b = min(max(rank_offsets[r + 1], a), n);
  int64_t t = 0;
  for (int32_t j = a + lane(); j < b; j += kWave) {
    const int32_t s = perm[j];
    if (s < 0 || s >= n) continue;
    const int32_t Lr = uih_len[s];
    const int64_t L = Lr < 0 ? 0 : (Lr > FS_MAX_UIH ? FS_MAX_UIH : Lr);
    t += c2 * L * L + c1 * L + c0;
  }
  t = wave_sum(t);
  if (lane() == 0) cost[r] = t;
}

__global__ void __launch_bounds__(kTuneThreads)
k_vbs_autotune(const int64_t* __restrict__ times, int32_t W, int32_t step_num,
               int32_t step_den, int32_t tol_num, int32_t tol_den, int64_t* __restrict__ shares,
               int32_t* __restrict__ err) {
  __shared__ int64_t tmp[17];
  const int32_t r = threadIdx.x;
  int64_t t = 0, s = 1;
  bool bad = false;
  if (r < W) {
    t = times[r];
    s = shares[r];
    bad = t < 0 || t > kTimeMax || s < 1 || s > kShareMax;
    t = t < 0 ? 0 : (t > kTimeMax ? kTimeMax : t);
    s = s < 1 ? 1 : (s > kShareMax ? kShareMax : s);
  }
  flag_err(err, bad, FS_EF_SHAPE);
  int64_t sum;
  block_excl_scan<int64_t>(r < W ? t : 0, tmp, &sum);
  if (r >= W) return;
  const i128 lhs = (i128)W * t * tol_den;
  int64_t d = s * step_num / step_den;
  d = d < 1 ? 1 : d;
  if (lhs > (i128)sum * (tol_den + tol_num)) {  // slower than the mean: give up weight
    s = s - d < 1 ? 1 : s - d;
  } else if (lhs < (i128)sum * (tol_den - tol_num)) {  // faster: take more
    s = s + d > kShareMax ? kShareMax : s + d;
  }
  shares[r] = s;
}

}  // namespace
}  // namespace fs

using namespace fs;

extern "C" int fs_rank_cost(const int32_t* uih_len, int32_t n, const int32_t* perm,
                            const int32_t* rank_offsets, int32_t W, int64_t c2, int64_t c1,
                            int64_t c0, int64_t* cost, hipStream_t stream) {
  if (n < 0 || n > FS_MAX_SAMPLES || W < 1 || W > FS_MAX_RANKS || !rank_offsets || !cost)
    return FS_ERR_INVALID_ARG;
  if (n > 0 && (!uih_len || !perm)) return FS_ERR_INVALID_ARG;
  // c2 * 65535^2 * 16384 + ... stays below 2^63 for coefficients up to 2^16
  const int64_t cmax = (int64_t)1 << 16;
  if (c2 < 0 || c1 < 0 || c0 < 0 || c2 > cmax || c1 > cmax || c0 > cmax)
    return FS_ERR_INVALID_ARG;
  hipLaunchKernelGGL(k_rank_cost, dim3((unsigned)cdiv(W, kCostThreads / kWave)),
                     dim3(kCostThreads), 0, stream, uih_len, n, perm, rank_offsets, W, c2, c1, c0,
                     cost);
  FS_LAUNCH_CHECK();
  return FS_OK;
}

extern "C" int fs_vbs_autotune(const int64_t* times, int32_t W, int32_t step_num,
                               int32_t step_den, int32_t tol_num, int32_t tol_den,
                               int64_t* shares, int32_t* err, hipStream_t stream) {
  if (W < 1 || W > FS_MAX_RANKS || !times || !shares) return FS_ERR_INVALID_ARG;
  const int32_t lim = 1 << 20;
  if (step_den < 1 || step_den > lim || step_num < 0 || step_num > step_den || tol_den < 1 ||
      tol_den > lim || tol_num < 0 || tol_num > tol_den)
    return FS_ERR_INVALID_ARG;
  hipLaunchKernelGGL(k_vbs_autotune, dim3(1), dim3(kTuneThreads), 0, stream, times, W, step_num,
                     step_den, tol_num, tol_den, shares, err);
  FS_LAUNCH_CHECK();
  return FS_OK;
}
