// Exclusive column scans of a row-major matrix of 32-bit counts (rows =
// tiles in output order, columns = bins), in place. Lanes are columns, so
// every row load is coalesced. Large matrices: each wave takes 32
// consecutive rows, each workgroup 128, in two launches over (row blocks) x
// (column groups of 64): k_colsum stores each row block's column sums,
// k_colscan adds the sums of the row blocks before its own and rewrites the
// rows as exclusive prefixes. Small matrices: one launch (k_colscan1).
// A caller that knows on the device how many leading rows are in use passes
// that count (g_used, nullable): rows past it are all zero, so they are
// neither read nor rewritten.
#pragma once

#include "common.hpp"

namespace fs {
namespace {

constexpr int kColThreads = 256;
constexpr int kColRows = 32;
constexpr int kColBlockRows = kColRows * (kColThreads / kWave);

__global__ void __launch_bounds__(kColThreads)
k_colsum(const uint32_t* __restrict__ counts, int32_t ld, int32_t G, int32_t C,
         uint32_t* __restrict__ part, const int32_t* __restrict__ g_used) {
  __shared__ uint32_t wsum[kColThreads / kWave][kWave];
  if (g_used) G = max(1, min(G, *g_used));
  const int w = threadIdx.x / kWave, l = lane();
  const int32_t c = blockIdx.y * kWave + l;
  const int32_t r0 = blockIdx.x * kColBlockRows + w * kColRows;
  // rows past G read row G - 1 and count zero: the loads stay unconditional,
  // so all 32 are in flight at once
  const int32_t cc = c < C ? c : C - 1;
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < kColRows; ++i) {
    const uint32_t x = counts[(int64_t)min(r0 + i, G - 1) * ld + cc];
    s += (c < C && r0 + i < G) ? x : 0u;
  }
  wsum[w][l] = s;
  __syncthreads();
  if (w == 0 && c < C)
    part[(int64_t)blockIdx.x * ld + c] = wsum[0][l] + wsum[1][l] + wsum[2][l] + wsum[3][l];
}

// counts[r][c] <- sum of counts[r'][c] over r' < r; tot[c] <- column total.
__global__ void __launch_bounds__(kColThreads)
k_colscan(uint32_t* __restrict__ counts, int32_t ld, int32_t G, int32_t C,
          const uint32_t* __restrict__ part, uint32_t* __restrict__ tot,
          const int32_t* __restrict__ g_used) {
  __shared__ uint32_t wsum[kColThreads / kWave][kWave];
  if (g_used) G = max(1, min(G, *g_used));
  const int w = threadIdx.x / kWave, l = lane();
  const int32_t c = blockIdx.y * kWave + l;
  const int32_t r0 = blockIdx.x * kColBlockRows + w * kColRows;
  const bool on = c < C;
  const int32_t cc = on ? c : C - 1;
  uint32_t v[kColRows];
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < kColRows; ++i) {
    const uint32_t x = counts[(int64_t)min(r0 + i, G - 1) * ld + cc];
    v[i] = (on && r0 + i < G) ? x : 0u;
    s += v[i];
  }
  // sums of the earlier row blocks, 8 independent loads at a time
  uint32_t base = 0;
  for (int32_t k0 = 0; k0 < (int32_t)blockIdx.x; k0 += 8) {
    uint32_t b8[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      b8[j] = part[(int64_t)min(k0 + j, (int32_t)blockIdx.x - 1) * ld + cc];
#pragma unroll
    for (int j = 0; j < 8; ++j) base += (k0 + j < (int32_t)blockIdx.x) ? b8[j] : 0u;
  }
  wsum[w][l] = s;
  __syncthreads();
  for (int x = 0; x < w; ++x) base += wsum[x][l];
  if (!on) return;
#pragma unroll
  for (int i = 0; i < kColRows; ++i) {
    if (r0 + i < G) counts[(int64_t)(r0 + i) * ld + c] = base;
    base += v[i];
  }
  if (blockIdx.x == gridDim.x - 1 && w == kColThreads / kWave - 1) tot[c] = base;
}

// Small matrices (G <= kColOneRows): one launch, one workgroup of eight
// waves per group of 64 columns. Each wave sums a contiguous slice of the
// rows (kColBatch loads in flight per lane), the waves' slice sums are
// combined in LDS, then each wave rereads its slice and writes the exclusive
// prefixes. Eight waves halve each wave's chain of dependent loads against
// four (measured: workload 3 step 0.293 -> 0.282 ms).
constexpr int kColOneRows = 1024;
constexpr int kColBatch = 32;
constexpr int kColOneThreads = 512;

__global__ void __launch_bounds__(kColOneThreads)
k_colscan1(uint32_t* __restrict__ counts, int32_t ld, int32_t G, int32_t C,
           uint32_t* __restrict__ tot, const int32_t* __restrict__ g_used) {
  __shared__ uint32_t wsum[kColOneThreads / kWave][kWave];
  if (g_used) G = min(G, *g_used);
  constexpr int nw = kColOneThreads / kWave;
  // the wave index made provably uniform: row addresses then live in scalar
  // registers and each load needs only the lane's column offset
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), l = lane();
  const int32_t c = blockIdx.x * kWave + l;
  const bool on = c < C;
  const uint32_t cc = (uint32_t)(on ? c : C - 1);
  const int32_t per = (int32_t)cdiv(G, nw);
  const int32_t r0 = min(G, w * per), r1 = min(G, r0 + per);
  uint32_t s = 0;
  for (int32_t rb = r0; rb < r1; rb += kColBatch) {
    uint32_t v[kColBatch];
#pragma unroll
    for (int i = 0; i < kColBatch; ++i)
      v[i] = (counts + (int64_t)min(rb + i, G - 1) * ld)[cc];
#pragma unroll
    for (int i = 0; i < kColBatch; ++i) s += rb + i < r1 ? v[i] : 0u;
  }
  wsum[w][l] = s;
  __syncthreads();
  uint32_t base = 0;
  for (int x = 0; x < w; ++x) base += wsum[x][l];
  if (w == nw - 1 && on) tot[c] = base + s;
  if (!on) return;
  for (int32_t rb = r0; rb < r1; rb += kColBatch) {
    uint32_t v[kColBatch];
#pragma unroll
    for (int i = 0; i < kColBatch; ++i)
      v[i] = (counts + (int64_t)min(rb + i, G - 1) * ld)[cc];
#pragma unroll
    for (int i = 0; i < kColBatch; ++i) {
      if (rb + i < r1) {
        (counts + (int64_t)(rb + i) * ld)[cc] = base;
        base += v[i];
      }
    }
  }
}

// The column scan of a G x C matrix with leading dimension ld: one launch
// when G <= one_rows, else block sums then prefixes; part holds
// cdiv(G, 128) * ld entries, tot C. g_used: see above.
inline int launch_colscan(uint32_t* counts, int32_t ld, int32_t G, int32_t C, uint32_t* part,
                          uint32_t* tot, hipStream_t stream, const int32_t* g_used = nullptr,
                          int32_t one_rows = kColOneRows) {
  if (G <= one_rows) {
    hipLaunchKernelGGL(k_colscan1, dim3((unsigned)cdiv(C, kWave)), dim3(kColOneThreads), 0,
                       stream, counts, ld, G, C, tot, g_used);
    FS_LAUNCH_CHECK();
    return FS_OK;
  }
  const dim3 grid((unsigned)cdiv(G, kColBlockRows), (unsigned)cdiv(C, kWave));
  hipLaunchKernelGGL(k_colsum, grid, dim3(kColThreads), 0, stream, counts, ld, G, C, part,
                     g_used);
  FS_LAUNCH_CHECK();
  hipLaunchKernelGGL(k_colscan, grid, dim3(kColThreads), 0, stream, counts, ld, G, C, part, tot,
                     g_used);
  FS_LAUNCH_CHECK();
  return FS_OK;
}

}  // namespace
}  // namespace fs
