// Keyed transpose: a jagged tensor keyed by feature, from feature-major to
// batch-major order.
//
// "FreeScale: distributed training for sequence recommendation models",
// section 4.2 lists the keyed transpose among its jagged-tensor kernels: the
// values of F features over B samples arrive feature by feature (list (f, b)
// of lengths[f*B + b] values after every list (f', b') with f' < f, or
// f' = f and b' < b) and leave sample by sample (list (b, f) after every
// (b', f') with b' < b, or b' = b and f' < f); each list keeps its order.
//
// Offsets, three launches over tiles of kTile list entries:
//   k_kt_sums     each tile's length sum in both orders
//   k_kt_scan     one workgroup: exclusive prefixes of the tile sums
//   k_kt_offsets  each tile's exclusive prefixes -- the feature-major starts
//                 to the workspace, the batch-major ones to out_offsets
// Values, one launch (k_kt_copy): a merge-path split of the batch-major
// sequence in which every list contributes one start item followed by one
// item per value. Each workgroup takes kItems consecutive items, so lists of
// any length mix (empty, one value, thousands) cost the same per item; it
// finds its first and last list by a search over out_offsets, stages its
// lists' starts in LDS and each value finds its list there by binary search.
// Loads and stores are one element per lane, in output order.
#include "common.hpp"
#include "divu32.hpp"

namespace fs {
namespace {

constexpr int kThreads = 256;
constexpr int kPer = 8;                    // list entries (or values) per thread
constexpr int kTile = kThreads * kPer;     // list entries per offsets tile
constexpr int kItems = kThreads * kPer;    // merged items per copy workgroup
constexpr int kScanThreads = 1024;

// Sums of the lengths of tile blockIdx.x in feature-major order (entries
// e = f*B + b) and in batch-major order (entries e = b*F + f, length
// lengths[f*B + b]). Negative lengths count as zero and flag FS_EF_SHAPE.
__global__ void __launch_bounds__(kThreads)
k_kt_sums(const int32_t* __restrict__ lengths, uint32_t F, uint32_t B, uint32_t FB,
          DivU32 divF, int64_t* __restrict__ tsum_f, int64_t* __restrict__ tsum_b,
          int32_t* __restrict__ err) {
  __shared__ int64_t tmp[17];
  const uint32_t tile0 = blockIdx.x * (uint32_t)kTile;
  // feature-major: lane-strided, so each load instruction is coalesced
  int32_t vf[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const uint32_t e = tile0 + threadIdx.x + i * kThreads;
    vf[i] = e < FB ? lengths[e] : 0;
  }
  // batch-major: kPer consecutive entries per thread, (b, f) stepped along
  const uint32_t e0 = tile0 + threadIdx.x * kPer;
  uint32_t b = divu32(e0, divF), f = e0 - b * F;
  int32_t vb[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    vb[i] = e0 + i < FB ? lengths[(int64_t)f * B + b] : 0;
    if (++f == F) {
      f = 0;
      ++b;
    }
  }
  int64_t sf = 0, sb = 0;
  bool neg = false;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    neg |= vf[i] < 0;
    sf += vf[i] > 0 ? vf[i] : 0;
    sb += vb[i] > 0 ? vb[i] : 0;
  }
  flag_err(err, neg, FS_EF_SHAPE);
  sf = wave_sum(sf);
  sb = wave_sum(sb);
  const int w = threadIdx.x / kWave;
  if (lane() == 0) {
    tmp[w] = sf;
    tmp[8 + w] = sb;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t a = 0, c = 0;
    for (int x = 0; x < kThreads / kWave; ++x) {
      a += tmp[x];
      c += tmp[8 + x];
    }
    tsum_f[blockIdx.x] = a;
    tsum_b[blockIdx.x] = c;
  }
}

// Tile sums -> exclusive tile prefixes (in place), one workgroup. Writes the
// total to out_offsets[FB] and flags FS_EF_SHAPE when it is not n_vals.
__global__ void __launch_bounds__(kScanThreads)
k_kt_scan(int64_t* __restrict__ tsum_f, int64_t* __restrict__ tsum_b, int32_t G, uint32_t FB,
          int64_t n_vals, int64_t* __restrict__ out_offsets, int32_t* __restrict__ err) {
  __shared__ int64_t tmp[17];
  const int32_t per = (int32_t)cdiv(G, kScanThreads);
  const int32_t g0 = min(G, (int32_t)threadIdx.x * per), g1 = min(G, g0 + per);
  int64_t sf = 0, sb = 0;
  for (int32_t g = g0; g < g1; ++g) {
    sf += tsum_f[g];
    sb += tsum_b[g];
  }
  int64_t tot_f, tot_b;
  int64_t bf = block_excl_scan(sf, tmp, &tot_f);
  int64_t bb = block_excl_scan(sb, tmp, &tot_b);
  for (int32_t g = g0; g < g1; ++g) {
    const int64_t xf = tsum_f[g], xb = tsum_b[g];
    tsum_f[g] = bf;
    tsum_b[g] = bb;
    bf += xf;
    bb += xb;
  }
  if (threadIdx.x == 0) {
    out_offsets[FB] = tot_b;
    if (tot_b != n_vals && err) atomicOr(err, FS_EF_SHAPE);
  }
}

// Exclusive prefixes of tile blockIdx.x in both orders.
__global__ void __launch_bounds__(kThreads)
k_kt_offsets(const int32_t* __restrict__ lengths, uint32_t F, uint32_t B, uint32_t FB,
             DivU32 divF, const int64_t* __restrict__ tbase_f,
             const int64_t* __restrict__ tbase_b, int64_t* __restrict__ in_off,
             int64_t* __restrict__ out_offsets) {
  __shared__ int64_t tmp[17];
  const uint32_t e0 = blockIdx.x * (uint32_t)kTile + threadIdx.x * kPer;
  uint32_t b = divu32(e0, divF), f = e0 - b * F;
  int32_t vf[kPer], vb[kPer];
  int64_t sf = 0, sb = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const bool on = e0 + i < FB;
    vf[i] = on ? lengths[e0 + i] : 0;
    vb[i] = on ? lengths[(int64_t)f * B + b] : 0;
    vf[i] = vf[i] > 0 ? vf[i] : 0;
    vb[i] = vb[i] > 0 ? vb[i] : 0;
    sf += vf[i];
    sb += vb[i];
    if (++f == F) {
      f = 0;
      ++b;
    }
  }
  int64_t tot;
  int64_t xf = block_excl_scan(sf, tmp, &tot) + tbase_f[blockIdx.x];
  int64_t xb = block_excl_scan(sb, tmp, &tot) + tbase_b[blockIdx.x];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (e0 + i < FB) {
      in_off[e0 + i] = xf;
      out_offsets[e0 + i] = xb;
    }
    xf += vf[i];
    xb += vb[i];
  }
}

// Values: workgroup blockIdx.x copies the values among merged items
// [d0, d0 + kItems). List s (batch-major index s = b*F + f) has its start
// item at out_offsets[s] + s, followed by its values; a value at output
// position p belongs to the last list whose start is at or before p.
template <typename V>
__global__ void __launch_bounds__(kThreads)
k_kt_copy(const V* __restrict__ values, V* __restrict__ out,
          const int64_t* __restrict__ out_offsets, const int64_t* __restrict__ in_off,
          uint32_t F, uint32_t B, uint32_t FB, DivU32 divF, int64_t n_vals) {
  __shared__ int32_t s_rel[kItems + 1];    // list start - p0, clamped at 0
  __shared__ int64_t s_delta[kItems + 1];  // input start - output start
  __shared__ int64_t s_c[2];
  const int64_t n_dev = out_offsets[FB];
  const int64_t d_end = (int64_t)FB + min(n_dev, n_vals);
  const int64_t d0 = (int64_t)blockIdx.x * kItems;
  if (d0 >= d_end) return;
  const int64_t d1 = min(d0 + kItems, d_end);
  // lists with a start item before d0 and before d1
  const int w = threadIdx.x / kWave;
  if (w < 2) {
    const int64_t d = w == 0 ? d0 : d1;
    const int64_t c = wave_partition_point(
        0, (int64_t)FB, [&](int64_t s) { return out_offsets[s] + s < d; });
    if (lane() == 0) s_c[w] = c;
  }
  __syncthreads();
  const int64_t c0 = s_c[0], c1 = s_c[1];
  const int64_t p0 = d0 - c0, p1 = d1 - c1;  // output positions [p0, p1)
  // lists sa .. c1-1 cover them; list sa starts at or before p0
  const int64_t sa = c0 > 0 ? c0 - 1 : 0;
  const int32_t nseg = (int32_t)(c1 - sa);
  for (int32_t j = threadIdx.x; j < nseg; j += kThreads) {
    const uint32_t s = (uint32_t)(sa + j);
    const int64_t lo = out_offsets[s];
    const uint32_t b = divu32(s, divF), f = s - b * F;
    s_rel[j] = (int32_t)max(lo - p0, (int64_t)0);
    s_delta[j] = in_off[(int64_t)f * B + b] - lo;
  }
  __syncthreads();
  if (nseg <= 0) return;
  const int32_t m = (int32_t)(p1 - p0);
  int64_t src[kPer];
  int32_t jlo = 0;  // a thread's positions ascend: each search starts at the last hit
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int32_t q = threadIdx.x + i * kThreads;
    int32_t lo = jlo, hi = nseg;  // last j with s_rel[j] <= q
    while (hi - lo > 1) {
      const int32_t mid = (lo + hi) >> 1;
      if (s_rel[mid] <= q) lo = mid;
      else hi = mid;
    }
    jlo = lo;
    const int64_t p = p0 + q;
    const int64_t sp = s_delta[lo] + p;
    src[i] = (q < m && p < n_vals && sp >= 0 && sp < n_vals) ? sp : -1;
  }
  V v[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if (src[i] >= 0) v[i] = __builtin_nontemporal_load(values + src[i]);
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if (src[i] >= 0)
      __builtin_nontemporal_store(v[i], out + p0 + threadIdx.x + i * kThreads);
}

struct KtLayout {
  int64_t *tsum_f, *tsum_b, *in_off;
  size_t bytes;
};

KtLayout kt_layout(void* ws, int64_t FB) {
  Carve c(ws);
  KtLayout L;
  const int64_t G = cdiv(FB, kTile);
  L.tsum_f = c.take<int64_t>((size_t)(G > 0 ? G : 1));
  L.tsum_b = c.take<int64_t>((size_t)(G > 0 ? G : 1));
  L.in_off = c.take<int64_t>((size_t)(FB > 0 ? FB : 1));
  L.bytes = align_up(c.used, 256);
  return L;
}

}  // namespace
}  // namespace fs

using namespace fs;

extern "C" size_t fs_keyed_transpose_workspace_size(int32_t F, int32_t B) {
  if (F < 0 || B < 0) return 0;
  return kt_layout(nullptr, (int64_t)F * B).bytes;
}

extern "C" int fs_keyed_transpose(const void* values, int64_t n_vals, int32_t elem_bytes,
                                  const int32_t* lengths, int32_t F, int32_t B,
                                  void* out_values, int64_t* out_offsets, int32_t* err,
                                  void* ws, size_t ws_bytes, hipStream_t stream) {
  if (F < 0 || B < 0 || (int64_t)F * B >= (int64_t)INT32_MAX || n_vals < 0 || !out_offsets)
    return FS_ERR_INVALID_ARG;
  if (elem_bytes != 4 && elem_bytes != 8) return FS_ERR_UNSUPPORTED;
  const int64_t FB = (int64_t)F * B;
  if (FB > 0 && !lengths) return FS_ERR_INVALID_ARG;
  if (n_vals > 0 && (!values || !out_values || ((uintptr_t)values % elem_bytes) ||
                     ((uintptr_t)out_values % elem_bytes)))
    return FS_ERR_INVALID_ARG;
  if (n_vals > (INT64_MAX - FB - kItems) / 2) return FS_ERR_INVALID_ARG;
  const int64_t blocks = cdiv(FB + n_vals, kItems);
  if (blocks > (int64_t)INT32_MAX) return FS_ERR_UNSUPPORTED;
  const KtLayout L = kt_layout(ws, FB);
  if (!ws || ws_bytes < L.bytes) return FS_ERR_WORKSPACE;
  const int32_t G = (int32_t)cdiv(FB, kTile);
  const DivU32 divF = make_divu32(F > 0 ? (uint32_t)F : 1u);
  if (G > 0) {
    hipLaunchKernelGGL(k_kt_sums, dim3((unsigned)G), dim3(kThreads), 0, stream, lengths,
                       (uint32_t)F, (uint32_t)B, (uint32_t)FB, divF, L.tsum_f, L.tsum_b, err);
    FS_LAUNCH_CHECK();
  }
  hipLaunchKernelGGL(k_kt_scan, dim3(1), dim3(kScanThreads), 0, stream, L.tsum_f, L.tsum_b, G,
                     (uint32_t)FB, n_vals, out_offsets, err);
  FS_LAUNCH_CHECK();
  if (G == 0) return FS_OK;
  hipLaunchKernelGGL(k_kt_offsets, dim3((unsigned)G), dim3(kThreads), 0, stream, lengths,
                     (uint32_t)F, (uint32_t)B, (uint32_t)FB, divF, L.tsum_f, L.tsum_b, L.in_off,
                     out_offsets);
  FS_LAUNCH_CHECK();
  if (n_vals == 0) return FS_OK;
  if (elem_bytes == 8)
    hipLaunchKernelGGL(k_kt_copy<uint64_t>, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                       (const uint64_t*)values, (uint64_t*)out_values, out_offsets, L.in_off,
                       (uint32_t)F, (uint32_t)B, (uint32_t)FB, divF, n_vals);
  else
    hipLaunchKernelGGL(k_kt_copy<uint32_t>, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                       (const uint32_t*)values, (uint32_t*)out_values, out_offsets, L.in_off,
                       (uint32_t)F, (uint32_t)B, (uint32_t)FB, divF, n_vals);
  FS_LAUNCH_CHECK();
  return FS_OK;
}
