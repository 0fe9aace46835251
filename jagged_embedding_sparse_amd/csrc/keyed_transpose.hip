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
// Offsets: the feature-major starts go to the workspace, the batch-major
// ones to out_offsets. Up to kOneMax lists one workgroup scans both orders
// (k_kt_offsets1); beyond that, three launches over tiles of kTile lists:
//   k_kt_sums     each tile's length sum in both orders
//   k_kt_scan     one workgroup: exclusive prefixes of the tile sums
//   k_kt_offsets  each tile's exclusive prefixes
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
constexpr int kPer = 8;                     // list entries per thread
constexpr int kTile = kThreads * kPer;      // list entries per offsets tile
constexpr int kScanThreads = 1024;
// lists for the one-workgroup offsets (measured at 4096 lists: 10.5 us
// against 14 us for the tiled launches; at 16384, 24 us against 14) ...
constexpr int kOneMax = 8192;
constexpr int kOneLds = 9216;  // ... whose rows padded to an odd length fit this
constexpr int kCopyThreads = 512;
constexpr int kCopyPer = 8;                        // values per thread
constexpr int kItems = kCopyThreads * kCopyPer;    // merged items per copy workgroup

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

// Both orders' exclusive prefixes in one workgroup (F*B <= kOneMax): the
// lengths are staged in LDS with coalesced loads, all of a thread's loads
// in flight at once (the rows of Bp = B | 1 entries: an odd row stride puts
// the F lists of one sample in different banks); wave w then owns a
// contiguous chunk of entries of each order, sums it, and after the wave
// sums are combined scans it, eight consecutive entries per lane. Writes the
// total to out_offsets[FB]; flags FS_EF_SHAPE for negative lengths (counted
// as zero) and when the total is not n_vals.
__global__ void __launch_bounds__(kScanThreads)
k_kt_offsets1(const int32_t* __restrict__ lengths, uint32_t F, uint32_t B, uint32_t FB,
              DivU32 divF, DivU32 divB, int64_t n_vals, int64_t* __restrict__ in_off,
              int64_t* __restrict__ out_offsets, int32_t* __restrict__ err) {
  constexpr int nw = kScanThreads / kWave;
  constexpr int kStage = kOneMax / kScanThreads;
  __shared__ int32_t s_len[kOneLds];
  __shared__ int64_t s_wf[nw], s_wb[nw];
  const int w = threadIdx.x / kWave, l = lane();
  const uint32_t Bp = B | 1u;
  int32_t x[kStage];
#pragma unroll
  for (int i = 0; i < kStage; ++i) {
    const uint32_t e = threadIdx.x + i * kScanThreads;
    x[i] = e < FB ? lengths[e] : 0;
  }
  bool neg = false;
#pragma unroll
  for (int i = 0; i < kStage; ++i) {
    const uint32_t e = threadIdx.x + i * kScanThreads;
    neg |= x[i] < 0;
    if (e < FB) {
      const uint32_t f = divu32(e, divB), b = e - f * B;
      s_len[f * Bp + b] = x[i] > 0 ? x[i] : 0;
    }
  }
  flag_err(err, neg, FS_EF_SHAPE);
  __syncthreads();
  // wave w owns entries [c0, c1) of each order, taken 512 at a time: lane l
  // scans entries 8l .. 8l+7 of the 512 in registers, so one wave scan (a
  // chain of cross-lane steps) serves 512 entries
  constexpr int R = 8;
  const uint32_t C = (uint32_t)cdiv(FB, nw * kWave * R) * (kWave * R);
  const uint32_t c0 = min(FB, w * C), c1 = min(FB, c0 + C);
  // entry e of the feature-major order is list (e / B, e % B), entry e of
  // the batch-major order list (e % F, e / F)
  auto at_f = [&](uint32_t e) {
    const uint32_t f = divu32(e, divB);
    return s_len[f * Bp + (e - f * B)];
  };
  auto at_b = [&](uint32_t e) {
    const uint32_t b = divu32(e, divF);
    return s_len[(e - b * F) * Bp + b];
  };
  int64_t sf = 0, sb = 0;
  for (uint32_t e = c0 + l; e < c1; e += kWave) {
    sf += at_f(e);
    sb += at_b(e);
  }
  sf = wave_sum(sf);
  sb = wave_sum(sb);
  if (l == 0) {
    s_wf[w] = sf;
    s_wb[w] = sb;
  }
  __syncthreads();
  int64_t xf = 0, xb = 0, tot = 0;
  for (int k = 0; k < nw; ++k) {
    xf += k < w ? s_wf[k] : 0;
    xb += k < w ? s_wb[k] : 0;
    tot += s_wb[k];
  }
  for (uint32_t e0 = c0; e0 < c1; e0 += kWave * R) {
    const uint32_t e1 = e0 + l * R;
    int32_t vf[R], vb[R];
    int64_t lf = 0, lb = 0;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      vf[i] = e1 + i < c1 ? at_f(e1 + i) : 0;
      vb[i] = e1 + i < c1 ? at_b(e1 + i) : 0;
      lf += vf[i];
      lb += vb[i];
    }
    const int64_t incf = wave_incl_scan(lf), incb = wave_incl_scan(lb);
    int64_t pf = xf + incf - lf, pb = xb + incb - lb;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      if (e1 + i < c1) {
        in_off[e1 + i] = pf;
        out_offsets[e1 + i] = pb;
      }
      pf += vf[i];
      pb += vb[i];
    }
    xf += __shfl(incf, kWave - 1, kWave);
    xb += __shfl(incb, kWave - 1, kWave);
  }
  if (threadIdx.x == 0) {
    out_offsets[FB] = tot;
    if (tot != n_vals && err) atomicOr(err, FS_EF_SHAPE);
  }
}

// Values: workgroup blockIdx.x copies the values among merged items
// [d0, d0 + kItems). List s (batch-major index s = b*F + f) has its start
// item at out_offsets[s] + s, followed by its values; a value at output
// position p belongs to the last list whose start is at or before p.
template <typename V>
__global__ void __launch_bounds__(kCopyThreads)
k_kt_copy(const V* __restrict__ values, V* __restrict__ out,
          const int64_t* __restrict__ out_offsets, const int64_t* __restrict__ in_off,
          uint32_t F, uint32_t B, uint32_t FB, DivU32 divF, int64_t n_vals) {
  __shared__ int32_t s_rel[kItems + 1];    // list start - p0, clamped at 0
  __shared__ int64_t s_delta[kItems + 1];  // input start - output start
  __shared__ int64_t s_c[3];
  const int64_t d0 = (int64_t)blockIdx.x * kItems;
  // lists with a start item before d0 and before d0 + kItems, and the value
  // count, fetched side by side
  const int w = threadIdx.x / kWave;
  auto lists_before = [&](int64_t d) {
    return wave_partition_point(0, (int64_t)FB,
                                [&](int64_t s) { return out_offsets[s] + s < d; });
  };
  if (w < 2) {
    const int64_t c = lists_before(d0 + w * kItems);
    if (lane() == 0) s_c[w] = c;
  } else if (w == 2 && lane() == 0) {
    s_c[2] = out_offsets[FB];
  }
  __syncthreads();
  const int64_t d_end = (int64_t)FB + min(s_c[2], n_vals);
  if (d0 >= d_end) return;
  int64_t d1 = d0 + kItems;
  if (d1 > d_end) {  // the last workgroup: the sequence ends inside it
    d1 = d_end;
    if (w == 0) {
      const int64_t c = lists_before(d1);
      if (lane() == 0) s_c[1] = c;
    }
    __syncthreads();
  }
  const int64_t c0 = s_c[0], c1 = s_c[1];
  const int64_t p0 = d0 - c0, p1 = d1 - c1;  // output positions [p0, p1)
  // lists sa .. c1-1 cover them; list sa starts at or before p0
  const int64_t sa = c0 > 0 ? c0 - 1 : 0;
  const int32_t nseg = (int32_t)(c1 - sa);
  for (int32_t j = threadIdx.x; j < nseg; j += kCopyThreads) {
    const uint32_t s = (uint32_t)(sa + j);
    const int64_t lo = out_offsets[s];
    const uint32_t b = divu32(s, divF), f = s - b * F;
    s_rel[j] = (int32_t)max(lo - p0, (int64_t)0);
    s_delta[j] = in_off[(int64_t)f * B + b] - lo;
  }
  __syncthreads();
  if (nseg <= 0) return;
  const int32_t m = (int32_t)(p1 - p0);
  int64_t src[kCopyPer];
  int32_t jlo = 0;  // a thread's positions ascend: each search starts at the last hit
#pragma unroll
  for (int i = 0; i < kCopyPer; ++i) {
    const int32_t q = threadIdx.x + i * kCopyThreads;
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
  V v[kCopyPer];
#pragma unroll
  for (int i = 0; i < kCopyPer; ++i)
    if (src[i] >= 0) v[i] = __builtin_nontemporal_load(values + src[i]);
#pragma unroll
  for (int i = 0; i < kCopyPer; ++i)
    if (src[i] >= 0)
      __builtin_nontemporal_store(v[i], out + p0 + threadIdx.x + i * kCopyThreads);
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
  if (FB <= kOneMax && (int64_t)F * (B | 1) <= kOneLds) {
    hipLaunchKernelGGL(k_kt_offsets1, dim3(1), dim3(kScanThreads), 0, stream, lengths,
                       (uint32_t)F, (uint32_t)B, (uint32_t)FB, divF,
                       make_divu32(B > 0 ? (uint32_t)B : 1u), n_vals, L.in_off, out_offsets,
                       err);
    FS_LAUNCH_CHECK();
  } else {
    hipLaunchKernelGGL(k_kt_sums, dim3((unsigned)G), dim3(kThreads), 0, stream, lengths,
                       (uint32_t)F, (uint32_t)B, (uint32_t)FB, divF, L.tsum_f, L.tsum_b, err);
    FS_LAUNCH_CHECK();
    hipLaunchKernelGGL(k_kt_scan, dim3(1), dim3(kScanThreads), 0, stream, L.tsum_f, L.tsum_b,
                       G, (uint32_t)FB, n_vals, out_offsets, err);
    FS_LAUNCH_CHECK();
    hipLaunchKernelGGL(k_kt_offsets, dim3((unsigned)G), dim3(kThreads), 0, stream, lengths,
                       (uint32_t)F, (uint32_t)B, (uint32_t)FB, divF, L.tsum_f, L.tsum_b,
                       L.in_off, out_offsets);
    FS_LAUNCH_CHECK();
  }
  if (FB == 0 || n_vals == 0) return FS_OK;
  if (elem_bytes == 8)
    hipLaunchKernelGGL(k_kt_copy<uint64_t>, dim3((unsigned)blocks), dim3(kCopyThreads), 0,
                       stream, (const uint64_t*)values, (uint64_t*)out_values, out_offsets, L.in_off,
                       (uint32_t)F, (uint32_t)B, (uint32_t)FB, divF, n_vals);
  else
    hipLaunchKernelGGL(k_kt_copy<uint32_t>, dim3((unsigned)blocks), dim3(kCopyThreads), 0,
                       stream, (const uint32_t*)values, (uint32_t*)out_values, out_offsets, L.in_off,
                       (uint32_t)F, (uint32_t)B, (uint32_t)FB, divF, n_vals);
  FS_LAUNCH_CHECK();
  return FS_OK;
}
