// Device and host helpers shared by the gfx950 kernels of libfs_sparse.
//
// Wavefronts are 64 lanes wide (CDNA). Scans and match-by-value use ballots
// and cross-lane shuffles; workgroup scans go through LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fs_sparse.h"

namespace fs {

constexpr int kWave = 64;

// ---------------------------------------------------------------- lanes
__device__ __forceinline__ int lane() { return (int)__lane_id(); }

// bits of the lanes below this one
__device__ __forceinline__ uint64_t lanemask_lt() {
  int l = lane();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

__device__ __forceinline__ int popc(uint64_t x) { return __popcll(x); }

// lanes of the wave holding the same `bits`-bit value v (all lanes active)
__device__ __forceinline__ uint64_t match_bits(uint32_t v, int bits) {
  uint64_t m = ~0ull;
  for (int b = 0; b < bits; ++b) {
    uint64_t on = __ballot((v >> b) & 1u);
    m &= ((v >> b) & 1u) ? on : ~on;
  }
  return m;
}

// Same as match_bits for any value below the table size, at a few LDS
// operations instead of two VALU steps per bit: every active lane sets its
// bit in tab[v] (a per-wave table of 64-bit lane masks, all zero on entry),
// reads the entry back and the lowest peer clears it again. A wave's LDS
// operations complete in issue order, so the read sees every peer's bit and
// the clear follows every peer's read. Inactive lanes get 0.
__device__ __forceinline__ uint64_t lds_peers(uint64_t* tab, uint32_t v, bool active) {
  const uint64_t me = 1ull << lane();
  uint64_t peers = 0;
  if (active) {
    __hip_atomic_fetch_or(&tab[v], me, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
    peers = __hip_atomic_load(&tab[v], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
  }
  if (active && (peers & (me - 1)) == 0)
    __hip_atomic_store(&tab[v], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
  return peers;
}

template <typename T>
__device__ __forceinline__ T wave_incl_scan(T v) {
  int l = lane();
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    T t = __shfl_up(v, d, kWave);
    if (l >= d) v += t;
  }
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int d = kWave / 2; d > 0; d >>= 1) v += __shfl_xor(v, d, kWave);
  return v;
}

// Exclusive scan over the workgroup (blockDim.x a multiple of 64, <= 1024).
// `tmp` is LDS scratch of at least 17 elements. Returns the exclusive prefix;
// *total receives the workgroup sum. Contains barriers: call uniformly.
template <typename T>
__device__ T block_excl_scan(T v, T* tmp, T* total) {
  int w = threadIdx.x / kWave, nw = blockDim.x / kWave;
  T inc = wave_incl_scan(v);
  if (lane() == kWave - 1) tmp[w] = inc;
  __syncthreads();
  if (w == 0) {
    T x = lane() < nw ? tmp[lane()] : T(0);
    T xi = wave_incl_scan(x);
    if (lane() < nw) tmp[lane()] = xi - x;
    if (lane() == nw - 1) tmp[16] = xi;
  }
  __syncthreads();
  T r = tmp[w] + inc - v;
  *total = tmp[16];
  __syncthreads();
  return r;
}

// Smallest i in [lo, hi] with pred(i) false, for a predicate that is true
// then false over [lo, hi). All lanes of the wave call it with the same
// arguments; each round probes 64 positions in parallel and keeps the gap
// between the last true and the first false probe, so a range of 2^k takes
// about k/6 dependent rounds instead of k.
template <typename P>
__device__ __forceinline__ int64_t wave_partition_point(int64_t lo, int64_t hi, P pred) {
  while (hi - lo > kWave) {
    const int64_t span = hi - lo;
    const int64_t p = lo + (span * (lane() + 1)) / (kWave + 1);
    const int k = popc(__ballot(pred(p)));
    const int64_t nlo = k > 0 ? __shfl(p, k - 1, kWave) + 1 : lo;
    const int64_t nhi = k < kWave ? __shfl(p, k < kWave ? k : 0, kWave) : hi;
    lo = nlo;
    hi = nhi;
  }
  const int64_t p = lo + lane();
  const bool t = p < hi && pred(p);
  return lo + popc(__ballot(t));
}

// ---------------------------------------------------------------- XCDs
// Workgroups are dealt to the 8 XCDs round-robin. With a grid that is a
// multiple of 8, XCD x runs the x-th eighth of the tiles, so neighbouring
// tiles (whose outputs often share cache lines) meet in one L2.
constexpr int kXcd = 8;

__device__ __forceinline__ int32_t xcd_tile(int32_t bid, int32_t G) {
  return (bid % kXcd) * (G / kXcd) + bid / kXcd;
}

// ---------------------------------------------------------------- errors
__device__ __forceinline__ void flag_err(int32_t* err, bool bad, int bit) {
  if (__ballot(bad) && err != nullptr) {
    if (lane() == __ffsll((unsigned long long)__ballot(bad)) - 1) atomicOr(err, bit);
  }
}

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// round-to-nearest-even of the top 16 bits; NaN stays a (quiet) NaN
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (u >> 16) | 0x40u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// ---------------------------------------------------------------- tables
// Row and state strides of a table (0 = dense) and their checks for the
// calls that touch weights: weights 16-byte aligned, row stride a multiple of
// 16 covering the row; with the state (the update): state stride a multiple
// of 4 of at least 4, and a state inside the first row's stride must sit
// past that row's weights.
__host__ inline int64_t table_row_bytes(const fs_table& t) {
  return (int64_t)t.dim * (t.dtype == FS_F32 ? 4 : 2);
}
__host__ inline int64_t table_stride(const fs_table& t) {
  return t.stride ? t.stride : table_row_bytes(t);
}
__host__ inline int64_t table_state_stride(const fs_table& t) {
  return t.state_stride ? t.state_stride : 4;
}
__host__ inline bool table_layout_ok(const fs_table& t, bool with_state) {
  const int64_t rb = table_row_bytes(t), st = table_stride(t), ss = table_state_stride(t);
  if (st < rb || (st & 15) || t.stride < 0) return false;
  if (t.weights && ((uintptr_t)t.weights & 15)) return false;
  if (!with_state) return true;
  if (ss < 4 || (ss & 3) || t.state_stride < 0) return false;
  if (t.state) {
    if ((uintptr_t)t.state & 3) return false;
    const intptr_t off = (intptr_t)t.state - (intptr_t)t.weights;
    if (t.weights && off >= 0 && off < st && (off < rb || off + 4 > st)) return false;
  }
  return true;
}

// ---------------------------------------------------------------- misc
__host__ __device__ __forceinline__ int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

__host__ __device__ __forceinline__ size_t align_up(size_t x, size_t a) {
  return (x + a - 1) / a * a;
}

// bump allocator over a caller workspace
struct Carve {
  char* base;
  size_t used = 0;
  explicit Carve(void* b) : base((char*)b) {}
  template <typename T>
  T* take(size_t count) {
    used = align_up(used, 256);
    T* p = (T*)(base ? base + used : nullptr);
    used += sizeof(T) * count;
    return p;
  }
};

}  // namespace fs

#define FS_LAUNCH_CHECK()                         \
  do {                                            \
    if (hipGetLastError() != hipSuccess) return FS_ERR_HIP; \
  } while (0)
