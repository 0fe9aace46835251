// Gradient segment-reduce per unique row, fused with the row-wise update.
//
// "FreeScale: distributed training for sequence recommendation models",
// Algorithm 2: backward splits the batch-major gradients into collision and
// exclusive parts and sends them to the row shards, where update_embedding
// applies them; collision rows first, so the next iteration reads them
// updated (section 3.2), exclusive rows at leisure. The optimizer is not
// named on the pages; SGD and row-wise Adagrad are supported.
//
// g_u = sum of grad[bm] over u's occurrences, accumulated in fp64 and rounded
// once to fp32, so the result does not depend on how the sum is split.
// Zipf IDs make segment lengths span 1 .. ~10^5, so three kernels:
//   short rows (<= kShort = 4 occurrences, most rows): one lane group per
//     row, grid-stride over the table's unique rows; all of a row's loads
//     are in flight at once, then the group sums and updates the row.
//   medium rows (kShort < len < kChunkMin = 65): one lane group per row as
//     well; the group loads all of the row's occurrence indices with one
//     load and streams its gradient rows 8 or 16 at a time.
//   long rows: the table's occurrence range is cut into chunks (128 to 512
//     occurrences, smaller for smaller batches so that the grid still has
//     about two chunks per resident wave);
//     a wave streams each long row's piece of its chunk (all lane groups of
//     the wave interleaved), updates rows that lie inside the chunk and
//     leaves fp64 partials for the rest; a fix-up sums each row's partials
//     in chunk order and updates it.
// Lanes: a group of LPG = min(64, D/4) lanes covers a row, 4*CPL/4 columns
// per lane (16-byte gradient loads); weights use the same column mapping.
#include <mutex>

#include "common.hpp"

namespace fs {
namespace {

constexpr int kThreads = 256;
constexpr int kShort = 4;      // rows whose loads all go out at once
constexpr int kChunkMin = 65;  // rows this long or longer take the chunked path
constexpr int kMedBatch = 8;   // gradient rows in flight per lane group (medium rows)
// occurrences per long-path chunk (one wave): the largest of 512, 256, 128
// that leaves about two chunks per resident wave (5 per SIMD)
constexpr int64_t kChunkTarget = 2 * 256 * 4 * 5;
constexpr int64_t kChunk256From = 256 * kChunkTarget;  // first n_tok with 256-chunks
constexpr int64_t kChunk512From = 512 * kChunkTarget;  // first n_tok with 512-chunks
inline int64_t chunk_for(int64_t n_tok) {
  return n_tok >= kChunk512From ? 512 : (n_tok >= kChunk256From ? 256 : 128);
}
constexpr int kShortBlocks = 4096;
// gradient rows in flight per lane group on the long-row path (8, 12 and 16
// measured the same: the path runs at the device's rate for random 512-B rows)
constexpr int kLongBatch = 8;
// waves of the short-row kernel the GPU holds at once (256 CUs x 4 SIMDs x
// 5 waves of ~90 registers); the unit size aims at two or more units each
constexpr int64_t kResident = 256 * 4 * 5;

struct RUArgs {
  void* weights;
  float* state;
  int64_t stride;        // bytes between weight rows
  int64_t state_stride;  // bytes between rows' states
  const float* grad;
  float* reduced;  // may be null
  const int64_t* unique;
  const int64_t* unique_offsets;
  const int32_t* seg_offsets;
  const int32_t* occ_bm;
  const int32_t* occ_uid;
  const uint8_t* cls;
  double* partials;  // [chunks][2][D]
  int64_t chunk;     // occurrences per long-path chunk
  int64_t row_base;
  int64_t n_cap;  // occurrences this table can have
  int32_t g_lo, g_hi;
  int32_t which, optim;
  float lr, eps;
};

template <int D>
struct Map {
  static constexpr int LPG = (D / 4) < kWave ? (D / 4) : kWave;  // lanes per row
  static constexpr int CPL = D / LPG;                            // columns per lane
  static constexpr int NV = CPL / 4;                             // float4 per lane
  static constexpr int GPW = kWave / LPG;                        // groups per wave
  __device__ static int col(int sub, int v) { return 4 * (sub + v * LPG); }
};

// Gradient rows are read exactly once: streaming (non-temporal) loads keep
// them from displacing the weight rows, Adagrad state and fp64 partials in
// the caches (measured: 1060 -> 1021 us per update at workload 5).
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 ld_stream(const float4* p) {
  const f32x4 v = __builtin_nontemporal_load((const f32x4*)p);
  return make_float4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float* state_at(const RUArgs& a, int64_t row) {
  return (float*)((char*)a.state + row * a.state_stride);
}

__device__ __forceinline__ bool class_ok(const RUArgs& a, int64_t u) {
  return a.which < 0 || a.cls[u] == (uint8_t)a.which;
}

template <int D>
__device__ __forceinline__ void add_row(double (&acc)[Map<D>::CPL], const float* grad, int64_t bm,
                                        int sub) {
  using M = Map<D>;
  const float4* p = (const float4*)(grad + bm * D);
#pragma unroll
  for (int v = 0; v < M::NV; ++v) {
    const float4 g = p[sub + v * M::LPG];
    acc[4 * v + 0] += (double)g.x;
    acc[4 * v + 1] += (double)g.y;
    acc[4 * v + 2] += (double)g.z;
    acc[4 * v + 3] += (double)g.w;
  }
}

// Weight columns of one lane, widened to fp32.
template <int D, typename WT>
struct RowW {
  float w[Map<D>::CPL];
};

template <int D, typename WT>
__device__ __forceinline__ void load_w(const RUArgs& a, int64_t row, int sub, RowW<D, WT>& r) {
  using M = Map<D>;
  if constexpr (sizeof(WT) == 4) {
    const float4* w = (const float4*)((const char*)a.weights + row * a.stride);
#pragma unroll
    for (int v = 0; v < M::NV; ++v) {
      const float4 x = w[sub + v * M::LPG];
      r.w[4 * v] = x.x;
      r.w[4 * v + 1] = x.y;
      r.w[4 * v + 2] = x.z;
      r.w[4 * v + 3] = x.w;
    }
  } else {
    const uint2* w = (const uint2*)((const char*)a.weights + row * a.stride);
#pragma unroll
    for (int v = 0; v < M::NV; ++v) {
      const uint2 x = w[sub + v * M::LPG];
      r.w[4 * v] = bf16_bits_to_f32(x.x & 0xFFFFu);
      r.w[4 * v + 1] = bf16_bits_to_f32(x.x >> 16);
      r.w[4 * v + 2] = bf16_bits_to_f32(x.y & 0xFFFFu);
      r.w[4 * v + 3] = bf16_bits_to_f32(x.y >> 16);
    }
  }
}

// Applies the optimizer to row u (weights already loaded into r) with the
// group's fp64 sums. Every lane of the group calls it: the Adagrad sum of
// squares is a reduction over the group's lanes (all of which hold the same
// u and `active`).
template <int D, typename WT>
__device__ __forceinline__ void apply_row(const RUArgs& a, int64_t u, int64_t row, float st,
                                          int sub, const double (&acc)[Map<D>::CPL],
                                          RowW<D, WT>& r, bool active) {
  using M = Map<D>;
  float g[M::CPL];
#pragma unroll
  for (int c = 0; c < M::CPL; ++c) g[c] = (float)acc[c];
  float m = a.lr;
  if (a.optim == FS_RW_ADAGRAD) {
    double ss = 0.0;
#pragma unroll
    for (int c = 0; c < M::CPL; ++c) ss += (double)g[c] * (double)g[c];
#pragma unroll
    for (int off = M::LPG / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off, kWave);
    if (active) {
      const float mean_sq = (float)(ss / (double)D);
      const float s = st + mean_sq;
      if (sub == 0) *state_at(a, row) = s;
      const float denom = sqrtf(s) + a.eps;
      m = a.lr / denom;
    }
  }
  if (!active) return;
  if (a.reduced) {
    const int64_t lu = u - a.unique_offsets[a.g_lo];
    float4* rp = (float4*)(a.reduced + lu * D);
#pragma unroll
    for (int v = 0; v < M::NV; ++v)
      rp[sub + v * M::LPG] = make_float4(g[4 * v], g[4 * v + 1], g[4 * v + 2], g[4 * v + 3]);
  }
#pragma unroll
  for (int c = 0; c < M::CPL; ++c) {
    const float step = m * g[c];
    r.w[c] = r.w[c] - step;
  }
  if constexpr (sizeof(WT) == 4) {
    float4* w = (float4*)((char*)a.weights + row * a.stride);
#pragma unroll
    for (int v = 0; v < M::NV; ++v)
      w[sub + v * M::LPG] = make_float4(r.w[4 * v], r.w[4 * v + 1], r.w[4 * v + 2], r.w[4 * v + 3]);
  } else {
    uint2* w = (uint2*)((char*)a.weights + row * a.stride);
#pragma unroll
    for (int v = 0; v < M::NV; ++v) {
      uint2 x;
      x.x = f32_to_bf16_bits(r.w[4 * v]) | (f32_to_bf16_bits(r.w[4 * v + 1]) << 16);
      x.y = f32_to_bf16_bits(r.w[4 * v + 2]) | (f32_to_bf16_bits(r.w[4 * v + 3]) << 16);
      w[sub + v * M::LPG] = x;
    }
  }
}

template <int D, typename WT>
__device__ __forceinline__ void update_row(const RUArgs& a, int64_t u, int sub,
                                           const double (&acc)[Map<D>::CPL], bool active) {
  RowW<D, WT> r;
  int64_t row = 0;
  float st = 0.f;
  if (active) {
    row = a.unique[u] - a.row_base;
    load_w<D, WT>(a, row, sub, r);
    if (a.optim == FS_RW_ADAGRAD) st = *state_at(a, row);
  }
  apply_row<D, WT>(a, u, row, st, sub, acc, r, active);
}

// ---------------------------------------------------------------- short rows
// Grid-stride over the table's unique rows in units of `unit` rows per wave.
// The wave loads the unit's CSR bounds, keys, classes and Adagrad state with
// one coalesced or gathered load each; lane groups then take the rows in
// turn, R at a time, fetch their metadata by shuffle and keep R weight rows
// and R gradient rows in flight. The unit is 64 rows when the table has
// enough rows to give every wave of the grid several units, and shrinks to
// 32 or 16 otherwise, so that small batches spread over more waves and each
// wave's chain of dependent rounds stays short.
template <int D, typename WT>
__device__ __forceinline__ void short_rows(const RUArgs& a, int64_t bid, int64_t nblk) {
  using M = Map<D>;
  // rows per lane group and batch: 2 keeps the register count at 90 (five
  // waves per SIMD), which measured faster than 4 rows at four waves
  constexpr int R = M::CPL <= 8 ? 2 : 1;
  constexpr int PER = M::GPW * R;  // rows per batch of the wave
  const int64_t u_lo = a.unique_offsets[a.g_lo], u_hi = a.unique_offsets[a.g_hi];
  const int l = lane(), grp = l / M::LPG, sub = l % M::LPG;
  const bool ada = a.optim == FS_RW_ADAGRAD;
  const int64_t wid = bid * (kThreads / kWave) + threadIdx.x / kWave;
  const int64_t nwaves = nblk * (kThreads / kWave);
  const int64_t n_rows = u_hi - u_lo;
  const int unit = n_rows >= 2 * kWave * kResident ? kWave
                   : (n_rows >= 2 * 32 * kResident ? 32 : 16);
  for (int64_t ub = u_lo + wid * unit; ub < u_hi; ub += nwaves * unit) {
    const int64_t uu = ub + l;
    const bool in = l < unit && uu < u_hi;
    const int32_t lo = in ? a.seg_offsets[uu] : 0;
    const int32_t hi = in ? a.seg_offsets[uu + 1] : 0;
    const int32_t len = hi - lo;
    const bool act = in && len <= kShort && class_ok(a, uu);
    const uint64_t actm = __ballot(act);
    if (!actm) continue;
    const uint32_t row = act ? (uint32_t)(a.unique[uu] - a.row_base) : 0u;
    const float st = (act && ada) ? *state_at(a, row) : 0.f;
    // the row's (at most kShort) gradient slots, loaded once per unit beside
    // its key and state: a batch below then waits for one round of loads
    // (its gradient and weight rows), not for the slots first
    int32_t obm[kShort];
#pragma unroll
    for (int m = 0; m < kShort; ++m) obm[m] = (act && m < len) ? a.occ_bm[lo + m] : 0;
#pragma unroll 1
    for (int j0 = 0; j0 < unit; j0 += PER) {
      const uint64_t win = (PER >= kWave) ? ~0ull : (((1ull << PER) - 1ull) << j0);
      if (!(actm & win)) continue;
      int32_t jlen[R], jj[R];
      uint32_t jrow[R];
      float jst[R];
      bool ja[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int j = j0 + r * M::GPW + grp;
        jj[r] = j;
        ja[r] = (actm >> j) & 1ull;
        jlen[r] = __shfl(hi - lo, j, kWave);
        jrow[r] = (uint32_t)__shfl((int)row, j, kWave);
        jst[r] = __shfl(st, j, kWave);
      }
      // a short row has at most kShort occurrences: its weight row and all of
      // its gradient rows load at once
      RowW<D, WT> wr[R];
      double acc[R][M::CPL];
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (ja[r]) load_w<D, WT>(a, jrow[r], sub, wr[r]);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int rlen = ja[r] ? jlen[r] : 0;
        float4 gv[kShort][M::NV];
#pragma unroll
        for (int m = 0; m < kShort; ++m) {
          const int32_t bm = __shfl(obm[m], jj[r], kWave);
          if (m < rlen) {
            const float4* gp = (const float4*)(a.grad + (int64_t)bm * D);
#pragma unroll
            for (int v = 0; v < M::NV; ++v) gv[m][v] = ld_stream(gp + sub + v * M::LPG);
          }
        }
#pragma unroll
        for (int c = 0; c < M::CPL; ++c) acc[r][c] = 0.0;
#pragma unroll
        for (int m = 0; m < kShort; ++m) {
          if (m < rlen) {
#pragma unroll
            for (int v = 0; v < M::NV; ++v) {
              acc[r][4 * v + 0] += (double)gv[m][v].x;
              acc[r][4 * v + 1] += (double)gv[m][v].y;
              acc[r][4 * v + 2] += (double)gv[m][v].z;
              acc[r][4 * v + 3] += (double)gv[m][v].w;
            }
          }
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r)
        apply_row<D, WT>(a, ub + j0 + r * M::GPW + grp, jrow[r], jst[r], sub, acc[r], wr[r],
                         ja[r]);
    }
  }
}

// ---------------------------------------------------------------- medium rows
// Rows of kShort < len < kChunkMin occurrences (about 4% of the rows and 13%
// of the occurrences at workload 5's Zipf IDs). Grid-stride over the table's
// unique rows in units of 64: the wave finds the unit's medium rows by one
// ballot, then each lane group takes one of them: the group's lanes load all
// of the row's occurrence slots with one load (kMedSlots per lane), its
// weight row and state go out beside them, and its gradient rows stream
// MB at a time. A wave thus has GPW rows in progress instead of walking them
// one after another inside a chunk.
template <int D, typename WT, int MB = kMedBatch>
__device__ __forceinline__ void medium_rows(const RUArgs& a, int64_t bid, int64_t nblk) {
  using M = Map<D>;
  constexpr int kMedSlots = (kChunkMin - 1 + M::LPG - 1) / M::LPG;
  static_assert(M::LPG % MB == 0, "a batch must not straddle slot registers");
  const int64_t u_lo = a.unique_offsets[a.g_lo], u_hi = a.unique_offsets[a.g_hi];
  const int l = lane(), grp = l / M::LPG, sub = l % M::LPG;
  const bool ada = a.optim == FS_RW_ADAGRAD;
  const int64_t wid = bid * (kThreads / kWave) + threadIdx.x / kWave;
  const int64_t nwaves = nblk * (kThreads / kWave);
  for (int64_t ub = u_lo + wid * kWave; ub < u_hi; ub += nwaves * kWave) {
    const int64_t uu = ub + l;
    const bool in = uu < u_hi;
    const int32_t lo = in ? a.seg_offsets[uu] : 0;
    const int32_t len = in ? a.seg_offsets[uu + 1] - lo : 0;
    const bool med = in && len > kShort && len < kChunkMin && class_ok(a, uu);
    uint64_t medm = __ballot(med);
    if (!medm) continue;
    const uint32_t row = med ? (uint32_t)(a.unique[uu] - a.row_base) : 0u;
    const float st = (med && ada) ? *state_at(a, row) : 0.f;
    while (medm) {
      uint64_t mm = medm;
      int myj = -1;
#pragma unroll
      for (int g = 0; g < M::GPW; ++g) {
        const int j = mm ? __ffsll((unsigned long long)mm) - 1 : -1;
        mm &= mm ? mm - 1 : 0ull;
        if (g == grp) myj = j;
      }
      medm = mm;
      const bool on = myj >= 0;
      const int js = on ? myj : 0;
      const int32_t mlen = __shfl(len, js, kWave), mlo = __shfl(lo, js, kWave);
      const uint32_t mrow = (uint32_t)__shfl((int)row, js, kWave);
      const float mst = __shfl(st, js, kWave);
      const int glen = on ? mlen : 0;
      RowW<D, WT> wr;
      if (on) load_w<D, WT>(a, mrow, sub, wr);
      int32_t mb[kMedSlots];
#pragma unroll
      for (int q = 0; q < kMedSlots; ++q) {
        const int m = q * M::LPG + sub;
        mb[q] = m < glen ? a.occ_bm[mlo + m] : 0;
      }
      int wlen = glen;  // longest row of this round (wave-uniform)
#pragma unroll
      for (int off = M::LPG; off < kWave; off <<= 1) wlen = max(wlen, __shfl_xor(wlen, off, kWave));
      double acc[M::CPL];
#pragma unroll
      for (int c = 0; c < M::CPL; ++c) acc[c] = 0.0;
      // a batch of MB (a divisor of LPG) lies inside one slot register
#pragma unroll 1
      for (int m0 = 0; m0 < wlen; m0 += MB) {
        const int q = m0 / M::LPG;
        int32_t slot = mb[0];
#pragma unroll
        for (int x = 1; x < kMedSlots; ++x) slot = q == x ? mb[x] : slot;
        float4 gv[MB][M::NV];
#pragma unroll
        for (int e = 0; e < MB; ++e) {
          const int m = m0 + e;
          const int32_t bm = __shfl(slot, grp * M::LPG + (m % M::LPG), kWave);
          if (m < glen) {
            const float4* gp = (const float4*)(a.grad + (int64_t)bm * D);
#pragma unroll
            for (int v = 0; v < M::NV; ++v) gv[e][v] = ld_stream(gp + sub + v * M::LPG);
          }
        }
#pragma unroll
        for (int e = 0; e < MB; ++e) {
          if (m0 + e < glen) {
#pragma unroll
            for (int v = 0; v < M::NV; ++v) {
              acc[4 * v + 0] += (double)gv[e][v].x;
              acc[4 * v + 1] += (double)gv[e][v].y;
              acc[4 * v + 2] += (double)gv[e][v].z;
              acc[4 * v + 3] += (double)gv[e][v].w;
            }
          }
        }
      }
      apply_row<D, WT>(a, ub + js, mrow, mst, sub, acc, wr, on);
    }
  }
}

// ---------------------------------------------------------------- long rows
template <int D, typename WT>
__device__ __forceinline__ void long_chunk(const RUArgs& a, int64_t o_lo, int64_t o_hi,
                                           int64_t c) {
  using M = Map<D>;
  const int64_t cb = o_lo + c * a.chunk;
  const int64_t ce = min(cb + a.chunk, o_hi);
  const int grp = lane() / M::LPG, sub = lane() % M::LPG;
  const int32_t u_first = a.occ_uid[cb], u_last = a.occ_uid[ce - 1];
  for (int32_t ub = u_first; ub <= u_last; ub += kWave) {
    const int32_t uu = ub + lane();
    const bool in = uu <= u_last;
    const int32_t lo = in ? a.seg_offsets[uu] : 0, hi = in ? a.seg_offsets[uu + 1] : 0;
    uint64_t todo = __ballot(in && hi - lo >= kChunkMin && class_ok(a, uu));
    while (todo) {
      const int j = __ffsll((unsigned long long)todo) - 1;
      todo &= todo - 1;
      const int64_t s_lo = __shfl(lo, j, kWave), s_hi = __shfl(hi, j, kWave);
      const int64_t u = ub + j;
      const int64_t p0 = max(s_lo, cb), p1 = min(s_hi, ce);
      const bool complete = s_lo >= cb && s_hi <= ce;
      // a row that lies inside the chunk is updated here: fetch its weights
      // and state now, while its gradients stream in
      RowW<D, WT> wr;
      int64_t row = 0;
      float st = 0.f;
      if (complete) {
        row = a.unique[u] - a.row_base;
        if (grp == 0) load_w<D, WT>(a, row, sub, wr);
        if (a.optim == FS_RW_ADAGRAD) st = *state_at(a, row);
      }
      double acc[M::CPL];
#pragma unroll
      for (int x = 0; x < M::CPL; ++x) acc[x] = 0.0;
      for (int64_t ob = p0; ob < p1; ob += kWave) {
        const int nblk = (int)min((int64_t)kWave, p1 - ob);
        const int32_t bmv = lane() < nblk ? a.occ_bm[ob + lane()] : 0;
        // group g takes rows g, g + GPW, ... of this block of 64
        for (int m0 = 0; m0 < nblk; m0 += kLongBatch * M::GPW) {
          float4 gv[kLongBatch][M::NV];
#pragma unroll
          for (int e = 0; e < kLongBatch; ++e) {
            const int m = m0 + e * M::GPW + grp;
            const int32_t bm = __shfl(bmv, m < kWave ? m : 0, kWave);
            if (m < nblk) {
              const float4* gp = (const float4*)(a.grad + (int64_t)bm * D);
#pragma unroll
              for (int v = 0; v < M::NV; ++v) gv[e][v] = ld_stream(gp + sub + v * M::LPG);
            }
          }
#pragma unroll
          for (int e = 0; e < kLongBatch; ++e) {
            if (m0 + e * M::GPW + grp < nblk) {
#pragma unroll
              for (int v = 0; v < M::NV; ++v) {
                acc[4 * v + 0] += (double)gv[e][v].x;
                acc[4 * v + 1] += (double)gv[e][v].y;
                acc[4 * v + 2] += (double)gv[e][v].z;
                acc[4 * v + 3] += (double)gv[e][v].w;
              }
            }
          }
        }
      }
      // combine the interleaved groups (fixed order)
#pragma unroll
      for (int off = M::LPG; off < kWave; off <<= 1)
#pragma unroll
        for (int x = 0; x < M::CPL; ++x) acc[x] += __shfl_xor(acc[x], off, kWave);
      if (complete) {
        apply_row<D, WT>(a, u, row, st, sub, acc, wr, grp == 0);
      } else if (grp == 0) {
        const int slot = s_lo >= cb ? 1 : 0;
        double* p = a.partials + ((c - 0) * 2 + slot) * D;
#pragma unroll
        for (int v = 0; v < M::NV; ++v)
#pragma unroll
          for (int e = 0; e < 4; ++e) p[M::col(sub, v) + e] = acc[4 * v + e];
      }
    }
  }
}

// Chunks in grid-stride order, one per wave at a time.
template <int D, typename WT>
__device__ __forceinline__ void long_rows(const RUArgs& a, int64_t bid, int64_t nblk) {
  const int64_t o_lo = a.seg_offsets[a.unique_offsets[a.g_lo]];
  const int64_t o_hi = a.seg_offsets[a.unique_offsets[a.g_hi]];
  const int64_t nwaves = nblk * (kThreads / kWave);
  for (int64_t c = bid * (kThreads / kWave) + threadIdx.x / kWave; o_lo + c * a.chunk < o_hi;
       c += nwaves)
    long_chunk<D, WT>(a, o_lo, o_hi, c);
}

// ---------------------------------------------------------------- fix-up
// Chunk c owns the long row that starts in it and runs past its end: sum the
// row's partials (slot 1 of c, slot 0 of each later chunk it covers), four
// waves in contiguous slices with E partials in flight per lane group,
// combined in wave order.
template <int D>
struct FixShape {
  static constexpr int E = D >= 1024 ? 1 : (D >= 512 ? 2 : 4);
};

// part: LDS of kThreads / kWave rows of D doubles (the waves' sums)
template <int D, typename WT>
__device__ __forceinline__ void fix_rows(const RUArgs& a, int64_t bid, double* part) {
  using M = Map<D>;
  constexpr int E = FixShape<D>::E;
  const int64_t o_lo = a.seg_offsets[a.unique_offsets[a.g_lo]];
  const int64_t o_hi = a.seg_offsets[a.unique_offsets[a.g_hi]];
  const int64_t c = bid;
  const int64_t cb = o_lo + c * a.chunk;
  if (cb >= o_hi) return;
  const int64_t ce = min(cb + a.chunk, o_hi);
  const int64_t u = a.occ_uid[ce - 1];
  const int64_t s_lo = a.seg_offsets[u], s_hi = a.seg_offsets[u + 1];
  if (!(s_hi - s_lo >= kChunkMin && s_lo >= cb && s_hi > ce && class_ok(a, u))) return;
  const int64_t c_last = (s_hi - 1 - o_lo) / a.chunk;  // slot 0 of chunks c+1..c_last
  const int64_t n_parts = 1 + (c_last - c);
  const int w = threadIdx.x / kWave;
  const int grp = lane() / M::LPG, sub = lane() % M::LPG;
  // part k of the row: k == 0 -> chunk c slot 1; k >= 1 -> chunk c+k slot 0
  const int64_t per = cdiv(n_parts, kThreads / kWave);
  const int64_t k0 = min(n_parts, w * per), k1 = min(n_parts, k0 + per);
  double acc[M::CPL];
#pragma unroll
  for (int x = 0; x < M::CPL; ++x) acc[x] = 0.0;
  for (int64_t kb = k0; kb < k1; kb += E * M::GPW) {
    double pv[E][M::CPL];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int64_t k = kb + e * M::GPW + grp;
      if (k < k1) {
        const double* p = a.partials + ((c + k) * 2 + (k == 0 ? 1 : 0)) * D;
#pragma unroll
        for (int v = 0; v < M::NV; ++v)
#pragma unroll
          for (int q = 0; q < 4; ++q) pv[e][4 * v + q] = p[M::col(sub, v) + q];
      }
    }
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (kb + e * M::GPW + grp < k1)
#pragma unroll
        for (int x = 0; x < M::CPL; ++x) acc[x] += pv[e][x];
  }
#pragma unroll
  for (int off = M::LPG; off < kWave; off <<= 1)
#pragma unroll
    for (int x = 0; x < M::CPL; ++x) acc[x] += __shfl_xor(acc[x], off, kWave);
  if (grp == 0) {
#pragma unroll
    for (int v = 0; v < M::NV; ++v)
#pragma unroll
      for (int q = 0; q < 4; ++q) part[w * D + M::col(sub, v) + q] = acc[4 * v + q];
  }
  __syncthreads();
  if (w == 0) {
#pragma unroll
    for (int x = 0; x < M::CPL; ++x) acc[x] = 0.0;
    for (int ww = 0; ww < kThreads / kWave; ++ww)
#pragma unroll
      for (int v = 0; v < M::NV; ++v)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[4 * v + q] += part[ww * D + M::col(sub, v) + q];
    update_row<D, WT>(a, u, sub, acc, grp == 0);
  }
}

// ---------------------------------------------------------------- launches
// One launch per kernel kind for every table of the call: two or more tables
// of at most kSetMaxDim columns share one launch (workgroup ranges per table,
// each workgroup running its table's row shape), wider tables get launches
// of their own (their shapes need more registers, which a shared kernel
// would impose on every table), and so does a narrow table alone (the shared
// kernel's registers cost one wave per SIMD on the short rows: workload 5
// ran 2% slower through it). Multi-table calls thus make four launches
// instead of four per table (workload 4's update: 0.40 -> 0.26 ms). Each table's fp64 partial sums have their own region of
// the workspace, so the tables' long rows can run side by side.
enum Kind { kShortRows = 0, kMediumRows = 1, kLongRows = 2, kFixRows = 3 };
constexpr int kSetMaxDim = 256;

template <int K, int D, typename WT>
__device__ __forceinline__ void run_kind(const RUArgs& a, int64_t bid, int64_t nblk,
                                         double* part) {
  if constexpr (K == kShortRows) short_rows<D, WT>(a, bid, nblk);
  else if constexpr (K == kMediumRows) medium_rows<D, WT>(a, bid, nblk);
  else if constexpr (K == kLongRows) long_rows<D, WT>(a, bid, nblk);
  else fix_rows<D, WT>(a, bid, part);
}

// the tables of one shared launch; table k owns workgroups [first[k], first[k+1])
struct RUSet {
  RUArgs a[FS_MAX_TABLES];
  int32_t first[FS_MAX_TABLES + 1];
  int32_t shape[FS_MAX_TABLES];  // 2 * log2(D / 64) + (bf16 ? 1 : 0), D <= kSetMaxDim
  int32_t n;
};

template <int K>
__device__ __forceinline__ void set_body(const RUSet& s, double* part) {
  int k = 0;
  while (k + 1 < s.n && (int32_t)blockIdx.x >= s.first[k + 1]) ++k;
  const int64_t bid = (int64_t)blockIdx.x - s.first[k], nblk = s.first[k + 1] - s.first[k];
  switch (s.shape[k]) {
    case 0: run_kind<K, 64, float>(s.a[k], bid, nblk, part); break;
    case 1: run_kind<K, 64, uint16_t>(s.a[k], bid, nblk, part); break;
    case 2: run_kind<K, 128, float>(s.a[k], bid, nblk, part); break;
    case 3: run_kind<K, 128, uint16_t>(s.a[k], bid, nblk, part); break;
    case 4: run_kind<K, 256, float>(s.a[k], bid, nblk, part); break;
    case 5: run_kind<K, 256, uint16_t>(s.a[k], bid, nblk, part); break;
  }
}

// the shared launches, one kernel per kind
__global__ void __launch_bounds__(kThreads) k_short_set(RUSet s) {
  set_body<kShortRows>(s, nullptr);
}
__global__ void __launch_bounds__(kThreads) k_medium_set(RUSet s) {
  set_body<kMediumRows>(s, nullptr);
}
__global__ void __launch_bounds__(kThreads) k_long_set(RUSet s) { set_body<kLongRows>(s, nullptr); }
__global__ void __launch_bounds__(kThreads) k_fix_set(RUSet s) {
  __shared__ double part[(kThreads / kWave) * kSetMaxDim];
  set_body<kFixRows>(s, part);
}

// one table's own launches (a table alone in its width class, or a wide one):
// each kernel holds one row shape, so its register count is that shape's
template <int D, typename WT>
__global__ void __launch_bounds__(kThreads) k_short(RUArgs a) {
  short_rows<D, WT>(a, blockIdx.x, gridDim.x);
}
// A table's own medium-row kernel streams 16 gradient rows at a time when a
// lane holds one float4 of a row (rows of up to 256 columns): a medium row
// (about 13 occurrences on average at Zipf IDs) then takes one round of
// gradient loads instead of two, for 120 instead of 88 VGPRs (four waves per
// SIMD instead of five). Alone on the GPU the kernel takes the same time
// (121 us at workload 5); beside the long-row part of the same update the step
// gains (same box, two runs each): workload 5 1.546/1.545 -> 1.535/1.530 ms,
// workload 3 0.238/0.248 -> 0.222/0.230. The shared launch of several tables
// keeps 8 (with 16 it drops to three waves per SIMD and workload 4 gains
// nothing), as does the one-launch kernel of small calls.
template <int D>
struct MedBatch {
  static constexpr int V = Map<D>::NV == 1 ? 16 : kMedBatch;
};

template <int D, typename WT>
__global__ void __launch_bounds__(kThreads) k_medium(RUArgs a) {
  medium_rows<D, WT, MedBatch<D>::V>(a, blockIdx.x, gridDim.x);
}
template <int D, typename WT>
__global__ void __launch_bounds__(kThreads) k_long(RUArgs a) {
  long_rows<D, WT>(a, blockIdx.x, gridDim.x);
}
template <int D, typename WT>
__global__ void __launch_bounds__(kThreads) k_fix(RUArgs a) {
  __shared__ double part[(kThreads / kWave) * D];
  fix_rows<D, WT>(a, blockIdx.x, part);
}

// Small calls of one table: long, medium and short rows in one launch (the
// long rows' workgroups first, as their chunks are the longest work), the
// fix-up after it -- two launches instead of four, where a call of a few
// thousand occurrences is a chain of launches more than a stream of bytes.
constexpr int64_t kFusedMax = 1 << 17;  // occurrences

template <int D, typename WT>
__global__ void __launch_bounds__(kThreads) k_rows3(RUArgs a, int32_t b_long, int32_t b_medium,
                                                   int32_t b_short) {
  const int32_t b = blockIdx.x;
  if (b < b_long) long_rows<D, WT>(a, b, b_long);
  else if (b < b_long + b_medium) medium_rows<D, WT>(a, b - b_long, b_medium);
  else short_rows<D, WT>(a, b - b_long - b_medium, b_short);
}

// workgroups of each kind for one table with n_cap occurrences
int64_t blocks_of(int K, int64_t n_cap, int64_t chunk) {
  int64_t b;
  if (K == kShortRows) b = cdiv(n_cap, kThreads);  // 64 rows per wave, 4 waves per block
  else if (K == kMediumRows) b = cdiv(n_cap, 2 * kWave * (kThreads / kWave));  // ~2 units per wave
  else if (K == kLongRows) return cdiv(cdiv(n_cap, chunk), kThreads / kWave);
  else return cdiv(n_cap, chunk);
  return b > kShortBlocks ? kShortBlocks : (b < 1 ? 1 : b);
}

template <int K, int D, typename WT>
int launch_one(const RUArgs& a, hipStream_t stream) {
  const int64_t b = blocks_of(K, a.n_cap, a.chunk);
  if (b <= 0) return FS_OK;
  const dim3 g((unsigned)b), tb(kThreads);
  if constexpr (K == kShortRows) hipLaunchKernelGGL((k_short<D, WT>), g, tb, 0, stream, a);
  else if constexpr (K == kMediumRows) hipLaunchKernelGGL((k_medium<D, WT>), g, tb, 0, stream, a);
  else if constexpr (K == kLongRows) hipLaunchKernelGGL((k_long<D, WT>), g, tb, 0, stream, a);
  else hipLaunchKernelGGL((k_fix<D, WT>), g, tb, 0, stream, a);
  FS_LAUNCH_CHECK();
  return FS_OK;
}

template <int D, typename WT>
int launch_rows3(const RUArgs& a, hipStream_t stream) {
  const int64_t bl = blocks_of(kLongRows, a.n_cap, a.chunk);
  const int64_t bm = blocks_of(kMediumRows, a.n_cap, a.chunk);
  const int64_t bs = blocks_of(kShortRows, a.n_cap, a.chunk);
  hipLaunchKernelGGL((k_rows3<D, WT>), dim3((unsigned)(bl + bm + bs)), dim3(kThreads), 0, stream,
                     a, (int32_t)bl, (int32_t)bm, (int32_t)bs);
  FS_LAUNCH_CHECK();
  return launch_one<kFixRows, D, WT>(a, stream);
}

template <typename WT>
int launch_rows3_dim(int dim, const RUArgs& a, hipStream_t stream) {
  switch (dim) {
    case 64: return launch_rows3<64, WT>(a, stream);
    case 128: return launch_rows3<128, WT>(a, stream);
    case 256: return launch_rows3<256, WT>(a, stream);
    case 512: return launch_rows3<512, WT>(a, stream);
    case 1024: return launch_rows3<1024, WT>(a, stream);
  }
  return FS_ERR_UNSUPPORTED;
}

template <int K, typename WT>
int launch_dim(int dim, const RUArgs& a, hipStream_t stream) {
  switch (dim) {
    case 64: return launch_one<K, 64, WT>(a, stream);
    case 128: return launch_one<K, 128, WT>(a, stream);
    case 256: return launch_one<K, 256, WT>(a, stream);
    case 512: return launch_one<K, 512, WT>(a, stream);
    case 1024: return launch_one<K, 1024, WT>(a, stream);
  }
  return FS_ERR_UNSUPPORTED;
}

template <int K>
int launch_table(int dim, bool bf16, const RUArgs& a, hipStream_t stream) {
  return bf16 ? launch_dim<K, uint16_t>(dim, a, stream) : launch_dim<K, float>(dim, a, stream);
}

int shape_of(int dim, bool bf16) {
  const int l = dim == 64 ? 0 : (dim == 128 ? 1 : 2);
  return 2 * l + (bf16 ? 1 : 0);
}

// every kind of the requested rows in order (short and medium rows: FS_ROWS_FEW;
// long rows, then the fix-up of their partial sums: FS_ROWS_MANY), each kind
// one launch for the narrow tables (a table's own launch when it is the only
// narrow one) and one per wide table
int launch_tables(const RUArgs* args, const int* dims, const bool* bf16, int T, int32_t rows,
                  hipStream_t stream) {
  if (T == 1 && rows == FS_ROWS_ALL && args[0].n_cap <= kFusedMax)
    return bf16[0] ? launch_rows3_dim<uint16_t>(dims[0], args[0], stream)
                   : launch_rows3_dim<float>(dims[0], args[0], stream);
  int narrow = 0;
  for (int t = 0; t < T; ++t) narrow += dims[t] <= kSetMaxDim;
  for (int K = 0; K < 4; ++K) {
    const int32_t part = (K == kShortRows || K == kMediumRows) ? FS_ROWS_FEW : FS_ROWS_MANY;
    if (!(rows & part)) continue;
    RUSet set;
    set.n = 0;
    int64_t total = 0;
    for (int t = 0; t < T; ++t) {
      if (dims[t] > kSetMaxDim || narrow < 2) continue;
      const int64_t b = blocks_of(K, args[t].n_cap, args[t].chunk);
      set.a[set.n] = args[t];
      set.shape[set.n] = shape_of(dims[t], bf16[t]);
      set.first[set.n] = (int32_t)total;
      total += b > 0 ? b : 0;
      ++set.n;
    }
    if (set.n > 0 && total > 0) {
      set.first[set.n] = (int32_t)total;
      const dim3 g((unsigned)total), tb(kThreads);
      switch (K) {
        case kShortRows: hipLaunchKernelGGL(k_short_set, g, tb, 0, stream, set); break;
        case kMediumRows: hipLaunchKernelGGL(k_medium_set, g, tb, 0, stream, set); break;
        case kLongRows: hipLaunchKernelGGL(k_long_set, g, tb, 0, stream, set); break;
        default: hipLaunchKernelGGL(k_fix_set, g, tb, 0, stream, set);
      }
      FS_LAUNCH_CHECK();
    }
    for (int t = 0; t < T; ++t) {
      if (dims[t] <= kSetMaxDim && narrow >= 2) continue;
      int rc = FS_OK;
      switch (K) {
        case kShortRows: rc = launch_table<kShortRows>(dims[t], bf16[t], args[t], stream); break;
        case kMediumRows: rc = launch_table<kMediumRows>(dims[t], bf16[t], args[t], stream); break;
        case kLongRows: rc = launch_table<kLongRows>(dims[t], bf16[t], args[t], stream); break;
        default: rc = launch_table<kFixRows>(dims[t], bf16[t], args[t], stream);
      }
      if (rc) return rc;
    }
  }
  return FS_OK;
}

bool dim_ok(int d) { return d == 64 || d == 128 || d == 256 || d == 512 || d == 1024; }

}  // namespace
}  // namespace fs

using namespace fs;

// Long-path chunks of a call with n occurrences; the workspace holds two fp64
// partial rows per chunk. chunk_for grows with n, so the count drops where
// the chunk size steps up: the query takes the largest count of any n' <= n
// (the last n' before each step), so that a workspace sized for a capacity
// serves every smaller call.
static int64_t max_chunks(int64_t n) {
  int64_t m = cdiv(n, chunk_for(n));
  const int64_t last128 = (n < kChunk256From ? n : kChunk256From - 1);
  const int64_t last256 = (n < kChunk512From ? n : kChunk512From - 1);
  const int64_t c128 = cdiv(last128, 128), c256 = cdiv(last256, chunk_for(last256));
  m = c128 > m ? c128 : m;
  return c256 > m ? c256 : m;
}

// doubles of one table's region of partial sums
static size_t partial_doubles(int64_t n_tok, int32_t max_dim) {
  const int64_t n = n_tok > 0 ? n_tok : 1;
  return (size_t)(max_chunks(n) * 2) * (size_t)(max_dim > 0 ? max_dim : 1);
}

extern "C" size_t fs_grad_reduce_update_workspace_size(int64_t n_tok, int32_t T,
                                                      int32_t max_dim) {
  Carve c(nullptr);
  c.take<double>(partial_doubles(n_tok, max_dim) * (size_t)(T > 0 ? T : 1));
  return c.used + 256;
}

namespace {

// Host-side checks shared by both entry points: arguments, shapes, and a
// scratch area of ws_bytes for the long rows' fp64 partial sums.
int ru_check(const fs_table* tables, int32_t T, int32_t W, const float* const* grad,
             int64_t n_tok, const int64_t* unique, const int64_t* unique_offsets,
             const int32_t* seg_offsets, const int32_t* occ_bm, const int32_t* occ_uid,
             const uint8_t* cls, int32_t which, int32_t rows, int32_t optim, size_t ws_bytes,
             int too_small) {
  if (!tables || T < 1 || T > FS_MAX_TABLES || W < 1 || W > FS_MAX_RANKS || n_tok < 0 ||
      (int64_t)T * n_tok >= (int64_t)INT32_MAX || !grad || !unique_offsets || !seg_offsets)
    return FS_ERR_INVALID_ARG;
  if (which != FS_ALL && which != FS_EXCLUSIVE && which != FS_COLLISION) return FS_ERR_INVALID_ARG;
  if (which != FS_ALL && !cls) return FS_ERR_INVALID_ARG;
  if (rows != FS_ROWS_FEW && rows != FS_ROWS_MANY && rows != FS_ROWS_ALL)
    return FS_ERR_INVALID_ARG;
  if (optim != FS_SGD && optim != FS_RW_ADAGRAD) return FS_ERR_INVALID_ARG;
  if (n_tok > 0 && (!unique || !occ_bm || !occ_uid)) return FS_ERR_INVALID_ARG;
  int max_dim = 0;
  int64_t base = 0;
  for (int t = 0; t < T; ++t) {
    const fs_table& tb = tables[t];
    if (tb.rows < 1 || (tb.dtype != FS_F32 && tb.dtype != FS_BF16)) return FS_ERR_INVALID_ARG;
    if (!dim_ok(tb.dim)) return FS_ERR_UNSUPPORTED;
    if (n_tok > 0 && (!tb.weights || !grad[t])) return FS_ERR_INVALID_ARG;
    if (optim == FS_RW_ADAGRAD && n_tok > 0 && !tb.state) return FS_ERR_INVALID_ARG;
    if (!table_layout_ok(tb, optim == FS_RW_ADAGRAD)) return FS_ERR_INVALID_ARG;
    max_dim = tb.dim > max_dim ? tb.dim : max_dim;
    base += tb.rows;
  }
  if (base > (int64_t)UINT32_MAX) return FS_ERR_UNSUPPORTED;
  if (ws_bytes < fs_grad_reduce_update_workspace_size(n_tok, T, max_dim)) return too_small;
  return FS_OK;
}

int ru_launch(const fs_table* tables, int32_t T, int32_t W, const float* const* grad,
              int64_t n_tok, const int64_t* unique, const int64_t* unique_offsets,
              const int32_t* seg_offsets, const int32_t* occ_bm, const int32_t* occ_uid,
              const uint8_t* cls, int32_t which, int32_t rows, int32_t optim, float lr,
              float eps, float* const* reduced_out, void* ws, hipStream_t stream) {
  RUArgs args[FS_MAX_TABLES];
  int dims[FS_MAX_TABLES];
  bool bf16[FS_MAX_TABLES];
  int max_dim = 0;
  for (int t = 0; t < T; ++t) max_dim = tables[t].dim > max_dim ? tables[t].dim : max_dim;
  const size_t region = partial_doubles(n_tok, max_dim);
  int64_t base = 0;
  for (int t = 0; t < T; ++t) {
    const fs_table& tb = tables[t];
    RUArgs& a = args[t];
    a.weights = tb.weights;
    a.state = tb.state;
    a.stride = table_stride(tb);
    a.state_stride = table_state_stride(tb);
    a.grad = grad[t];
    a.reduced = reduced_out ? reduced_out[t] : nullptr;
    a.unique = unique;
    a.unique_offsets = unique_offsets;
    a.seg_offsets = seg_offsets;
    a.occ_bm = occ_bm;
    a.occ_uid = occ_uid;
    a.cls = cls;
    a.partials = (double*)ws + region * (size_t)t;  // each table its own region
    a.chunk = chunk_for(n_tok > 0 ? n_tok : 1);
    a.row_base = base;
    a.n_cap = n_tok;
    a.g_lo = t * W;
    a.g_hi = (t + 1) * W;
    a.which = which;
    a.optim = optim;
    a.lr = lr;
    a.eps = eps;
    base += tb.rows;
    dims[t] = tb.dim;
    bf16[t] = tb.dtype == FS_BF16;
  }
  if (n_tok == 0) return FS_OK;
  return launch_tables(args, dims, bf16, T, rows, stream);
}

// The allocation-free variant's scratch: one array per GPU the library runs
// on, held until the process ends. Host code never passes the array's name
// (a host-side stand-in); it passes the device address that
// hipGetSymbolAddress returns, queried once per device with that device
// current.
__device__ __align__(256) unsigned char scratch[FS_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_for(hipStream_t stream, void** out) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return FS_ERR_HIP;
  int dev = cur;
  if (stream) {
    hipDevice_t d = 0;
    if (hipStreamGetDevice(stream, &d) != hipSuccess) return FS_ERR_HIP;
    dev = (int)d;
  }
  if (dev < 0 || dev >= kMaxDevices) return FS_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return FS_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return FS_ERR_HIP;
    if (e != hipSuccess || !p) return FS_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FS_OK;
}

}  // namespace

extern "C" int fs_grad_reduce_update(const fs_table* tables, int32_t T, int32_t W,
                                     const float* const* grad, int64_t n_tok,
                                     const int64_t* unique, const int64_t* unique_offsets,
                                     const int32_t* seg_offsets, const int32_t* occ_bm,
                                     const int32_t* occ_uid, const uint8_t* cls, int32_t which,
                                     int32_t rows, int32_t optim, float lr, float eps,
                                     float* const* reduced_out, void* ws, size_t ws_bytes,
                                     hipStream_t stream) {
  int rc = ru_check(tables, T, W, grad, n_tok, unique, unique_offsets, seg_offsets, occ_bm,
                    occ_uid, cls, which, rows, optim, ws ? ws_bytes : 0, FS_ERR_WORKSPACE);
  if (rc) return rc;
  return ru_launch(tables, T, W, grad, n_tok, unique, unique_offsets, seg_offsets, occ_bm,
                   occ_uid, cls, which, rows, optim, lr, eps, reduced_out, ws, stream);
}

extern "C" int fs_grad_reduce_update_noalloc(const fs_table* tables, int32_t T, int32_t W,
                                             const float* const* grad, int64_t n_tok,
                                             const int64_t* unique,
                                             const int64_t* unique_offsets,
                                             const int32_t* seg_offsets, const int32_t* occ_bm,
                                             const int32_t* occ_uid, const uint8_t* cls,
                                             int32_t which, int32_t rows, int32_t optim, float lr,
                                             float eps, float* const* reduced_out,
                                             hipStream_t stream) {
  int rc = ru_check(tables, T, W, grad, n_tok, unique, unique_offsets, seg_offsets, occ_bm,
                    occ_uid, cls, which, rows, optim, FS_NOALLOC_SCRATCH_BYTES,
                    FS_ERR_TOO_LARGE);
  if (rc) return rc;
  void* ws = nullptr;
  rc = scratch_for(stream, &ws);
  if (rc) return rc;
  // every fp64 partial a launch reads is written earlier in the same launch
  // sequence, so the scratch needs no clearing between calls
  return ru_launch(tables, T, W, grad, n_tok, unique, unique_offsets, seg_offsets, occ_bm,
                   occ_uid, cls, which, rows, optim, lr, eps, reduced_out, ws, stream);
}
