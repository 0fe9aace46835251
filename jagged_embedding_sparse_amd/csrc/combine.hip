// Ranged combine: shard-major rows back to each table's batch-major slots.
//
// "FreeScale: distributed training for sequence recommendation models",
// section 4.2: the ranged combine kernel lays out the output of the embedding
// AllToAll -- the rows a source rank receives from the shards, range by
// range -- in that rank's original (batch-major) order. With every virtual
// rank on one GPU the rows arrive in the shard-major order of the dispatch
// (fs_bucketize_permute), so item k's row goes to slot shard_bm[k] of the
// output of its table (the table whose key range holds shard_keys[k]). The
// sparse step itself does not call this: its lookup writes the batch-major
// slots directly.
//
// One wave per 64 consecutive items: their keys and slots are loaded
// coalesced once and handed to lane groups of 16 lanes by shuffles; each
// group copies one row at a time in 16-byte vectors, four rows in flight,
// reading in shard-major order and writing the scattered slots with
// streaming stores.
#include "common.hpp"

namespace fs {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kLanesPerRow = 16;                    // 256 bytes per row pass
constexpr int kRowsPerStep = kWave / kLanesPerRow;  // rows per wave instruction
constexpr int kBatch = 4;                           // rows in flight per lane group

struct CombineArgs {
  const char* src;
  int64_t stride;                // bytes between consecutive rows of src
  const int64_t* shard_keys;
  const int32_t* shard_bm;
  const int64_t* shard_offsets;  // items [0, shard_offsets[W]) are valid
  int32_t W, T;
  int64_t row_base[FS_MAX_TABLES + 1];
  int32_t vpr[FS_MAX_TABLES];    // 16-byte vectors per row of each table
  char* out[FS_MAX_TABLES];
};

__global__ void __launch_bounds__(kThreads) k_combine(CombineArgs a) {
  // per-table values in LDS: a lane's table is a runtime index
  __shared__ char* s_out[FS_MAX_TABLES];
  __shared__ int32_t s_vpr[FS_MAX_TABLES];
  if (threadIdx.x < (unsigned)a.T) {
    s_out[threadIdx.x] = a.out[threadIdx.x];
    s_vpr[threadIdx.x] = a.vpr[threadIdx.x];
  }
  __syncthreads();
  const int64_t nv = a.shard_offsets[a.W];
  const int w = threadIdx.x / kWave, l = lane();
  const int64_t k0 = ((int64_t)blockIdx.x * (kThreads / kWave) + w) * kWave;
  if (k0 >= nv) return;
  const int nvalid = (int)min((int64_t)kWave, nv - k0);
  int32_t t = 0, bm = 0;
  if (l < nvalid) {
    const int64_t key = a.shard_keys[k0 + l];
    bm = a.shard_bm[k0 + l];
#pragma unroll
    for (int q = 1; q < FS_MAX_TABLES; ++q) t += (q < a.T && key >= a.row_base[q]) ? 1 : 0;
  }
  const int grp = l / kLanesPerRow, sub = l % kLanesPerRow;
  for (int s0 = 0; s0 < kWave / kRowsPerStep; s0 += kBatch) {
    int32_t tj[kBatch], bj[kBatch], vj[kBatch];
    bool on[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int j = (s0 + b) * kRowsPerStep + grp;
      tj[b] = __shfl(t, j, kWave);
      bj[b] = __shfl(bm, j, kWave);
      on[b] = j < nvalid;
      vj[b] = on[b] ? s_vpr[tj[b]] : 0;
    }
    // rows of more than 256 bytes take several passes of the lane group
    for (int v0 = 0;; v0 += kLanesPerRow) {
      u32x4 x[kBatch];
      bool go[kBatch];
      bool any = false;
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        go[b] = v0 + sub < vj[b];
        any |= v0 < vj[b];
        if (go[b]) {
          const int j = (s0 + b) * kRowsPerStep + grp;
          const u32x4* sp = (const u32x4*)(a.src + (k0 + j) * a.stride);
          x[b] = __builtin_nontemporal_load(sp + v0 + sub);
        }
      }
#pragma unroll
      for (int b = 0; b < kBatch; ++b) {
        if (go[b]) {
          u32x4* dp = (u32x4*)(s_out[tj[b]] + (int64_t)bj[b] * vj[b] * 16);
          __builtin_nontemporal_store(x[b], dp + v0 + sub);
        }
      }
      if (!any) break;
    }
  }
}

}  // namespace
}  // namespace fs

using namespace fs;

extern "C" int fs_ranged_combine(const void* src, int64_t src_stride, const int64_t* shard_keys,
                                 const int32_t* shard_bm, const int64_t* shard_offsets,
                                 int32_t W, const fs_table* tables, int32_t T, void* const* out,
                                 int64_t n_tok, hipStream_t stream) {
  if (!tables || T < 1 || T > FS_MAX_TABLES || W < 1 || W > FS_MAX_RANKS || n_tok < 0 ||
      (int64_t)T * n_tok >= (int64_t)INT32_MAX || !shard_offsets || !out)
    return FS_ERR_INVALID_ARG;
  if (n_tok > 0 && (!src || !shard_keys || !shard_bm)) return FS_ERR_INVALID_ARG;
  CombineArgs a;
  a.src = (const char*)src;
  a.stride = src_stride;
  a.shard_keys = shard_keys;
  a.shard_bm = shard_bm;
  a.shard_offsets = shard_offsets;
  a.W = W;
  a.T = T;
  int64_t base = 0, max_bytes = 0;
  for (int t = 0; t < T; ++t) {
    const fs_table& tb = tables[t];
    if (tb.rows < 1 || tb.dim < 1 || (tb.dtype != FS_F32 && tb.dtype != FS_BF16))
      return FS_ERR_INVALID_ARG;
    const int64_t rb = (int64_t)tb.dim * (tb.dtype == FS_F32 ? 4 : 2);
    if (rb != 64 && rb != 128 && rb != 256 && rb != 512 && rb != 1024 && rb != 2048)
      return FS_ERR_UNSUPPORTED;
    if (n_tok > 0 && (!out[t] || ((uintptr_t)out[t] & 15))) return FS_ERR_INVALID_ARG;
    a.row_base[t] = base;
    a.vpr[t] = (int32_t)(rb / 16);
    a.out[t] = (char*)out[t];
    base += tb.rows;
    max_bytes = rb > max_bytes ? rb : max_bytes;
  }
  a.row_base[T] = base;
  if (base > (int64_t)UINT32_MAX) return FS_ERR_UNSUPPORTED;
  if (n_tok > 0 && (src_stride < max_bytes || (src_stride & 15) || ((uintptr_t)src & 15)))
    return FS_ERR_INVALID_ARG;
  const int64_t cap = (int64_t)T * n_tok;  // items the dispatch can have produced
  if (cap == 0) return FS_OK;
  hipLaunchKernelGGL(k_combine, dim3((unsigned)cdiv(cap, kThreads)), dim3(kThreads), 0, stream,
                     a);
  FS_LAUNCH_CHECK();
  return FS_OK;
}
