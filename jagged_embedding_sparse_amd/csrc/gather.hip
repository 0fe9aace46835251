// Jagged embedding lookup: unique rows -> batch-major output slots.
//
// "FreeScale: distributed training for sequence recommendation models",
// Algorithm 2: Lookup of the (exclusive or collision) rows, the AllToAll back
// to batch-major form and the merge of both classes into one batch. On one
// GPU the three fuse: each occurrence's batch-major slot receives a bit copy
// of its row.
//
// Work is spread over occurrences in CSR order, not over unique rows: hot
// rows (tens of thousands of occurrences under Zipf IDs) split evenly, and
// consecutive occurrences of one row re-read it from L1/L2, so HBM sees
// each unique row about once. A lane group of row_bytes/16 lanes (at most
// 64) copies one row with 16-byte loads and streaming stores.
#include "common.hpp"

namespace fs {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

struct LookupArgs {
  const char* weights;
  char* out;
  int64_t stride;  // bytes between weight rows
  int64_t row_base;
  int64_t n_cap;  // occurrences this table can have (n_tok)
  const int64_t* unique;
  const int64_t* unique_offsets;
  const int32_t* seg_offsets;
  const int32_t* occ_bm;
  const int32_t* occ_uid;
  const uint8_t* cls;
  int32_t g_lo, g_hi;  // group range of the table: [t*W, (t+1)*W]
  int32_t which;
  int32_t vpr;  // 16-byte vectors per row
};

// Every table of a call in one launch: workgroups [lo_t, lo_{t+1}) copy
// table t.
struct LookupBatch {
  LookupArgs t[FS_MAX_TABLES];
  int32_t block_lo[FS_MAX_TABLES + 1];
  int32_t n;
};

// Occurrences per wave: 64 for rows of up to 256 B, fewer for larger rows,
// so that a wave copies its rows in one batch and more waves share the work.
template <int VPR>
struct LookupShape {
  static constexpr int OPW = VPR <= 16 ? kWave : (VPR == 32 ? 32 : 16);
};

// One wave per OPW consecutive occurrences (CSR order). Index data is read
// coalesced once per wave -- occurrence -> (unique, slot), then the <= OPW
// unique rows those occurrences span -> (key, class) -- and handed to the
// copying lanes with cross-lane shuffles, so rows start loading after two
// dependent index loads and up to 16 rows per lane group are in flight.
template <int VPR>  // 16-byte vectors per row
__device__ __forceinline__ void lookup_rows(const LookupArgs& a, int64_t blk) {
  constexpr int LPR = VPR < kWave ? VPR : kWave;  // lanes per row
  constexpr int RPW = kWave / LPR;                // rows per wave instruction
  constexpr int VPL = VPR / LPR;                  // vectors per lane
  constexpr int OPW = LookupShape<VPR>::OPW;      // occurrences per wave
  constexpr int STEPS = OPW / RPW;                // row steps for OPW occurrences
  // rows per lane group in flight; 128-B rows take two batches of four (all
  // eight at once compiled to 252 VGPRs, four to 90)
  constexpr int BATCH = VPR == 8 ? 4 : (STEPS < 16 / VPL ? STEPS : 16 / VPL);
  const int64_t o_lo = a.seg_offsets[a.unique_offsets[a.g_lo]];
  const int64_t o_hi = a.seg_offsets[a.unique_offsets[a.g_hi]];
  const int w = threadIdx.x / kWave, l = lane();
  const int64_t o0 = o_lo + (blk * (kThreads / kWave) + w) * OPW;
  if (o0 >= o_hi) return;
  const int nvalid = (int)min((int64_t)OPW, o_hi - o0);
  const bool valid = l < nvalid;
  const int32_t u = valid ? a.occ_uid[o0 + l] : 0;
  const int32_t bm = valid ? a.occ_bm[o0 + l] : -1;
  const int32_t u0 = __shfl(u, 0, kWave);
  const int32_t span = __shfl(u, nvalid - 1, kWave) - u0 + 1;  // <= OPW
  uint32_t key = 0;
  int c = 0;
  if (l < span) {
    key = (uint32_t)(a.unique[u0 + l] - a.row_base);
    if (a.which >= 0) c = a.cls[u0 + l];
  }
  const int src = valid ? u - u0 : 0;
  const uint32_t row = (uint32_t)__shfl((int)key, src, kWave);
  const int cc = __shfl(c, src, kWave);
  const int32_t dst = (valid && (a.which < 0 || cc == a.which)) ? bm : -1;
  if (!__ballot(dst >= 0)) return;
  const int grp = l / LPR, sub = l % LPR;
#pragma unroll
  for (int s0 = 0; s0 < STEPS; s0 += BATCH) {
    u32x4 v[BATCH][VPL];
    int32_t d[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int j = (s0 + b) * RPW + grp;
      const uint32_t r = (uint32_t)__shfl((int)row, j, kWave);
      d[b] = __shfl(dst, j, kWave);
      if (d[b] >= 0) {
        const u32x4* sp = (const u32x4*)(a.weights + (int64_t)r * a.stride);
#pragma unroll
        for (int k = 0; k < VPL; ++k) v[b][k] = sp[sub + k * LPR];
      }
    }
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      if (d[b] < 0) continue;
      u32x4* dp = (u32x4*)(a.out + (int64_t)d[b] * (VPR * 16));
#pragma unroll
      for (int k = 0; k < VPL; ++k) __builtin_nontemporal_store(v[b][k], dp + sub + k * LPR);
    }
  }
}

// Each workgroup takes its table's row-size instance of the copy (all share
// one register allocation: the largest instance needs 102 VGPRs).
__global__ void __launch_bounds__(kThreads) k_lookup(LookupBatch batch) {
  int ti = 0;
  while (ti + 1 < batch.n && (int32_t)blockIdx.x >= batch.block_lo[ti + 1]) ++ti;
  const LookupArgs& a = batch.t[ti];
  const int64_t blk = (int64_t)blockIdx.x - batch.block_lo[ti];
  switch (a.vpr) {
    case 4: lookup_rows<4>(a, blk); break;
    case 8: lookup_rows<8>(a, blk); break;
    case 16: lookup_rows<16>(a, blk); break;
    case 32: lookup_rows<32>(a, blk); break;
    case 64: lookup_rows<64>(a, blk); break;
    default: lookup_rows<128>(a, blk); break;
  }
}

int occ_per_wave(int vpr) {
  switch (vpr) {
    case 4: return LookupShape<4>::OPW;
    case 8: return LookupShape<8>::OPW;
    case 16: return LookupShape<16>::OPW;
    case 32: return LookupShape<32>::OPW;
    case 64: return LookupShape<64>::OPW;
    default: return LookupShape<128>::OPW;
  }
}

}  // namespace
}  // namespace fs

using namespace fs;

extern "C" int fs_jagged_lookup(const fs_table* tables, int32_t T, int32_t W,
                                const int64_t* unique, const int64_t* unique_offsets,
                                const int32_t* seg_offsets, const int32_t* occ_bm,
                                const int32_t* occ_uid, const uint8_t* cls, int32_t which,
                                void* const* out, int64_t n_tok, hipStream_t stream) {
  if (!tables || T < 1 || T > FS_MAX_TABLES || W < 1 || W > FS_MAX_RANKS || n_tok < 0 ||
      (int64_t)T * n_tok >= (int64_t)INT32_MAX || !out || !unique_offsets || !seg_offsets)
    return FS_ERR_INVALID_ARG;
  if (which != FS_ALL && which != FS_EXCLUSIVE && which != FS_COLLISION) return FS_ERR_INVALID_ARG;
  if (which != FS_ALL && !cls) return FS_ERR_INVALID_ARG;
  if (n_tok > 0 && (!unique || !occ_bm || !occ_uid)) return FS_ERR_INVALID_ARG;
  int64_t base = 0;
  for (int t = 0; t < T; ++t) {
    const fs_table& tb = tables[t];
    if (tb.rows < 1 || tb.dim < 1 || (tb.dtype != FS_F32 && tb.dtype != FS_BF16))
      return FS_ERR_INVALID_ARG;
    if (n_tok > 0 && (!tb.weights || !out[t])) return FS_ERR_INVALID_ARG;
    const int64_t rb = (int64_t)tb.dim * (tb.dtype == FS_F32 ? 4 : 2);
    if (rb != 64 && rb != 128 && rb != 256 && rb != 512 && rb != 1024 && rb != 2048)
      return FS_ERR_UNSUPPORTED;
    if (!table_layout_ok(tb, false)) return FS_ERR_INVALID_ARG;
    base += tb.rows;
  }
  if (base > (int64_t)UINT32_MAX) return FS_ERR_UNSUPPORTED;
  // one launch for every table
  LookupBatch b;
  b.n = T;
  b.block_lo[0] = 0;
  base = 0;
  for (int t = 0; t < T; ++t) {
    const fs_table& tb = tables[t];
    LookupArgs& a = b.t[t];
    a.weights = (const char*)tb.weights;
    a.out = (char*)out[t];
    a.stride = table_stride(tb);
    a.row_base = base;
    a.n_cap = n_tok;
    a.unique = unique;
    a.unique_offsets = unique_offsets;
    a.seg_offsets = seg_offsets;
    a.occ_bm = occ_bm;
    a.occ_uid = occ_uid;
    a.cls = cls;
    a.g_lo = t * W;
    a.g_hi = (t + 1) * W;
    a.which = which;
    a.vpr = (int32_t)(tb.dim * (tb.dtype == FS_F32 ? 4 : 2) / 16);
    base += tb.rows;
    const int64_t occ_per_block = (int64_t)occ_per_wave(a.vpr) * (kThreads / kWave);
    b.block_lo[t + 1] = b.block_lo[t] + (int32_t)cdiv(n_tok, occ_per_block);
  }
  if (b.block_lo[T] > 0) {
    hipLaunchKernelGGL(k_lookup, dim3((unsigned)b.block_lo[T]), dim3(kThreads), 0, stream, b);
    FS_LAUNCH_CHECK();
  }
  return FS_OK;
}
