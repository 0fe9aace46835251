/*
 * fs_sparse.h -- C ABI of the MI355X (gfx950) jagged sparse step.
 *
 * The library runs, on one GPU, the per-step sparse path of row-wise sharded
 * sequence-recommender training as one rank of a virtual W-rank job would:
 * balance the global batch, permute and bucketize its IDs into per-shard
 * (shard-major) buffers, dedup each shard, split the unique rows into the
 * ones that collide with the previous iteration and the exclusive rest, gather
 * embeddings, segment-reduce gradients per unique row and apply a row-wise
 * SGD / Adagrad update. The method is the one of "FreeScale: distributed
 * training for sequence recommendation models" (arXiv 2604.24073), cited
 * below as [FS] with its section, algorithm or equation.
 *
 * Conventions for every call:
 *  - Array arguments are DEVICE pointers unless marked "host". The caller owns
 *    all memory; no call allocates or frees, and none keeps state between
 *    calls. Scratch memory comes from a caller workspace (ws, ws_bytes) whose
 *    size a host-only fs_*_workspace_size() query returns; it depends only on
 *    capacities, never on data, and never decreases as they shrink. (The one
 *    exception, fs_grad_reduce_update_noalloc, uses a fixed device array of
 *    the library's instead of a workspace.)
 *  - Every call is asynchronous on `stream`, makes no host synchronisation and
 *    may be captured. Data-dependent counts (unique rows, collisions, valid
 *    items) are written to device memory only; grids are sized by capacity.
 *    The caller orders streams (events), e.g. so that a lookup of iteration
 *    i+1 runs after the collision-row update of iteration i.
 *  - Return value: FS_OK or a negative FS_ERR_* code for what the host can
 *    check before launching (null pointers, sizes, unsupported shapes, a
 *    workspace that is too small, a failed launch). On error nothing is
 *    launched, except FS_ERR_HIP where earlier launches of the call may run.
 *  - Data faults found on the device are OR-ed into a caller-owned sticky
 *    int32 flag word `err` (FS_EF_* bits); the offending element is handled
 *    as documented per call and the rest of the output stays defined.
 *  - Integer types: IDs, keys and offsets into token arrays are int64;
 *    positions inside one call's arrays are int32, so one call handles fewer
 *    than 2^31 items.
 *  - Tables: `fs_table` describes table t of T. Keys are global row numbers:
 *    key = row_base_t + id with row_base_t = rows_0 + ... + rows_{t-1}; the
 *    sum of all rows must be below 2^32. Table t is row-wise sharded into W
 *    contiguous blocks of ceil(rows_t / W) rows: shard(t, id) = id / that.
 */
#ifndef FS_SPARSE_H
#define FS_SPARSE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* return codes */
#define FS_OK 0
#define FS_ERR_INVALID_ARG (-1)
#define FS_ERR_WORKSPACE (-2)
#define FS_ERR_HIP (-3)
#define FS_ERR_UNSUPPORTED (-4)
#define FS_ERR_TOO_LARGE (-5) /* beyond an allocation-free call's fixed scratch */

/* sticky device error bits */
#define FS_EF_ID_RANGE 1  /* an ID outside [0, rows_t) was dropped */
#define FS_EF_SHAPE 2     /* sample_offsets[n] != n_tok, or offsets decrease */
#define FS_EF_LEN_RANGE 4 /* a UIH length outside [0, FS_MAX_UIH] was clamped */

/* limits */
#define FS_MAX_SAMPLES 16384 /* samples per balance / bucketize call */
#define FS_MAX_RANKS 1024    /* virtual ranks = shards, W */
#define FS_MAX_TABLES 8
#define FS_MAX_UIH 65535

/* enums */
#define FS_F32 0
#define FS_BF16 1
#define FS_SGD 0
#define FS_RW_ADAGRAD 1
#define FS_ALL (-1)
#define FS_EXCLUSIVE 0
#define FS_COLLISION 1
/* rows of an update call by occurrence count (a bit mask) */
#define FS_ROWS_FEW 1  /* at most 64 occurrences: each row summed whole */
#define FS_ROWS_MANY 2 /* more than 64: summed in chunks, then combined */
#define FS_ROWS_ALL 3

typedef struct fs_table {
  void* weights;  /* device: rows rows of dim elements, dtype FS_F32 or FS_BF16 */
  float* state;   /* device fp32 row-wise Adagrad accumulator per row, or NULL */
  int64_t rows;   /* R_t */
  int32_t dim;    /* D_t */
  int32_t dtype;  /* FS_F32 or FS_BF16 */
  int64_t stride;       /* bytes from one weight row to the next; 0: dim * sizeof(dtype) */
  int64_t state_stride; /* bytes from one row's state to the next; 0: 4 */
} fs_table;
/* Layouts: dense ([rows][dim] weights and a separate [rows] state, strides  */
/* 0), rows spaced `stride` bytes apart, or each row's state in its own row */
/* slot -- stride >= dim * sizeof(dtype) + 4, state = weights + dim *        */
/* sizeof(dtype) bytes, state_stride = stride -- so that a row's update     */
/* reads and writes one slot instead of a slot and a separate state entry.  */
/* Slots of a power of two keep rows aligned to the memory's 128-byte lines */
/* (a 256-byte row in a 272-byte slot straddles an extra line). The lookup  */
/* and the update need weights 16-byte aligned, a stride that is a multiple */
/* of 16 and at least the row size, and a state stride that is a multiple  */
/* of 4 and at least 4 (else FS_ERR_INVALID_ARG); the state of a row must   */
/* not overlap its weights. Other calls read only rows, dim and dtype.      */

/* ------------------------------------------------------------------------ */
/* Load balancing -- [FS] section 4.1 (partitioning algorithms), run inside  */
/* the protocol of section 3.1 / Algorithm 1 (the partition function P      */
/* maps the gathered global batch to ranks). Every rank computes the same   */
/* result from the gathered lengths.                                        */
/*                                                                          */
/* Both sort the n samples of the global batch by UIH length, ascending,    */
/* ties by global sample index (stable).                                    */
/*  uih_len      [n] int32, UIH length of global sample s (s = the rank-major */
/*               gather order). Values outside [0, FS_MAX_UIH] are clamped   */
/*               and flag FS_EF_LEN_RANGE.                                   */
/*  perm         [n] int32 out: the balanced batch, rank-major: rank r's      */
/*               samples are perm[rank_offsets[r] .. rank_offsets[r+1]).      */
/*  rank_offsets [W+1] int32 out.                                            */
/*  err          sticky flags (may be NULL: faults then go unreported).      */
/*  ws, ws_bytes workspace of at least fs_balance_workspace_size(n, W) bytes */
/*               (else FS_ERR_WORKSPACE): per-slice sort counts, and VBS's    */
/*               weights and prefix sums.                                    */
/* n in [0, FS_MAX_SAMPLES], W in [1, FS_MAX_RANKS].                         */

/* FBS: zig-zag (snake) deal of the sorted samples. [FS] 4.1 prints rank i's */
/* positions as i, 2n-i, 2n+i, 4n-i, ... which is not a partition as printed; */
/* the build reads it as the snake draft i, 2W-1-i, 2W+i, 4W-1-i, ... (0-based). */
/* Each rank keeps its samples in dealing order. Counts differ by at most 1. */
int fs_balance_fbs(const int32_t* uih_len, int32_t n, int32_t W, int32_t* perm,
                   int32_t* rank_offsets, int32_t* err, void* ws, size_t ws_bytes,
                   hipStream_t stream);

/* VBS: weights w = round(L^alpha), alpha = alpha_num / alpha_den, exact in   */
/* integers (alpha in {0, 1/2, 1, 3/2, 2}; else FS_ERR_UNSUPPORTED). The     */
/* sorted samples are cut into W contiguous segments of about equal weight: */
/* rank r starts at the first prefix position whose weight sum reaches       */
/* r/W of the total, so each segment is within one boundary sample's weight */
/* of total/W; empty segments are legal. perm is the sorted order.           */
/*  rank_weight  [W] int64 out, weight of each segment (may be NULL).        */
int fs_balance_vbs(const int32_t* uih_len, int32_t n, int32_t W, int32_t alpha_num,
                   int32_t alpha_den, int32_t* perm, int32_t* rank_offsets,
                   int64_t* rank_weight, int32_t* err, void* ws, size_t ws_bytes,
                   hipStream_t stream);

size_t fs_balance_workspace_size(int32_t n, int32_t W);

/* ------------------------------------------------------------------------ */
/* VBS AutoTune -- [FS] 4.1: because the weights L^alpha need not match the */
/* real execution time, VBS raises or lowers each rank's local batch size by */
/* how its execution time compares with the global average (Figure 4's      */
/* AutoTune module; Algorithm 1's input R). The pages give no arithmetic;   */
/* the built reading moves per-rank shares s_r of the weight:               */
/*                                                                          */
/* fs_balance_vbs_shares: fs_balance_vbs with the cut at the shares: with   */
/* Q_r = s_0 + ... + s_{r-1}, Q = Q_W and S_k the weight of the first k     */
/* sorted samples (T = S_n), rank r starts at the first k with              */
/* Q * S_k >= Q_r * T, so each segment is within one boundary sample's      */
/* weight of T * s_r / Q. Equal shares give exactly fs_balance_vbs's cuts.  */
/*  shares       device int64 [W], each in [1, 2^40]; others are clamped and */
/*               flag FS_EF_SHAPE. Other arguments as fs_balance_vbs.        */
int fs_balance_vbs_shares(const int32_t* uih_len, int32_t n, int32_t W, int32_t alpha_num,
                          int32_t alpha_den, const int64_t* shares, int32_t* perm,
                          int32_t* rank_offsets, int64_t* rank_weight, int32_t* err, void* ws,
                          size_t ws_bytes, hipStream_t stream);

/* fs_rank_cost: modelled execution time of each rank of a partition, for   */
/* when no measured time exists: cost[r] = the sum over positions j in      */
/* [rank_offsets[r], rank_offsets[r+1]) of c2 L^2 + c1 L + c0 with          */
/* L = uih_len[perm[j]] clamped to [0, FS_MAX_UIH] (quadratic attention-like */
/* plus linear work). Coefficients in [0, 2^16] (else FS_ERR_INVALID_ARG).  */
/* Offsets are clipped to [0, n]; perm entries outside [0, n) count nothing. */
/*  uih_len [n], perm [n], rank_offsets [W+1]: a balance call's inputs and  */
/*  outputs; cost [W] int64 out.                                            */
int fs_rank_cost(const int32_t* uih_len, int32_t n, const int32_t* perm,
                 const int32_t* rank_offsets, int32_t W, int64_t c2, int64_t c1, int64_t c0,
                 int64_t* cost, hipStream_t stream);

/* fs_vbs_autotune: one AutoTune step on shares[W] in place. With the mean  */
/* m = (t_0 + ... + t_{W-1}) / W of the per-rank times, a rank with         */
/* t_r > m (1 + tol) gives up d_r = max(1, floor(s_r * step)) of its share,  */
/* one with t_r < m (1 - tol) gains d_r, the rest keep theirs; shares stay  */
/* in [1, 2^40]. All integer: W t_r tol_den is compared with                 */
/* (sum t)(tol_den +- tol_num), step = step_num / step_den.                 */
/*  times   device int64 [W] in [0, 2^52] (measured, e.g. in ns, or           */
/*          fs_rank_cost's); values outside are clamped and flag FS_EF_SHAPE, */
/*          as do shares outside [1, 2^40].                                  */
/*  0 <= step_num <= step_den <= 2^20, 0 <= tol_num <= tol_den <= 2^20       */
/*  (else FS_ERR_INVALID_ARG).                                              */
int fs_vbs_autotune(const int64_t* times, int32_t W, int32_t step_num, int32_t step_den,
                    int32_t tol_num, int32_t tol_den, int64_t* shares, int32_t* err,
                    hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Indexed permute + ranged dispatch -- [FS] 4.2 (the indexed-permute kernel */
/* applies the partition to the gathered IDs; the ranged-dispatch kernel    */
/* prepares the ID AllToAll's per-destination ranges) and 3.2 (batch-major  */
/* vs shard-major forms).                                                   */
/*                                                                          */
/*  ids            [T][n_tok] int64, table-major: ids[t*n_tok + k] is table t's */
/*                 ID of token k of the unbalanced batch.                   */
/*  sample_offsets [n+1] int64: sample s owns tokens [so[s], so[s+1]) (UIH   */
/*                 tokens, then candidate tokens). so[n] must equal n_tok.   */
/*  tables         host [T]: rows and dim are read (weights may be NULL).    */
/*  perm, rank_offsets: a balance call's output for the same n and W.        */
/* Outputs:                                                                  */
/*  bal_offsets    [n+1] int64: the q-th balanced sample s = perm[q] owns     */
/*                 batch-major tokens [bal[q], bal[q+1]); token j of it has   */
/*                 batch-major index bm = bal[q] + j.                          */
/*  shard_keys     [T*n_tok] int64, shard_bm [T*n_tok] int32: every valid    */
/*                 (table, token) item as key = row_base_t + id and its bm,  */
/*                 in shard-major order: destination shard d, then source    */
/*                 rank r, then table t, then balanced sample, then token    */
/*                 (what a W-way AllToAll of per-destination, table-major     */
/*                 send buffers delivers). Entries past shard_offsets[W] are  */
/*                 unspecified.                                               */
/*  splits         [W*W] int64: splits[d*W + r] = items rank r sends to d.    */
/*  shard_offsets  [W+1] int64: shard d's items are [so_d, so_{d+1}).        */
/*  err            IDs outside [0, rows_t) are dropped (FS_EF_ID_RANGE).     */
/*                 Sample offsets not rising from 0 to n_tok, a perm entry   */
/*                 outside [0, n), rank offsets not rising from 0 to n, or   */
/*                 lengths under perm not summing to n_tok flag FS_EF_SHAPE: */
/*                 then no item is written, shard_offsets and splits are     */
/*                 all zero and bal_offsets is unspecified.                  */
int fs_bucketize_permute(const int64_t* ids, int64_t n_tok, const int64_t* sample_offsets,
                         int32_t n, const fs_table* tables, int32_t T, const int32_t* perm,
                         const int32_t* rank_offsets, int32_t W, int64_t* bal_offsets,
                         int64_t* shard_keys, int32_t* shard_bm, int64_t* splits,
                         int64_t* shard_offsets, int32_t* err, void* ws, size_t ws_bytes,
                         hipStream_t stream);

size_t fs_bucketize_workspace_size(int64_t n_tok, int32_t n, int32_t T, int32_t W);

/* ------------------------------------------------------------------------ */
/* Dedup + collision split -- [FS] 3.2 and Algorithm 2 (compute_collision on */
/* the shard-major indices of iterations i and i+1): a row of iteration i+1 */
/* collides when iteration i updates it; only those rows need the write-    */
/* then-read order, every other (exclusive) row can be fetched ahead.       */
/*                                                                          */
/*  shard_keys, shard_bm, shard_offsets: a bucketize call's output (items   */
/*                 of shard d in [so_d, so_{d+1}), each a row of shard d,    */
/*                 bm rising within a shard; the dedup keeps the items'      */
/*                 order within each row, so occ_bm rises within each row).  */
/*                 Offsets are clamped into [0, n_cap] and made rising, and  */
/*                 a key outside its range's shard is clamped into it: such  */
/*                 input gives unspecified results but writes nothing past    */
/*                 the outputs.                                               */
/*  n_cap          host: capacity of the shard arrays (T*n_tok).             */
/*  prev_unique, prev_unique_offsets, prev_counts: the previous call's        */
/*                 unique, unique_offsets and counts (device; a call with the */
/*                 same tables and W), or all three NULL for the first        */
/*                 iteration (all rows exclusive). Offsets are clamped into   */
/*                 [0, prev U] and made rising.                               */
/*  prev_cap       host: capacity of prev_unique / prev_cls (0 when NULL).   */
/* Outputs (capacities n_cap unless noted):                                  */
/*  unique         int64 unique keys, ascending (= by table, then row). The   */
/*                 rows of (table t, shard d) are the contiguous range        */
/*                 unique_offsets[t*W+d] .. unique_offsets[t*W+d+1].          */
/*  unique_offsets [T*W+1] int64; the last entry is U.                        */
/*  seg_offsets    [n_cap+1] int32 CSR: unique row u's occurrences are        */
/*                 occ_bm[seg_offsets[u] .. seg_offsets[u+1]).                */
/*  occ_bm         int32 batch-major index of each occurrence, ascending      */
/*                 within each row.                                           */
/*  occ_uid        int32 unique index of each occurrence (CSR order).          */
/*  cls            uint8 [U]: FS_COLLISION if the row is in prev_unique.      */
/*  prev_cls       uint8 [prev U] (NULL when prev_unique is NULL):            */
/*                 FS_COLLISION if the previous row is in unique.             */
/*  counts         [4] int64: U, collisions C, U - C, prev U - C.             */
int fs_unique_collision_split(const int64_t* shard_keys, const int32_t* shard_bm,
                              const int64_t* shard_offsets, int64_t n_cap,
                              const fs_table* tables, int32_t T, int32_t W,
                              const int64_t* prev_unique, const int64_t* prev_unique_offsets,
                              const int64_t* prev_counts, int64_t prev_cap, int64_t* unique,
                              int64_t* unique_offsets,
                              int32_t* seg_offsets, int32_t* occ_bm, int32_t* occ_uid,
                              uint8_t* cls, uint8_t* prev_cls, int64_t* counts, void* ws,
                              size_t ws_bytes, hipStream_t stream);

size_t fs_unique_workspace_size(int64_t n_cap, int64_t prev_cap, int32_t T, int32_t W);

/* Collision split alone -- Algorithm 2's compute_collision on two dedup      */
/* results, for a caller that deduplicates an iteration before the previous  */
/* iteration's rows exist (fs_unique_collision_split with the three prev     */
/* pointers NULL), so that consecutive dedups need not wait for each other.  */
/* Together the two calls give exactly the outputs of one                     */
/* fs_unique_collision_split call with the previous rows.                     */
/*  unique, unique_offsets  a dedup call's outputs for T tables and W shards  */
/*                 (rows of (t, d) in unique_offsets[t*W+d] .. [t*W+d+1]).    */
/*  n_cap          host: capacity of unique and cls (the dedup call's n_cap). */
/*  prev_unique, prev_unique_offsets, prev_counts, prev_cap: as in            */
/*                 fs_unique_collision_split (all three NULL: every row       */
/*                 exclusive).                                               */
/*  cls            uint8 [U]: FS_COLLISION if the row is in prev_unique.      */
/*  prev_cls       uint8 [prev U] (NULL when prev_unique is NULL).            */
/*  counts         [4] int64, in/out: counts[0] = U as the dedup call wrote   */
/*                 it (read); counts[1..3] = C, U - C, prev U - C (written).  */
/*  ws, ws_bytes   at least fs_collision_split_workspace_size(n_cap, T, W).   */
int fs_collision_split(const int64_t* unique, const int64_t* unique_offsets, int64_t n_cap,
                       int32_t T, int32_t W, const int64_t* prev_unique,
                       const int64_t* prev_unique_offsets, const int64_t* prev_counts,
                       int64_t prev_cap, uint8_t* cls, uint8_t* prev_cls, int64_t* counts,
                       void* ws, size_t ws_bytes, hipStream_t stream);

size_t fs_collision_split_workspace_size(int64_t n_cap, int32_t T, int32_t W);

/* ------------------------------------------------------------------------ */
/* Jagged lookup -- Algorithm 2's Lookup, the batch-major transform that     */
/* follows it, and merge: every occurrence of a unique row of class `which`  */
/* (FS_ALL, FS_EXCLUSIVE or FS_COLLISION) gets a bit copy of the row, at its */
/* batch-major slot: out[t][bm] = weights_t[unique - row_base_t]. Other rows */
/* of out are not written.                                                   */
/*  tables   host [T] (weights, rows, dim, dtype are read).                  */
/*  unique .. occ_uid, cls: the split call's outputs for this iteration      */
/*           (cls may be NULL when which == FS_ALL).                          */
/*  out      host [T] of device [n_tok][dim_t] pointers, table dtype.         */
/* Row sizes dim_t * sizeof(dtype) must be 64, 128, 256, 512, 1024 or 2048    */
/* bytes (else FS_ERR_UNSUPPORTED).                                           */
int fs_jagged_lookup(const fs_table* tables, int32_t T, int32_t W, const int64_t* unique,
                     const int64_t* unique_offsets, const int32_t* seg_offsets,
                     const int32_t* occ_bm, const int32_t* occ_uid, const uint8_t* cls,
                     int32_t which, void* const* out, int64_t n_tok, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Ranged combine -- [FS] 4.2: the kernel that lays out the output of the    */
/* embedding AllToAll (the rows a rank receives from the shards, range by    */
/* range) in the rank's batch-major order. With every virtual rank on one GPU */
/* the rows come in the dispatch's shard-major order: row k of src belongs   */
/* to item k of fs_bucketize_permute's output and is copied to              */
/*   out[t][shard_bm[k]],  t = the table whose key range holds shard_keys[k], */
/* for k < shard_offsets[W] (the valid items; dropped IDs are not combined). */
/* Slots no item maps to are not written. The sparse step does not need it   */
/* (fs_jagged_lookup writes batch-major slots itself); it is the standalone  */
/* combine of the dispatch.                                                  */
/*  src, src_stride  device rows, 16-byte aligned, src_stride bytes apart    */
/*               (a multiple of 16, at least every table's row size).        */
/*  shard_keys, shard_bm, shard_offsets, W: fs_bucketize_permute's outputs   */
/*               for this batch (shard_bm < n_tok; other values write out of  */
/*               bounds).                                                    */
/*  tables   host [T]: rows, dim and dtype set the key ranges and row sizes  */
/*           (dim_t * sizeof(dtype) in {64, 128, ..., 2048} bytes, else      */
/*           FS_ERR_UNSUPPORTED); weights are not read.                      */
/*  out      host [T] of device [n_tok][dim_t] pointers, 16-byte aligned.    */
int fs_ranged_combine(const void* src, int64_t src_stride, const int64_t* shard_keys,
                      const int32_t* shard_bm, const int64_t* shard_offsets, int32_t W,
                      const fs_table* tables, int32_t T, void* const* out, int64_t n_tok,
                      hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Keyed transpose -- [FS] 4.2: a jagged tensor of F features (keys) over B  */
/* samples goes from feature-major to batch-major order. Input list (f, b)   */
/* holds lengths[f*B + b] values and the lists lie in the order (0,0),       */
/* (0,1), .., (0,B-1), (1,0), ..; the output holds the same lists in the     */
/* order (b=0,f=0), (0,1), .., (0,F-1), (1,0), .., each list's values in    */
/* their input order.                                                        */
/*  values       device [n_vals] elements of elem_bytes (4 or 8, else        */
/*               FS_ERR_UNSUPPORTED; aligned to it); copied bit for bit.     */
/*  lengths      device int32 [F][B]; negative lengths count as zero and     */
/*               flag FS_EF_SHAPE. F * B < 2^31; F or B may be 0.            */
/*  out_values   device [n_vals] elements, not aliasing values.              */
/*  out_offsets  device int64 [F*B + 1]: out_offsets[b*F + f] = where list   */
/*               (b, f) starts in out_values; out_offsets[F*B] = the total.  */
/*  err          nullable; FS_EF_SHAPE when the lengths do not sum to       */
/*               n_vals -- then values whose output position or input       */
/*               position is not below n_vals are not copied.               */
/*  ws, ws_bytes at least fs_keyed_transpose_workspace_size(F, B) bytes.    */
int fs_keyed_transpose(const void* values, int64_t n_vals, int32_t elem_bytes,
                       const int32_t* lengths, int32_t F, int32_t B, void* out_values,
                       int64_t* out_offsets, int32_t* err, void* ws, size_t ws_bytes,
                       hipStream_t stream);

size_t fs_keyed_transpose_workspace_size(int32_t F, int32_t B);

/* ------------------------------------------------------------------------ */
/* Gradient segment-reduce + row update -- Algorithm 2's backward (split the */
/* batch-major gradients into collision and exclusive parts, send them to    */
/* the shards, update_embedding) and its forward (the previous iteration's   */
/* exclusive rows are updated before the next exchange). For every unique    */
/* row u of class `which`: g_u = sum over its occurrences of grad[t][bm]     */
/* (fp64 accumulation in CSR order, rounded once to fp32), then              */
/*   FS_SGD:        w -= lr * g                                              */
/*   FS_RW_ADAGRAD: s += mean_d(g_d^2); w -= lr / (sqrt(s) + eps) * g        */
/* in fp32 with one rounding per operation; bf16 rows are widened exactly and */
/* stored round-to-nearest-even. Collision rows must be updated before the   */
/* next iteration's lookup of the same rows ([FS] 3.2).                      */
/*  grad         host [T] of device fp32 [n_tok][dim_t], batch-major.         */
/*  cls          the class of THIS iteration's rows against the next one: the */
/*               next split call's prev_cls (NULL with which == FS_ALL).      */
/*  rows         which of those rows by occurrence count: FS_ROWS_ALL,       */
/*               FS_ROWS_FEW or FS_ROWS_MANY (else FS_ERR_INVALID_ARG). The   */
/*               two parts update disjoint rows and only FS_ROWS_MANY uses    */
/*               the workspace, so they may run at the same time on two       */
/*               streams with one workspace; together they give exactly the  */
/*               FS_ROWS_ALL result. One update as two concurrent parts has  */
/*               one launch boundary fewer on each stream.                    */
/*  reduced_out  host [T] of device fp32 [U_t][dim_t] (or NULL array / NULL   */
/*               entries): row u of table t is written at u - unique_offsets[t*W]. */
/* dim_t must be 64, 128, 256, 512 or 1024 (else FS_ERR_UNSUPPORTED);        */
/* FS_RW_ADAGRAD needs every table's state.                                   */
/*  ws, ws_bytes  at least fs_grad_reduce_update_workspace_size(n_tok, T,    */
/*               max dim_t) bytes (fp64 partial sums of rows longer than a   */
/*               chunk, a region per table so that the tables' rows run side */
/*               by side), else FS_ERR_WORKSPACE.                             */
int fs_grad_reduce_update(const fs_table* tables, int32_t T, int32_t W,
                          const float* const* grad, int64_t n_tok, const int64_t* unique,
                          const int64_t* unique_offsets, const int32_t* seg_offsets,
                          const int32_t* occ_bm, const int32_t* occ_uid, const uint8_t* cls,
                          int32_t which, int32_t rows, int32_t optim, float lr, float eps,
                          float* const* reduced_out, void* ws, size_t ws_bytes,
                          hipStream_t stream);

size_t fs_grad_reduce_update_workspace_size(int64_t n_tok, int32_t T, int32_t max_dim);

/* fs_grad_reduce_update_noalloc: the same call for callers that cannot      */
/* allocate (code under HIP graph capture, tight serving loops, harnesses    */
/* that forbid hipMalloc): no workspace argument and no allocation of any   */
/* kind; the fp64 partial sums live in a fixed device array of              */
/* FS_NOALLOC_SCRATCH_BYTES per GPU, held from the first call on a device   */
/* until the process ends. Arguments, results and errors are those of        */
/* fs_grad_reduce_update, except that sizes whose                           */
/* fs_grad_reduce_update_workspace_size(n_tok, T, max dim_t) exceeds        */
/* FS_NOALLOC_SCRATCH_BYTES return FS_ERR_TOO_LARGE (one table of the       */
/* widest width: n_tok up to 33 553 920 at 64 columns, 16 776 704 at 128,  */
/* 2 097 024 at 256, 1 048 448 at 512, 524 160 at 1024; T tables need T    */
/* times the space). Every call on one GPU */
/* uses the same array: calls that overlap on one GPU (on different streams */
/* without an order between them) race and give undefined results; calls   */
/* ordered on one stream, or by events, are safe; so are an FS_ROWS_FEW     */
/* call and an FS_ROWS_MANY call that overlap (only the latter uses the     */
/* array). Nothing in the array needs clearing: each call writes every      */
/* partial it reads.                                                         */
#define FS_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int fs_grad_reduce_update_noalloc(const fs_table* tables, int32_t T, int32_t W,
                                  const float* const* grad, int64_t n_tok, const int64_t* unique,
                                  const int64_t* unique_offsets, const int32_t* seg_offsets,
                                  const int32_t* occ_bm, const int32_t* occ_uid,
                                  const uint8_t* cls, int32_t which, int32_t rows,
                                  int32_t optim, float lr, float eps, float* const* reduced_out,
                                  hipStream_t stream);

/* ------------------------------------------------------------------------ */
const char* fs_strerror(int code);
int fs_version(void);

#ifdef __cplusplus
}
#endif
#endif /* FS_SPARSE_H */
