/*
 * fs_oracle.c -- plain, slow, single-threaded CPU reference of the jagged
 * sparse step of FreeScale-style sequence-recommender training.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or call
 * this file; only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark do. It shares no source, header, table or helper with the HIP
 * library, and is built with gcc -O2 -ffp-contract=off so that every float
 * operation below is one IEEE operation in the order written.
 *
 * Source pages: "FreeScale: distributed training for sequence recommendation
 * models" (arXiv 2604.24073), abbreviated [FS]. Section numbers are that
 * paper's.
 *
 * Every function is written from the definition it cites, not from any
 * listing, and uses the plainest loop that states the definition.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_EF_ID_RANGE 1
#define OR_EF_LEN_RANGE 4

/* ------------------------------------------------------------------------ */
/* Balancing: [FS] section 4.1 "Partitioning Algorithms".                   */
/* Both partitioners order the global batch by UIH length. Reading: ascending */
/* length, ties by global sample index (the rank-major order in which the   */
/* lengths were gathered, [FS] section 3.1, Algorithm 1 stage I).           */

typedef struct { int64_t len; int64_t idx; } or_pair;

static int or_cmp_pair(const void* a, const void* b) {
  const or_pair* x = (const or_pair*)a;
  const or_pair* y = (const or_pair*)b;
  if (x->len != y->len) return x->len < y->len ? -1 : 1;
  if (x->idx != y->idx) return x->idx < y->idx ? -1 : 1;
  return 0;
}

/* order[p] = the sample at sorted position p. */
static void or_sorted_order(const int32_t* len, int32_t N, int32_t* order) {
  or_pair* v = (or_pair*)malloc(sizeof(or_pair) * (size_t)(N > 0 ? N : 1));
  for (int32_t s = 0; s < N; ++s) { v[s].len = len[s]; v[s].idx = s; }
  qsort(v, (size_t)N, sizeof(or_pair), or_cmp_pair);
  for (int32_t p = 0; p < N; ++p) order[p] = (int32_t)v[p].idx;
  free(v);
}

/* FBS rank of sorted position p. [FS] 4.1 prints the zig-zag as rank i taking
 * positions "i, 2n-i, 2n+i, 4n-i, ...", which is not a partition when read
 * literally. Reading: the snake draft, 0-based -- rank i takes i, 2n-1-i,
 * 2n+i, 4n-1-i, ...: even rounds of n positions go to ranks 0..n-1 in order,
 * odd rounds in reverse. */
int32_t or_fbs_rank_of_position(int64_t p, int32_t W) {
  int64_t round = p / W, off = p % W;
  return (int32_t)((round % 2 == 0) ? off : (W - 1 - off));
}

/* perm: rank-major concatenation of each rank's samples, in dealing order
 * (ascending sorted position). rank_offsets[W+1]. */
int or_balance_fbs(const int32_t* len, int32_t N, int32_t W,
                   int32_t* perm, int32_t* rank_offsets) {
  if (N < 0 || W < 1) return -1;
  int32_t* order = (int32_t*)malloc(sizeof(int32_t) * (size_t)(N > 0 ? N : 1));
  int32_t* fill = (int32_t*)calloc((size_t)W, sizeof(int32_t));
  or_sorted_order(len, N, order);
  /* count per rank */
  for (int32_t r = 0; r <= W; ++r) rank_offsets[r] = 0;
  for (int64_t p = 0; p < N; ++p) rank_offsets[or_fbs_rank_of_position(p, W) + 1] += 1;
  for (int32_t r = 0; r < W; ++r) rank_offsets[r + 1] += rank_offsets[r];
  /* place in ascending p within each rank */
  for (int64_t p = 0; p < N; ++p) {
    int32_t r = or_fbs_rank_of_position(p, W);
    perm[rank_offsets[r] + fill[r]] = order[p];
    fill[r] += 1;
  }
  free(order);
  free(fill);
  return 0;
}

static int64_t or_isqrt(int64_t x) { /* floor(sqrt(x)) for x >= 0, exact */
  if (x <= 0) return 0;
  int64_t r = (int64_t)sqrt((double)x);
  while (r > 0 && r * r > x) --r;
  while ((r + 1) * (r + 1) <= x) ++r;
  return r;
}

/* VBS weight round(L^alpha), alpha = num/den, computed exactly in integers.
 * [FS] 4.1 gives the weight as L to the power alpha; rounding to the nearest
 * integer makes prefix sums exact. Supported: den = 1 (integer powers) and
 * den = 2 (half-integer powers, via an integer square root: L^(num/2) is an
 * integer or irrational, so no ties arise and round(x) = (isqrt(4 x^2)+1)/2).
 * Returns -1 when unsupported. */
int64_t or_vbs_weight(int64_t L, int32_t num, int32_t den) {
  if (L < 0) return -1;
  if (den == 1) {
    if (num < 0 || num > 3) return -1;
    int64_t w = 1;
    for (int32_t k = 0; k < num; ++k) w *= L;
    return w;
  }
  if (den == 2) {
    if (num % 2 == 0) return or_vbs_weight(L, num / 2, 1);
    if (num < 0 || num > 3) return -1;
    int64_t p = 1; /* L^num */
    for (int32_t k = 0; k < num; ++k) p *= L;
    return (or_isqrt(4 * p) + 1) / 2;
  }
  return -1;
}

/* [FS] 4.1: VBS cuts the globally sorted samples into n contiguous segments of
 * approximately equal total weight. Reading: with S_k the prefix sum of the
 * first k sorted weights and T = S_N, rank r starts at
 *   c_r = min{ k in [0, N] : W * S_k >= r * T },
 * the lower bound of the ideal cut r*T/W; each segment then differs from T/W
 * by less than one boundary sample's weight. Segments may be empty.
 * perm = the sorted order; rank_offsets = c; rank_weight[r] = S_{c_{r+1}} - S_{c_r}. */
int or_balance_vbs(const int32_t* len, int32_t N, int32_t W, int32_t num, int32_t den,
                   int32_t* perm, int32_t* rank_offsets, int64_t* rank_weight) {
  if (N < 0 || W < 1) return -1;
  int32_t* order = (int32_t*)malloc(sizeof(int32_t) * (size_t)(N > 0 ? N : 1));
  int64_t* S = (int64_t*)malloc(sizeof(int64_t) * (size_t)(N + 1));
  or_sorted_order(len, N, order);
  S[0] = 0;
  for (int32_t k = 0; k < N; ++k) {
    int64_t w = or_vbs_weight(len[order[k]], num, den);
    if (w < 0) { free(order); free(S); return -2; }
    S[k + 1] = S[k] + w;
  }
  int64_t T = S[N];
  for (int32_t r = 0; r <= W; ++r) {
    int32_t c = 0;
    while (c < N && (int64_t)W * S[c] < (int64_t)r * T) ++c; /* linear search: plain */
    rank_offsets[r] = c;
  }
  rank_offsets[W] = N;
  for (int32_t k = 0; k < N; ++k) perm[k] = order[k];
  if (rank_weight)
    for (int32_t r = 0; r < W; ++r) rank_weight[r] = S[rank_offsets[r + 1]] - S[rank_offsets[r]];
  free(order);
  free(S);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* VBS AutoTune: [FS] 4.1 (VBS: the weights L^alpha may not track the real   */
/* execution time, so an autotune step raises or lowers a rank's local      */
/* batch size by how its execution time compares with the global average;   */
/* Figure 4's AutoTune module) and 3.1 (Algorithm 1's input R, the runtime  */
/* execution time information). The pages name the mechanism, not its       */
/* arithmetic. Readings:                                                    */
/*  - rank r holds a share s_r >= 1 of the batch weight; with Q_r = s_0 +   */
/*    ... + s_{r-1} and Q = Q_W, rank r starts at                           */
/*      c_r = min{ k in [0, N] : Q * S_k >= Q_r * T },                      */
/*    the lower bound of the ideal cut T * Q_r / Q. Equal shares give the   */
/*    plain VBS cut above.                                                  */
/*  - one AutoTune step: with times t_r and their mean m = (t_0 + ... +     */
/*    t_{W-1}) / W, a rank slower than m (1 + tol) gives up                 */
/*    d_r = max(1, floor(s_r * step)) of its share, a rank faster than      */
/*    m (1 - tol) gains d_r, the others keep theirs; shares stay in         */
/*    [1, 2^40]. The comparisons are made in integers:                      */
/*    W t_r tol_den > (sum t)(tol_den + tol_num), and < with tol_den - tol_num. */
/*  - without a dense model, R is modelled: t_r = the sum over the rank's   */
/*    samples of c2 L^2 + c1 L + c0 (quadratic attention plus linear work). */

#define OR_SHARE_MAX ((int64_t)1 << 40)

int or_balance_vbs_shares(const int32_t* len, int32_t N, int32_t W, int32_t num, int32_t den,
                          const int64_t* shares, int32_t* perm, int32_t* rank_offsets,
                          int64_t* rank_weight) {
  if (N < 0 || W < 1) return -1;
  for (int32_t r = 0; r < W; ++r)
    if (shares[r] < 1 || shares[r] > OR_SHARE_MAX) return -1;
  int32_t* order = (int32_t*)malloc(sizeof(int32_t) * (size_t)(N > 0 ? N : 1));
  int64_t* S = (int64_t*)malloc(sizeof(int64_t) * (size_t)(N + 1));
  or_sorted_order(len, N, order);
  S[0] = 0;
  for (int32_t k = 0; k < N; ++k) {
    int64_t w = or_vbs_weight(len[order[k]], num, den);
    if (w < 0) { free(order); free(S); return -2; }
    S[k + 1] = S[k] + w;
  }
  int64_t T = S[N];
  int64_t Q = 0;
  for (int32_t r = 0; r < W; ++r) Q += shares[r];
  int64_t Qr = 0;
  for (int32_t r = 0; r <= W; ++r) {
    int32_t c = 0;
    while (c < N && (__int128)Q * S[c] < (__int128)Qr * T) ++c; /* linear search: plain */
    rank_offsets[r] = c;
    if (r < W) Qr += shares[r];
  }
  rank_offsets[W] = N;
  for (int32_t k = 0; k < N; ++k) perm[k] = order[k];
  if (rank_weight)
    for (int32_t r = 0; r < W; ++r) rank_weight[r] = S[rank_offsets[r + 1]] - S[rank_offsets[r]];
  free(order);
  free(S);
  return 0;
}

/* cost[r] = sum over positions j in [rank_offsets[r], rank_offsets[r+1]) of */
/* c2 L^2 + c1 L + c0, L = len[perm[j]].                                     */
void or_rank_cost(const int32_t* len, const int32_t* perm, const int32_t* rank_offsets,
                  int32_t W, int64_t c2, int64_t c1, int64_t c0, int64_t* cost) {
  for (int32_t r = 0; r < W; ++r) {
    int64_t t = 0;
    for (int32_t j = rank_offsets[r]; j < rank_offsets[r + 1]; ++j) {
      int64_t L = len[perm[j]];
      t += c2 * L * L + c1 * L + c0;
    }
    cost[r] = t;
  }
}

/* One AutoTune step on shares[W] in place (readings above). */
void or_vbs_autotune(const int64_t* times, int32_t W, int32_t step_num, int32_t step_den,
                     int32_t tol_num, int32_t tol_den, int64_t* shares) {
  int64_t sum = 0;
  for (int32_t r = 0; r < W; ++r) sum += times[r];
  for (int32_t r = 0; r < W; ++r) {
    __int128 lhs = (__int128)W * times[r] * tol_den;
    int64_t d = shares[r] * step_num / step_den;
    if (d < 1) d = 1;
    if (lhs > (__int128)sum * (tol_den + tol_num)) {        /* slower than the mean */
      shares[r] -= d;
      if (shares[r] < 1) shares[r] = 1;
    } else if (lhs < (__int128)sum * (tol_den - tol_num)) { /* faster */
      shares[r] += d;
      if (shares[r] > OR_SHARE_MAX) shares[r] = OR_SHARE_MAX;
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Indexed permute and bucketize: [FS] 4.2 ("indexed permute" applies the    */
/* partition to the gathered IDs; "ranged dispatch" builds the per-destination */
/* ranges that the ID AllToAll sends) and 3.2 (batch-major vs shard-major).  */
/*                                                                          */
/* Readings:                                                                */
/*  - sample s has n_s = sample_offsets[s+1]-sample_offsets[s] tokens; the  */
/*    balanced batch lays samples out in perm order, so token j of the q-th */
/*    balanced sample has batch-major index bm = bal_offsets[q] + j.        */
/*  - table t is row-wise sharded into W contiguous blocks of               */
/*    ceil(R_t / W) rows: shard(t, id) = id / ceil(R_t / W).                */
/*  - shard-major order: destination shard, then source rank, then table,   */
/*    then balanced sample, then token -- what a W-way AllToAll of           */
/*    per-destination, table-major send buffers delivers.                    */
/*  - the key of (t, id) is row_base[t] + id; an ID outside [0, R_t) is      */
/*    dropped and flagged.                                                   */
/* splits[d*W + r] = items sent from rank r to shard d.                      */

int64_t or_bucketize(const int64_t* ids, int64_t n_tok, const int64_t* sample_offsets, int32_t N,
                     int32_t T, const int64_t* rows, const int64_t* row_base,
                     const int32_t* perm, const int32_t* rank_offsets, int32_t W,
                     int64_t* bal_offsets, int64_t* shard_keys, int32_t* shard_bm,
                     int64_t* splits, int64_t* shard_offsets, int32_t* err) {
  bal_offsets[0] = 0;
  for (int32_t q = 0; q < N; ++q) {
    int32_t s = perm[q];
    bal_offsets[q + 1] = bal_offsets[q] + (sample_offsets[s + 1] - sample_offsets[s]);
  }
  for (int64_t k = 0; k < (int64_t)W * W; ++k) splits[k] = 0;
  int64_t* count = (int64_t*)calloc((size_t)W, sizeof(int64_t));
  int64_t* fill = (int64_t*)calloc((size_t)W, sizeof(int64_t));
  /* two passes over the same enumeration: count, then append */
  for (int pass = 0; pass < 2; ++pass) {
    for (int32_t r = 0; r < W; ++r)
      for (int32_t t = 0; t < T; ++t) {
        int64_t block = (rows[t] + W - 1) / W;
        for (int32_t q = rank_offsets[r]; q < rank_offsets[r + 1]; ++q) {
          int32_t s = perm[q];
          int64_t ns = sample_offsets[s + 1] - sample_offsets[s];
          for (int64_t j = 0; j < ns; ++j) {
            int64_t id = ids[(int64_t)t * n_tok + sample_offsets[s] + j];
            if (id < 0 || id >= rows[t]) { if (pass == 0) *err |= OR_EF_ID_RANGE; continue; }
            int32_t d = (int32_t)(id / block);
            if (pass == 0) {
              count[d] += 1;
              splits[(int64_t)d * W + r] += 1;
            } else {
              int64_t pos = shard_offsets[d] + fill[d];
              shard_keys[pos] = row_base[t] + id;
              shard_bm[pos] = (int32_t)(bal_offsets[q] + j);
              fill[d] += 1;
            }
          }
        }
      }
    if (pass == 0) {
      shard_offsets[0] = 0;
      for (int32_t d = 0; d < W; ++d) shard_offsets[d + 1] = shard_offsets[d] + count[d];
    }
  }
  int64_t n_valid = shard_offsets[W];
  free(count);
  free(fill);
  return n_valid;
}

/* ------------------------------------------------------------------------ */
/* Ranged combine: [FS] 4.2 names the kernel that lays out the output of the  */
/* embedding AllToAll. Reading for one GPU that holds every virtual rank: row */
/* k of src belongs to item k of the shard-major order (what the shards send  */
/* back, block by block), and the combine puts it in the item's batch-major   */
/* slot of its own table: out_t[shard_bm[k]] = src_k, where t is the table    */
/* whose key range [row_base[t], row_base[t+1]) holds shard_keys[k]. Rows are */
/* opaque bytes (row_bytes[t] of them); slots no item maps to are untouched.  */
void or_ranged_combine(const uint8_t* src, int64_t src_stride, const int64_t* shard_keys,
                       const int32_t* shard_bm, int64_t n_valid, int32_t T,
                       const int64_t* row_base, const int64_t* row_bytes, uint8_t** out) {
  for (int64_t k = 0; k < n_valid; ++k) {
    int32_t t = 0;
    while (t + 1 < T && shard_keys[k] >= row_base[t + 1]) ++t;
    memcpy(out[t] + (int64_t)shard_bm[k] * row_bytes[t], src + k * src_stride,
           (size_t)row_bytes[t]);
  }
}

/* ------------------------------------------------------------------------ */
/* Keyed transpose: [FS] 4.2 names the kernel that turns a jagged tensor from */
/* the feature-major form to the batch-major form. Reading: F features, B    */
/* samples, lengths[f*B + b] values of feature f for sample b; the input     */
/* lists feature 0's values sample by sample, then feature 1's, and so on;   */
/* the output lists sample 0's values feature by feature, then sample 1's.   */
/* out_offsets[b*F + f] = where (b, f) starts in the output; its last entry  */
/* is the total.                                                            */
void or_keyed_transpose(const int64_t* values, const int32_t* lengths, int32_t F, int32_t B,
                        int64_t* out_values, int64_t* out_offsets) {
  int64_t* in_off = (int64_t*)malloc(sizeof(int64_t) * ((size_t)F * B + 1));
  int64_t x = 0;
  for (int64_t e = 0; e < (int64_t)F * B; ++e) {  /* feature-major starts */
    in_off[e] = x;
    x += lengths[e];
  }
  x = 0;
  for (int32_t b = 0; b < B; ++b)  /* batch-major starts */
    for (int32_t f = 0; f < F; ++f) {
      out_offsets[(int64_t)b * F + f] = x;
      x += lengths[(int64_t)f * B + b];
    }
  out_offsets[(int64_t)F * B] = x;
  for (int32_t b = 0; b < B; ++b)
    for (int32_t f = 0; f < F; ++f) {
      int64_t n = lengths[(int64_t)f * B + b];
      for (int64_t j = 0; j < n; ++j)
        out_values[out_offsets[(int64_t)b * F + f] + j] = values[in_off[(int64_t)f * B + b] + j];
    }
  free(in_off);
}

/* ------------------------------------------------------------------------ */
/* Dedup: [FS] 3.2 / Algorithm 2 compute the collision sets on shard-major   */
/* unique rows. Reading of the layout: unique rows ascending by key         */
/* (= by table, then row); since shards are contiguous row blocks of a      */
/* table, the rows of (table t, shard d) form one contiguous range,         */
/* unique_offsets[t*W + d] .. unique_offsets[t*W + d + 1]. Every unique row */
/* lists its occurrences (CSR) by ascending batch-major index.              */

typedef struct { int64_t key; int64_t bm; } or_item;

static int or_cmp_item(const void* a, const void* b) {
  const or_item* x = (const or_item*)a;
  const or_item* y = (const or_item*)b;
  if (x->key != y->key) return x->key < y->key ? -1 : 1;
  if (x->bm != y->bm) return x->bm < y->bm ? -1 : 1;
  return 0;
}

/* Returns U. occ_uid[o] = the unique index of occurrence o (CSR order). */
int64_t or_unique(const int64_t* shard_keys, const int32_t* shard_bm, int64_t n,
                  int32_t T, const int64_t* rows, const int64_t* row_base, int32_t W,
                  int64_t* unique, int64_t* unique_offsets, int32_t* seg_offsets,
                  int32_t* occ_bm, int32_t* occ_uid) {
  or_item* v = (or_item*)malloc(sizeof(or_item) * (size_t)(n > 0 ? n : 1));
  for (int64_t i = 0; i < n; ++i) { v[i].key = shard_keys[i]; v[i].bm = shard_bm[i]; }
  qsort(v, (size_t)n, sizeof(or_item), or_cmp_item);
  int64_t U = 0;
  for (int64_t i = 0; i < n; ++i) {
    if (i == 0 || v[i].key != v[i - 1].key) {
      unique[U] = v[i].key;
      seg_offsets[U] = (int32_t)i;
      ++U;
    }
    occ_bm[i] = (int32_t)v[i].bm;
    occ_uid[i] = (int32_t)(U - 1);
  }
  seg_offsets[U] = (int32_t)n;
  /* (table, shard) group starts: first unique key >= the group's first row
   * (a shard past the end of a small table starts at the table's end). The
   * group starts ascend, so one forward sweep finds them all. */
  int64_t u = 0;
  for (int32_t t = 0; t < T; ++t) {
    int64_t block = (rows[t] + W - 1) / W;
    for (int32_t d = 0; d < W; ++d) {
      int64_t first = (int64_t)d * block;
      int64_t lo_key = row_base[t] + (first < rows[t] ? first : rows[t]);
      while (u < U && unique[u] < lo_key) ++u;
      unique_offsets[(int64_t)t * W + d] = u;
    }
  }
  unique_offsets[(int64_t)T * W] = U;
  free(v);
  return U;
}

/* ------------------------------------------------------------------------ */
/* Collision split: [FS] 2.3 and 3.2, Algorithm 2 (compute_collision). A     */
/* collision row of iteration i+1 is one that iteration i also updates;     */
/* every other row is exclusive. cls[u] = [unique[u] in prev_unique];       */
/* prev_cls[v] = [prev_unique[v] in unique]. counts = (U, C, U-C, Up-C).    */
/* Plain membership by binary search over the sorted other set.             */

static int or_contains(const int64_t* a, int64_t n, int64_t key) {
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    int64_t mid = lo + (hi - lo) / 2;
    if (a[mid] < key) lo = mid + 1; else hi = mid;
  }
  return lo < n && a[lo] == key;
}

void or_collision(const int64_t* unique, int64_t U, const int64_t* prev_unique, int64_t Up,
                  uint8_t* cls, uint8_t* prev_cls, int64_t* counts) {
  int64_t C = 0;
  for (int64_t u = 0; u < U; ++u) {
    cls[u] = (uint8_t)or_contains(prev_unique, Up, unique[u]);
    C += cls[u];
  }
  for (int64_t v = 0; v < Up; ++v) prev_cls[v] = (uint8_t)or_contains(unique, U, prev_unique[v]);
  counts[0] = U;
  counts[1] = C;
  counts[2] = U - C;
  counts[3] = Up - C;
}

/* ------------------------------------------------------------------------ */
/* Row store: the rows of one table that a run touches, keyed by table-local */
/* row id (ascending), values in the table dtype (fp32, or bf16 as uint16), */
/* and one fp32 row-wise Adagrad accumulator per row.                       */

typedef struct {
  const int64_t* row_ids; /* ascending */
  int64_t n_rows;
  void* vals;             /* [n_rows][dim] */
  float* state;           /* [n_rows] or NULL */
  int32_t dim;
  int32_t bf16;
} or_store;

static int64_t or_store_find(const or_store* s, int64_t row) {
  int64_t lo = 0, hi = s->n_rows;
  while (lo < hi) {
    int64_t mid = lo + (hi - lo) / 2;
    if (s->row_ids[mid] < row) lo = mid + 1; else hi = mid;
  }
  return (lo < s->n_rows && s->row_ids[lo] == row) ? lo : -1;
}

/* bf16 <-> fp32. Widening is exact; narrowing is round-to-nearest-even of
 * the top 16 bits, with NaN kept quiet. */
float or_bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

uint16_t or_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------------ */
/* Lookup: Algorithm 2's Lookup and merge -- every occurrence of a unique    */
/* row gets a bit copy of the row as it stands after all earlier updates,   */
/* written at its batch-major slot: out[bm] of table t is [n_tok][dim].     */
/* which: -1 = all rows, 0 = exclusive only, 1 = collision only.           */
/* Returns the number of rows missing from the store (expected 0).          */

int64_t or_lookup(const or_store* st, int64_t row_base, int64_t u_lo, int64_t u_hi,
                  const int64_t* unique, const int32_t* seg_offsets, const int32_t* occ_bm,
                  const uint8_t* cls, int32_t which, void* out) {
  int64_t missing = 0;
  size_t esz = st->bf16 ? 2 : 4;
  size_t rb = esz * (size_t)st->dim;
  for (int64_t u = u_lo; u < u_hi; ++u) {
    if (which >= 0 && cls[u] != (uint8_t)which) continue;
    int64_t idx = or_store_find(st, unique[u] - row_base);
    if (idx < 0) { ++missing; continue; }
    for (int32_t o = seg_offsets[u]; o < seg_offsets[u + 1]; ++o)
      memcpy((char*)out + rb * (size_t)occ_bm[o], (const char*)st->vals + rb * (size_t)idx, rb);
  }
  return missing;
}

/* ------------------------------------------------------------------------ */
/* Gradient reduce: Algorithm 2's backward sends each occurrence's gradient  */
/* to the row's shard, where update_embedding combines them. The combined   */
/* gradient of row u is the sum over its occurrences (ascending bm) of the  */
/* batch-major gradient rows, accumulated in fp64 and rounded once to fp32.  */
/* grad is [n_tok][dim] fp32; g is [u_hi-u_lo][dim].                        */

void or_reduce(int32_t dim, int64_t u_lo, int64_t u_hi, const int32_t* seg_offsets,
               const int32_t* occ_bm, const float* grad, float* g) {
  double* acc = (double*)malloc(sizeof(double) * (size_t)dim);
  for (int64_t u = u_lo; u < u_hi; ++u) {
    for (int32_t d = 0; d < dim; ++d) acc[d] = 0.0;
    for (int32_t o = seg_offsets[u]; o < seg_offsets[u + 1]; ++o)
      for (int32_t d = 0; d < dim; ++d) acc[d] += (double)grad[(size_t)occ_bm[o] * dim + d];
    for (int32_t d = 0; d < dim; ++d) g[(size_t)(u - u_lo) * dim + d] = (float)acc[d];
  }
  free(acc);
}

/* ------------------------------------------------------------------------ */
/* Row update (the optimizer is not named on the pages; the workloads name   */
/* SGD and row-wise Adagrad). fp32 arithmetic, one rounding per operation:  */
/*   SGD:     w_d <- w_d - lr * g_d                                          */
/*   RW-Ada:  s <- s + mean_d(g_d^2);  m = lr / (sqrt(s) + eps);            */
/*            w_d <- w_d - m * g_d                                           */
/* mean_d(g_d^2) is summed in fp64 over d ascending, divided by dim in fp64 */
/* and rounded once to fp32. bf16 rows are widened exactly and stored with  */
/* round-to-nearest-even. optim: 0 = SGD, 1 = row-wise Adagrad.             */
/* Returns the number of rows missing from the store (expected 0).          */

int64_t or_update(or_store* st, int64_t row_base, int64_t u_lo, int64_t u_hi,
                  const int64_t* unique, const uint8_t* cls, int32_t which,
                  const float* g, int32_t optim, float lr, float eps) {
  int64_t missing = 0;
  int32_t D = st->dim;
  for (int64_t u = u_lo; u < u_hi; ++u) {
    if (which >= 0 && cls[u] != (uint8_t)which) continue;
    int64_t idx = or_store_find(st, unique[u] - row_base);
    if (idx < 0) { ++missing; continue; }
    const float* gu = g + (size_t)(u - u_lo) * D;
    float m = lr;
    if (optim == 1) {
      double ss = 0.0;
      for (int32_t d = 0; d < D; ++d) ss += (double)gu[d] * (double)gu[d];
      float mean_sq = (float)(ss / (double)D);
      float s = st->state[idx] + mean_sq;
      st->state[idx] = s;
      float denom = sqrtf(s) + eps;
      m = lr / denom;
    }
    for (int32_t d = 0; d < D; ++d) {
      float w, step = m * gu[d];
      if (st->bf16) {
        uint16_t* p = (uint16_t*)st->vals + (size_t)idx * D + d;
        w = or_bf16_to_f32(*p);
        *p = or_f32_to_bf16(w - step);
      } else {
        float* p = (float*)st->vals + (size_t)idx * D + d;
        w = *p;
        *p = w - step;
      }
    }
  }
  return missing;
}
