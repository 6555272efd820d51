/*
 * mog.h -- C ABI of libmog, Mixture-of-Gaussians (Iceberg) decode attention
 * for AMD Instinct MI355X (gfx950).
 *
 * The method is the one of "Iceberg Attention: Sublinear Long-Context
 * Decoding with Mixture-of-Gaussians" (abstract): after prefill the keys of
 * every attention head are partitioned into about sqrt(N) clusters, each
 * split into about log2(N) subclusters, and every group is summarised by a
 * Gaussian; at each decode step the query is scored against the summaries,
 * the best clusters and subclusters are attended exactly and the rest of the
 * cache is estimated from the groups' means and variances.  Following the
 * retrieval-completion attention page (abstract), sink and tail anchor
 * tokens are always attended exactly, and the exact and estimated parts are
 * added as unnormalised numerator and denominator before one normalisation.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer marked DEVICE is caller-owned device memory; the library
 *    never allocates, frees or synchronises.  HOST pointers are read during
 *    the call only.
 *  - All GPU work is enqueued on the caller's stream; the call returns as
 *    soon as it is enqueued.  A fault inside a kernel shows up at the
 *    caller's next synchronisation, not as a return code.
 *  - Arguments are validated before anything is enqueued; a call that
 *    returns an error has enqueued nothing.  mog_last_error() then returns a
 *    description (per thread).
 *  - Layouts: keys/values are row-major with head_dim contiguous elements per
 *    token.  Queries and outputs are float32 [n_seq][n_q_heads][head_dim];
 *    query head h reads KV head h / (n_q_heads / n_kv_heads).
 *  - NaN or Inf in inputs propagate; they are not checked.
 *
 * Limits: head_dim 64 or 128; 1 <= n_q_heads / n_kv_heads <= 8;
 * n_seq <= MOG_MAX_SEQ; per-sequence length N with n_sink + n_recent < N and
 * N <= MOG_MAX_LEN; keys within |k| < 65536 (the build sums them in 64-bit
 * fixed point); at most MOG_MAX_FOLD tokens folded per unit between builds.
 */
#ifndef MOG_H
#define MOG_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOG_MAX_SEQ 256
#define MOG_MAX_LEN (1 << 22)
#define MOG_MAX_FOLD (1 << 15)

typedef enum {
  MOG_OK = 0,
  MOG_ERR_INVALID_ARG = 1, /* null pointer, bad size, inconsistent shapes   */
  MOG_ERR_UNSUPPORTED = 2, /* a valid request the library does not cover  */
  MOG_ERR_WORKSPACE = 3,   /* workspace or layout buffer too small          */
  MOG_ERR_HIP = 4,         /* a HIP launch or runtime call failed           */
  MOG_ERR_CAPACITY = 5,    /* a layout's fold area is full: build again     */
  /* Not statuses: these two give the type the range of int32_t, so any int
   * a C caller passes (e.g. to mog_status_string) is a valid value of it. */
  MOG_STATUS_RANGE_MIN_ = -0x7fffffff - 1,
  MOG_STATUS_RANGE_MAX_ = 0x7fffffff
} mog_status;

typedef enum { MOG_F32 = 0, MOG_BF16 = 1 } mog_dtype;

typedef enum { MOG_KV_CONTIGUOUS = 0, MOG_KV_PAGED = 1 } mog_kv_format;

/* The KV cache of a batch of sequences.
 *
 * CONTIGUOUS: k and v are DEVICE arrays [n_seq][n_kv_heads][max_len][head_dim]
 *   of `dtype`; sequence s uses its first seq_lens[s] rows.
 * PAGED: k and v are DEVICE page pools [n_pages][n_kv_heads][page_size][head_dim];
 *   block_table is a DEVICE int32 array [n_seq][max_blocks]; token t of
 *   sequence s lives in page block_table[s][t / page_size], slot
 *   t % page_size.  The table must hold valid page ids for every used block.
 * seq_lens is a HOST int32 array [n_seq]. */
typedef struct {
  int32_t format;     /* mog_kv_format */
  int32_t dtype;      /* mog_dtype     */
  int32_t n_seq;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t max_len;    /* CONTIGUOUS: rows per (seq, head); PAGED: unused   */
  int32_t page_size;  /* PAGED only (any power of two, 1..256)             */
  int32_t n_pages;    /* PAGED only: pages in the pool                     */
  int32_t max_blocks; /* PAGED only: columns of block_table                */
  const int32_t* seq_lens;    /* HOST   [n_seq]                  */
  const void* k;              /* DEVICE                          */
  const void* v;              /* DEVICE                          */
  const int32_t* block_table; /* DEVICE [n_seq][max_blocks], PAGED only */
} mog_kv;

/* Shape of a layout (what mog_layout_size needs). */
typedef struct {
  int32_t n_seq;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t dtype;            /* dtype of the reordered K/V copy (= the cache's) */
  int32_t n_sink;           /* anchors at the start of every sequence */
  int32_t n_recent;         /* anchors at the end of every sequence   */
  int32_t fold_capacity;    /* rows per unit kept for mog_append, 0..MOG_MAX_FOLD */
  int32_t fm_dim;           /* features per group summary: 0 (none), 64, 128, 256 */
  int32_t rows_external;    /* 1: k_mid / v_mid are caller arrays outside the
                               layout buffer (mog_layout_rows gives their
                               size), e.g. pinned host memory the GPU reads
                               over the host link; 0: carved from the buffer */
  const int32_t* seq_lens;  /* HOST [n_seq] lengths at the build */
} mog_dims;

/* Per-unit geometry, one unit = one (sequence, KV head); unit id
 * u = seq * n_kv_heads + kv_head.  With N_b the length at the build:
 * C = min(ceil(sqrt(N_b)), n_mid) clusters, S = ceil(log2(N_b)) subclusters
 * per cluster, n_mid = N_b - n_sink - n_recent middle-region tokens (the
 * clustered part).  N is the current length, N_b + n_fold: mog_append
 * folds the tokens that leave the recent window into the partition. */
typedef struct {
  int32_t seq, kv_head;
  int32_t N, n_mid;
  int32_t C, S;
  int32_t n_fold;   /* tokens folded since the build (rows in the fold area)  */
  int32_t reserved1;
  int64_t row_base; /* first row of this unit in k_mid / v_mid / perm        */
  int64_t cl_base;  /* first cluster of this unit in cl_ms / cl_vbar         */
  int64_t sub_base; /* first subcluster of this unit in sub_ms / sub_vbar    */
  int64_t off_base; /* first entry of this unit's C*S+1 offsets in sub_off   */
} mog_unit;

/* A built (or imported) cluster layout.  Plain descriptor: every pointer
 * points into the caller's layout buffer.
 *  k_mid, v_mid  [total_mid + n_units * fold_capacity][head_dim] dtype: the
 *                middle region of every unit, rows ordered by (cluster,
 *                subcluster, token position); then the fold area: row
 *                total_mid + u * fold_capacity + f holds the f-th token
 *                folded into unit u.
 *  perm          [total_mid] int32: token position of every reordered row.
 *  sub_off       per unit C*S+1 int32 row offsets relative to row_base;
 *                subcluster i of cluster j owns rows [sub_off[j*S+i],
 *                sub_off[j*S+i+1]); cluster j owns [sub_off[j*S], sub_off[(j+1)*S]).
 *  cl_ms, sub_ms [groups][2*head_dim] float32: mean key (first head_dim
 *                entries) then diagonal population variance of the keys.
 *  cl_vbar, sub_vbar [groups][head_dim] float32: mean value.
 *                Group statistics cover the folded tokens too.
 *  cl_ms16, cl_vbar16, sub_ms16, sub_vbar16  the same four arrays in bf16
 *                (bits as uint16, rounded to nearest, ties to even): the
 *                statistics the decode reads.  mog_build and mog_append
 *                keep them in step with the float32 arrays; a caller that
 *                writes the float32 arrays itself calls
 *                mog_layout_sync_stats before decoding.
 *  fold_sub      [n_units][fold_capacity] int32: subcluster (j*S+i, within
 *                the unit) of every folded token, in fold order.
 *  fold_pos      [n_units][fold_capacity] int32: its token position.
 *  cl_fold, sub_fold [groups] int32: folded tokens per cluster / subcluster
 *                (a group holds its sub_off rows plus these).
 *  fm_w          [fm_dim][head_dim] float32: the feature map's projection
 *                (a copy of the build's), fm_scale its logit scale.
 *  cl_fz, sub_fz [groups][fm_dim] float32: per group the sum over its
 *                members of phi(sqrt(fm_scale) k), phi(x) = exp(W x -
 *                |x|^2 / 2) / sqrt(fm_dim) (NULL when fm_dim is 0).
 *  units         DEVICE copy of the mog_unit table (n_units entries).
 *  append_scratch  library-internal working memory of mog_append.
 *  seq_lens      current lengths; fold_count[s] of them were folded, so
 *                seq_lens[s] - fold_count[s] is the length at the build. */
typedef struct {
  int32_t n_seq, n_kv_heads, head_dim, dtype, n_sink, n_recent;
  int32_t n_units;
  int32_t max_C, max_S;
  int32_t fold_capacity;
  int32_t fm_dim;
  float fm_scale;
  int32_t seq_lens[MOG_MAX_SEQ];
  int32_t fold_count[MOG_MAX_SEQ];
  int64_t total_mid, total_cl, total_sub, total_off;
  mog_unit* units;
  void* k_mid;
  void* v_mid;
  int32_t* perm;
  int32_t* sub_off;
  float* cl_ms;
  float* cl_vbar;
  float* sub_ms;
  float* sub_vbar;
  uint16_t* cl_ms16;
  uint16_t* cl_vbar16;
  uint16_t* sub_ms16;
  uint16_t* sub_vbar16;
  int32_t* fold_sub;
  int32_t* fold_pos;
  int32_t* cl_fold;
  int32_t* sub_fold;
  void* append_scratch;
  float* fm_w;
  float* cl_fz;
  float* sub_fz;
  int32_t rows_external;  /* k_mid / v_mid live outside the layout buffer */
} mog_layout;

typedef struct {
  int32_t kmeans_iters; /* Lloyd rounds before the final assignment (10)   */
  int32_t n_sink;
  int32_t n_recent;
  int32_t fold_capacity; /* rows per unit kept for mog_append (0: none)    */
  uint64_t seed;        /* seeds the Forgy initialisation of every unit    */
  int32_t fm_dim;       /* feature-map summaries: 0 (none), 64, 128, 256   */
  float fm_scale;       /* their logit scale; 0 selects 1/sqrt(head_dim)   */
  const float* fm_w;    /* DEVICE [fm_dim][head_dim] float32, rows drawn from
                           N(0, I) by the caller; read during the build    */
  void* rows_k;         /* NULL, or caller arrays of mog_layout_rows rows of */
  void* rows_v;         /* head_dim elements each, 16-byte aligned, that the
                           GPU can address (device memory, or pinned host
                           memory: the KV-offload setting of the retrieval-
                           completion page's abstract, where only the rows a
                           step selects cross the host link); they then hold
                           k_mid / v_mid instead of the layout buffer      */
} mog_build_params;

typedef struct {
  int32_t n_q_heads;            /* Hq; Hq / n_kv_heads query heads per KV head */
  int32_t top_c;                /* clusters attended exactly per query head     */
  int32_t top_s;                /* subclusters per chosen cluster               */
  int32_t residual;             /* 1: add the Gaussian estimate of the rest;
                                   2: add the feature-map estimate of the rest
                                   (retrieval-completion page, abstract: each
                                   left-out group's mass is phi(sqrt(s) q).Z_g
                                   from the layout's summaries, its value the
                                   mean value; needs fm_dim > 0 and the scale
                                   the summaries were built with);
                                   0: exact part only, renormalised            */
  float scale;                  /* logit scale; 0 selects 1/sqrt(head_dim)      */
  int32_t splits;               /* 0: automatic; else 1..8192.  mog_decode: the
                                   exact-attention blocks shared by all units in
                                   proportion to the rows each reads (plus one
                                   per unit); mog_dense_decode: blocks per unit */
  int32_t shared_selection;     /* 0: every query head selects its own clusters
                                   and subclusters; 1: one selection per KV
                                   head, by the sum over its query heads of
                                   each head's estimated mass fraction
                                   exp(score - LSE_head) (DuoAttention review,
                                   page 2, Limitations: heads sharing a KV head
                                   couple their needs); the exact read per KV
                                   head is then capped at one head's budget   */
  const int32_t* top_c_per_seq; /* HOST [n_seq] or NULL (then top_c)           */
  const int32_t* top_s_per_seq; /* HOST [n_seq] or NULL (then top_s)           */
  hipEvent_t exact_begin;       /* optional (NULL: unused): set by the dispatch */
  hipEvent_t exact_end;         /* of the exact-attention kernel itself to its  */
                                /* start / end time (hipExtLaunchKernel), for  */
                                /* timing that kernel alone                    */
  int32_t exact_repeat;         /* timing aid: 0 or 1 launches the exact-      */
                                /* attention kernel once; n in 2..64 launches  */
                                /* it n times back to back (each launch redoes */
                                /* the same work, results are unchanged), the  */
                                /* events then spanning the first start to the */
                                /* last end                                    */
} mog_decode_params;

typedef enum {
  MOG_OP_BUILD = 0,
  MOG_OP_DECODE = 1,
  MOG_OP_DENSE = 2,
  /* not operations: the range of int32_t, as for mog_status */
  MOG_OP_RANGE_MIN_ = -0x7fffffff - 1,
  MOG_OP_RANGE_MAX_ = 0x7fffffff
} mog_op;

/* ---------------------------------------------------------------------- */

/* Bytes of the layout buffer for `dims`.  Pure host computation. */
mog_status mog_layout_size(const mog_dims* dims, size_t* bytes);

/* Rows of k_mid (and of v_mid) for `dims`: the middle regions of every unit
 * plus their fold areas, sum over units of (N - n_sink - n_recent) +
 * n_units * fold_capacity.  An external row array holds rows * head_dim
 * elements of the dtype.  Pure host computation. */
mog_status mog_layout_rows(const mog_dims* dims, int64_t* rows);

/* Carve `layout_mem` (DEVICE, >= mog_layout_size bytes, 256-byte aligned)
 * into a layout for `dims`, fill `out` (host) and enqueue the write of the
 * device unit table and the zeroing of the fold counts.  mog_build calls
 * this itself; it is exported so a caller can import a layout computed
 * elsewhere by writing the arrays (cl_fold / sub_fold must stay zero).
 * With dims->rows_external the caller also sets out->k_mid / out->v_mid. */
mog_status mog_layout_init(const mog_dims* dims, void* layout_mem, size_t layout_bytes,
                           mog_layout* out, hipStream_t stream);

/* Enqueue the rewrite of a layout's bf16 statistics (cl_ms16, cl_vbar16,
 * sub_ms16, sub_vbar16) from its float32 ones, every group of every unit,
 * for a caller that wrote cl_ms, cl_vbar, sub_ms or sub_vbar itself (an
 * imported layout).  The decode reads group statistics in bf16 (the storage
 * precision of the group means and variances is left open by the Iceberg
 * and MoG write-ups; bf16 halves the bytes the latency-bound kernels move).
 * Allocates nothing.  Errors: MOG_ERR_INVALID_ARG for a NULL or incomplete
 * layout, MOG_ERR_HIP if the launch fails. */
mog_status mog_layout_sync_stats(const mog_layout* layout, hipStream_t stream);

/* Host copy of the geometry of unit `unit` of a layout. */
mog_status mog_layout_unit(const mog_layout* layout, int32_t unit, mog_unit* out);

/* Workspace bytes for an operation.
 *  MOG_OP_BUILD : `kv` and `bp` used (layout geometry follows from them).
 *  MOG_OP_DECODE: `layout` and `dp` used.
 *  MOG_OP_DENSE : `kv` and `dp` used (n_q_heads, splits).
 * Unused arguments may be NULL. */
mog_status mog_workspace_size(mog_op op, const mog_kv* kv, const mog_layout* layout,
                              const mog_build_params* bp, const mog_decode_params* dp,
                              size_t* bytes);

/* Prefill-side build (Iceberg Attention abstract: hierarchical partition of
 * each head's keys, one Gaussian per group): for every unit, seeded Forgy
 * k-means of the middle-region keys into C clusters (kmeans_iters rounds,
 * then a final assignment), k-means of every cluster into min(S, n)
 * subclusters, reordering of K/V into cluster-contiguous rows, and the
 * per-group statistics.  Fills `out`.  `ws`: DEVICE scratch of
 * mog_workspace_size(MOG_OP_BUILD) bytes. */
mog_status mog_build(const mog_kv* kv, const mog_build_params* params, void* layout_mem,
                     size_t layout_bytes, void* ws, size_t ws_bytes, mog_layout* out,
                     hipStream_t stream);

/* One decode step (Iceberg Attention abstract; merge rule of the
 * retrieval-completion page's abstract).  Per query head: score every
 * cluster by ln n + scale q.mu + scale^2/2 sum q_i^2 var_i, take the top_c
 * clusters, score their subclusters the same way, take top_s in each;
 * attend exactly over the anchors (read from `kv`) and the chosen
 * subclusters' rows (read from the layout); add exp(score) and
 * exp(score) * vbar of every group left out; normalise once.
 *  q    DEVICE float32 [n_seq][n_q_heads][head_dim]
 *  out  DEVICE float32 [n_seq][n_q_heads][head_dim]
 *  lse  DEVICE float32 [n_seq][n_q_heads] natural-log normaliser, or NULL
 *  sel_c DEVICE int32 [n_seq][n_q_heads][cmax] chosen cluster ids, ascending,
 *        padded with -1 (cmax = max over sequences of top_c), or NULL
 *  sel_s DEVICE int32 [n_seq][n_q_heads][cmax][smax] chosen subcluster ids
 *        (0..S-1) of the k-th chosen cluster, ascending, padded with -1
 *        (smax = max top_s), or NULL.  Selection outputs are left
 *        untouched when the corresponding maximum budget is 0.
 *  ws   DEVICE scratch of mog_workspace_size(MOG_OP_DECODE) bytes.  Its first
 *        256 bytes must be zero before the first call; the library leaves
 *        them zero.
 * Calls that share a workspace must not overlap. */
mog_status mog_decode(const mog_layout* layout, const mog_kv* kv, const float* q,
                      const mog_decode_params* params, float* out, float* lse,
                      int32_t* sel_c, int32_t* sel_s, void* ws, size_t ws_bytes,
                      hipStream_t stream);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * decode step as mog_decode (same arguments, kernels and results) with the
 * workspace taken from the library's own static device scratch of
 * MOG_DECODE_NOALLOC_MAX_WS bytes instead of a caller buffer.  Allocates
 * nothing, on the host or the device.
 *  - The scratch is one file-scope device array: every GPU the library runs
 *    on holds its own copy of MOG_DECODE_NOALLOC_MAX_WS bytes until the
 *    process ends.  Its address on a device is looked up on the first call
 *    made with that device current, and kept.
 *  - Every call on a GPU uses that GPU's one scratch, which keeps the last
 *    call's contents: calls that overlap on one GPU (other streams, other
 *    threads) race and must not be issued.  No part of it has to start at
 *    zero: each call writes every entry before reading it.
 *  - MOG_ERR_WORKSPACE (nothing enqueued) when the step needs more than
 *    MOG_DECODE_NOALLOC_MAX_WS bytes (mog_workspace_size(MOG_OP_DECODE)
 *    tells how many it needs); mog_decode with a caller workspace then
 *    serves it. */
#define MOG_DECODE_NOALLOC_MAX_WS ((size_t)64 << 20)
mog_status mog_decode_noalloc(const mog_layout* layout, const mog_kv* kv, const float* q,
                              const mog_decode_params* params, float* out, float* lse,
                              int32_t* sel_c, int32_t* sel_s, hipStream_t stream);

/* Incremental decode (Iceberg Attention abstract: the partition is built
 * once after prefill and then serves every decode step).  The sequences of
 * `kv` are the layout's sequences grown by a_s = kv->seq_lens[s] -
 * layout->seq_lens[s] >= 0 tokens.  The a_s tokens that leave the recent
 * window, positions [N_s - n_recent, N_s - n_recent + a_s) with N_s =
 * layout->seq_lens[s], are folded into the partition one by one, oldest
 * first: each joins the nonempty cluster whose mean key is nearest (squared
 * distance in float64, ties to the lower id), then the nearest nonempty
 * subcluster of that cluster; both groups' count, mean key, population
 * variance and mean value are updated by Welford's running formulas
 * (float64 from the stored float32, stored float32), and the token's K/V
 * rows are copied into the unit's fold area, from which mog_decode reads
 * them whenever their subcluster is chosen.  C, S and the rest of the
 * partition are kept.  Updates layout->seq_lens and layout->fold_count
 * (HOST) and enqueues the device updates on `stream`; no workspace.
 * MOG_ERR_CAPACITY (nothing enqueued, layout unchanged) when a sequence's
 * folded tokens would exceed layout->fold_capacity: build again.  Calls on
 * one layout must not overlap with each other or with mog_decode. */
mog_status mog_append(const mog_kv* kv, mog_layout* layout, hipStream_t stream);

/* Exact dense decode attention over all tokens of every sequence (the
 * in-library baseline): out = softmax(scale K q)^T V.  Same q/out/lse/ws
 * conventions as mog_decode; only n_q_heads, scale and splits of `params`
 * are used. */
mog_status mog_dense_decode(const mog_kv* kv, const float* q, const mog_decode_params* params,
                            float* out, float* lse, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/* Static text of a status code. */
const char* mog_status_string(mog_status status);

/* Description of the last error raised on the calling thread ("" if none). */
const char* mog_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOG_H */
