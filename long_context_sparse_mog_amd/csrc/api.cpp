// Host side of the libmog C ABI: argument validation, sizes, layout carving
// and kernel launch.  Nothing here allocates device memory, copies between
// host and device, or synchronises.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "mog_internal.h"

using namespace mog;

namespace {

thread_local std::string g_last_error;

mog_status fail(mog_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
mog_status fail(mog_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

mog_status ok() {
  g_last_error.clear();
  return MOG_OK;
}

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int esize(int dtype) { return dtype == MOG_BF16 ? 2 : 4; }

// ------------------------------------------------------------------------
// Layout geometry
// ------------------------------------------------------------------------
struct Totals {
  int64_t mid = 0, cl = 0, sub = 0, off = 0;
  int max_C = 0, max_S = 0;
};

struct LayoutPlan {
  Totals t;
  size_t o_units, o_kmid, o_vmid, o_perm, o_suboff, o_clms, o_clvb, o_subms, o_subvb;
  size_t o_clms16, o_clvb16, o_subms16, o_subvb16;
  size_t o_foldsub, o_foldpos, o_clfold, o_subfold, o_appws, o_fmw, o_clfz, o_subfz, bytes;
};

mog_status check_dims(const mog_dims* d) {
  if (!d) return fail(MOG_ERR_INVALID_ARG, "dims is NULL");
  if (d->n_seq < 1 || d->n_seq > MOG_MAX_SEQ)
    return fail(MOG_ERR_INVALID_ARG, "n_seq=%d outside [1, %d]", d->n_seq, MOG_MAX_SEQ);
  if (d->n_kv_heads < 1) return fail(MOG_ERR_INVALID_ARG, "n_kv_heads=%d < 1", d->n_kv_heads);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(MOG_ERR_UNSUPPORTED, "head_dim=%d (supported: 64, 128)", d->head_dim);
  if (d->dtype != MOG_F32 && d->dtype != MOG_BF16) return fail(MOG_ERR_UNSUPPORTED, "dtype=%d", d->dtype);
  if (d->n_sink < 0 || d->n_recent < 0)
    return fail(MOG_ERR_INVALID_ARG, "negative anchor count (n_sink=%d, n_recent=%d)", d->n_sink, d->n_recent);
  if (d->fold_capacity < 0 || d->fold_capacity > MOG_MAX_FOLD)
    return fail(MOG_ERR_INVALID_ARG, "fold_capacity=%d outside [0, %d]", d->fold_capacity, MOG_MAX_FOLD);
  if (d->fm_dim != 0 && d->fm_dim != 64 && d->fm_dim != 128 && d->fm_dim != 256)
    return fail(MOG_ERR_UNSUPPORTED, "fm_dim=%d (supported: 0, 64, 128, 256)", d->fm_dim);
  if (d->rows_external != 0 && d->rows_external != 1)
    return fail(MOG_ERR_INVALID_ARG, "rows_external=%d (0 or 1)", d->rows_external);
  if (!d->seq_lens) return fail(MOG_ERR_INVALID_ARG, "seq_lens is NULL");
  for (int s = 0; s < d->n_seq; ++s) {
    const int N = d->seq_lens[s];
    if (N > MOG_MAX_LEN) return fail(MOG_ERR_UNSUPPORTED, "seq_lens[%d]=%d > %d", s, N, MOG_MAX_LEN);
    if ((int64_t)N - d->n_sink - d->n_recent < 1)
      return fail(MOG_ERR_INVALID_ARG, "seq_lens[%d]=%d leaves no middle region after %d+%d anchors", s, N,
                  d->n_sink, d->n_recent);
  }
  return MOG_OK;
}

LayoutPlan plan_layout(const mog_dims* d) {
  LayoutPlan p;
  for (int s = 0; s < d->n_seq; ++s) {
    const UnitSizes z = unit_sizes(d->seq_lens[s], d->n_sink, d->n_recent);
    p.t.mid += (int64_t)d->n_kv_heads * z.n_mid;
    p.t.cl += (int64_t)d->n_kv_heads * z.C;
    p.t.sub += (int64_t)d->n_kv_heads * z.C * z.S;
    p.t.off += (int64_t)d->n_kv_heads * (z.C * z.S + 1);
    p.t.max_C = std::max(p.t.max_C, z.C);
    p.t.max_S = std::max(p.t.max_S, z.S);
  }
  const int64_t nu = (int64_t)d->n_seq * d->n_kv_heads;
  const int D = d->head_dim;
  // K/V rows: the reordered middle regions, then each unit's fold area
  // (none in the buffer when the caller keeps them elsewhere)
  const size_t rows = d->rows_external ? 0 : (size_t)p.t.mid + (size_t)nu * d->fold_capacity;
  size_t o = 0;
  p.o_units = o; o = align_up(o + nu * sizeof(mog_unit));
  p.o_kmid = o; o = align_up(o + rows * D * esize(d->dtype));
  p.o_vmid = o; o = align_up(o + rows * D * esize(d->dtype));
  p.o_perm = o; o = align_up(o + (size_t)p.t.mid * 4);
  p.o_suboff = o; o = align_up(o + (size_t)p.t.off * 4);
  p.o_clms = o; o = align_up(o + (size_t)p.t.cl * 2 * D * 4);
  p.o_clvb = o; o = align_up(o + (size_t)p.t.cl * D * 4);
  p.o_subms = o; o = align_up(o + (size_t)p.t.sub * 2 * D * 4);
  p.o_subvb = o; o = align_up(o + (size_t)p.t.sub * D * 4);
  p.o_clms16 = o; o = align_up(o + (size_t)p.t.cl * 2 * D * 2);
  p.o_clvb16 = o; o = align_up(o + (size_t)p.t.cl * D * 2);
  p.o_subms16 = o; o = align_up(o + (size_t)p.t.sub * 2 * D * 2);
  p.o_subvb16 = o; o = align_up(o + (size_t)p.t.sub * D * 2);
  p.o_foldsub = o; o = align_up(o + (size_t)nu * d->fold_capacity * 4);
  p.o_foldpos = o; o = align_up(o + (size_t)nu * d->fold_capacity * 4);
  p.o_clfold = o; o = align_up(o + (size_t)p.t.cl * 4);
  p.o_subfold = o; o = align_up(o + (size_t)p.t.sub * 4);
  p.o_appws = o; o = align_up(o + append_scratch_bytes(nu));
  const size_t F = (size_t)d->fm_dim;
  p.o_fmw = o; o = align_up(o + F * D * 4);
  p.o_clfz = o; o = align_up(o + (size_t)p.t.cl * F * 4);
  p.o_subfz = o; o = align_up(o + (size_t)p.t.sub * F * 4);
  p.bytes = o;
  return p;
}

void fill_seq_args(SeqArgs& sa, int n_seq, const int32_t* lens) {
  memset(&sa, 0, sizeof(sa));
  sa.n_seq = n_seq;
  for (int s = 0; s < n_seq; ++s) sa.len[s] = lens[s];
}

// ------------------------------------------------------------------------
// KV validation
// ------------------------------------------------------------------------
mog_status check_kv(const mog_kv* kv) {
  if (!kv) return fail(MOG_ERR_INVALID_ARG, "kv is NULL");
  if (kv->format != MOG_KV_CONTIGUOUS && kv->format != MOG_KV_PAGED)
    return fail(MOG_ERR_INVALID_ARG, "kv->format=%d", kv->format);
  if (kv->dtype != MOG_F32 && kv->dtype != MOG_BF16) return fail(MOG_ERR_UNSUPPORTED, "kv->dtype=%d", kv->dtype);
  if (kv->n_seq < 1 || kv->n_seq > MOG_MAX_SEQ)
    return fail(MOG_ERR_INVALID_ARG, "kv->n_seq=%d outside [1, %d]", kv->n_seq, MOG_MAX_SEQ);
  if (kv->n_kv_heads < 1) return fail(MOG_ERR_INVALID_ARG, "kv->n_kv_heads=%d", kv->n_kv_heads);
  if (kv->head_dim != 64 && kv->head_dim != 128)
    return fail(MOG_ERR_UNSUPPORTED, "kv->head_dim=%d (supported: 64, 128)", kv->head_dim);
  if (!kv->seq_lens) return fail(MOG_ERR_INVALID_ARG, "kv->seq_lens is NULL");
  if (!kv->k || !kv->v) return fail(MOG_ERR_INVALID_ARG, "kv->k or kv->v is NULL");
  if (!aligned(kv->k, 16) || !aligned(kv->v, 16))
    return fail(MOG_ERR_INVALID_ARG, "kv->k and kv->v must be 16-byte aligned");
  int max_len = 0;
  for (int s = 0; s < kv->n_seq; ++s) {
    if (kv->seq_lens[s] < 1 || kv->seq_lens[s] > MOG_MAX_LEN)
      return fail(MOG_ERR_INVALID_ARG, "kv->seq_lens[%d]=%d outside [1, %d]", s, kv->seq_lens[s], MOG_MAX_LEN);
    max_len = std::max(max_len, kv->seq_lens[s]);
  }
  if (kv->format == MOG_KV_CONTIGUOUS) {
    if (kv->max_len < max_len)
      return fail(MOG_ERR_INVALID_ARG, "kv->max_len=%d below the longest sequence (%d)", kv->max_len, max_len);
  } else {
    const int P = kv->page_size;
    if (P < 1 || P > 256 || (P & (P - 1)))
      return fail(MOG_ERR_INVALID_ARG, "kv->page_size=%d is not a power of two in [1, 256]", P);
    if (!kv->block_table) return fail(MOG_ERR_INVALID_ARG, "kv->block_table is NULL");
    if (kv->n_pages < 1) return fail(MOG_ERR_INVALID_ARG, "kv->n_pages=%d", kv->n_pages);
    if ((int64_t)kv->max_blocks * P < max_len)
      return fail(MOG_ERR_INVALID_ARG, "kv->max_blocks=%d pages of %d tokens cannot hold %d tokens",
                  kv->max_blocks, P, max_len);
  }
  return MOG_OK;
}

KVRef make_kvref(const mog_kv* kv) {
  KVRef r;
  r.k = kv->k;
  r.v = kv->v;
  r.block_table = kv->block_table;
  r.paged = kv->format == MOG_KV_PAGED;
  r.n_kv_heads = kv->n_kv_heads;
  r.max_len = kv->max_len;
  int sh = 0;
  if (r.paged)
    while ((1 << sh) < kv->page_size) ++sh;
  r.page_shift = sh;
  r.max_blocks = kv->max_blocks;
  return r;
}

// ------------------------------------------------------------------------
// Decode geometry
// ------------------------------------------------------------------------
struct DecodePlan {
  int G, c_stride, s_stride, splits, nblk, nb_res, nb_chosen, half;
  size_t o_clscore, o_cllse, o_clmask, o_cltiles, o_clrow0, o_chrow0, o_chnm, o_clrank, o_urows, o_list, o_nch, o_uinfo, o_tbase, o_ntl, o_tiles, o_res, o_ex;
  size_t o_fq, bytes;
};

int seq_top(const int32_t* per, int dflt, int s) { return per ? per[s] : dflt; }

mog_status check_decode_params(const mog_decode_params* p, int n_kv_heads, int n_seq) {
  if (!p) return fail(MOG_ERR_INVALID_ARG, "params is NULL");
  if (p->n_q_heads < 1 || p->n_q_heads % n_kv_heads)
    return fail(MOG_ERR_INVALID_ARG, "n_q_heads=%d is not a positive multiple of n_kv_heads=%d", p->n_q_heads,
                n_kv_heads);
  const int G = p->n_q_heads / n_kv_heads;
  if (G > kMaxG) return fail(MOG_ERR_UNSUPPORTED, "%d query heads per KV head (max %d)", G, kMaxG);
  if (p->splits < 0 || p->splits > 8192) return fail(MOG_ERR_INVALID_ARG, "splits=%d outside [0, 8192]", p->splits);
  if (p->residual < 0 || p->residual > 2)
    return fail(MOG_ERR_INVALID_ARG, "residual=%d (0: none, 1: Gaussian, 2: feature map)", p->residual);
  if (p->shared_selection != 0 && p->shared_selection != 1)
    return fail(MOG_ERR_INVALID_ARG, "shared_selection=%d (0 or 1)", p->shared_selection);
  if (p->exact_repeat < 0 || p->exact_repeat > 64)
    return fail(MOG_ERR_INVALID_ARG, "exact_repeat=%d outside [0, 64]", p->exact_repeat);
  if (!(p->scale >= 0.f) || isinf(p->scale)) return fail(MOG_ERR_INVALID_ARG, "scale must be finite and >= 0");
  for (int s = 0; s < n_seq; ++s) {
    const int c = seq_top(p->top_c_per_seq, p->top_c, s);
    const int sk = seq_top(p->top_s_per_seq, p->top_s, s);
    if (c < 0 || c > 32767) return fail(MOG_ERR_INVALID_ARG, "top_c=%d for sequence %d outside [0, 32767]", c, s);
    if (sk < 0 || sk > 127) return fail(MOG_ERR_INVALID_ARG, "top_s=%d for sequence %d outside [0, 127]", sk, s);
  }
  return MOG_OK;
}

DecodePlan plan_decode(const mog_layout* L, const mog_decode_params* p) {
  DecodePlan d;
  d.G = p->n_q_heads / L->n_kv_heads;
  d.c_stride = 0;
  d.s_stride = 0;
  d.nb_chosen = 0;
  for (int s = 0; s < L->n_seq; ++s) {
    const int c = seq_top(p->top_c_per_seq, p->top_c, s);
    const int sk = seq_top(p->top_s_per_seq, p->top_s, s);
    d.c_stride = std::max(d.c_stride, c);
    d.s_stride = std::max(d.s_stride, sk);
    const UnitSizes z = unit_sizes(L->seq_lens[s] - L->fold_count[s], L->n_sink, L->n_recent);
    d.nb_chosen = std::max<int>(d.nb_chosen, std::min(z.C, d.G * std::min(c, z.C)));
  }
  if (p->splits > 0) {
    d.splits = p->splits;
  } else {
    // one round of blocks: the exact kernel holds 2 blocks of 4 waves per
    // compute unit, 512 on the chip; launching more leaves a second round
    // that runs behind the first
    d.splits = std::max(1, kExactResidentBlocks - L->n_units);
  }
  d.nblk = d.splits + L->n_units;
  // exact blocks in halves of 2 waves with units of their own (finer shares)
  // when more than 16 units split the blocks and every unit's chosen list
  // fits a wave's own list
  d.half = (L->n_units > kExactResidentBlocks / 32 && d.nb_chosen <= kWaveListMax) ? 1 : 0;
  d.nb_res = d.nb_chosen + (int)ceil_div(L->max_C, kRestClustersSmall);  // (the smaller residual blocks: most records)
  const int D = L->head_dim, G = d.G, RS = D + kPartPad;
  const int64_t nu = L->n_units;
  size_t o = kAlign;  // first 256 bytes: reserved, kept zero
  // per-cluster entries: max_C per unit, so a unit's entries start at
  // u * max_C and kernels can address them before reading the unit table
  const size_t ncw = (size_t)nu * L->max_C;
  d.o_clscore = o; o = align_up(o + ncw * G * 4);
  d.o_cllse = o; o = align_up(o + (size_t)nu * G * 4);
  d.o_clmask = o; o = align_up(o + ncw * 4);
  d.o_cltiles = o; o = align_up(o + ncw * 4);
  d.o_clrow0 = o; o = align_up(o + ncw * 4);
  d.o_chrow0 = o; o = align_up(o + ncw * 4);
  d.o_chnm = o; o = align_up(o + ncw * 4);
  d.o_clrank = o; o = align_up(o + ncw * G * 4);
  d.o_urows = o; o = align_up(o + (size_t)nu * 4);
  d.o_list = o; o = align_up(o + ncw * 4);
  d.o_nch = o; o = align_up(o + (size_t)nu * 4);
  d.o_uinfo = o; o = align_up(o + (size_t)nu * 2 * 4);
  d.o_tbase = o; o = align_up(o + ncw * 4);
  d.o_ntl = o; o = align_up(o + ncw * 4);
  d.o_tiles = o;
  o = align_up(o + (size_t)(tile_unit_base(L->total_mid, L->total_cl, (int)nu, L->fold_capacity) + 2) *
                       sizeof(TileRec));
  d.o_res = o; o = align_up(o + (size_t)nu * d.nb_res * G * RS * 4);
  d.o_ex = o; o = align_up(o + (size_t)d.nblk * (d.half ? 2 : 1) * G * RS * 4);
  // feature-map residual: each query head's features, [n_units][G][fm_dim]
  d.o_fq = o;
  if (p->residual == 2) o = align_up(o + (size_t)nu * G * L->fm_dim * 4);
  d.bytes = o;
  return d;
}

struct DensePlan {
  int G, splits;
  size_t o_ex, bytes;
};

DensePlan plan_dense(const mog_kv* kv, const mog_decode_params* p) {
  DensePlan d;
  d.G = p->n_q_heads / kv->n_kv_heads;
  const int64_t nu = (int64_t)kv->n_seq * kv->n_kv_heads;
  int maxN = 1;
  for (int s = 0; s < kv->n_seq; ++s) maxN = std::max(maxN, kv->seq_lens[s]);
  if (p->splits > 0) {
    d.splits = p->splits;
  } else {
    int sp = (int)std::min<int64_t>(1024, ceil_div(2048, nu));
    sp = std::min<int64_t>(sp, ceil_div(maxN, 256));
    d.splits = std::max(1, sp);
  }
  const int RS = kv->head_dim + kPartPad;
  d.o_ex = kAlign;
  d.bytes = align_up(d.o_ex + (size_t)nu * d.splits * d.G * RS * 4);
  return d;
}

mog_status check_layout_arrays(const mog_layout* L) {
  if (!L->units || !L->k_mid || !L->v_mid || !L->sub_off || !L->cl_ms || !L->cl_vbar || !L->sub_ms ||
      !L->sub_vbar || !L->cl_ms16 || !L->cl_vbar16 || !L->sub_ms16 || !L->sub_vbar16 || !L->cl_fold ||
      !L->sub_fold || !L->append_scratch)
    return fail(MOG_ERR_INVALID_ARG, "layout has NULL arrays (not initialised?)");
  if (L->fold_capacity < 0 || L->fold_capacity > MOG_MAX_FOLD)
    return fail(MOG_ERR_INVALID_ARG, "layout fold_capacity=%d outside [0, %d]", L->fold_capacity, MOG_MAX_FOLD);
  if (L->fold_capacity > 0 && (!L->fold_sub || !L->fold_pos))
    return fail(MOG_ERR_INVALID_ARG, "layout has NULL fold arrays");
  if (L->fm_dim != 0 && L->fm_dim != 64 && L->fm_dim != 128 && L->fm_dim != 256)
    return fail(MOG_ERR_INVALID_ARG, "layout fm_dim=%d", L->fm_dim);
  if (L->fm_dim && (!L->fm_w || !L->cl_fz || !L->sub_fz || !(L->fm_scale > 0.f) || isinf(L->fm_scale)))
    return fail(MOG_ERR_INVALID_ARG, "layout has fm_dim=%d but no feature-map arrays or scale", L->fm_dim);
  for (int s = 0; s < L->n_seq; ++s)
    if (L->fold_count[s] < 0 || L->fold_count[s] > L->fold_capacity)
      return fail(MOG_ERR_INVALID_ARG, "layout fold_count[%d]=%d outside [0, %d]", s, L->fold_count[s],
                  L->fold_capacity);
  return MOG_OK;
}

mog_status check_layout_vs_kv(const mog_layout* L, const mog_kv* kv) {
  if (!L) return fail(MOG_ERR_INVALID_ARG, "layout is NULL");
  if (L->n_seq != kv->n_seq || L->n_kv_heads != kv->n_kv_heads || L->head_dim != kv->head_dim ||
      L->dtype != kv->dtype)
    return fail(MOG_ERR_INVALID_ARG, "layout (n_seq=%d, n_kv_heads=%d, head_dim=%d, dtype=%d) does not match kv "
                "(%d, %d, %d, %d)", L->n_seq, L->n_kv_heads, L->head_dim, L->dtype, kv->n_seq, kv->n_kv_heads,
                kv->head_dim, kv->dtype);
  for (int s = 0; s < L->n_seq; ++s)
    if (L->seq_lens[s] != kv->seq_lens[s])
      return fail(MOG_ERR_INVALID_ARG, "sequence %d: layout length %d, kv length %d", s, L->seq_lens[s],
                  kv->seq_lens[s]);
  return check_layout_arrays(L);
}

// ------------------------------------------------------------------------
// Build
// ------------------------------------------------------------------------
mog_status check_build(const mog_kv* kv, const mog_build_params* bp, mog_dims* dims_out) {
  mog_status st;
  if ((st = check_kv(kv)) != MOG_OK) return st;
  if (!bp) return fail(MOG_ERR_INVALID_ARG, "build params is NULL");
  if (bp->kmeans_iters < 0 || bp->kmeans_iters > 1000)
    return fail(MOG_ERR_INVALID_ARG, "kmeans_iters=%d outside [0, 1000]", bp->kmeans_iters);
  mog_dims d;
  d.n_seq = kv->n_seq;
  d.n_kv_heads = kv->n_kv_heads;
  d.head_dim = kv->head_dim;
  d.dtype = kv->dtype;
  d.n_sink = bp->n_sink;
  d.n_recent = bp->n_recent;
  d.fold_capacity = bp->fold_capacity;
  d.fm_dim = bp->fm_dim;
  d.rows_external = (bp->rows_k || bp->rows_v) ? 1 : 0;
  if (d.rows_external && !(bp->rows_k && bp->rows_v))
    return fail(MOG_ERR_INVALID_ARG, "rows_k and rows_v must both be set or both be NULL");
  if (d.rows_external && (!aligned(bp->rows_k, 16) || !aligned(bp->rows_v, 16)))
    return fail(MOG_ERR_INVALID_ARG, "rows_k and rows_v must be 16-byte aligned");
  d.seq_lens = kv->seq_lens;
  if ((st = check_dims(&d)) != MOG_OK) return st;
  if (bp->fm_dim) {
    if (!bp->fm_w) return fail(MOG_ERR_INVALID_ARG, "fm_dim=%d but fm_w is NULL", bp->fm_dim);
    if (!aligned(bp->fm_w, 16)) return fail(MOG_ERR_INVALID_ARG, "fm_w must be 16-byte aligned");
    if (!(bp->fm_scale >= 0.f) || isinf(bp->fm_scale))
      return fail(MOG_ERR_INVALID_ARG, "fm_scale must be finite and >= 0");
  }
  *dims_out = d;
  return MOG_OK;
}

struct BuildPlan {
  size_t o_cent, o_norm, o_sums, o_counts, o_labels, o_clstart, o_members, o_sublab, bytes;
};

BuildPlan plan_build(const mog_dims* d) {
  const LayoutPlan lp = plan_layout(d);
  BuildPlan b;
  const int D = d->head_dim;
  size_t o = kAlign;
  b.o_cent = o; o = align_up(o + (size_t)lp.t.cl * D * 4);
  b.o_norm = o; o = align_up(o + (size_t)lp.t.cl * 4);
  b.o_sums = o; o = align_up(o + (size_t)lp.t.cl * D * 8);
  b.o_counts = o; o = align_up(o + (size_t)lp.t.cl * 4);
  b.o_labels = o; o = align_up(o + (size_t)lp.t.mid * 4);
  b.o_clstart = o; o = align_up(o + (size_t)lp.t.cl * 4);
  b.o_members = o; o = align_up(o + (size_t)lp.t.mid * 4);
  b.o_sublab = o; o = align_up(o + (size_t)lp.t.mid * 4);
  b.bytes = o;
  return b;
}

mog_status build_workspace_bytes(const mog_kv* kv, const mog_build_params* bp, size_t* bytes) {
  mog_dims d;
  mog_status st = check_build(kv, bp, &d);
  if (st != MOG_OK) return st;
  *bytes = plan_build(&d).bytes;
  return ok();
}

}  // namespace

// ==========================================================================
// Exported entry points
// ==========================================================================
extern "C" {

const char* mog_status_string(mog_status st) {
  switch ((int)st) {
    case MOG_OK: return "ok";
    case MOG_ERR_INVALID_ARG: return "invalid argument";
    case MOG_ERR_UNSUPPORTED: return "unsupported";
    case MOG_ERR_WORKSPACE: return "workspace too small";
    case MOG_ERR_HIP: return "HIP error";
    case MOG_ERR_CAPACITY: return "fold area full (build again)";
  }
  return "unknown status";
}

const char* mog_last_error(void) { return g_last_error.c_str(); }

mog_status mog_layout_rows(const mog_dims* dims, int64_t* rows) {
  mog_status st = check_dims(dims);
  if (st != MOG_OK) return st;
  if (!rows) return fail(MOG_ERR_INVALID_ARG, "rows is NULL");
  const LayoutPlan p = plan_layout(dims);
  *rows = p.t.mid + (int64_t)dims->n_seq * dims->n_kv_heads * dims->fold_capacity;
  return ok();
}

mog_status mog_layout_size(const mog_dims* dims, size_t* bytes) {
  mog_status st = check_dims(dims);
  if (st != MOG_OK) return st;
  if (!bytes) return fail(MOG_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = plan_layout(dims).bytes;
  return ok();
}

static mog_status layout_carve(const mog_dims* dims, void* mem, size_t mem_bytes, mog_layout* out) {
  mog_status st = check_dims(dims);
  if (st != MOG_OK) return st;
  if (!out) return fail(MOG_ERR_INVALID_ARG, "out is NULL");
  if (!mem) return fail(MOG_ERR_INVALID_ARG, "layout_mem is NULL");
  if (!aligned(mem, kAlign)) return fail(MOG_ERR_INVALID_ARG, "layout_mem must be 256-byte aligned");
  const LayoutPlan p = plan_layout(dims);
  if (mem_bytes < p.bytes)
    return fail(MOG_ERR_WORKSPACE, "layout buffer has %zu bytes, %zu needed", mem_bytes, p.bytes);
  char* b = static_cast<char*>(mem);
  mog_layout L;
  memset(&L, 0, sizeof(L));
  L.n_seq = dims->n_seq;
  L.n_kv_heads = dims->n_kv_heads;
  L.head_dim = dims->head_dim;
  L.dtype = dims->dtype;
  L.n_sink = dims->n_sink;
  L.n_recent = dims->n_recent;
  L.n_units = dims->n_seq * dims->n_kv_heads;
  L.max_C = p.t.max_C;
  L.max_S = p.t.max_S;
  L.fold_capacity = dims->fold_capacity;
  for (int s = 0; s < dims->n_seq; ++s) L.seq_lens[s] = dims->seq_lens[s];
  L.total_mid = p.t.mid;
  L.total_cl = p.t.cl;
  L.total_sub = p.t.sub;
  L.total_off = p.t.off;
  L.units = reinterpret_cast<mog_unit*>(b + p.o_units);
  L.rows_external = dims->rows_external;
  L.k_mid = dims->rows_external ? nullptr : b + p.o_kmid;  // external: set by the caller
  L.v_mid = dims->rows_external ? nullptr : b + p.o_vmid;
  L.perm = reinterpret_cast<int32_t*>(b + p.o_perm);
  L.sub_off = reinterpret_cast<int32_t*>(b + p.o_suboff);
  L.cl_ms = reinterpret_cast<float*>(b + p.o_clms);
  L.cl_vbar = reinterpret_cast<float*>(b + p.o_clvb);
  L.sub_ms = reinterpret_cast<float*>(b + p.o_subms);
  L.sub_vbar = reinterpret_cast<float*>(b + p.o_subvb);
  L.cl_ms16 = reinterpret_cast<uint16_t*>(b + p.o_clms16);
  L.cl_vbar16 = reinterpret_cast<uint16_t*>(b + p.o_clvb16);
  L.sub_ms16 = reinterpret_cast<uint16_t*>(b + p.o_subms16);
  L.sub_vbar16 = reinterpret_cast<uint16_t*>(b + p.o_subvb16);
  L.fold_sub = dims->fold_capacity ? reinterpret_cast<int32_t*>(b + p.o_foldsub) : nullptr;
  L.fold_pos = dims->fold_capacity ? reinterpret_cast<int32_t*>(b + p.o_foldpos) : nullptr;
  L.cl_fold = reinterpret_cast<int32_t*>(b + p.o_clfold);
  L.sub_fold = reinterpret_cast<int32_t*>(b + p.o_subfold);
  L.append_scratch = b + p.o_appws;
  L.fm_dim = dims->fm_dim;
  L.fm_scale = 1.0f / sqrtf((float)dims->head_dim);
  if (dims->fm_dim) {
    L.fm_w = reinterpret_cast<float*>(b + p.o_fmw);
    L.cl_fz = reinterpret_cast<float*>(b + p.o_clfz);
    L.sub_fz = reinterpret_cast<float*>(b + p.o_subfz);
  }
  *out = L;
  return MOG_OK;
}

mog_status mog_layout_init(const mog_dims* dims, void* layout_mem, size_t layout_bytes, mog_layout* out,
                           hipStream_t stream) {
  mog_layout L;
  mog_status st = layout_carve(dims, layout_mem, layout_bytes, &L);
  if (st != MOG_OK) return st;
  SeqArgs sa;
  fill_seq_args(sa, dims->n_seq, dims->seq_lens);
  hipError_t e = launch_layout_table(L, sa, stream);
  if (e != hipSuccess) return fail(MOG_ERR_HIP, "layout table launch: %s", hipGetErrorString(e));
  *out = L;
  return ok();
}

mog_status mog_layout_sync_stats(const mog_layout* L, hipStream_t stream) {
  if (!L) return fail(MOG_ERR_INVALID_ARG, "layout is NULL");
  mog_status st = check_layout_arrays(L);
  if (st != MOG_OK) return st;
  if (L->head_dim != 64 && L->head_dim != 128) return fail(MOG_ERR_INVALID_ARG, "layout head_dim=%d", L->head_dim);
  if (L->total_cl < 0 || L->total_sub < 0) return fail(MOG_ERR_INVALID_ARG, "layout has negative group counts");
  hipError_t e = launch_stats16(*L, stream);
  if (e != hipSuccess) return fail(MOG_ERR_HIP, "statistics copy launch: %s", hipGetErrorString(e));
  return ok();
}

mog_status mog_layout_unit(const mog_layout* L, int32_t unit, mog_unit* out) {
  if (!L || !out) return fail(MOG_ERR_INVALID_ARG, "NULL argument");
  if (unit < 0 || unit >= L->n_units) return fail(MOG_ERR_INVALID_ARG, "unit %d outside [0, %d)", unit, L->n_units);
  const int s = unit / L->n_kv_heads, kvh = unit % L->n_kv_heads;
  // geometry follows from the lengths at the build
  int64_t row = 0, cl = 0, sub = 0, offb = 0;
  for (int s2 = 0; s2 < s; ++s2) {
    const UnitSizes z = unit_sizes(L->seq_lens[s2] - L->fold_count[s2], L->n_sink, L->n_recent);
    row += (int64_t)L->n_kv_heads * z.n_mid;
    cl += (int64_t)L->n_kv_heads * z.C;
    sub += (int64_t)L->n_kv_heads * z.C * z.S;
    offb += (int64_t)L->n_kv_heads * (z.C * z.S + 1);
  }
  const UnitSizes z = unit_sizes(L->seq_lens[s] - L->fold_count[s], L->n_sink, L->n_recent);
  mog_unit U;
  U.seq = s;
  U.kv_head = kvh;
  U.N = L->seq_lens[s];
  U.n_mid = z.n_mid;
  U.C = z.C;
  U.S = z.S;
  U.n_fold = L->fold_count[s];
  U.reserved1 = 0;
  U.row_base = row + (int64_t)kvh * z.n_mid;
  U.cl_base = cl + (int64_t)kvh * z.C;
  U.sub_base = sub + (int64_t)kvh * z.C * z.S;
  U.off_base = offb + (int64_t)kvh * (z.C * z.S + 1);
  *out = U;
  return ok();
}

mog_status mog_workspace_size(mog_op op, const mog_kv* kv, const mog_layout* layout, const mog_build_params* bp,
                              const mog_decode_params* dp, size_t* bytes) {
  if (!bytes) return fail(MOG_ERR_INVALID_ARG, "bytes is NULL");
  mog_status st;
  switch ((int)op) {
    case MOG_OP_DECODE: {
      if (!layout) return fail(MOG_ERR_INVALID_ARG, "layout is NULL");
      if ((st = check_decode_params(dp, layout->n_kv_heads, layout->n_seq)) != MOG_OK) return st;
      *bytes = plan_decode(layout, dp).bytes;
      return ok();
    }
    case MOG_OP_DENSE: {
      if ((st = check_kv(kv)) != MOG_OK) return st;
      if ((st = check_decode_params(dp, kv->n_kv_heads, kv->n_seq)) != MOG_OK) return st;
      *bytes = plan_dense(kv, dp).bytes;
      return ok();
    }
    case MOG_OP_BUILD:
      return build_workspace_bytes(kv, bp, bytes);
  }
  return fail(MOG_ERR_INVALID_ARG, "unknown op %d", (int)op);
}

// The decode step with its workspace (`static_ws`: the library's own scratch
// of mog_decode_noalloc, whose size limit gets its own error text).
static mog_status decode_with_ws(const mog_layout* layout, const mog_kv* kv, const float* q,
                                 const mog_decode_params* params, float* out, float* lse, int32_t* sel_c,
                                 int32_t* sel_s, void* ws, size_t ws_bytes, bool static_ws, hipStream_t stream) {
  mog_status st;
  if ((st = check_kv(kv)) != MOG_OK) return st;
  if ((st = check_layout_vs_kv(layout, kv)) != MOG_OK) return st;
  if ((st = check_decode_params(params, kv->n_kv_heads, kv->n_seq)) != MOG_OK) return st;
  if (!q || !out) return fail(MOG_ERR_INVALID_ARG, "q or out is NULL");
  if (!ws) return fail(MOG_ERR_INVALID_ARG, "workspace is NULL");
  if (!aligned(ws, kAlign)) return fail(MOG_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (!aligned(layout->k_mid, 16) || !aligned(layout->v_mid, 16))
    return fail(MOG_ERR_INVALID_ARG, "layout rows must be 16-byte aligned");
  for (int s = 0; s < kv->n_seq; ++s)
    if (kv->seq_lens[s] - layout->n_sink - layout->n_recent < 1)
      return fail(MOG_ERR_INVALID_ARG, "sequence %d has no middle region", s);
  const float scale = params->scale > 0.f ? params->scale : 1.0f / sqrtf((float)kv->head_dim);
  if (params->residual == 2) {
    if (layout->fm_dim == 0)
      return fail(MOG_ERR_INVALID_ARG, "residual=2 needs a layout built with feature-map summaries (fm_dim > 0)");
    if (scale != layout->fm_scale)
      return fail(MOG_ERR_INVALID_ARG, "residual=2: decode scale %g differs from the summaries' scale %g", scale,
                  layout->fm_scale);
  }
  const DecodePlan d = plan_decode(layout, params);
  if (ws_bytes < d.bytes) {
    if (static_ws)
      return fail(MOG_ERR_WORKSPACE,
                  "this decode needs %zu bytes of scratch, above the %zu of the library's static scratch "
                  "(MOG_DECODE_NOALLOC_MAX_WS); call mog_decode with a workspace instead", d.bytes, ws_bytes);
    return fail(MOG_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, d.bytes);
  }
  // with a zero budget there is nothing to report
  if (d.c_stride == 0) sel_c = sel_s = nullptr;
  if (d.s_stride == 0) sel_s = nullptr;

  DecodeLaunch x;
  memset(&x, 0, sizeof(x));
  x.L = *layout;
  x.kv = make_kvref(kv);
  fill_seq_args(x.seq, kv->n_seq, kv->seq_lens);
  for (int s = 0; s < kv->n_seq; ++s) {
    x.seq.top_c[s] = (int16_t)seq_top(params->top_c_per_seq, params->top_c, s);
    x.seq.top_s[s] = (int8_t)seq_top(params->top_s_per_seq, params->top_s, s);
  }
  x.q = q;
  x.out = out;
  x.lse = lse;
  x.sel_c = sel_c;
  x.sel_s = sel_s;
  x.c_stride = d.c_stride;
  x.s_stride = std::max(d.s_stride, 1);
  x.Hq = params->n_q_heads;
  x.G = d.G;
  x.D = kv->head_dim;
  x.dtype = kv->dtype;
  x.residual = params->residual;
  x.shared = params->shared_selection;
  x.splits = d.splits;
  x.nblk = d.nblk;
  x.half = d.half;
  x.nb_res = d.nb_res;
  x.nb_chosen = d.nb_chosen;
  // whole-cluster step: every chosen cluster is read entirely, so there are
  // no subclusters to score or rank
  x.whole = layout->fold_capacity == 0 && sel_s == nullptr && d.nb_chosen <= kWaveListMax;
  for (int s = 0; s < kv->n_seq && x.whole; ++s) {
    const UnitSizes z = unit_sizes(layout->seq_lens[s] - layout->fold_count[s], layout->n_sink, layout->n_recent);
    x.whole = x.seq.top_s[s] >= z.S;
  }
  x.scale = scale;
  x.ev_begin = params->exact_begin;
  x.ev_end = params->exact_end;
  x.repeat = std::max(1, params->exact_repeat);
  char* w = static_cast<char*>(ws);
  x.ws.fq = params->residual == 2 ? reinterpret_cast<float*>(w + d.o_fq) : nullptr;
  x.ws.cl_score = reinterpret_cast<float*>(w + d.o_clscore);
  x.ws.cl_lse = reinterpret_cast<float*>(w + d.o_cllse);
  x.ws.cl_mask = reinterpret_cast<uint32_t*>(w + d.o_clmask);
  x.ws.cl_tiles = reinterpret_cast<int32_t*>(w + d.o_cltiles);
  x.ws.cl_row0 = reinterpret_cast<int32_t*>(w + d.o_clrow0);
  x.ws.ch_row0 = reinterpret_cast<int32_t*>(w + d.o_chrow0);
  x.ws.ch_nm = reinterpret_cast<uint32_t*>(w + d.o_chnm);
  x.ws.cl_rank = reinterpret_cast<int32_t*>(w + d.o_clrank);
  x.ws.unit_rows = reinterpret_cast<int32_t*>(w + d.o_urows);
  x.ws.cl_list = reinterpret_cast<int32_t*>(w + d.o_list);
  x.ws.n_chosen = reinterpret_cast<int32_t*>(w + d.o_nch);
  x.ws.uinfo = reinterpret_cast<int32_t*>(w + d.o_uinfo);
  x.ws.ch_tbase = reinterpret_cast<int32_t*>(w + d.o_tbase);
  x.ws.ch_ntiles = reinterpret_cast<int32_t*>(w + d.o_ntl);
  x.ws.tiles = reinterpret_cast<TileRec*>(w + d.o_tiles);
  x.ws.res_part = reinterpret_cast<float*>(w + d.o_res);
  x.ws.ex_part = reinterpret_cast<float*>(w + d.o_ex);
  hipError_t e = launch_decode(x, stream);
  if (e != hipSuccess) return fail(MOG_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"

// Scratch of mog_decode_noalloc: device memory of the code object, one copy
// on every GPU the library runs on, held until the process ends.  In host
// code `scratch` only names the symbol; its device address on the current
// GPU comes from hipGetSymbolAddress, looked up once per device and kept.
static __device__ __align__(256) unsigned char scratch[MOG_DECODE_NOALLOC_MAX_WS];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

mog_status static_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOG_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MOG_ERR_UNSUPPORTED, "device %d (the scratch table holds %d)", dev,
                                                 kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MOG_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MOG_OK;
}

}  // namespace

extern "C" {

mog_status mog_decode(const mog_layout* layout, const mog_kv* kv, const float* q, const mog_decode_params* params,
                      float* out, float* lse, int32_t* sel_c, int32_t* sel_s, void* ws, size_t ws_bytes,
                      hipStream_t stream) {
  return decode_with_ws(layout, kv, q, params, out, lse, sel_c, sel_s, ws, ws_bytes, false, stream);
}

mog_status mog_decode_noalloc(const mog_layout* layout, const mog_kv* kv, const float* q,
                              const mog_decode_params* params, float* out, float* lse, int32_t* sel_c,
                              int32_t* sel_s, hipStream_t stream) {
  void* ws = nullptr;
  const mog_status st = static_scratch(&ws);
  if (st != MOG_OK) return st;
  return decode_with_ws(layout, kv, q, params, out, lse, sel_c, sel_s, ws, MOG_DECODE_NOALLOC_MAX_WS, true, stream);
}

mog_status mog_append(const mog_kv* kv, mog_layout* layout, hipStream_t stream) {
  mog_status st;
  if ((st = check_kv(kv)) != MOG_OK) return st;
  if (!layout) return fail(MOG_ERR_INVALID_ARG, "layout is NULL");
  const mog_layout* L = layout;
  if (L->n_seq != kv->n_seq || L->n_kv_heads != kv->n_kv_heads || L->head_dim != kv->head_dim ||
      L->dtype != kv->dtype)
    return fail(MOG_ERR_INVALID_ARG, "layout (n_seq=%d, n_kv_heads=%d, head_dim=%d, dtype=%d) does not match kv "
                "(%d, %d, %d, %d)", L->n_seq, L->n_kv_heads, L->head_dim, L->dtype, kv->n_seq, kv->n_kv_heads,
                kv->head_dim, kv->dtype);
  if ((st = check_layout_arrays(L)) != MOG_OK) return st;
  AppendLaunch x;
  memset(&x, 0, sizeof(x));
  int total = 0;
  for (int s = 0; s < L->n_seq; ++s) {
    const int a = kv->seq_lens[s] - L->seq_lens[s];
    if (a < 0)
      return fail(MOG_ERR_INVALID_ARG, "sequence %d: kv length %d below the layout's %d", s, kv->seq_lens[s],
                  L->seq_lens[s]);
    if (L->fold_count[s] + a > L->fold_capacity)
      return fail(MOG_ERR_CAPACITY, "sequence %d: %d folded + %d new tokens exceed the fold capacity %d", s,
                  L->fold_count[s], a, L->fold_capacity);
    x.seq[s].len = L->seq_lens[s];
    x.seq[s].n_new = (uint16_t)a;
    x.seq[s].f0 = (uint16_t)L->fold_count[s];
    total += a;
  }
  if (total == 0) return ok();
  x.L = *L;
  x.kv = make_kvref(kv);
  x.n_seq = L->n_seq;
  hipError_t e = launch_append(x, stream);
  if (e != hipSuccess) return fail(MOG_ERR_HIP, "append launch: %s", hipGetErrorString(e));
  for (int s = 0; s < L->n_seq; ++s) {
    layout->fold_count[s] += x.seq[s].n_new;
    layout->seq_lens[s] += x.seq[s].n_new;
  }
  return ok();
}

mog_status mog_dense_decode(const mog_kv* kv, const float* q, const mog_decode_params* params, float* out,
                            float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  mog_status st;
  if ((st = check_kv(kv)) != MOG_OK) return st;
  if ((st = check_decode_params(params, kv->n_kv_heads, kv->n_seq)) != MOG_OK) return st;
  if (!q || !out) return fail(MOG_ERR_INVALID_ARG, "q or out is NULL");
  if (!ws) return fail(MOG_ERR_INVALID_ARG, "workspace is NULL");
  if (!aligned(ws, kAlign)) return fail(MOG_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const DensePlan d = plan_dense(kv, params);
  if (ws_bytes < d.bytes) return fail(MOG_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, d.bytes);
  DenseLaunch x;
  memset(&x, 0, sizeof(x));
  x.kv = make_kvref(kv);
  fill_seq_args(x.seq, kv->n_seq, kv->seq_lens);
  x.q = q;
  x.out = out;
  x.lse = lse;
  x.Hq = params->n_q_heads;
  x.G = d.G;
  x.D = kv->head_dim;
  x.dtype = kv->dtype;
  x.n_kv_heads = kv->n_kv_heads;
  x.splits = d.splits;
  x.scale = params->scale > 0.f ? params->scale : 1.0f / sqrtf((float)kv->head_dim);
  x.ev_begin = params->exact_begin;
  x.ev_end = params->exact_end;
  x.repeat = std::max(1, params->exact_repeat);
  x.ex_part = reinterpret_cast<float*>(static_cast<char*>(ws) + d.o_ex);
  hipError_t e = launch_dense(x, stream);
  if (e != hipSuccess) return fail(MOG_ERR_HIP, "dense launch: %s", hipGetErrorString(e));
  return ok();
}

mog_status mog_build(const mog_kv* kv, const mog_build_params* params, void* layout_mem, size_t layout_bytes,
                     void* ws, size_t ws_bytes, mog_layout* out, hipStream_t stream) {
  mog_dims d;
  mog_status st = check_build(kv, params, &d);
  if (st != MOG_OK) return st;
  if (!out) return fail(MOG_ERR_INVALID_ARG, "out is NULL");
  if (!ws) return fail(MOG_ERR_INVALID_ARG, "workspace is NULL");
  if (!aligned(ws, kAlign)) return fail(MOG_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const BuildPlan bpn = plan_build(&d);
  if (ws_bytes < bpn.bytes) return fail(MOG_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, bpn.bytes);
  mog_layout L;
  if ((st = layout_carve(&d, layout_mem, layout_bytes, &L)) != MOG_OK) return st;
  if (d.rows_external) {
    L.k_mid = params->rows_k;
    L.v_mid = params->rows_v;
  }
  SeqArgs sa;
  fill_seq_args(sa, d.n_seq, d.seq_lens);
  hipError_t e = launch_layout_table(L, sa, stream);
  if (e != hipSuccess) return fail(MOG_ERR_HIP, "layout table launch: %s", hipGetErrorString(e));
  BuildLaunch x;
  memset(&x, 0, sizeof(x));
  x.L = L;
  x.kv = make_kvref(kv);
  x.seq = sa;
  x.D = d.head_dim;
  x.dtype = d.dtype;
  x.iters = params->kmeans_iters;
  x.seed = params->seed;
  if (params->fm_dim) {
    L.fm_scale = params->fm_scale > 0.f ? params->fm_scale : 1.0f / sqrtf((float)d.head_dim);
    x.L = L;
    x.fm_w = params->fm_w;
  }
  char* w = static_cast<char*>(ws);
  x.ws.cent = reinterpret_cast<float*>(w + bpn.o_cent);
  x.ws.cent_norm = reinterpret_cast<float*>(w + bpn.o_norm);
  x.ws.sums = reinterpret_cast<unsigned long long*>(w + bpn.o_sums);
  x.ws.counts = reinterpret_cast<int32_t*>(w + bpn.o_counts);
  x.ws.labels = reinterpret_cast<int32_t*>(w + bpn.o_labels);
  x.ws.cl_start = reinterpret_cast<int32_t*>(w + bpn.o_clstart);
  x.ws.members = reinterpret_cast<int32_t*>(w + bpn.o_members);
  x.ws.sublab = reinterpret_cast<int32_t*>(w + bpn.o_sublab);
  e = launch_build(x, stream);
  if (e != hipSuccess) return fail(MOG_ERR_HIP, "build launch: %s", hipGetErrorString(e));
  *out = L;
  return ok();
}

}  // extern "C"
