// Decode-side kernels of libmog: Gaussian log-mass scoring of clusters and
// subclusters, top-c / top-s selection, exact split-K attention over the
// anchors and the chosen subclusters, the residual estimate of every group
// left out, and the single-normalisation merge; plus the dense baseline.
//
// Method: "Iceberg Attention: Sublinear Long-Context Decoding with
// Mixture-of-Gaussians" (abstract) -- score the query against per-group
// Gaussians, attend exactly to the best clusters/subclusters, estimate the
// rest from means and variances.  Merge rule: retrieval-completion attention
// page (abstract) -- exact anchors + retrieved tokens and the estimated
// remainder are added as unnormalised numerator/denominator and normalised
// once.
//
// All softmax bookkeeping is in the base-2 log domain: a logit x is carried
// as x*log2(e) so every exponential is an exp2.
#include <hip/hip_ext.h>

#include "attn_tile.h"
#include "mog_internal.h"

namespace mog {

struct LayoutRef {
  const mog_unit* units;
  const void* k_mid;
  const void* v_mid;
  const int32_t* sub_off;
  // group statistics in bf16 (the layout's copies of its float32 ones):
  // [groups][2 D] key mean | variance, [groups][D] value mean
  const uint16_t* cl_ms;
  const uint16_t* cl_vbar;
  const uint16_t* sub_ms;
  const uint16_t* sub_vbar;
  // folded tokens (incremental decode): per-group counts, and per unit the
  // subcluster of every fold row; unit u's fold rows start at layout row
  // fold_row0 + u * fold_cap
  const int32_t* cl_fold;
  const int32_t* sub_fold;
  const int32_t* fold_sub;
  int64_t fold_row0;
  int32_t fold_cap;
  // feature-map summaries: projection [fm_dim][D], per-group feature sums
  const float* fm_w;
  const float* cl_fz;
  const float* sub_fz;
  int32_t fm_dim;
};

struct DArgs {
  LayoutRef L;
  KVRef kv;
  const float* q;
  float* out;
  float* lse;
  int32_t* sel_c;
  int32_t* sel_s;
  int32_t c_stride, s_stride, Hq, Hkv, n_sink, n_recent, residual, shared, splits, nb_res, n_units, nblk;
  int32_t cstride;   // per-cluster workspace entries per unit (the largest C)
  float scale_l2;    // scale * log2(e)
  float half_s2_l2;  // scale^2 / 2 * log2(e)
  float sqrt_scale;  // feature-map residual: the map is applied to sqrt(scale) q
  int32_t score_blocks;  // blocks of the cluster-score kernel per unit that score clusters
  int32_t L_head_dim;
  int32_t whole;          // whole-cluster step (top-c lists the tiles, no subcluster kernel)
  int32_t half;           // exact blocks in halves of 2 waves, each with a unit share of its own
  int32_t rest_cl;        // clusters per residual block (rest_clusters_per_block)
  int32_t rest_per_unit;  // residual blocks per unit: ceil(largest C / rest_cl)
  // every unit has the same geometry (equal lengths and fold counts at the
  // build): its record follows from its index (uni_C > 0), else it is loaded
  int32_t uni_C, uni_S, uni_nmid, uni_N, uni_nfold;
  DecodeWS ws;
};

// Unit u's record: computed from the index for a layout of equal units (the
// unit table's own rule: units in order, C clusters, C*S subclusters, C*S+1
// offsets and n_mid rows each), else loaded.
// A block-uniform value by a scalar load (through the scalar cache, whose
// round trip is shorter than a vector load's); only for memory no launch of
// the step writes while the reading kernel runs.
template <typename T>
__device__ inline T scalar_load(const T* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}

// A unit record by scalar loads: the table is read-only while a decode runs
// (the layout's own launches write it before), and every lane of the wave
// reads the same address, so the record can come through the scalar cache,
// whose round trip is shorter than a vector load's.
__device__ inline mog_unit unit_scalar(const mog_unit* p) {
  typedef const __attribute__((address_space(4))) mog_unit* const_unit_ptr;
  const const_unit_ptr c = (const_unit_ptr)p;
  mog_unit U;
  U.seq = c->seq;
  U.kv_head = c->kv_head;
  U.N = c->N;
  U.n_mid = c->n_mid;
  U.C = c->C;
  U.S = c->S;
  U.n_fold = c->n_fold;
  U.reserved1 = 0;
  U.row_base = c->row_base;
  U.cl_base = c->cl_base;
  U.sub_base = c->sub_base;
  U.off_base = c->off_base;
  return U;
}

__device__ inline mog_unit unit_record(const DArgs& a, int u) {
  if (a.uni_C > 0) {
    mog_unit U;
    U.seq = u / a.Hkv;
    U.kv_head = u % a.Hkv;
    U.N = a.uni_N;
    U.n_mid = a.uni_nmid;
    U.C = a.uni_C;
    U.S = a.uni_S;
    U.n_fold = a.uni_nfold;
    U.reserved1 = 0;
    U.row_base = (int64_t)u * a.uni_nmid;
    U.cl_base = (int64_t)u * a.uni_C;
    U.sub_base = (int64_t)u * a.uni_C * a.uni_S;
    U.off_base = (int64_t)u * (a.uni_C * a.uni_S + 1);
    return U;
  }
  return unit_scalar(a.L.units + u);
}

struct BudgetArgs {
  int16_t top_c[MOG_MAX_SEQ];
  int8_t top_s[MOG_MAX_SEQ];
};

// ---------------------------------------------------------------------------
// Block-wide helpers (NT threads, a multiple of 64)
// ---------------------------------------------------------------------------
template <int NT>
__device__ inline int block_excl_scan(int v, int* sh, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    int t = sh[w];
    off += (w < wave) ? t : 0;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return off + x - v;
}

template <int NT>
__device__ inline float block_max(float v, float* sh) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = -INFINITY;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) r = fmaxf(r, sh[w]);
  __syncthreads();
  return r;
}

template <int NT>
__device__ inline float block_sum(float v, float* sh) {
  v = wave_sum_dpp(v);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = 0.f;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) r += sh[w];
  __syncthreads();
  return r;
}

// exp-weighted accumulation of one estimated group (log2 weight w, mean
// value vb) into a running (m, l, o) state.
template <int VPL>
__device__ inline void add_group(float& m, float& l, float (&o)[VPL], float w, const float (&vb)[VPL]) {
  const float mn = fmaxf(m, w);
  const float a = (m == -INFINITY) ? 0.f : exp2f(m - mn);
  const float p = exp2f(w - mn);
  l = l * a + p;
#pragma unroll
  for (int e = 0; e < VPL; ++e) o[e] = o[e] * a + p * vb[e];
  m = mn;
}

// N consecutive floats of a group-statistics row.  Each row is read once per
// step, so the loads are non-temporal (they leave the L2 to the small
// per-unit arrays and the kernels' code).
template <int N>
__device__ inline void load_floats(const float* p, float (&x)[N]) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  if constexpr (N == 4) {
    const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    x[0] = t.x; x[1] = t.y; x[2] = t.z; x[3] = t.w;
  } else if constexpr (N == 2) {
    const f32x2 t = __builtin_nontemporal_load(reinterpret_cast<const f32x2*>(p));
    x[0] = t.x; x[1] = t.y;
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = __builtin_nontemporal_load(p + i);
  }
}

// N consecutive bf16 statistics as float32 (exact), one load; non-temporal
// like the float32 rows above.
template <int N>
__device__ inline void load_floats(const uint16_t* p, float (&x)[N]) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  if constexpr (N == 4) {
    const u32x2 t = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    x[0] = bf16_lo(t.x); x[1] = bf16_hi(t.x); x[2] = bf16_lo(t.y); x[3] = bf16_hi(t.y);
  } else if constexpr (N == 2) {
    const uint32_t t = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
    x[0] = bf16_lo(t); x[1] = bf16_hi(t);
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = __uint_as_float((uint32_t)__builtin_nontemporal_load(p + i) << 16);
  }
}

// N consecutive bf16 statistics (N even) as N / 2 packed pairs, one
// non-temporal load.
template <int N>
__device__ inline void load_bf16_pairs(const uint16_t* p, uint32_t (&r)[N / 2]) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  if constexpr (N == 4) {
    const u32x2 t = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    r[0] = t.x; r[1] = t.y;
  } else {
    static_assert(N == 2, "rows of 2 or 4 statistics a lane");
    r[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
  }
}

// N (1 or 2) consecutive bf16 statistics as the bits of one 32-bit word
// (the first in the low half), one non-temporal load.
template <int N>
__device__ inline uint32_t load_bf16_bits(const uint16_t* p) {
  static_assert(N == 1 || N == 2, "one or two statistics a lane");
  if constexpr (N == 2) return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
  else return (uint32_t)__builtin_nontemporal_load(p);
}

// Per-lane coefficients of the score: lanes 0-31 hold scale*log2e*q_i for the
// mean half of a [mu | var] row, lanes 32-63 hold scale^2/2*log2e*q_i^2 for the
// variance half, so one coalesced load of a group row and one wave sum give
// log2e * (scale q.mu + scale^2/2 sum q_i^2 var_i).
template <int D, int G>
__device__ inline void score_coefs(const DArgs& a, const float* qb, float (&coef)[G][D / 32]) {
  constexpr int EPL = D / 32;
  const int lane = threadIdx.x & 63;
  const bool var_half = lane >= 32;
  const int e0 = (lane & 31) * EPL;
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const float qv = qb[h * D + e0 + e];
      coef[h][e] = var_half ? a.half_s2_l2 * qv * qv : a.scale_l2 * qv;
    }
  }
}

// ---------------------------------------------------------------------------
// 1. Cluster scores: score[g][h] = log2 n_g + log2e (scale q_h.mu_g +
//    scale^2/2 sum_i q_{h,i}^2 var_{g,i}); -inf for an empty cluster.
//    Grid (ceil(maxC/16), units); each wave loads 4 cluster rows at once.
// ---------------------------------------------------------------------------
constexpr int kScoreRowsPerWave = 4;  // clusters scored per wave (16 per block)

// Feature-map residual: log2 of the features of every query head of unit u,
// fq[u][h][i] = log2(e) (sqrt(s) w_i.q_h - s |q_h|^2 / 2) (the 1/sqrt(m) factor
// is applied where the features are used).  Block f of the unit takes
// features [64 f, 64 f + 64): their rows of W and the unit's queries pass
// through LDS (`lds`, dynamic; the rows padded to D + 1 floats, so that the
// 64 lanes reading 64 rows hit 64 banks), lane i takes feature 64 f + i and
// wave w heads w, w + 4.
template <int D, int G>
__host__ __device__ constexpr int query_features_lds() {
  return (64 * (D + 1) + G * D) * (int)sizeof(float);
}

template <int D, int G>
__device__ inline void query_features(const DArgs& a, int u, int f, float* lds) {
  constexpr int P = D + 1, R4 = D / 4;  // (LDS row pitch; float4s per row)
  float* wr = lds;           // [64][P]
  float* qs = lds + 64 * P;  // [G][D]
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int m = a.L.fm_dim;
  const int seq = u / a.Hkv, kvh = u % a.Hkv;
  const float* qb = a.q + ((int64_t)seq * a.Hq + (int64_t)kvh * G) * D;
  const float* wb = a.L.fm_w + (int64_t)64 * f * D;
  constexpr int NL = 64 * R4 / 256;  // float4s of the block's rows per thread
  float4 w[NL];
#pragma unroll
  for (int k = 0; k < NL; ++k) w[k] = *reinterpret_cast<const float4*>(wb + 4 * (t + 256 * k));
  for (int k = t; k < G * D; k += 256) qs[k] = qb[k];
#pragma unroll
  for (int k = 0; k < NL; ++k) {
    const int r = (t + 256 * k) / R4, c = (t + 256 * k) % R4;
    float* d = wr + r * P + 4 * c;
    d[0] = w[k].x;
    d[1] = w[k].y;
    d[2] = w[k].z;
    d[3] = w[k].w;
  }
  __syncthreads();
  const float s = a.sqrt_scale;
  const float* wi = wr + lane * P;
#pragma unroll
  for (int h = wave; h < G; h += 4) {
    const float* qh = qs + h * D;
    float dot = 0.f, qq = 0.f;
#pragma unroll 16
    for (int e = 0; e < D; ++e) {
      const float qv = qh[e];
      dot += wi[e] * qv;
      qq += qv * qv;
    }
    a.ws.fq[((int64_t)u * G + h) * m + 64 * f + lane] = kLog2e * (s * dot - 0.5f * s * s * qq);
  }
}

template <int D, int G>
__global__ __launch_bounds__(256) void k_score_clusters(DArgs a) {
  constexpr int EPL = D / 32;
  const int u = blockIdx.y;
  if ((int)blockIdx.x >= a.score_blocks) {
    extern __shared__ float fq_lds[];  // (sized only when these blocks exist)
    query_features<D, G>(a, u, blockIdx.x - a.score_blocks, fq_lds);
    return;
  }
  const mog_unit U = unit_record(a, u);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // (a subcluster step's kernels add the unit's exact rows to this count)
  if (blockIdx.x == 0 && threadIdx.x == 0 && !a.whole) a.ws.unit_rows[u] = 0;
  const int g0 = blockIdx.x * (4 * kScoreRowsPerWave) + wave * kScoreRowsPerWave;
  if (g0 >= U.C) return;
  const float* qb = a.q + ((int64_t)U.seq * a.Hq + (int64_t)U.kv_head * G) * D;
  float coef[G][EPL];
  score_coefs<D, G>(a, qb, coef);
  const int32_t* off = a.L.sub_off + U.off_base;
  float x[kScoreRowsPerWave][EPL];
#pragma unroll
  for (int k = 0; k < kScoreRowsPerWave; ++k) {
    const int g = min(g0 + k, U.C - 1);
    load_floats<EPL>(a.L.cl_ms + (U.cl_base + g) * (2 * D) + lane * EPL, x[k]);
  }
  // the R x G partial dot products, summed over the lanes by one
  // reduce-scatter: one lane then holds each (cluster, head) score; the
  // lane's cluster is known now, so its bounds load with the rows
  constexpr int R = kScoreRowsPerWave;
  const int j = rs_index<R * G>(lane), g = g0 + j / G;
  const int gc = min(g, U.C - 1);
  const int ob0 = off[gc * U.S], ob1 = off[(gc + 1) * U.S];
  const int nf = a.L.fold_cap ? a.L.cl_fold[U.cl_base + gc] : 0;
  float part[R * G];
#pragma unroll
  for (int k = 0; k < R; ++k) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float t = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) t += coef[h][e] * x[k][e];
      part[k * G + h] = t;
    }
  }
  const float t = wave_reduce_scatter<R * G>(part);
  if (rs_owner<R * G>(lane) && g < U.C) {
    const int nr = ob1 - ob0;
    const int n = nr + nf;
    a.ws.cl_score[((int64_t)u * G + j % G) * a.cstride + g] = n > 0 ? t + log2f((float)n) : -INFINITY;
    // the most tile slots the cluster can need if chosen (one partial tile
    // per run, at most S runs, a folded row alone at worst), read by the
    // top-c kernel with the scores; a whole-cluster step reads every row of
    // a chosen cluster, one run: its size and first row instead
    if (j % G == 0) {
      const int64_t cg = (int64_t)u * a.cstride + g;
      if (a.whole) {
        a.ws.cl_tiles[cg] = nr;
        a.ws.cl_row0[cg] = ob0;
      } else {
        a.ws.cl_tiles[cg] = (nr + 31) / 32 + U.S + nf;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 2. Top-c clusters of every head of a unit, one wave per head.  Cluster i
//    sits in lane i % 64, slot i / 64 of the wave's registers (KPL slots,
//    enough for the largest unit).  A radix select, most significant bits
//    first, finds the key of the c-th largest score: bits every valid key
//    shares are decided at once, the next (up to) 8 varying bits by a
//    histogram in the wave's LDS bins (suffix counts by a DPP scan), and it
//    stops as soon as every remaining candidate is needed.  The keys above
//    it and the lowest-index keys equal to it are chosen.  Empty clusters are
//    never chosen.  The block then writes every cluster's head mask, the
//    ascending list of clusters some head chose and their tile-slot bases
//    (wave w takes the slots w, w + G, ...).  A whole-cluster step writes,
//    in place of the list and the slot bases, each chosen cluster's first
//    row and (rows | head mask << 24), which the exact kernel cuts into
//    tiles, and the unit's exact row count, which the subcluster kernel
//    writes otherwise.  Grid (units), 64 G threads.
// ---------------------------------------------------------------------------
// s_waitcnt immediate of "vmcnt(0)" on gfx9-family chips (vmcnt in bits 3:0
// and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima)
constexpr int kWaitVmcnt0 = 0x0F70;

// bits 0..b set (b in [-1, 31])
__device__ inline uint32_t mask_upto(int b) { return b >= 31 ? ~0u : ((1u << (b + 1)) - 1u); }

// The selection of one wave: its keys sit in KPL slots (slot j of lane l:
// item 64 j + l; key 0: not valid), c_eff of the nvalid valid ones are to be
// taken, hb is the wave's LDS bins (256 + 64 ints).  On return the chosen
// are the keys above prefix on the bits of hi_mask, then the first kk (by
// index) of the cand keys equal to prefix there (hi_mask: decided bits,
// prefix: their values).  No barrier: a wave's LDS operations run in order.
template <int KPL>
__device__ inline void wave_select(const float (&scv)[KPL], const uint32_t (&key)[KPL], int c_eff, int nvalid, int* hb,
                                   int& kk, int& cand, uint32_t& prefix, uint32_t& hi_mask) {
  const int lane = threadIdx.x & 63;
  kk = c_eff;
  cand = nvalid;
  prefix = 0u;
  hi_mask = 0u;
  bool resolved = false;
  if (kk > 0 && kk < nvalid) {
    // One 256-bin histogram of the valid values over [lo, hi]: value x goes
    // to bin floor((hi - x) * 256 / (hi - lo)) (at most 255).  Rounded
    // subtraction and scaling are monotone, so a value in a lower bin is
    // strictly larger than every value in a higher bin: the chosen keys are
    // those of the bins before the one where the count reaches c, plus the
    // best of that boundary bin, ranked exactly by key and index when it
    // holds at most 64 keys.  A more crowded boundary bin falls back to the
    // radix select below.
    float vhi = -INFINITY, vlo = INFINITY;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      if (key[j] != 0u) {
        vhi = fmaxf(vhi, scv[j]);
        vlo = fminf(vlo, scv[j]);
      }
    }
    vhi = __uint_as_float(wave_reduce_uniform(
        __float_as_uint(vhi), [](uint32_t x, uint32_t y) { return __float_as_uint(fmaxf(__uint_as_float(x), __uint_as_float(y))); },
        __float_as_uint(-INFINITY)));
    vlo = __uint_as_float(wave_reduce_uniform(
        __float_as_uint(vlo), [](uint32_t x, uint32_t y) { return __float_as_uint(fminf(__uint_as_float(x), __uint_as_float(y))); },
        __float_as_uint(INFINITY)));
    const float inv = vhi > vlo ? 256.f / (vhi - vlo) : 0.f;
    int bin[KPL];
#pragma unroll
    for (int j = 0; j < KPL; ++j) bin[j] = key[j] != 0u ? (int)fminf(255.f, (vhi - scv[j]) * inv) : 256 + lane;
    int* hh = hb;
    *reinterpret_cast<int4*>(&hh[4 * lane]) = make_int4(0, 0, 0, 0);
    __asm__ volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < KPL; ++j) atomicAdd(&hh[bin[j]], 1);
    __asm__ volatile("" ::: "memory");
    // lane l holds bins 4l .. 4l+3 (bins in increasing order = values in
    // decreasing order); the keys before its bins come from the lanes before
    const int4 cv = *reinterpret_cast<const int4*>(&hh[4 * lane]);
    const int part = cv.x + cv.y + cv.z + cv.w;
    const int b0 = wave_incl_scan(part) - part, b1 = b0 + cv.x, b2 = b1 + cv.y, b3 = b2 + cv.z;
    int dsel = -1, dbef = 0, dcnt = 0;
    if (b0 < kk && kk <= b1) { dsel = 4 * lane; dbef = b0; dcnt = cv.x; }
    else if (b1 < kk && kk <= b2) { dsel = 4 * lane + 1; dbef = b1; dcnt = cv.y; }
    else if (b2 < kk && kk <= b3) { dsel = 4 * lane + 2; dbef = b2; dcnt = cv.z; }
    else if (b3 < kk && kk <= b3 + cv.w) { dsel = 4 * lane + 3; dbef = b3; dcnt = cv.w; }
    const unsigned long long fb = __ballot(dsel >= 0);
    const int src = fb ? __ffsll((long long)fb) - 1 : 0;
    const int bsel = __builtin_amdgcn_readlane(dsel, src);
    const int nbef = __builtin_amdgcn_readlane(dbef, src);
    const int nbin = __builtin_amdgcn_readlane(dcnt, src);
    if (fb != 0ull && nbin <= 64) {
      // the boundary bin's keys, one per lane, in the wave's LDS bins
      // (every lane has read its bins above; a wave's LDS operations run
      // in order)
      int nmine = 0;
#pragma unroll
      for (int j = 0; j < KPL; ++j) nmine += bin[j] == bsel;
      int pos = wave_incl_scan(nmine) - nmine;
      uint32_t* lk = reinterpret_cast<uint32_t*>(hh);
      int* li = hh + 64;
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        if (bin[j] == bsel) {
          lk[pos] = key[j];
          li[pos] = 64 * j + lane;
          ++pos;
        }
      }
      __asm__ volatile("" ::: "memory");
      const uint32_t myk = lane < nbin ? lk[lane] : 0u;
      const int myi = lane < nbin ? li[lane] : 0;
      int rk = 0;
      for (int t = 0; t < nbin; ++t) {
        const uint32_t kt = lk[t];
        const int it = li[t];
        rk += (int)((kt > myk) | ((kt == myk) & (it < myi)));
      }
      const int need = kk - nbef;  // keys still to be taken from the bin (>= 1)
      const unsigned long long cb = __ballot(lane < nbin && rk == need - 1);
      const uint32_t kcut = (uint32_t)__builtin_amdgcn_readlane((int)myk, __ffsll((long long)cb) - 1);
      const int n_gt = __popcll(__ballot(lane < nbin && myk > kcut));
      const int n_eq = __popcll(__ballot(lane < nbin && myk == kcut));
      prefix = kcut;
      hi_mask = ~0u;
      kk = need - n_gt;
      cand = n_eq;
      resolved = true;
    }
  }
  if (kk > 0 && !resolved) {
    uint32_t kor = 0u, kand = ~0u;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      kor |= key[j];
      kand &= key[j] != 0u ? key[j] : ~0u;
    }
    kor = wave_reduce_uniform(kor, [](uint32_t x, uint32_t y) { return x | y; }, 0u);
    kand = wave_reduce_uniform(kand, [](uint32_t x, uint32_t y) { return x & y; }, ~0u);
    const uint32_t varying = kor ^ kand;
    int* hh = hb;
    int top = 31;  // highest undecided bit
    while (cand > kk && top >= 0) {
      const uint32_t low = mask_upto(top);
      const uint32_t rem = varying & low;
      if (rem == 0u) {  // the candidates are all equal
        prefix |= kand & low;
        hi_mask |= low;
        break;
      }
      const int nb = 31 - __clz(rem);  // next varying bit; bits (nb, top] shared
      const uint32_t shared_bits = low & ~mask_upto(nb);
      prefix |= kand & shared_bits;
      hi_mask |= shared_bits;
      const int w = nb + 1 < 8 ? nb + 1 : 8;
      const int shift = nb - w + 1;
      const uint32_t dmask = (1u << w) - 1u;
      // histogram of the candidates' next digit; keys that are not
      // candidates go to the lane's spare bin, so there is no branch (a wave
      // executes its LDS operations in order)
      *reinterpret_cast<int4*>(&hh[4 * lane]) = make_int4(0, 0, 0, 0);
      __asm__ volatile("" ::: "memory");
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        const uint32_t kv = key[j];
        const bool m = kv != 0u && (kv & hi_mask) == prefix;
        atomicAdd(&hh[m ? (int)((kv >> shift) & dmask) : 256 + lane], 1);
      }
      __asm__ volatile("" ::: "memory");
      // lane l holds digits 252-4l .. 255-4l; candidates above its digits
      // come from the lanes before it
      const int4 cv = *reinterpret_cast<const int4*>(&hh[4 * (63 - lane)]);
      const int c0 = cv.x, c1 = cv.y, c2 = cv.z, c3 = cv.w;
      const int part = c0 + c1 + c2 + c3;
      const int a3 = wave_incl_scan(part) - part, a2 = a3 + c3, a1 = a2 + c2, a0 = a1 + c1;
      const int dbase = 4 * (63 - lane);
      int dsel = -1, dab = 0, dcnt = 0;
      if (a3 < kk && kk <= a2) { dsel = dbase + 3; dab = a3; dcnt = c3; }
      else if (a2 < kk && kk <= a1) { dsel = dbase + 2; dab = a2; dcnt = c2; }
      else if (a1 < kk && kk <= a0) { dsel = dbase + 1; dab = a1; dcnt = c1; }
      else if (a0 < kk && kk <= a0 + c0) { dsel = dbase; dab = a0; dcnt = c0; }
      const unsigned long long fb = __ballot(dsel >= 0);
      const int src = fb ? __ffsll((long long)fb) - 1 : 0;
      const int d = __builtin_amdgcn_readlane(dsel, src);
      prefix |= (uint32_t)d << shift;
      hi_mask |= dmask << shift;
      kk -= __builtin_amdgcn_readlane(dab, src);
      cand = __builtin_amdgcn_readlane(dcnt, src);
      top = shift - 1;
    }
  }
}

template <int G, int KPL>
__global__ __launch_bounds__(64 * G) void k_select_topc(DArgs a, BudgetArgs b) {
  constexpr int NSW = (KPL + G - 1) / G;  // tail slots per wave
  __shared__ int hist[G][256 + 64];       // 256 digit bins, then one spare bin per lane
  __shared__ uint32_t lmask[64 * KPL];     // per cluster: the heads that chose it
  __shared__ int slot_cnt[KPL], slot_tiles[KPL];
  __shared__ int wave_rows[G];  // whole-cluster step: rows of each wave's chosen clusters
  __shared__ float gfr[G][64 * KPL];  // shared selection: each head's mass fractions
  const int u = blockIdx.x, tid = threadIdx.x, lane = tid & 63, h = tid >> 6;
  const int want_raw = b.top_c[u / a.Hkv];
  // the scores need only the unit index: their loads go out with the unit
  // record's (entries past the unit's C are masked below)
  const int64_t cw = (int64_t)u * a.cstride;
  float scv[KPL];
#pragma unroll
  for (int j = 0; j < KPL; ++j) scv[j] = a.ws.cl_score[((int64_t)u * G + h) * a.cstride + min(64 * j + lane, a.cstride - 1)];
  // the tile-slot bounds of the clusters of this wave's tail slots (written
  // by the score kernel beside the scores)
  int bound[NSW], row0[NSW];
#pragma unroll
  for (int t = 0; t < NSW; ++t) {
    const int64_t cg = cw + min(64 * (h + G * t) + lane, a.cstride - 1);
    bound[t] = a.ws.cl_tiles[cg];
    row0[t] = a.whole ? a.ws.cl_row0[cg] : 0;
  }
  const mog_unit U = unit_scalar(a.L.units + u);
  const int C = U.C;
  if (tid == 0 && !a.whole) a.ws.unit_rows[u] = 0;  // the subcluster kernel adds to it
  // (cleared while the score loads are in flight; the heads OR their bits in
  // after the barrier)
  for (int i = tid; i < 64 * KPL; i += 64 * G) lmask[i] = 0u;
  __syncthreads();
  if (a.shared) {
    // one selection per KV head: the key of a cluster is the sum over the
    // heads of the head's estimated mass fraction 2^(score - L_h), L_h the
    // log2 of the head's total over its nonempty clusters; each head's
    // fractions go to its own LDS row, and after one barrier every wave adds
    // the rows in head order, so every wave holds the same keys
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < KPL; ++j)
      if (64 * j + lane < C) mx = fmaxf(mx, scv[j]);
    mx = wave_max(mx);
    float sm = 0.f;
#pragma unroll
    for (int j = 0; j < KPL; ++j) sm += (64 * j + lane < C && scv[j] != -INFINITY) ? exp2f(scv[j] - mx) : 0.f;
    const float lh = mx + log2f(wave_sum_uniform(sm));
    if (lane == 0) a.ws.cl_lse[(int64_t)u * G + h] = lh;
#pragma unroll
    for (int j = 0; j < KPL; ++j)
      gfr[h][64 * j + lane] = (64 * j + lane < C && scv[j] != -INFINITY) ? exp2f(scv[j] - lh) : 0.f;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      if (scv[j] != -INFINITY) {
        float t = gfr[0][64 * j + lane];
        for (int hh = 1; hh < G; ++hh) t += gfr[hh][64 * j + lane];
        scv[j] = t;
      }
    }
  }
  uint32_t key[KPL];
  int nvalid = 0;
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const bool in = 64 * j + lane < C && scv[j] != -INFINITY;
    key[j] = in ? float_key(scv[j]) : 0u;
    nvalid += in;
  }
  if (a.shared) {
    // the selection's histogram bins on log2 of the summed fractions (a
    // monotone map, clamped away from 0): the sums crowd near 0, where bins
    // over their linear range would put the c-th key among hundreds of tiny
    // ones.  The keys, which rank the boundary bin, stay the sums themselves.
#pragma unroll
    for (int j = 0; j < KPL; ++j)
      if (key[j] != 0u) scv[j] = log2f(fmaxf(scv[j], 1e-30f));
  }
  nvalid = (int)wave_reduce_uniform((uint32_t)nvalid, [](uint32_t x, uint32_t y) { return x + y; }, 0u);
  const int want = want_raw < 0 ? 0 : want_raw;
  const int c_eff = want < nvalid ? want : nvalid;
  // hi_mask: decided bits, prefix: their values; cand: keys matching the
  // prefix there; kk: how many of those are still to be taken
  int kk, cand;
  uint32_t prefix, hi_mask;
  wave_select<KPL>(scv, key, c_eff, nvalid, hist[h], kk, cand, prefix, hi_mask);
  // chosen: keys above the prefix on the decided bits, then the first kk
  // (by index) of the keys that match it there.  When every key matching
  // the prefix is taken (cand == kk) no tie ranks are needed.
  const int hq = U.kv_head * G + h;
  const int64_t row = (int64_t)U.seq * a.Hq + hq;
  const unsigned long long below = (1ull << lane) - 1ull;
  const bool all_ties = cand == kk;
  const bool want_sel = a.sel_c != nullptr || a.sel_s != nullptr;
  int ties = 0, rank0 = 0;
  if (all_ties && !want_sel) {
    // (the usual case: no tie to rank and nothing to report) lane j keeps
    // slot j's chosen lanes and writes them
    if (c_eff > 0) {
#pragma unroll
      for (int j = 0; j < KPL; ++j)
        if ((key[j] != 0u) & ((key[j] & hi_mask) >= prefix)) atomicOr(&lmask[64 * j + lane], 1u << h);
    }
  } else {
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const int i = 64 * j + lane;
    const uint32_t kd = key[j] & hi_mask;
    const bool valid = c_eff > 0 && key[j] != 0u;
    bool sel;
    if (all_ties) {
      sel = valid && kd >= prefix;
    } else {
      const bool tie = valid && kd == prefix;
      const unsigned long long tb = __ballot(tie);
      sel = valid && (kd > prefix || (tie && ties + __popcll(tb & below) < kk));
      ties += __popcll(tb);
    }
    const unsigned long long sb = __ballot(sel);
    if (sel) atomicOr(&lmask[i], 1u << h);
    if (want_sel) {
      const int rank = sel ? rank0 + __popcll(sb & below) : -1;
      if (i < C) {
        if (a.sel_s) a.ws.cl_rank[(cw + i) * G + h] = rank;  // read back only for sel_s
        if (sel && a.sel_c) a.sel_c[row * a.c_stride + rank] = i;
      }
      rank0 += __popcll(sb);
    }
  }
  }
  if (a.sel_c)
    for (int j = c_eff + lane; j < a.c_stride; j += 64) a.sel_c[row * a.c_stride + j] = -1;
  if (a.sel_s) {
    const int64_t base = row * a.c_stride * a.s_stride;
    for (int j = c_eff * a.s_stride + lane; j < a.c_stride * a.s_stride; j += 64) a.sel_s[base + j] = -1;
  }
  __syncthreads();
  // tail: cluster i = 64 j + lane.  A chosen cluster takes ceil(rows/32) + S
  // + folded rows tile slots, the most its chosen subclusters can make.
  // First the per-slot counts, then each slot's list positions and slot
  // bases from the counts of the slots before it (a whole-cluster step needs
  // the positions only).
  uint32_t um[NSW];
  int tcnt[NSW], tinc[NSW];
  int wrows = 0;
#pragma unroll
  for (int t = 0; t < NSW; ++t) {
    const int j = h + G * t;
    um[t] = 0u;
    tcnt[t] = 0;
    tinc[t] = 0;
    if (j < KPL) {
      um[t] = lmask[64 * j + lane];
      if (64 * j + lane >= C) um[t] = 0u;
      const int n = __popcll(__ballot(um[t] != 0u));
      int nt = 0;
      if (a.whole) {
        wrows += um[t] != 0u ? bound[t] : 0;
      } else {
        tcnt[t] = um[t] != 0u ? bound[t] : 0;
        tinc[t] = wave_incl_scan(tcnt[t]);  // the slot's total in lane 63; the bases below
        nt = __builtin_amdgcn_readlane(tinc[t], 63);
      }
      if (lane == 0) {
        slot_cnt[j] = n;
        slot_tiles[j] = nt;
      }
    }
  }
  if (a.whole) {
    wrows = (int)wave_reduce_uniform((uint32_t)wrows, [](uint32_t x, uint32_t y) { return x + y; }, 0u);
    if (lane == 0) wave_rows[h] = wrows;
  }
  __syncthreads();
  // every load of the kernel has landed by now; waiting for them here, before
  // the list and tile stores, keeps the uses below from waiting on those
  // stores (the vector memory counter counts stores too)
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  // exclusive prefixes of the slots' counts (lane l: slot l), read per slot
  const int sc_l = lane < KPL ? slot_cnt[lane] : 0, st_l = lane < KPL ? slot_tiles[lane] : 0;
  const int sc_inc = wave_incl_scan(sc_l), st_inc = wave_incl_scan(st_l);
  const int sc_exc = sc_inc - sc_l, st_exc = st_inc - st_l;
#pragma unroll
  for (int t = 0; t < NSW; ++t) {
    const int j = h + G * t;
    if (j < KPL) {
      const int i = 64 * j + lane;
      const int pos0 = __builtin_amdgcn_readlane(sc_exc, j);
      const int tb0 = __builtin_amdgcn_readlane(st_exc, j);
      if (i < C) a.ws.cl_mask[cw + i] = um[t];
      const bool ch = um[t] != 0u;
      const int pos = pos0 + __popcll(__ballot(ch) & below);
      const int tb = tb0 + tinc[t] - tcnt[t];
      if (ch) {
        if (a.whole) {
          a.ws.ch_row0[cw + pos] = row0[t];
          a.ws.ch_nm[cw + pos] = (uint32_t)bound[t] | um[t] << 24;
        } else {
          a.ws.cl_list[cw + pos] = i;
          a.ws.ch_tbase[cw + pos] = tb;
        }
      }
    }
  }
  const int total = __builtin_amdgcn_readlane(sc_inc, 63);
  if (h == 0 && lane == 0) {
    a.ws.n_chosen[u] = total;
    if (a.whole) {
      int rows = 0;
      for (int w = 0; w < G; ++w) rows += wave_rows[w];
      a.ws.unit_rows[u] = rows;
    }
  }
}

// ---------------------------------------------------------------------------
// 3. Subclusters and residual, one block per chosen cluster: the steps
//    with shared selection or the feature-map residual (the others run the
//    one-wave-per-cluster kernel of 3b).  Grid (units,
//    n_rest + nb_chosen); blocks are numbered x (record slot order) as
//    below, but the rest blocks come
//    first in the grid, so the dispatcher starts them together with the
//    chosen-cluster blocks instead of after every chosen slot (most of which
//    find no cluster and leave):
//    * block x < nb_chosen takes the x-th chosen cluster of its unit (from
//      the ascending list the top-c pass wrote), if any: scores its S
//      subclusters for every head (one batch of row loads per wave), picks
//      the top-s of each head that chose the cluster, writes the subcluster
//      head masks, adds the rows read exactly to the unit's count, writes
//      the cluster's exact tiles (runs of chosen subclusters cut into tiles
//      of <= 32 rows) from its slot base, and accumulates the residual
//      terms of the subclusters a choosing head left out;
//    * block nb_chosen + y (feature-map residual only; the Gaussian
//      residual of whole clusters left out runs in blocks at the end of the
//      exact launch) covers clusters [R y, R y + R), R =
//      kRestClustersPerBlock: the residual terms of
//      every head that left a cluster out.
//    Every block writes one residual record per head: the chosen clusters'
//    in slots [0, n_chosen), the rest after them.
// ---------------------------------------------------------------------------
// Feature-map residual: the weight (log2 of the estimated mass) of a group
// whose feature sums z the wave holds (z[k]: feature lane + 64 k), for head h:
// log2(sum_i e_h[i] z[i]) + max_h, with e_h = 2^(fq_h - max_h) in LDS.
__device__ inline float fm_weight(const float (&z)[4], const float* e_h, float base_h, int FM) {
  const int lane = threadIdx.x & 63;
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (64 * k < FM) s += e_h[lane + 64 * k] * z[k];
  s = wave_sum_uniform(s);
  return s > 0.f ? base_h + log2f(s) : -INFINITY;
}

__device__ inline void load_fz(const float* row, int FM, float (&z)[4]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 0; k < 4; ++k) z[k] = 64 * k < FM ? row[lane + 64 * k] : 0.f;
}

// Gaussian residual of clusters [R y, R y + R) of unit u (R = 4 RCW): every
// head that left a cluster out adds its term 2^score v-bar.  A wave takes RCW
// clusters, in batches whose loads are all issued before any is used: the
// whole share at once where its registers stay within 128 per lane (clusters past C re-read the last one and are
// skipped; an empty cluster scores -inf for every head, so its size is not
// needed).
template <int D, int G, int RCW>
__device__ inline void rest_clusters(const DArgs& a, int u, int C, int64_t cl_base, int y, float (&rm)[G],
                                     float (&rl)[G], float (&ro)[G][D / 64]) {
  constexpr int VPL = D / 64;
  constexpr int RB = (VPL + G + 1) * RCW <= 128 ? RCW : RCW / 2;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t cw = (int64_t)u * a.cstride;
  const uint32_t all = (1u << G) - 1u;
  const int g0 = (y * 4 + wave) * RCW;
#pragma unroll
  for (int k0 = 0; k0 < RCW; k0 += RB) {
    uint32_t mask[RB];
    float vb[RB][VPL], sc[RB][G];
#pragma unroll
    for (int k = 0; k < RB; ++k) {
      const int g = min(g0 + k0 + k, C - 1);
      mask[k] = a.ws.cl_mask[cw + g];
      load_floats<VPL>(a.L.cl_vbar + (cl_base + g) * D + lane * VPL, vb[k]);
#pragma unroll
      for (int h = 0; h < G; ++h) sc[k][h] = a.ws.cl_score[((int64_t)u * G + h) * a.cstride + g];
    }
#pragma unroll
    for (int k = 0; k < RB; ++k) {
      const bool in_c = g0 + k0 + k < C;
      const uint32_t unchosen = in_c && sc[k][0] != -INFINITY ? (all & ~mask[k]) : 0u;
#pragma unroll
      for (int h = 0; h < G; ++h)
        if ((unchosen >> h) & 1u) add_group<VPL>(rm[h], rl[h], ro[h], sc[k][h], vb[k]);
    }
  }
}

// A wave's per-head states into rows wave * G + h of st (stride D + kPartPad),
// as write_block_record reads them.
template <int D, int G>
__device__ inline void store_wave_states(float* st, const float (&rm)[G], const float (&rl)[G],
                                         const float (&ro)[G][D / 64]) {
  constexpr int VPL = D / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float* r = st + (wave * G + h) * (D + kPartPad);
#pragma unroll
    for (int e = 0; e < VPL; ++e) r[lane * VPL + e] = ro[h][e];
    if (lane == 0) {
      r[D] = rm[h];
      r[D + 1] = rl[h];
    }
  }
}

// The feature table of unit u's G heads, for the feature-map residual:
// fe[256 h + i] = 2^(fq[h][i] - max_h) and fbase[h] = max_h - log2(m) / 2
// (waves h, h + 4, ... of the block; visible after the caller's barrier).
template <int G>
__device__ inline void fm_table(const DArgs& a, int u, float* fe, float* fbase) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int FM = a.L.fm_dim;
  for (int h = wave; h < G; h += 4) {
    const float* fqh = a.ws.fq + ((int64_t)u * G + h) * FM;
    float v[4], mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[k] = 64 * k < FM ? fqh[lane + 64 * k] : -INFINITY;
      mx = fmaxf(mx, v[k]);
    }
    mx = wave_max(mx);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (64 * k < FM) fe[256 * h + lane + 64 * k] = exp2f(v[k] - mx);
    if (lane == 0) fbase[h] = mx - 0.5f * log2f((float)FM);
  }
}

// Feature-map residual of clusters [R y, R y + R) of unit u (R =
// kRestClustersPerBlock, R / 4 per wave): every head that left a cluster out
// adds its term with the cluster's feature-map mass estimate.  A wave takes
// NB clusters at a time, their loads issued before any is used (clusters past
// C re-read the last one and are skipped); the NB G dot products of feature
// sums with the heads' feature exponentials (held in registers) are summed
// over the lanes by one reduce-scatter, each lane takes the log of its sum,
// and every weight is then read from the lane that holds it.
template <int D, int G, int NB>
__device__ inline void rest_clusters_fm(const DArgs& a, int u, const mog_unit& U, int y, const float* fe,
                                        const float* fbase, float (&rm)[G], float (&rl)[G],
                                        float (&ro)[G][D / 64]) {
  constexpr int VPL = D / 64;
  constexpr int RCW = kRestClustersPerBlock / 4;
  constexpr int V = NB * G;
  static_assert(RCW % NB == 0 && V <= 64, "batches of whole clusters, one reduce-scatter each");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int C = U.C, S = U.S, FM = a.L.fm_dim;
  const int64_t cw = (int64_t)u * a.cstride;
  const int32_t* off = a.L.sub_off + U.off_base;
  const uint32_t all = (1u << G) - 1u;
  float e[G][4];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int k = 0; k < 4; ++k) e[h][k] = 64 * k < FM ? fe[256 * h + lane + 64 * k] : 0.f;
  const float base = fbase[rs_index<V>(lane) % G];  // (of the head whose sum the lane receives)
  const int g0 = y * kRestClustersPerBlock + wave * RCW;
#pragma unroll 1
  for (int k0 = 0; k0 < RCW; k0 += NB) {
    uint32_t mask[NB];
    int n_g[NB];
    float vb[NB][VPL], z[NB][4];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int g = min(g0 + k0 + k, C - 1);
      mask[k] = a.ws.cl_mask[cw + g];
      n_g[k] = off[(g + 1) * S] - off[g * S] + (a.L.fold_cap ? a.L.cl_fold[U.cl_base + g] : 0);
      load_floats<VPL>(a.L.cl_vbar + (U.cl_base + g) * D + lane * VPL, vb[k]);
      load_fz(a.L.cl_fz + (U.cl_base + g) * FM, FM, z[k]);
    }
    float part[V];
#pragma unroll
    for (int k = 0; k < NB; ++k)
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float t = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) t += e[h][j] * z[k][j];
        part[k * G + h] = t;
      }
    const float t = wave_reduce_scatter<V>(part);
    const float wl = t > 0.f ? base + log2f(t) : -INFINITY;
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const uint32_t unchosen = (g0 + k0 + k < C && n_g[k] > 0) ? (all & ~mask[k]) : 0u;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        if (!((unchosen >> h) & 1u)) continue;
        const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), rs_lane<V>(k * G + h)));
        if (w != -INFINITY) add_group<VPL>(rm[h], rl[h], ro[h], w, vb[k]);
      }
    }
  }
}

// Exact tiles of a chosen cluster (lane i: subcluster i, rows [st, en) of
// the unit's middle rows, head mask m; m = 0 for a subcluster no head
// chose): a run is a maximal sequence of chosen nonempty subclusters with
// one head mask whose rows are contiguous; each run is cut into tiles of
// <= 32 rows, written run after run to ctiles.  Returns the tile count
// (wave-uniform).  Called by a whole wave.
__device__ inline int write_run_tiles(TileRec* ctiles, int64_t row_base, int64_t row_elems, int st, int en,
                                      uint32_t m) {
  const int lane = threadIdx.x & 63;
  const bool live = m != 0u && en > st;
  const unsigned long long below = (1ull << lane) - 1ull;
  const unsigned long long lb = __ballot(live);
  const unsigned long long lbb = lb & below;
  const int prv = lbb ? 63 - __clzll((long long)lbb) : 0;
  const uint32_t m_prv = (uint32_t)__shfl((int)m, prv, 64);
  const int en_prv = __shfl(en, prv, 64);
  const bool head = live && !(lbb != 0ull && m_prv == m && en_prv == st);
  const unsigned long long hb = __ballot(head);
  const unsigned long long later = hb & ~(below | (1ull << lane));
  const int nxt = later ? __ffsll((long long)later) - 1 : 64;
  const unsigned long long in_run = lb & (nxt >= 64 ? ~0ull : ((1ull << nxt) - 1ull));
  const int last = in_run ? 63 - __clzll((long long)in_run) : 0;
  const int run_en = __shfl(en, last, 64);
  const int ntl = head ? (run_en - st + 31) / 32 : 0;
  const int incl = wave_incl_scan(ntl);
  const int n_tiles = __builtin_amdgcn_readlane(incl, 63);
  // the tiles are written by every lane (tiles t = lane, lane + 64, ...):
  // tile t belongs to the run whose head lane j has tile range
  // [incl_j - ntl_j, incl_j); the runs are visited in a wave-uniform loop
  const int tfirst = incl - ntl;
  for (int t0 = 0; t0 < n_tiles; t0 += 64) {
    const int t = t0 + lane;
    int64_t toff = 0;
    int tn = 0;
    uint32_t tm = 0u;
    for (unsigned long long bits = hb; bits; bits &= bits - 1ull) {
      const int j = __ffsll((long long)bits) - 1;
      const int ts = __builtin_amdgcn_readlane(tfirst, j);
      const int tc = __builtin_amdgcn_readlane(ntl, j);
      if (t >= ts && t < ts + tc) {
        const int r = __builtin_amdgcn_readlane(st, j) + 32 * (t - ts);
        toff = (row_base + r) * row_elems;
        tn = min(32, __builtin_amdgcn_readlane(run_en, j) - r);
        tm = (uint32_t)__builtin_amdgcn_readlane((int)m, j);
      }
    }
    if (t < n_tiles) ctiles[t] = TileRec{toff, tn, tm};
  }
  return n_tiles;
}

template <int D, int G>
__global__ __launch_bounds__(256) void k_subclusters(DArgs a, BudgetArgs b, int nb_chosen, int n_rest_blocks) {
  constexpr int EPL = D / 32;
  constexpr int VPL = D / 64;
  constexpr int RS = D + kPartPad;
  constexpr int SR = kDecodeSubRows;
  constexpr int RPW = SR / 4;   // subcluster rows per wave
  static_assert(SR * G <= 256, "one thread per (subcluster, head) score");
  __shared__ float st[4][G][D + kPartPad];  // wave states, as write_block_record reads them
  __shared__ float lds_sc[SR][G];
  __shared__ float lds_gs[SR];  // shared selection: summed mass fractions
  __shared__ uint32_t lds_sm[SR];
  __shared__ int lds_cnt[SR];   // reordered rows of each subcluster
  __shared__ int lds_fcnt[SR];  // folded rows of each subcluster
  __shared__ int lds_off[SR + 1];
  __shared__ int sh[16];
  __shared__ float lds_fe[G][256];  // feature-map residual: 2^(fq - max) per head
  __shared__ float lds_fbase[G];    // and max - log2(m) / 2
  const int u = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int s_keep_raw = b.top_s[u / a.Hkv];  // issued with the unit record
  const int64_t cw = (int64_t)u * a.cstride;  // the unit's per-cluster workspace entries
  // the x-th chosen cluster needs only the unit index: its loads go out with
  // the unit record's
  const int x = (int)blockIdx.y < n_rest_blocks ? nb_chosen + (int)blockIdx.y : (int)blockIdx.y - n_rest_blocks;
  const int n_ch_raw = a.ws.n_chosen[u];
  int g_x = 0, tb_x = 0;
  if (x < nb_chosen) {
    g_x = a.ws.cl_list[cw + x];
    tb_x = a.ws.ch_tbase[cw + x];
  }
  const mog_unit U = unit_scalar(a.L.units + u);
  const int S = U.S, C = U.C, n_ch = uni(n_ch_raw);
  // the unit's records: one per chosen cluster, then one per rest block;
  // slots past them (no such cluster in this unit) leave at once
  if (x < nb_chosen ? x >= n_ch : (x - nb_chosen) * kRestClustersPerBlock >= C) return;
  const uint32_t all = (1u << G) - 1u;
  const bool fmr = a.residual == 2;
  const int FM = a.L.fm_dim;
  if (fmr) fm_table<G>(a, u, &lds_fe[0][0], lds_fbase);  // (read after the next barrier)
  const int32_t* off = a.L.sub_off + U.off_base;
  float rm[G], rl[G], ro[G][VPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    rm[h] = -INFINITY;
    rl[h] = 0.f;
#pragma unroll
    for (int e = 0; e < VPL; ++e) ro[h][e] = 0.f;
  }
  float* dst = a.ws.res_part + ((int64_t)u * a.nb_res + (x < nb_chosen ? x : n_ch + x - nb_chosen)) * G * RS;

  if (x < nb_chosen) {
    // -------- the x-th chosen cluster ---------------------------------------
    // (x < nb_chosen <= the largest C, so the list entries are in range)
    const int g = uni(g_x);
    {
      const int64_t cg = cw + g;
      const int64_t sg0 = U.sub_base + (int64_t)g * S;
      const uint32_t mask = a.ws.cl_mask[cg];
      // a budget of S or more subclusters per chosen cluster reads every
      // nonempty one: no scores, no ranking, nothing left out of the cluster
      const bool whole = s_keep_raw >= S;
      float coef[G][EPL];
      // scores: wave w takes rows w, w+4, ...
      float xr[RPW][EPL];
      if (!whole) {
        const float* qb = a.q + ((int64_t)U.seq * a.Hq + (int64_t)U.kv_head * G) * D;
        score_coefs<D, G>(a, qb, coef);
#pragma unroll
        for (int k = 0; k < RPW; ++k) {
          const int i = min(wave + 4 * k, S - 1);
          load_floats<EPL>(a.L.sub_ms + (sg0 + i) * (2 * D) + lane * EPL, xr[k]);
        }
      }
      // subcluster bounds: thread i < S keeps subcluster i's for the tiles,
      // and every wave the sizes of its own rows for the count term
      {
        const int i = min(tid, S - 1);
        const int o0 = off[g * S + i], o1 = off[g * S + i + 1];
        const int fc = a.L.fold_cap ? a.L.sub_fold[sg0 + i] : 0;
        if (tid < S) {
          lds_cnt[tid] = o1 - o0;
          lds_fcnt[tid] = fc;
          lds_off[tid] = o0;
        }
        if (tid == S - 1) lds_off[S] = o1;
      }
      // the value means of the same rows, for the residual below: issued
      // with the score rows where the registers allow it (at G >= 2 the
      // occupancy is set by the other path), else after the ranking
      constexpr bool kEarlyVb = G >= 2;
      float vb[RPW][VPL];
      if (kEarlyVb && a.residual && !whole) {
#pragma unroll
        for (int k = 0; k < RPW; ++k)
          load_floats<VPL>(a.L.sub_vbar + (sg0 + min(wave + 4 * k, S - 1)) * D + lane * VPL, vb[k]);
      }
      // (the scheduler would otherwise sink these loads to their use)
      if constexpr (kEarlyVb) __builtin_amdgcn_sched_barrier(0);
      const int s_keep = s_keep_raw < 0 ? 0 : s_keep_raw;
      const int ti = tid / G, th = tid % G;
      bool tsel = false;
      if (whole) {
        __syncthreads();  // the bounds
        if (tid < SR) lds_sm[tid] = (tid < S && lds_cnt[tid] + lds_fcnt[tid] > 0) ? mask : 0u;
        __syncthreads();
        tsel = tid < SR * G && ((lds_sm[ti] >> th) & 1u);
      } else {
      int rcnt[RPW];
#pragma unroll
      for (int k = 0; k < RPW; ++k) {
        const int i = min(wave + 4 * k, S - 1);
        rcnt[k] = off[g * S + i + 1] - off[g * S + i] + (a.L.fold_cap ? a.L.sub_fold[sg0 + i] : 0);
      }
      if (tid < SR) lds_sm[tid] = 0u;
      // full scores (count term added; -inf for an empty subcluster and for
      // the rows past S, so the ranking below runs over all SR rows): the
      // wave's RPW x G partial dot products are summed over the lanes by one
      // reduce-scatter, after which one lane holds each (row, head) score
      {
        float part[RPW * G];
#pragma unroll
        for (int k = 0; k < RPW; ++k) {
#pragma unroll
          for (int h = 0; h < G; ++h) {
            float t = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) t += coef[h][e] * xr[k][e];
            part[k * G + h] = t;
          }
        }
        const float t = wave_reduce_scatter<RPW * G>(part);
        if (rs_owner<RPW * G>(lane)) {
          const int j = rs_index<RPW * G>(lane), k = j / G, h = j % G, i = wave + 4 * k;
          int cnt = 0;
#pragma unroll
          for (int kk = 0; kk < RPW; ++kk) cnt = kk == k ? rcnt[kk] : cnt;
          lds_sc[i][h] = (i < S && cnt > 0) ? t + log2f((float)cnt) : -INFINITY;
        }
      }
      __syncthreads();
      if (a.shared) {
        // one selection per KV head: a subcluster's key is the sum over the
        // heads of 2^(score - L_h), L_h the head's log2 total over clusters
        if (tid < SR) {
          float gsv = 0.f;
          bool any = false;
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const float v = lds_sc[tid][h];
            any |= v != -INFINITY;
            gsv += v != -INFINITY ? exp2f(v - a.ws.cl_lse[(int64_t)u * G + h]) : 0.f;
          }
          lds_gs[tid] = any ? gsv : -INFINITY;
        }
        __syncthreads();
      }
      // top-s of every choosing head at once: thread (i, h) ranks subcluster
      // i's score among head h's, or the shared keys (ties to the lower index)
      if (tid < SR * G) {
        const float my = a.shared ? lds_gs[ti] : lds_sc[ti][th];
        float osc[SR];
#pragma unroll
        for (int j = 0; j < SR; ++j) osc[j] = a.shared ? lds_gs[j] : lds_sc[j][th];
        // branch-free count (bitwise, not short-circuit, operators)
        int rank = 0;
#pragma unroll
        for (int j = 0; j < SR; ++j)
          rank += (int)((osc[j] != -INFINITY) & ((osc[j] > my) | ((osc[j] == my) & (j < ti))));
        tsel = my != -INFINITY && ((mask >> th) & 1u) && rank < s_keep;
        if (tsel) atomicOr(&lds_sm[ti], 1u << th);
      }
      __syncthreads();
      // (G = 1: issued now, so their registers are not held through the
      // ranking)
      if (!kEarlyVb && a.residual) {
#pragma unroll
        for (int k = 0; k < RPW; ++k)
          load_floats<VPL>(a.L.sub_vbar + (sg0 + min(wave + 4 * k, S - 1)) * D + lane * VPL, vb[k]);
      }
      }  // (not whole)
      if (a.sel_s && tid < SR * G && ((mask >> th) & 1u)) {
        // selection output: the head's chosen subclusters in index order,
        // under the cluster's rank for the head, then -1
        const int rch = a.ws.cl_rank[cg * G + th];
        const int hq = U.kv_head * G + th;
        const int64_t base = (((int64_t)U.seq * a.Hq + hq) * a.c_stride + rch) * a.s_stride;
        int before = 0, all_h = 0;
        for (int j = 0; j < SR; ++j) {
          const int bit = (int)((lds_sm[j] >> th) & 1u);
          before += j < ti ? bit : 0;
          all_h += bit;
        }
        if (tsel) a.sel_s[base + before] = ti;
        if (ti == 0)
          for (int j = all_h; j < a.s_stride; ++j) a.sel_s[base + j] = -1;
      }
      const int my_cnt = lane < S ? lds_cnt[lane] : 0;
      const int my_fcnt = lane < S ? lds_fcnt[lane] : 0;
      if (wave == 0) {
        const uint32_t rows = (lane < S && lds_sm[lane]) ? (uint32_t)(my_cnt + my_fcnt) : 0u;
        const int rsum = (int)wave_reduce_uniform(rows, [](uint32_t p, uint32_t q) { return p + q; }, 0u);
        if (lane == 0) atomicAdd(&a.ws.unit_rows[u], rsum);
        // exact tiles of the cluster, from its slot base
        const int st = lane < S ? lds_off[lane] : 0;
        const int en = lane < S ? lds_off[lane] + lds_cnt[lane] : 0;
        const uint32_t m = lane < S ? lds_sm[lane] : 0u;
        const unsigned long long below = (1ull << lane) - 1ull;
        TileRec* ctiles = a.ws.tiles + tile_unit_base(U.row_base, U.cl_base, u, a.L.fold_cap) + uni(tb_x);
        const int n_tiles = write_run_tiles(ctiles, U.row_base, a.L_head_dim, st, en, m);
        int n_all = n_tiles;
        // folded rows of the chosen subclusters, after the reordered ones:
        // the unit's fold rows are scanned 64 at a time (lane l: row f0 + l);
        // a tile is a run of consecutive fold rows with one head mask, cut at
        // every 32nd row
        if (__ballot(lane < S && m != 0u && my_fcnt > 0)) {
          const int nf = U.n_fold;
          const int32_t* fs = a.L.fold_sub + (int64_t)u * a.L.fold_cap;
          const int64_t frow = a.L.fold_row0 + (int64_t)u * a.L.fold_cap;
          TileRec* ft = ctiles + n_tiles;
          int nt = 0;
          for (int f0 = 0; f0 < nf; f0 += 64) {
            const int f = f0 + lane;
            const int li = (f < nf ? fs[f] : -1) - g * S;
            const uint32_t fm = (li >= 0 && li < S) ? lds_sm[li] : 0u;
            const uint32_t fm_prv = (uint32_t)__shfl_up((int)fm, 1, 64);
            const bool cont = fm != 0u && (lane & 31) != 0 && fm_prv == fm;
            const bool fhead = fm != 0u && !cont;
            const unsigned long long fhb = __ballot(fhead);
            const unsigned long long after = __ballot(!cont) & ~((2ull << lane) - 1ull);
            const int fend = after ? __ffsll((long long)after) - 1 : 64;
            if (fhead) ft[nt + __popcll(fhb & below)] = TileRec{(frow + f) * (int64_t)a.L_head_dim, fend - lane, fm};
            nt += __popcll(fhb);
          }
          n_all += nt;
        }
        if (lane == 0) a.ws.ch_ntiles[cw + x] = n_all;
      }
      // residual of the subclusters a choosing head left out: wave w takes
      // subclusters w, w+4, ...
      if (a.residual) {
        uint32_t need[RPW];
#pragma unroll
        for (int k = 0; k < RPW; ++k) {
          const int i = wave + 4 * k;
          need[k] = 0u;
          if (i < S && lds_cnt[i] + lds_fcnt[i] > 0) need[k] = mask & ~lds_sm[i];
        }
        if (fmr) {
          // the feature-map estimate of each left-out subcluster's mass (one
          // row at a time: this mode keeps the Gaussian path's registers)
#pragma unroll
          for (int k = 0; k < RPW; ++k) {
            if (!need[k]) continue;
            float z[4];
            load_fz(a.L.sub_fz + (sg0 + wave + 4 * k) * FM, FM, z);
#pragma unroll
            for (int h = 0; h < G; ++h) {
              if (!((need[k] >> h) & 1u)) continue;
              const float w = fm_weight(z, lds_fe[h], lds_fbase[h], FM);
              if (w != -INFINITY) add_group<VPL>(rm[h], rl[h], ro[h], w, vb[k]);
            }
          }
        } else {
#pragma unroll
          for (int k = 0; k < RPW; ++k) {
            if (!need[k]) continue;
            const int i = wave + 4 * k;
#pragma unroll
            for (int h = 0; h < G; ++h)
              if ((need[k] >> h) & 1u) add_group<VPL>(rm[h], rl[h], ro[h], lds_sc[i][h], vb[k]);
          }
        }
      }
    }
  } else {
    // -------- residual of clusters left out (feature-map residual) -----------
    const int y = x - nb_chosen;
    if (fmr && a.residual) {
      __syncthreads();  // the feature table
      rest_clusters_fm<D, G, 2>(a, u, U, y, &lds_fe[0][0], lds_fbase, rm, rl, ro);  // (this kernel's registers)
    }
  }

  store_wave_states<D, G>(&st[0][0][0], rm, rl, ro);
  __syncthreads();
  write_block_record<D, G>(&st[0][0][0], dst);
}

// ---------------------------------------------------------------------------
// 3b. Subclusters, one wave per chosen cluster (selection per query head,
//     Gaussian residual or none; folded rows count in their subcluster's
//     size and are read as tiles after the cluster's runs): wave w of block (u, y)
//     takes the unit's chosen cluster x = 4 y + w and does alone, with no
//     barrier, what a block of the kernel above does for it:
//     * the S subcluster scores (count term included) in chunks of
//       kSubChunk rows: each chunk's G x kSubChunk dot products are summed
//       over the lanes by one reduce-scatter while the next chunk's rows
//       load, and the scores go to the wave's LDS row, head-major;
//     * the top-s of each head that chose the cluster, by rank counts over
//       that row (ties to the lower index), lane i holding subcluster i's
//       head mask;
//     * the selection output, the rows read exactly added to the unit's
//       count, and the cluster's exact tiles from its slot base;
//     * the residual record of the subclusters a choosing head left out.
//     A chosen cluster's work is thus one wave's chain, and many more
//     chosen clusters are in flight per compute unit than with a block each.
// ---------------------------------------------------------------------------
constexpr int kSubChunk = 8;

// The work of one wave on the x-th chosen cluster g of unit u (slot base
// tbx, head mask `mask`): what 3b describes after the cluster is known.
// lsc is the wave's LDS row of scores.
template <int D, int G>
__device__ inline void sub_wave_cluster(const DArgs& a, int u, int x, const mog_unit& U, int g, int tbx,
                                        uint32_t mask, int s_keep_raw, float4 (&lsc)[G][kDecodeSubRows / 4],
                                        const float* fe, const float* fbase) {
  constexpr int EPL = D / 32;
  constexpr int VPL = D / 64;
  constexpr int RS = D + kPartPad;
  constexpr int SR = kDecodeSubRows;
  constexpr int RC = kSubChunk;
  constexpr int NCH = SR / RC;
  static_assert(SR % RC == 0 && SR % 4 == 0, "whole chunks, float4 rows");
  static_assert(RC * G <= 64, "one lane per (row, head) sum of a chunk");
  const int lane = threadIdx.x & 63;
  const int64_t cw = (int64_t)u * a.cstride;
  const int S = U.S;
  const int64_t cg = cw + g;
  const int64_t sg0 = U.sub_base + (int64_t)g * S;
  // subcluster bounds: lane i <= S holds offset i
  const int32_t* off = a.L.sub_off + U.off_base + (int64_t)g * S;
  const int o_i = off[min(lane, S)];
  const int o_n = __shfl_down(o_i, 1, 64);
  const int cnt = lane < S ? o_n - o_i : 0;
  // folded rows of each subcluster (incremental decode): they count in the
  // group's size and are read as tiles of their own
  const int fcnt = (a.L.fold_cap && lane < S) ? a.L.sub_fold[sg0 + lane] : 0;
  const int ncnt = cnt + fcnt;
  const int s_keep = s_keep_raw < 0 ? 0 : s_keep_raw;
  float* sc = reinterpret_cast<float*>(&lsc[0][0]);  // sc[h * SR + i]
  uint32_t sm = 0u;  // lane i: the heads that chose subcluster i
  // every subcluster's value mean (the lane's VPL bf16 elements, packed),
  // for the residual: loaded with the score rows, unpacked where used (a
  // load whose result is used inside a branch waits there)
  uint32_t vraw[SR];
  if (s_keep >= S) {
    // a budget of S or more reads every nonempty subcluster of the cluster
    sm = (lane < S && ncnt > 0) ? mask : 0u;
  } else {
    // every row of the cluster in one round trip: the bf16 pairs stay packed
    // (EPL / 2 registers a row) until their chunk is scored
    uint32_t raw[SR][EPL / 2];
#pragma unroll
    for (int k = 0; k < SR; ++k) load_bf16_pairs<EPL>(a.L.sub_ms + (sg0 + min(k, S - 1)) * (2 * D) + lane * EPL, raw[k]);
    float coef[G][EPL];
    score_coefs<D, G>(a, a.q + ((int64_t)U.seq * a.Hq + (int64_t)U.kv_head * G) * D, coef);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      float part[RC * G];
#pragma unroll
      for (int k = 0; k < RC; ++k) {
        float xk[EPL];
#pragma unroll
        for (int e = 0; e < EPL / 2; ++e) {
          xk[2 * e] = bf16_lo(raw[c * RC + k][e]);
          xk[2 * e + 1] = bf16_hi(raw[c * RC + k][e]);
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float t = 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) t += coef[h][e] * xk[e];
          part[k * G + h] = t;
        }
      }
      const float t = wave_reduce_scatter<RC * G>(part);
      const int j = rs_index<RC * G>(lane), i = c * RC + j / G, h = j % G;
      const int ci = __shfl(ncnt, i & 63, 64);
      // (rows past S score -inf, so every row of the LDS row is written)
      if (rs_owner<RC * G>(lane)) sc[h * SR + i] = (i < S && ci > 0) ? t + log2f((float)ci) : -INFINITY;
    }
    // (issued once the rows' registers are free: the launch then keeps
    // five waves a SIMD resident at one head per KV head)
    if (a.residual) {
#pragma unroll
      for (int k = 0; k < SR; ++k) vraw[k] = load_bf16_bits<VPL>(a.L.sub_vbar + (sg0 + min(k, S - 1)) * D + lane * VPL);
    }
    __asm__ volatile("" ::: "memory");  // (a wave's LDS operations run in order)
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (!((mask >> h) & 1u)) continue;
      const float my = lane < SR ? sc[h * SR + lane] : -INFINITY;
      // branch-free rank count (bitwise, not short-circuit, operators)
      int rank = 0;
#pragma unroll
      for (int j4 = 0; j4 < SR / 4; ++j4) {
        const float4 o4 = lsc[h][j4];
        const float ov[4] = {o4.x, o4.y, o4.z, o4.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int j = 4 * j4 + q;
          rank += (int)((ov[q] != -INFINITY) & ((ov[q] > my) | ((ov[q] == my) & (j < lane))));
        }
      }
      if (lane < S && my != -INFINITY && rank < s_keep) sm |= 1u << h;
    }
  }
  const unsigned long long below = (1ull << lane) - 1ull;
  if (a.sel_s) {
    // the head's chosen subclusters in index order, under the cluster's rank
    // for the head, then -1
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (!((mask >> h) & 1u)) continue;
      const bool mine = (sm >> h) & 1u;
      const unsigned long long bits = __ballot(mine);
      // (one head: the cluster's rank is its list position, which the fused
      // launch knows before the unit's ranks are written)
      const int rch = G == 1 ? x : a.ws.cl_rank[cg * G + h];
      const int64_t base = (((int64_t)U.seq * a.Hq + U.kv_head * G + h) * a.c_stride + rch) * a.s_stride;
      if (mine) a.sel_s[base + __popcll(bits & below)] = lane;
      for (int j = __popcll(bits) + lane; j < a.s_stride; j += 64) a.sel_s[base + j] = -1;
    }
  }
  // the residual first: its value-mean loads are then the wave's only
  // outstanding memory operations (the vector memory counter also counts
  // stores, so a wait issued after the tile stores and the row-count atomic
  // below would wait for them too)
  if (a.residual) {
    // residual of the subclusters a choosing head left out: every lane holds
    // VPL elements of each such subcluster's value mean
    const uint32_t need = (lane < S && ncnt > 0) ? (mask & ~sm) : 0u;
    const unsigned long long any_need = __ballot(need != 0u);
    float rm[G], rl[G], ro[G][VPL];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      rm[h] = -INFINITY;
      rl[h] = 0.f;
#pragma unroll
      for (int e = 0; e < VPL; ++e) ro[h][e] = 0.f;
    }
    if (a.residual == 2) {
      // the feature-map estimate of each left-out subcluster's mass (the
      // unit's feature table fe / fbase in LDS): ZB subclusters' feature sums
      // loaded at a time, unconditionally; their ZB G dot products with the
      // heads' features (held in registers) summed over the lanes by one
      // reduce-scatter, each lane taking the log of the sum it receives, and
      // every weight read from the lane that holds it
      constexpr int ZB = G <= 2 ? 8 : 4;
      constexpr int V = ZB * G;
      static_assert(SR % ZB == 0 && V <= 64, "whole batches, one reduce-scatter each");
      const int FM = a.L.fm_dim;
      float e[G][4];
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int j = 0; j < 4; ++j) e[h][j] = 64 * j < FM ? fe[256 * h + lane + 64 * j] : 0.f;
      const float base = fbase[rs_index<V>(lane) % G];  // (of the head whose sum the lane receives)
#pragma unroll
      for (int k0 = 0; k0 < SR; k0 += ZB) {
        if (!((any_need >> k0) & ((1ull << ZB) - 1ull))) continue;
        float z[ZB][4];
#pragma unroll
        for (int k = 0; k < ZB; ++k) load_fz(a.L.sub_fz + (sg0 + min(k0 + k, S - 1)) * FM, FM, z[k]);
        float part[V];
#pragma unroll
        for (int k = 0; k < ZB; ++k)
#pragma unroll
          for (int h = 0; h < G; ++h) {
            float t = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) t += e[h][j] * z[k][j];
            part[k * G + h] = t;
          }
        const float t = wave_reduce_scatter<V>(part);
        const float wl = t > 0.f ? base + log2f(t) : -INFINITY;
#pragma unroll
        for (int k = 0; k < ZB; ++k) {
          if (!((any_need >> (k0 + k)) & 1ull)) continue;
          const uint32_t nk = (uint32_t)__builtin_amdgcn_readlane((int)need, k0 + k);
          float vb[VPL];
          vb[0] = bf16_lo(vraw[k0 + k]);
          if constexpr (VPL == 2) vb[1] = bf16_hi(vraw[k0 + k]);
#pragma unroll
          for (int h = 0; h < G; ++h) {
            if (!((nk >> h) & 1u)) continue;
            const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), rs_lane<V>(k * G + h)));
            if (w != -INFINITY) add_group<VPL>(rm[h], rl[h], ro[h], w, vb);
          }
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < SR; ++k) {
        if (!((any_need >> k) & 1ull)) continue;
        const uint32_t nk = (uint32_t)__builtin_amdgcn_readlane((int)need, k);
        float vb[VPL];
        vb[0] = bf16_lo(vraw[k]);
        if constexpr (VPL == 2) vb[1] = bf16_hi(vraw[k]);
#pragma unroll
        for (int h = 0; h < G; ++h)
          if ((nk >> h) & 1u) add_group<VPL>(rm[h], rl[h], ro[h], sc[h * SR + k], vb);
      }
    }
    // the wave's record: one (o, m, l) row per head
    float* dst = a.ws.res_part + ((int64_t)u * a.nb_res + x) * G * RS;
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < VPL; ++e) dst[h * RS + lane * VPL + e] = ro[h][e];
      if (lane == 0) *reinterpret_cast<float2*>(dst + h * RS + D) = float2{rm[h], rl[h]};
    }
  }
  {
    const uint32_t rows = (lane < S && sm != 0u) ? (uint32_t)ncnt : 0u;
    const int rsum = (int)wave_reduce_uniform(rows, [](uint32_t p, uint32_t q) { return p + q; }, 0u);
    if (lane == 0) atomicAdd(&a.ws.unit_rows[u], rsum);
  }
  TileRec* ctiles = a.ws.tiles + tile_unit_base(U.row_base, U.cl_base, u, a.L.fold_cap) + tbx;
  const int n_tiles =
      write_run_tiles(ctiles, U.row_base, a.L_head_dim, lane < S ? o_i : 0, lane < S ? o_n : 0, lane < S ? sm : 0u);
  int n_all = n_tiles;
  if (__ballot(lane < S && sm != 0u && fcnt > 0)) {
    // folded rows of the chosen subclusters, after the reordered ones: the
    // unit's fold rows are scanned 64 at a time (lane l: row f0 + l), the
    // subclusters of FB such chunks loaded before any is used; a tile is a
    // run of consecutive fold rows with one head mask, cut at every 32nd row
    constexpr int FB = 8;
    const int nf = U.n_fold;
    const int32_t* fs = a.L.fold_sub + (int64_t)u * a.L.fold_cap;
    const int64_t frow = a.L.fold_row0 + (int64_t)u * a.L.fold_cap;
    TileRec* ft = ctiles + n_tiles;
    int nt = 0;
    for (int fb0 = 0; fb0 < nf; fb0 += 64 * FB) {
      int fsv[FB];
#pragma unroll
      for (int c = 0; c < FB; ++c) {
        const int f = fb0 + 64 * c + lane;
        fsv[c] = f < nf ? fs[f] : -1;
      }
#pragma unroll
      for (int c = 0; c < FB; ++c) {
        const int f0 = fb0 + 64 * c;
        if (f0 < nf) {
          const int f = f0 + lane;
          const int li = fsv[c] - g * S;
          const bool mine = li >= 0 && li < S;
          const uint32_t smi = (uint32_t)__shfl((int)sm, mine ? li : 0, 64);
          const uint32_t fm = mine ? smi : 0u;
          const uint32_t fm_prv = (uint32_t)__shfl_up((int)fm, 1, 64);
          const bool cont = fm != 0u && (lane & 31) != 0 && fm_prv == fm;
          const bool fhead = fm != 0u && !cont;
          const unsigned long long fhb = __ballot(fhead);
          const unsigned long long after = __ballot(!cont) & ~((2ull << lane) - 1ull);
          const int fend = after ? __ffsll((long long)after) - 1 : 64;
          if (fhead) ft[nt + __popcll(fhb & below)] = TileRec{(frow + f) * (int64_t)a.L_head_dim, fend - lane, fm};
          nt += __popcll(fhb);
        }
      }
    }
    n_all += nt;
  }
  if (lane == 0) a.ws.ch_ntiles[cw + x] = n_all;
}


template <int D, int G>
__global__ __launch_bounds__(256) void k_sub_wave(DArgs a, BudgetArgs b, int nb_chosen) {
  __shared__ float4 lsc4[4][G][kDecodeSubRows / 4];  // each wave's scores [head][subcluster]
  __shared__ float lds_fe[G][256];  // feature-map residual: 2^(fq - max) per head
  __shared__ float lds_fbase[G];    // and max - log2(m) / 2
  const int u = blockIdx.x, wave = threadIdx.x >> 6;
  const int x = (int)blockIdx.y * 4 + wave;
  const int64_t cw = (int64_t)u * a.cstride;
  const int s_keep_raw = b.top_s[u / a.Hkv];
  const int n_ch_raw = a.ws.n_chosen[u];
  // (entries below nb_chosen <= the largest C are in range; they are used
  // only for x < n_chosen)
  const int xs = min(x, nb_chosen - 1);
  const int g_raw = a.ws.cl_list[cw + xs];
  const int tb_raw = a.ws.ch_tbase[cw + xs];
  const mog_unit U = unit_scalar(a.L.units + u);
  if (a.residual == 2) {
    // (before any wave leaves: the table's barrier)
    fm_table<G>(a, u, &lds_fe[0][0], lds_fbase);
    __syncthreads();
  }
  if (x >= uni(n_ch_raw)) return;
  const int g = uni(g_raw);
  const uint32_t mask = (uint32_t)uni((int)a.ws.cl_mask[cw + g]);
  sub_wave_cluster<D, G>(a, u, x, U, g, uni(tb_raw), mask, s_keep_raw, lsc4[wave], &lds_fe[0][0], lds_fbase);
}

// ---------------------------------------------------------------------------
// 3c. Top-c and subclusters in one launch, for one query head per KV head
//     (the steps of 3b): every wave of block (u, y) selects its unit's top-c
//     itself (the selection of 2, on the unit's scores and tile bounds, which
//     the L2 serves to all of the unit's waves), takes the unit's x-th
//     chosen cluster, x = 4 y + w, with its slot base, and does 3b's work on
//     it.  Wave 0 of block (u, 0) also writes the unit's selection (head
//     masks, list, slot bases, count and the selection output) for the exact
//     and merge kernels.  The top-c launch and every wave's list loads drop
//     out of the step; the unit's exact row count is cleared by the score
//     kernel.
// ---------------------------------------------------------------------------
template <int D, int KPL>
__global__ __launch_bounds__(256) void k_select_sub1(DArgs a, BudgetArgs b) {
  __shared__ int hist[4][256 + 64];
  __shared__ float4 lsc4[4][1][kDecodeSubRows / 4];
  __shared__ float lds_fe[256];  // feature-map residual: the head's 2^(fq - max)
  __shared__ float lds_fbase[1];
  const int u = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (a.residual == 2) {
    fm_table<1>(a, u, lds_fe, lds_fbase);
    __syncthreads();
  }
  const int x = (int)blockIdx.y * 4 + wave;
  const int64_t cw = (int64_t)u * a.cstride;
  const int want_raw = b.top_c[u / a.Hkv];
  const int s_keep_raw = b.top_s[u / a.Hkv];
  // scores and tile bounds of the unit's clusters (slot j of lane l: cluster
  // 64 j + l; one head, so the head's scores start at u * cstride)
  float scv[KPL];
  int bound[KPL];
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const int i = min(64 * j + lane, a.cstride - 1);
    scv[j] = a.ws.cl_score[cw + i];
    bound[j] = a.ws.cl_tiles[cw + i];
  }
  const mog_unit U = unit_scalar(a.L.units + u);
  const int C = U.C;
  uint32_t key[KPL];
  int nvalid = 0;
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const bool in = 64 * j + lane < C && scv[j] != -INFINITY;
    key[j] = in ? float_key(scv[j]) : 0u;
    nvalid += in;
  }
  nvalid = (int)wave_reduce_uniform((uint32_t)nvalid, [](uint32_t p, uint32_t q) { return p + q; }, 0u);
  const int want = want_raw < 0 ? 0 : want_raw;
  const int c_eff = want < nvalid ? want : nvalid;
  int kk, cand;
  uint32_t prefix, hi_mask;
  wave_select<KPL>(scv, key, c_eff, nvalid, hist[wave], kk, cand, prefix, hi_mask);
  // the chosen clusters (the rule of 2), their positions in the ascending
  // list and their tile-slot bases; the wave's own cluster x
  const unsigned long long below = (1ull << lane) - 1ull;
  const bool all_ties = cand == kk;
  int ties = 0, n_before = 0, t_before = 0, g = 0, tbx = 0;
  bool sel[KPL];
  int pos[KPL], tbs[KPL];
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const uint32_t kd = key[j] & hi_mask;
    const bool valid = c_eff > 0 && key[j] != 0u;
    bool sj;
    if (all_ties) {
      sj = valid && kd >= prefix;
    } else {
      const bool tie = valid && kd == prefix;
      const unsigned long long tb = __ballot(tie);
      sj = valid && (kd > prefix || (tie && ties + __popcll(tb & below) < kk));
      ties += __popcll(tb);
    }
    sel[j] = sj;
    const unsigned long long sb = __ballot(sj);
    pos[j] = n_before + __popcll(sb & below);
    const int bnd = sj ? bound[j] : 0;
    const int incl = wave_incl_scan(bnd);
    tbs[j] = t_before + incl - bnd;
    const unsigned long long hit = __ballot(sj && pos[j] == x);
    if (hit) {
      const int src = __ffsll((long long)hit) - 1;
      g = 64 * j + src;
      tbx = __builtin_amdgcn_readlane(tbs[j], src);
    }
    n_before += __popcll(sb);
    t_before += __builtin_amdgcn_readlane(incl, 63);
  }
  const int n_ch = n_before;
  if (blockIdx.y == 0 && wave == 0) {
    const int64_t row = (int64_t)U.seq * a.Hq + U.kv_head;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const int i = 64 * j + lane;
      if (i < C) {
        a.ws.cl_mask[cw + i] = sel[j] ? 1u : 0u;
        if (a.sel_s) a.ws.cl_rank[cw + i] = sel[j] ? pos[j] : -1;  // read back only for sel_s
      }
      if (sel[j]) {
        a.ws.cl_list[cw + pos[j]] = i;
        a.ws.ch_tbase[cw + pos[j]] = tbs[j];
        if (a.sel_c) a.sel_c[row * a.c_stride + pos[j]] = i;
      }
    }
    if (a.sel_c)
      for (int j = n_ch + lane; j < a.c_stride; j += 64) a.sel_c[row * a.c_stride + j] = -1;
    if (a.sel_s) {
      const int64_t base = row * a.c_stride * a.s_stride;
      for (int j = n_ch * a.s_stride + lane; j < a.c_stride * a.s_stride; j += 64) a.sel_s[base + j] = -1;
    }
    if (lane == 0) a.ws.n_chosen[u] = n_ch;
  }
  if (x >= n_ch) return;
  sub_wave_cluster<D, 1>(a, u, x, U, g, tbx, 1u, s_keep_raw, lsc4[wave], lds_fe, lds_fbase);
}

// ---------------------------------------------------------------------------
// 4. Exact split-K pass.  The tiles a unit reads exactly are numbered
//    [sink anchor tiles | recent anchor tiles | tiles of the chosen clusters
//    in list order]; wave w of the unit takes [w*NT/NW, (w+1)*NT/NW).  Every
//    wave scans the chosen clusters' tile counts into LDS; a wave lists its
//    tiles (one per lane: binary search, then the 16-byte tile record) in
//    LDS and streams them.  Grid: the exact blocks of every unit.
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// 4a. Shares of the exact blocks.  Unit u reads T_u = anchors + rows of its
//     chosen subclusters exactly; it gets n_u(r) = 1 + floor(T_u * r) slots
//     (blocks, or half blocks when many units split them), numbered unit by
//     unit, for the largest scale r a 4-ary search finds with
//     sum_u n_u(r) <= B, B = min(slots, n_units + ceil(total / min_rows)) (so
//     no slot gets much under min_rows rows).  This bounds the heaviest slot
//     by the smallest load the slot count allows, up to rounding: with many
//     units of a few slots each, a fixed scale (r = (B - n_units) / total)
//     leaves up to one slot per unit unused and its siblings a third more
//     work.  With many slots per unit the fixed scale is kept.  Every wave of
//     every exact block recomputes the shares from the per-unit row counts
//     (a few KB): no table, no launch, no barrier.
// ---------------------------------------------------------------------------
struct BlockShare {
  int u;      // unit (-1: the slot has no work)
  int first;  // first slot of the unit
  int n;      // slots of the unit
};

// The share holding slot want_block of nblk, found by one wave on its own
// (every wave of a slot computes the same, so no barrier is needed): lane l
// holds the totals of units l + 64 k (k < kShareRegs) in registers, the
// counts are wave sums, the slot numbers a lane scan.  Past 64 kShareRegs
// units the scale is the fixed one, the units read 64 at a time.
constexpr int kShareRegs = 4;
constexpr int kShareRounds = 3;
// Rows a block gets at least (half of it for a half block): small steps
// (32K: about 25K rows over 8 units) then spread over more blocks, whose
// waves stream 2-3 tiles after their set-up instead of 7 (64 measured best
// against 256, 128, 32 and 16: 32K 24.6 -> 23.3 us per step).
constexpr int kShareMinRows = 64;

__device__ BlockShare wave_find_share(const int32_t* unit_rows, int n_units, int nblk, int A, int want_block,
                                      int min_rows) {
  const int lane = threadIdx.x & 63;
  const bool in_regs = n_units <= 64 * kShareRegs;
  float w[kShareRegs];
  long long part = 0;
  if (in_regs) {
#pragma unroll
    for (int k = 0; k < kShareRegs; ++k) {
      const int v = lane + 64 * k;
      const int t = v < n_units ? A + unit_rows[v] : -1;
      w[k] = (float)t;
      part += t < 0 ? 0 : t;
    }
  } else {
    for (int v = lane; v < n_units; v += 64) part += (long long)A + unit_rows[v];
  }
  long long total;
  if (in_regs) {
    // (at most 256 units of at most 2^22 + A rows: the sum fits 32 bits, and
    // DPP sums are cheaper than 64-bit lane exchanges)
    total = (long long)wave_reduce_uniform((uint32_t)part, [](uint32_t x, uint32_t y) { return x + y; }, 0u);
  } else {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
    total = part;
  }
  const long long by_rows = (total + min_rows - 1) / min_rows;
  const int B = (int)(nblk - n_units < by_rows ? nblk : n_units + by_rows);
  // blocks n_u(r) summed over the units (r >= 0: monotone in r)
  auto part_count = [&](float r) {
    int c = 0;
#pragma unroll
    for (int k = 0; k < kShareRegs; ++k) c += w[k] >= 0.f ? 1 + (int)floorf(w[k] * r) : 0;
    return (uint32_t)c;
  };
  auto add = [](uint32_t x, uint32_t y) { return x + y; };
  float r = total > 0 ? (float)(B - n_units) / (float)total : 0.f;
  // (with 32 or more blocks per unit beyond its first, the fixed scale
  // already leaves at most a few percent of a block per unit unused)
  if (in_regs && total > 0 && B - n_units < 32 * n_units) {
    // 4-ary search on [lo, hi): lo meets the bound (r = 0 always does, as
    // n_units <= nblk), hi = (B + 1) / total cannot (the sum exceeds
    // total * r); each round counts three interior points, whose wave sums
    // are independent of each other
    float lo = (int)wave_reduce_uniform(part_count(r), add, 0u) <= B ? r : 0.f;
    float hi = (float)(B + 1) / (float)total * 1.001f;
    for (int it = 0; it < kShareRounds; ++it) {
      const float d = 0.25f * (hi - lo);
      const float c1 = lo + d, c2 = lo + 2.f * d, c3 = lo + 3.f * d;
      const int n1 = (int)wave_reduce_uniform(part_count(c1), add, 0u);
      const int n2 = (int)wave_reduce_uniform(part_count(c2), add, 0u);
      const int n3 = (int)wave_reduce_uniform(part_count(c3), add, 0u);
      if (n3 <= B) lo = c3;
      else if (n2 <= B) { lo = c2; hi = c3; }
      else if (n1 <= B) { lo = c1; hi = c2; }
      else hi = c1;
    }
    r = lo;
  }
  BlockShare res{-1, 0, 0};
  int carry = 0;
  for (int base = 0, k = 0; base < n_units; base += 64, ++k) {
    const int v = base + lane;
    int sp = 0;
    if (in_regs) {
#pragma unroll
      for (int kk = 0; kk < kShareRegs; ++kk)
        if (kk == k && w[kk] >= 0.f) sp = 1 + (int)floorf(w[kk] * r);
    } else if (v < n_units) {
      // fixed scale in exact integers: sum <= n_units + (B - n_units)
      sp = 1 + (int)(total > 0 ? ((long long)A + unit_rows[v]) * (B - n_units) / total : 0);
    }
    const int incl = wave_incl_scan(sp);
    const int first = carry + incl - sp;
    const unsigned long long hit = __ballot(v < n_units && want_block >= first && want_block < first + sp);
    if (hit) {
      const int src = __ffsll((long long)hit) - 1;
      res = BlockShare{__builtin_amdgcn_readlane(v, src), __builtin_amdgcn_readlane(first, src),
                       __builtin_amdgcn_readlane(sp, src)};
      break;
    }
    carry += __builtin_amdgcn_readlane(incl, 63);
  }
  return res;
}

// A tile of at most 32 contiguous layout rows: element offset of its first
// row, row count (0: no more tiles), mask of the heads that read it.
struct TileDesc {
  int64_t off;
  int nrows;
  uint32_t mask;
  int src;  // 0: layout rows (k_mid / v_mid), 1: KV cache rows (anchors)
};

constexpr int kTileBatch = 64;  // tiles listed per wave before streaming them

template <int D, int G, typename Engine, typename T>
__global__ __launch_bounds__(256, 2) void k_exact(DArgs a) {
  constexpr int RS = D + kPartPad;
  __shared__ u32x4 kvbuf[4][Engine::BUF];
  // the wave states of the epilogue reuse the tile buffers when they are
  // large enough (after a barrier)
  constexpr int ST = 4 * G * (D + kPartPad);
  constexpr bool ALIAS = sizeof(u32x4) * 4 * Engine::BUF >= sizeof(float) * ST;
  __shared__ float st_own[ALIAS ? 1 : ST];
  float* st = ALIAS ? reinterpret_cast<float*>(&kvbuf[0][0]) : st_own;
  // the chosen clusters in list order, for the tile listing: the block's
  // (lists longer than kWaveListMax: exclusive prefix of the tile counts,
  // then tile-slot bases) or each wave's own copy (prefix | slot bases, or a
  // whole-cluster step's first rows | its rows and head masks)
  constexpr int kBlockList = 2 * kMaxC + 1, kWaveList = 3 * kWaveListMax + 1;
  __shared__ int lists[kBlockList > 4 * kWaveList ? kBlockList : 4 * kWaveList];
  __shared__ int sh[16];
  __shared__ TileRec tiles[4][kTileBatch];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  if ((int)blockIdx.x >= a.nblk) {
    // the residual of the clusters some head left out, in blocks after the
    // exact ones (dispatched as exact blocks retire): the Gaussian one, or a
    // whole-cluster step's feature-map one; record y of unit u covers
    // clusters [R y, R y + R) (R = rest_cl), after the unit's chosen-cluster
    // records (none for a whole-cluster step)
    const int r = (int)blockIdx.x - a.nblk;
    const int u = r / a.rest_per_unit, y = r % a.rest_per_unit;
    const int n_ch_raw = a.whole ? 0 : a.ws.n_chosen[u];
    const mog_unit U = uni_unit(a.L.units + u);
    if (y * a.rest_cl >= U.C) return;
    constexpr int VPL = D / 64;
    float rm[G], rl[G], ro[G][VPL];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      rm[h] = -INFINITY;
      rl[h] = 0.f;
#pragma unroll
      for (int e = 0; e < VPL; ++e) ro[h][e] = 0.f;
    }
    if (a.residual == 2) {
      // (the unit's feature table in the list LDS, which this path does not
      // otherwise use)
      float* fe = reinterpret_cast<float*>(lists);
      fm_table<G>(a, u, fe, fe + 256 * G);
      __syncthreads();
      rest_clusters_fm<D, G, (G <= 6 ? 8 : 4)>(a, u, U, y, fe, fe + 256 * G, rm, rl, ro);
    } else if (a.rest_cl == kRestClustersSmall) {
      rest_clusters<D, G, kRestClustersSmall / 4>(a, u, U.C, U.cl_base, y, rm, rl, ro);
    } else {
      rest_clusters<D, G, kRestClustersPerBlock / 4>(a, u, U.C, U.cl_base, y, rm, rl, ro);
    }
    store_wave_states<D, G>(st, rm, rl, ro);
    __syncthreads();
    write_block_record<D, G>(st, a.ws.res_part + ((int64_t)u * a.nb_res + uni(n_ch_raw) + y) * G * RS);
    return;
  }
  const int A = a.n_sink + a.n_recent;
  // Shares: one per block, or with `half` one per half block (waves 0-1
  // and 2-3 serve units of their own: finer shares when many units split
  // the blocks)
  const int WPS = a.half ? 2 : 4;                   // waves per share
  const int hf = a.half ? wave >> 1 : 0;            // the wave's share in the block
  const int ws_wave = a.half ? wave & 1 : wave;     // the wave's index in its share
  const int slot = a.half ? 2 * (int)blockIdx.x + hf : (int)blockIdx.x;
  const BlockShare bs = wave_find_share(a.ws.unit_rows, a.n_units, a.half ? 2 * a.nblk : a.nblk, A, slot,
                                        a.half ? kShareMinRows / 2 : kShareMinRows);
  const int u = bs.u;
  // (a share with no unit leaves; a half block's idle half still meets the
  // other half at the epilogue's barriers)
  if (u < 0 && !a.half) return;
  Engine acc;
  if (u >= 0) {
    const int p = slot - bs.first, splits_u = bs.n;
    if (p == 0 && ws_wave == 0 && lane == 0) {
      a.ws.uinfo[2 * u] = bs.first;
      a.ws.uinfo[2 * u + 1] = bs.n;
    }
    const mog_unit U = uni_unit(a.L.units + u);
    const int C = U.C, S = U.S;
    u32x4* buf = kvbuf[wave];
    // tile counts of the chosen clusters (in list order) -> exclusive prefix.
    // Lists of up to 256 clusters (the usual case): each wave loads the four
    // entries of each lane without waiting for the list length (issued before
    // the query's loads, so one wait covers both) and scans them itself into
    // its own LDS rows, with no barrier.  Longer lists: a block scan, E entries
    // per thread.
    const int64_t cw = (int64_t)u * a.cstride;
    const int n_ch_raw = a.ws.n_chosen[u];
    // (a whole-cluster step: rows | head mask << 24 and first rows)
    const int32_t* la = a.whole ? reinterpret_cast<const int32_t*>(a.ws.ch_nm) : a.ws.ch_ntiles;
    const int32_t* lb = a.whole ? a.ws.ch_row0 : a.ws.ch_tbase;
    int wl[4], wt[4];
  #pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int x = min(4 * lane + k, a.cstride - 1);
      wl[k] = la[cw + x];
      wt[k] = lb[cw + x];
    }
    // (unit u is sequence u / Hkv, KV head u % Hkv: the query's address does
    // not wait for the unit record)
    acc.init(a.q + ((int64_t)(u / a.Hkv) * a.Hq + (int64_t)(u % a.Hkv) * G) * D, a.scale_l2, buf);
    // (a whole-cluster step has at most kWaveListMax chosen clusters; the
    // clamp only keeps every list access in range)
    const int n_ch = a.whole ? min(uni(n_ch_raw), kWaveListMax) : uni(n_ch_raw);
    const int* tp = lists;  // the prefix the listing searches, and the slot bases (or first rows)
    const int* tb = lists + kMaxC + 1;
    const int* tn = nullptr;  // a whole-cluster step's rows | head masks
    if (n_ch <= kWaveListMax) {
      int* wp = lists + wave * kWaveList;
      int* wb = wp + kWaveListMax + 1;
      int* wn = wb + kWaveListMax;
      int cnt[4], sum = 0;
  #pragma unroll
      for (int k = 0; k < 4; ++k) {
        const bool in = 4 * lane + k < n_ch;
        cnt[k] = !in ? 0 : a.whole ? (int)((((uint32_t)wl[k] & 0xffffffu) + 31u) >> 5) : wl[k];
        sum += cnt[k];
      }
      const int incl = wave_incl_scan(sum);
      int base = incl - sum;
  #pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (4 * lane + k < n_ch) {
          wp[4 * lane + k] = base;
          wb[4 * lane + k] = wt[k];
          if (a.whole) wn[4 * lane + k] = wl[k];
        }
        base += cnt[k];
      }
      if (lane == 63) wp[n_ch] = incl;
      __asm__ volatile("" ::: "memory");  // (a wave's LDS operations run in order)
      tp = wp;
      tb = wb;
      tn = wn;
    } else {
      // (a whole block: half-block shares are used only when every unit's
      // list fits a wave's own list, so this branch has no idle half)
      int* tpre = lists;
      int* tbs = lists + kMaxC + 1;
      constexpr int EM = kMaxC / 256;
      const int E = (n_ch + 255) / 256;
      int loc[EM], tbl[EM];
  #pragma unroll
      for (int k = 0; k < EM; ++k) {
        const int x = min(tid * E + k, a.cstride - 1);
        loc[k] = a.ws.ch_ntiles[cw + x];
        tbl[k] = a.ws.ch_tbase[cw + x];
      }
      int sum = 0;
  #pragma unroll
      for (int k = 0; k < EM; ++k) {
        loc[k] = (k < E && tid * E + k < n_ch) ? loc[k] : 0;
        sum += loc[k];
      }
      int total;
      int base = block_excl_scan<256>(sum, sh, total);
  #pragma unroll
      for (int k = 0; k < EM; ++k) {
        const int x = tid * E + k;
        if (k < E && x < n_ch) {
          tpre[x] = base;
          tbs[x] = tbl[k];
        }
        base += loc[k];
      }
      if (tid == 0) tpre[n_ch] = total;
      __syncthreads();
    }
    // virtual tiles of the unit: [sink tiles | recent tiles | chosen clusters'
    // tiles in list order]; wave w of the unit takes [w NT / NW, (w+1) NT / NW)
    const int n_st = (a.n_sink + 31) / 32, n_rt = (a.n_recent + 31) / 32, n_at = n_st + n_rt;
    const int NT = n_at + uni(tp[n_ch]);
    const int NW = splits_u * WPS;
    const int w = p * WPS + ws_wave;
    int k0 = (int)((int64_t)w * NT / NW);
    const int k1 = (int)((int64_t)(w + 1) * NT / NW);
    const T* kc = static_cast<const T*>(a.kv.k);
    const T* vc = static_cast<const T*>(a.kv.v);
    const uint32_t all = (1u << G) - 1u;
    const KVRef kv = a.kv;
    // first token and row count of anchor tile k (< n_at)
    auto anchor_tile = [&](int k, int& tok, int& nr) {
      if (k < n_st) {
        tok = 32 * k;
        nr = min(32, a.n_sink - 32 * k);
      } else {
        const int j = k - n_st;
        tok = U.N - a.n_recent + 32 * j;
        nr = min(32, a.n_recent - 32 * j);
      }
    };
    if (kv.paged) {
      // anchors of a paged cache: rows gathered through the block table
      for (; k0 < k1 && k0 < n_at; ++k0) {
        int tok, nr;
        anchor_tile(k0, tok, nr);
        acc.tile_gather(buf, kc, vc, nr, all, [&](int i) { return kv_row_offset(kv, U.seq, U.kv_head, tok + i, D); });
      }
    }
    if (k0 < k1) {
      const T* km = static_cast<const T*>(a.L.k_mid);
      const T* vm = static_cast<const T*>(a.L.v_mid);
      const TileRec* utiles = a.ws.tiles + tile_unit_base(U.row_base, U.cl_base, u, a.L.fold_cap);
      TileRec* tl = tiles[wave];
      const int64_t anc_base = kv.paged ? 0 : kv_row_offset(kv, U.seq, U.kv_head, 0, D);
      while (k0 < k1) {
        // (1) list the next batch in LDS, one tile per lane: an anchor tile
        //     of a contiguous cache, or the chosen cluster's slot (binary
        //     search of the prefix, then one 16-byte load)
        const int nt = min(kTileBatch, k1 - k0);
        if (lane < nt) {
          const int k = k0 + lane;
          TileRec r;
          if (k < n_at) {
            int tok, nr;
            anchor_tile(k, tok, nr);
            r = TileRec{anc_base + (int64_t)tok * D, nr | (int)0x80000000, 0xffffffffu};
          } else {
            const int kv_ = k - n_at;
            int lo = 0, hi = n_ch;  // last x with tp[x] <= kv_
            while (hi - lo > 1) {
              const int mid = (lo + hi) >> 1;
              if (tp[mid] <= kv_) lo = mid; else hi = mid;
            }
            const int jt = kv_ - tp[lo];
            if (a.whole) {
              // tile jt of a whole cluster: its rows from the first, 32 at a time
              const uint32_t nm = (uint32_t)tn[lo];
              r = TileRec{(U.row_base + tb[lo] + 32 * jt) * (int64_t)D, min(32, (int)(nm & 0xffffffu) - 32 * jt),
                          nm >> 24};
            } else {
              r = utiles[tb[lo] + jt];
            }
          }
          tl[lane] = r;
        }
        k0 += nt;
        // (2) stream the batch: the next tile's loads are in flight while the
        //     current one is computed.  rd(i) is tile i of the batch, or past
        //     the end an empty tile (0 rows: its loads read nothing), so every
        //     load is issued unconditionally and the wait for a tile's
        //     registers never has to cover the next tile's loads.
        auto rd = [&](int i) {
          const TileRec r = tl[i < nt ? i : nt - 1];
          TileDesc t;
          t.off = uni(r.off);
          const int ns = uni(r.nrows_src);
          t.nrows = i < nt ? (ns & 0x7fffffff) : 0;
          t.src = (int)((uint32_t)ns >> 31);
          t.mask = (uint32_t)uni((int)r.mask);
          return t;
        };
        auto kp = [&](const TileDesc& t) { return (t.src ? kc : km) + t.off; };
        auto vp = [&](const TileDesc& t) { return (t.src ? vc : vm) + t.off; };
        if constexpr (Engine::PIPELINED) {
          typename Engine::Regs ra, rb;
          TileDesc ta = rd(0), tb;
          Engine::load(kp(ta), vp(ta), ta.nrows, ra.k, ra.v);
          // the scheduling barriers keep each tile's loads ahead of the
          // previous tile's arithmetic (the scheduler would otherwise sink them
          // to save registers and serialise load and compute)
          for (int i = 0; i < nt; i += 2) {
            tb = rd(i + 1);
            Engine::load(kp(tb), vp(tb), tb.nrows, rb.k, rb.v);
            __builtin_amdgcn_sched_barrier(0);
            acc.compute(buf, ra.k, ra.v, ta.nrows, ta.mask);
            if (i + 1 >= nt) break;
            ta = rd(i + 2);
            Engine::load(kp(ta), vp(ta), ta.nrows, ra.k, ra.v);
            __builtin_amdgcn_sched_barrier(0);
            acc.compute(buf, rb.k, rb.v, tb.nrows, tb.mask);
          }
        } else {
          for (int i = 0; i < nt; ++i) {
            const TileDesc t = rd(i);
            acc.tile(buf, kp(t), vp(t), t.nrows, t.mask);
          }
        }
      }
    }
  }
  __syncthreads();  // every wave is done with its tile buffer
  if (u >= 0) acc.to_lds(st);  // (an idle half's engine holds no state)
  __syncthreads();
  if (!a.half)
    write_record<D, G, 4>(st, 0, a.ws.ex_part + (int64_t)slot * G * RS, tid, 256);
  else if (u >= 0)
    write_record<D, G, 2>(st, 2 * hf, a.ws.ex_part + (int64_t)slot * G * RS, tid & 127, 128);
}

// ---------------------------------------------------------------------------
// 5. Merge: per query head, the exact records of its unit (n_part per unit,
//    or the range uinfo[u] the exact pass wrote) and the n_res residual
//    records of the unit, merged with one normalisation.  Grid (Hq, n_seq),
//    1024 threads: (D/8)-lane groups each fold every NG-th record into a
//    running (m, l, o) with two 16-byte loads per lane (one pass over the
//    records, NG of them in flight); then every group rescales its state to
//    the block maximum, the groups of a wave are summed by lane exchanges
//    and the waves' sums through LDS.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(1024) void k_merge(const float* part, int n_part, const int32_t* uinfo,
                                                const float* res, int res_stride, int rest_cl,
                                                const int32_t* n_chosen, const mog_unit* units, int G, int Hq,
                                                int Hkv, float* out, float* lse) {
  constexpr int RS = D + kPartPad;
  constexpr int QL = D / 8;        // lanes per record (8 elements each)
  constexpr int NG = 1024 / QL;    // records folded side by side
  constexpr int NW = 1024 / 64;
  __shared__ float4 wo[NW][QL][2];
  __shared__ float wm[NW], wl[NW];
  const int hq = blockIdx.x, seq = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int kvh = hq / G, h = hq % G;
  const int u = seq * Hkv + kvh;
  int64_t first = (int64_t)u * n_part;
  if (uinfo) {
    first = scalar_load(uinfo + 2 * u);
    n_part = scalar_load(uinfo + 2 * u + 1);
  }
  const int64_t stride = (int64_t)G * RS;
  const float* eb = part + (first * G + h) * RS;
  // residual records of the unit: one per chosen cluster (none without
  // n_chosen: a whole-cluster step leaves nothing out of a chosen cluster),
  // then one per rest_cl clusters
  int n_res = 0;
  if (res) n_res = (n_chosen ? scalar_load(n_chosen + u) : 0) + (scalar_load(&units[u].C) + rest_cl - 1) / rest_cl;
  const float* rb = res ? res + ((int64_t)u * res_stride * G + h) * RS : nullptr;
  const int total = n_part + (res ? n_res : 0);
  const int q = tid % QL, grp = tid / QL;
  float m = -INFINITY, l = 0.f;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // two records per group in flight: 2 NG = 128 records per pass at D = 128
  // (a unit has up to a few hundred), and registers for two blocks per
  // compute unit
#pragma unroll 2
  for (int i = grp; i < total; i += NG) {
    const float* r = i < n_part ? eb + i * stride : rb + (int64_t)(i - n_part) * stride;
    const float mi = r[D], li = r[D + 1];
    const float4 a0 = reinterpret_cast<const float4*>(r)[2 * q];
    const float4 a1 = reinterpret_cast<const float4*>(r)[2 * q + 1];
    const float oi[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    // branch-free, so the unrolled iterations' loads are all in flight
    const float mn = fmaxf(m, mi);
    const float fa = exp2_or_zero(m, mn), fb = exp2_or_zero(mi, mn);
    l = l * fa + li * fb;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = o[e] * fa + oi[e] * fb;
    m = mn;
  }
  // every group under the wave maximum, then the sum over the wave's groups
  // (lanes q, q + QL, q + 2 QL, ...); the waves' states meet in LDS after one
  // barrier and are rescaled to the block maximum there
  const float mw = wave_max(m);
  const float f = exp2_or_zero(m, mw);
  l *= f;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] *= f;
#pragma unroll
  for (int sft = QL; sft < 64; sft <<= 1) {
    l += __shfl_xor(l, sft, 64);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] += __shfl_xor(o[e], sft, 64);
  }
  if (lane < QL) {
    wo[wave][lane][0] = float4{o[0], o[1], o[2], o[3]};
    wo[wave][lane][1] = float4{o[4], o[5], o[6], o[7]};
    if (lane == 0) {
      wm[wave] = mw;
      wl[wave] = l;
    }
  }
  __syncthreads();
  // every thread: wave state w = tid % NW, elements 2p, 2p + 1 (p = tid / NW);
  // the NW states of one element pair sit in NW adjacent lanes, which take
  // the block maximum, the rescaled sums and the denominator by lane
  // exchanges
  static_assert(NW == 16 && 1024 / NW >= D / 2, "16 wave states, one element pair per 16 lanes");
  {
    const int w = tid % NW, pr = tid / NW;
    const float mv = wm[w];
    float M = mv;
#pragma unroll
    for (int sft = 1; sft < NW; sft <<= 1) M = fmaxf(M, __shfl_xor(M, sft, 64));
    const float fw = exp2_or_zero(mv, M);
    const float* ow = reinterpret_cast<const float*>(wo[w]);  // the state's D elements in order
    float t0 = 0.f, t1 = 0.f;
    if (pr < D / 2) {
      const float2 v = reinterpret_cast<const float2*>(ow)[pr];
      t0 = fw * v.x;
      t1 = fw * v.y;
    }
    float dn = fw * wl[w];
#pragma unroll
    for (int sft = 1; sft < NW; sft <<= 1) {
      t0 += __shfl_xor(t0, sft, 64);
      t1 += __shfl_xor(t1, sft, 64);
      dn += __shfl_xor(dn, sft, 64);
    }
    const int64_t orow = (int64_t)seq * Hq + hq;
    const float inv = dn > 0.f ? 1.f / dn : 0.f;
    if (w == 0 && pr < D / 2) reinterpret_cast<float2*>(out + orow * D)[pr] = float2{t0 * inv, t1 * inv};
    if (lse && tid == 0) lse[orow] = dn > 0.f ? (M + log2f(dn)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// Dense baseline: wave w of unit u covers tokens [w*N/NW, (w+1)*N/NW).
// ---------------------------------------------------------------------------
template <int D, int G, typename Engine, typename T>
__global__ __launch_bounds__(256, 2) void k_dense(KVRef kv, const float* q, int Hq, int Hkv, int splits,
                                               float scale_l2, SeqArgs seq_args, float* ex_part) {
  constexpr int RS = D + kPartPad;
  __shared__ u32x4 kvbuf[4][Engine::BUF];
  __shared__ float st[4 * G * (D + kPartPad)];
  const int u = blockIdx.y, p = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  const int seq = u / Hkv, kvh = u % Hkv;
  const int64_t N = seq_args.len[seq];
  const int NW = splits * 4;
  const int w = p * 4 + wave;
  const int t0 = (int)((int64_t)w * N / NW);
  const int t1 = (int)((int64_t)(w + 1) * N / NW);
  u32x4* buf = kvbuf[wave];
  Engine acc;
  acc.init(q + ((int64_t)seq * Hq + (int64_t)kvh * G) * D, scale_l2, buf);
  const T* kc = static_cast<const T*>(kv.k);
  const T* vc = static_cast<const T*>(kv.v);
  if (!kv.paged) {
    const T* kb = kc + kv_row_offset(kv, seq, kvh, 0, D);
    const T* vb = vc + kv_row_offset(kv, seq, kvh, 0, D);
    if constexpr (Engine::PIPELINED) {
      // rows of the tile at t (0 past the end: its loads read nothing, so
      // every load is issued unconditionally)
      auto nr = [&](int t) { return max(0, min(32, t1 - t)); };
      typename Engine::Regs ra, rb;
      int t = t0;
      Engine::load(kb + (int64_t)t * D, vb + (int64_t)t * D, nr(t), ra.k, ra.v);
      while (t < t1) {
        const int tb = t + 32;
        Engine::load(kb + (int64_t)tb * D, vb + (int64_t)tb * D, nr(tb), rb.k, rb.v);
        __builtin_amdgcn_sched_barrier(0);  // loads stay ahead of the arithmetic
        acc.compute(buf, ra.k, ra.v, nr(t), 0xffffffffu);
        if (tb >= t1) break;
        const int tc = tb + 32;
        Engine::load(kb + (int64_t)tc * D, vb + (int64_t)tc * D, nr(tc), ra.k, ra.v);
        __builtin_amdgcn_sched_barrier(0);
        acc.compute(buf, rb.k, rb.v, nr(tb), 0xffffffffu);
        t = tc;
      }
    } else {
      for (int t = t0; t < t1; t += 32)
        acc.tile(buf, kb + (int64_t)t * D, vb + (int64_t)t * D, min(32, t1 - t), 0xffffffffu);
    }
  } else {
    for (int t = t0; t < t1; t += 32)
      acc.tile_gather(buf, kc, vc, min(32, t1 - t), 0xffffffffu,
                      [&](int i) { return kv_row_offset(kv, seq, kvh, t + i, D); });
  }
  acc.to_lds(st);
  __syncthreads();
  write_block_record<D, G>(st, ex_part + ((int64_t)u * splits + p) * G * RS);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <int D, int G>
static hipError_t decode_impl(const DecodeLaunch& x, const DArgs& a, const BudgetArgs& b, hipStream_t s) {
  const int nu = x.L.n_units;
  const int fblocks = x.residual == 2 ? x.L.fm_dim / 64 : 0;
  const unsigned fq_lds = fblocks ? (unsigned)query_features_lds<D, G>() : 0u;
  hipLaunchKernelGGL((k_score_clusters<D, G>), dim3(a.score_blocks + fblocks, nu), dim3(256), fq_lds, s, a);
  // one query head per KV head and a subcluster step of 3b: top-c and the
  // subclusters in one launch (3c)
  const bool fused = G == 1 && !x.whole && !x.shared &&
                     x.nb_chosen > 0 && x.L.max_C <= 1024;
  if (fused) {
    const dim3 grid(nu, (x.nb_chosen + 3) / 4);
    if (x.L.max_C <= 256)
      hipLaunchKernelGGL((k_select_sub1<D, 4>), grid, dim3(256), 0, s, a, b);
    else if (x.L.max_C <= 512)
      hipLaunchKernelGGL((k_select_sub1<D, 8>), grid, dim3(256), 0, s, a, b);
    else
      hipLaunchKernelGGL((k_select_sub1<D, 16>), grid, dim3(256), 0, s, a, b);
  } else if (x.L.max_C <= 256)
    hipLaunchKernelGGL((k_select_topc<G, 4>), dim3(nu), dim3(64 * G), 0, s, a, b);
  else if (x.L.max_C <= 512)
    hipLaunchKernelGGL((k_select_topc<G, 8>), dim3(nu), dim3(64 * G), 0, s, a, b);
  else if (x.L.max_C <= 1024)
    hipLaunchKernelGGL((k_select_topc<G, 16>), dim3(nu), dim3(64 * G), 0, s, a, b);
  else
    hipLaunchKernelGGL((k_select_topc<G, kMaxC / 64>), dim3(nu), dim3(64 * G), 0, s, a, b);
  // the residual of the clusters left out runs in blocks after the exact
  // ones, in the spread of their end times (with shared selection, the
  // feature-map residual's in the subcluster block kernel); none without a
  // residual
  const bool sub_blocks = !x.whole && !fused && x.shared;
  if (!x.whole && !fused) {
    if (!x.shared) {
      // one wave per chosen cluster
      if (x.nb_chosen > 0)
        hipLaunchKernelGGL((k_sub_wave<D, G>), dim3(nu, (x.nb_chosen + 3) / 4), dim3(256), 0, s, a, b, x.nb_chosen);
    } else {
      const int nrest_sub = x.residual == 2 ? a.rest_per_unit : 0;
      // (no chosen cluster anywhere and no feature-map residual: nothing to do)
      if (x.nb_chosen + nrest_sub > 0)
        hipLaunchKernelGGL((k_subclusters<D, G>), dim3(nu, x.nb_chosen + nrest_sub), dim3(256), 0, s, a, b,
                           x.nb_chosen, nrest_sub);
    }
  }
  const int nrest = (x.residual == 1 || (x.residual == 2 && !sub_blocks)) ? nu * a.rest_per_unit : 0;
  // the timing events (if any) are taken by the dispatches themselves: the
  // start of the first exact launch and the end of the last
  for (int r = 0; r < x.repeat; ++r) {
    hipEvent_t e0 = r == 0 ? x.ev_begin : nullptr, e1 = r + 1 == x.repeat ? x.ev_end : nullptr;
    if (x.dtype == MOG_BF16) {
      hipExtLaunchKernelGGL((k_exact<D, G, MfmaTile<D, G>, uint16_t>), dim3(x.nblk + nrest), dim3(256), 0, s, e0,
                            e1, 0, a);
    } else {
      hipExtLaunchKernelGGL((k_exact<D, G, RowAcc<D, G>, float>), dim3(x.nblk + nrest), dim3(256), 0, s, e0, e1, 0,
                            a);
    }
  }
  hipLaunchKernelGGL((k_merge<D>), dim3(x.Hq, x.L.n_seq), dim3(1024), 0, s, a.ws.ex_part, 0,
                     (const int32_t*)a.ws.uinfo, x.residual ? (const float*)a.ws.res_part : nullptr, x.nb_res,
                     a.rest_cl, x.whole ? nullptr : (const int32_t*)a.ws.n_chosen, (const mog_unit*)x.L.units, G,
                     x.Hq, x.L.n_kv_heads, x.out, x.lse);
  return hipGetLastError();
}

template <int D>
static hipError_t decode_g(const DecodeLaunch& x, const DArgs& a, const BudgetArgs& b, hipStream_t s) {
  switch (x.G) {
    case 1: return decode_impl<D, 1>(x, a, b, s);
    case 2: return decode_impl<D, 2>(x, a, b, s);
    case 3: return decode_impl<D, 3>(x, a, b, s);
    case 4: return decode_impl<D, 4>(x, a, b, s);
    case 5: return decode_impl<D, 5>(x, a, b, s);
    case 6: return decode_impl<D, 6>(x, a, b, s);
    case 7: return decode_impl<D, 7>(x, a, b, s);
    case 8: return decode_impl<D, 8>(x, a, b, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeLaunch& x, hipStream_t s) {
  DArgs a;
  a.L.units = x.L.units;
  a.L.k_mid = x.L.k_mid;
  a.L.v_mid = x.L.v_mid;
  a.L.sub_off = x.L.sub_off;
  a.L.cl_ms = x.L.cl_ms16;
  a.L.cl_vbar = x.L.cl_vbar16;
  a.L.sub_ms = x.L.sub_ms16;
  a.L.sub_vbar = x.L.sub_vbar16;
  a.L.cl_fold = x.L.cl_fold;
  a.L.sub_fold = x.L.sub_fold;
  a.L.fold_sub = x.L.fold_sub;
  a.L.fold_row0 = x.L.total_mid;
  a.L.fold_cap = x.L.fold_capacity;
  a.L.fm_w = x.L.fm_w;
  a.L.cl_fz = x.L.cl_fz;
  a.L.sub_fz = x.L.sub_fz;
  a.L.fm_dim = x.L.fm_dim;
  a.sqrt_scale = sqrtf(x.scale);
  a.score_blocks = (x.L.max_C + 4 * kScoreRowsPerWave - 1) / (4 * kScoreRowsPerWave);
  a.kv = x.kv;
  a.q = x.q;
  a.out = x.out;
  a.lse = x.lse;
  a.sel_c = x.sel_c;
  a.sel_s = x.sel_s;
  a.c_stride = x.c_stride;
  a.s_stride = x.s_stride;
  a.Hq = x.Hq;
  a.Hkv = x.L.n_kv_heads;
  a.n_sink = x.L.n_sink;
  a.n_recent = x.L.n_recent;
  a.residual = x.residual;
  a.shared = x.shared;
  a.splits = x.splits;
  a.nb_res = x.nb_res;
  a.n_units = x.L.n_units;
  a.nblk = x.nblk;
  a.cstride = x.L.max_C;
  a.scale_l2 = x.scale * kLog2e;
  a.half_s2_l2 = 0.5f * x.scale * x.scale * kLog2e;
  a.L_head_dim = x.D;
  a.whole = x.whole;
  a.half = x.half;
  {
    // equal units: every sequence with the first one's length and fold count
    bool eq = true;
    for (int s = 1; s < x.L.n_seq; ++s)
      eq = eq && x.L.seq_lens[s] == x.L.seq_lens[0] && x.L.fold_count[s] == x.L.fold_count[0];
    const UnitSizes z = unit_sizes(x.L.seq_lens[0] - x.L.fold_count[0], x.L.n_sink, x.L.n_recent);
    a.uni_C = eq ? z.C : 0;
    a.uni_S = z.S;
    a.uni_nmid = z.n_mid;
    a.uni_N = x.L.seq_lens[0];
    a.uni_nfold = x.L.fold_count[0];
  }
  a.rest_cl = rest_clusters_per_block(x.residual, x.L.n_units, x.L.max_C);
  a.rest_per_unit = (x.L.max_C + a.rest_cl - 1) / a.rest_cl;
  a.ws = x.ws;
  BudgetArgs b;
  for (int i = 0; i < MOG_MAX_SEQ; ++i) {
    b.top_c[i] = x.seq.top_c[i];
    b.top_s[i] = x.seq.top_s[i];
  }
  return x.D == 128 ? decode_g<128>(x, a, b, s) : decode_g<64>(x, a, b, s);
}

template <int D, int G>
static hipError_t dense_impl(const DenseLaunch& x, hipStream_t s) {
  const int nu = x.seq.n_seq * x.n_kv_heads;
  for (int r = 0; r < x.repeat; ++r) {
    hipEvent_t e0 = r == 0 ? x.ev_begin : nullptr, e1 = r + 1 == x.repeat ? x.ev_end : nullptr;
    if (x.dtype == MOG_BF16) {
      hipExtLaunchKernelGGL((k_dense<D, G, MfmaTile<D, G>, uint16_t>), dim3(x.splits, nu), dim3(256), 0, s, e0, e1, 0,
                            x.kv, x.q, x.Hq, x.n_kv_heads, x.splits, x.scale * kLog2e, x.seq, x.ex_part);
    } else {
      hipExtLaunchKernelGGL((k_dense<D, G, RowAcc<D, G>, float>), dim3(x.splits, nu), dim3(256), 0, s, e0, e1, 0,
                            x.kv, x.q, x.Hq, x.n_kv_heads, x.splits, x.scale * kLog2e, x.seq, x.ex_part);
    }
  }
  hipLaunchKernelGGL((k_merge<D>), dim3(x.Hq, x.seq.n_seq), dim3(1024), 0, s, x.ex_part, x.splits,
                     (const int32_t*)nullptr, (const float*)nullptr, 0, 1, (const int32_t*)nullptr,
                     (const mog_unit*)nullptr, G, x.Hq, x.n_kv_heads, x.out, x.lse);
  return hipGetLastError();
}

template <int D>
static hipError_t dense_g(const DenseLaunch& x, hipStream_t s) {
  switch (x.G) {
    case 1: return dense_impl<D, 1>(x, s);
    case 2: return dense_impl<D, 2>(x, s);
    case 3: return dense_impl<D, 3>(x, s);
    case 4: return dense_impl<D, 4>(x, s);
    case 5: return dense_impl<D, 5>(x, s);
    case 6: return dense_impl<D, 6>(x, s);
    case 7: return dense_impl<D, 7>(x, s);
    case 8: return dense_impl<D, 8>(x, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_dense(const DenseLaunch& x, hipStream_t s) {
  return x.D == 128 ? dense_g<128>(x, s) : dense_g<64>(x, s);
}

}  // namespace mog
