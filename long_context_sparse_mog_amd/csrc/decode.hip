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
#include "attn_tile.h"
#include "mog_internal.h"

namespace mog {

struct LayoutRef {
  const mog_unit* units;
  const void* k_mid;
  const void* v_mid;
  const int32_t* sub_off;
  const float* cl_ms;
  const float* cl_vbar;
  const float* sub_ms;
  const float* sub_vbar;
};

struct DArgs {
  LayoutRef L;
  KVRef kv;
  const float* q;
  float* out;
  float* lse;
  int32_t* sel_c;
  int32_t* sel_s;
  int32_t c_stride, s_stride, Hq, Hkv, n_sink, n_recent, residual, splits, nb_res;
  float scale_l2;    // scale * log2(e)
  float half_s2_l2;  // scale^2 / 2 * log2(e)
  DecodeWS ws;
};

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

template <int N>
__device__ inline void load_floats(const float* p, float (&x)[N]) {
  if constexpr (N == 4) {
    float4 t = *reinterpret_cast<const float4*>(p);
    x[0] = t.x; x[1] = t.y; x[2] = t.z; x[3] = t.w;
  } else if constexpr (N == 2) {
    float2 t = *reinterpret_cast<const float2*>(p);
    x[0] = t.x; x[1] = t.y;
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = p[i];
  }
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

// Scores of R group rows (already loaded, x[r][EPL] per lane): lane r ends
// up holding the G scores of row r (without the count term).
template <int D, int G, int R>
__device__ inline void score_rows(const float (&x)[R][D / 32], const float (&coef)[G][D / 32], int lane,
                                  float (&mine)[G]) {
  constexpr int EPL = D / 32;
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float t = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) t += coef[h][e] * x[r][e];
      t = wave_sum_dpp(t);
      if (lane == r) mine[h] = t;
    }
  }
}

// ---------------------------------------------------------------------------
// 1. Cluster scores: score[g][h] = log2 n_g + log2e (scale q_h.mu_g +
//    scale^2/2 sum_i q_{h,i}^2 var_{g,i}); -inf for an empty cluster.
//    Grid (ceil(maxC/16), units); each wave loads 4 cluster rows at once.
// ---------------------------------------------------------------------------
template <int D, int G>
__global__ __launch_bounds__(256) void k_score_clusters(DArgs a) {
  constexpr int EPL = D / 32;
  const int u = blockIdx.y;
  const mog_unit U = a.L.units[u];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g0 = blockIdx.x * 16 + wave * 4;
  if (g0 >= U.C) return;
  const float* qb = a.q + ((int64_t)U.seq * a.Hq + (int64_t)U.kv_head * G) * D;
  float coef[G][EPL];
  score_coefs<D, G>(a, qb, coef);
  const int32_t* off = a.L.sub_off + U.off_base;
  float x[4][EPL];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int g = min(g0 + k, U.C - 1);
    load_floats<EPL>(a.L.cl_ms + (U.cl_base + g) * (2 * D) + lane * EPL, x[k]);
  }
  float mine[G];
#pragma unroll
  for (int h = 0; h < G; ++h) mine[h] = 0.f;
  score_rows<D, G, 4>(x, coef, lane, mine);
  // lane k (< 4) now holds the scores of cluster g0 + k
  const int g = g0 + lane;
  if (lane < 4 && g < U.C) {
    const int64_t cg = U.cl_base + g;
    const int n = off[(g + 1) * U.S] - off[g * U.S];
    const float lg = n > 0 ? log2f((float)n) : -INFINITY;
#pragma unroll
    for (int h = 0; h < G; ++h) a.ws.cl_score[cg * G + h] = n > 0 ? mine[h] + lg : -INFINITY;
    a.ws.cl_mask[cg] = 0u;
  }
}

// ---------------------------------------------------------------------------
// 2. Top-c clusters of one query head: radix select (four 8-bit digits, most
//    significant first) of the c-th largest order-preserving key, then the
//    keys above it and the lowest-index keys equal to it.  Empty clusters
//    are never chosen.  Grid (G, units), 256 threads.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_select_topc(DArgs a, BudgetArgs b, int G) {
  const int h = blockIdx.x, u = blockIdx.y, tid = threadIdx.x;
  const mog_unit U = a.L.units[u];
  const int C = U.C;
  __shared__ uint32_t keys[kMaxC];
  __shared__ int hist[256];
  __shared__ int sh[16];
  __shared__ int sh_b, sh_above;

  int nvalid = 0;
  for (int i = tid; i < C; i += 256) {
    const float sc = a.ws.cl_score[(U.cl_base + i) * G + h];
    const bool valid = sc != -INFINITY;
    keys[i] = valid ? float_key(sc) : 0u;
    nvalid += valid;
  }
  int total;
  block_excl_scan<256>(nvalid, sh, total);
  int want = b.top_c[U.seq];
  want = want < 0 ? 0 : want;
  int kk = want < total ? want : total;
  const int c_eff = kk;
  uint32_t prefix = 0u, pmask = 0u;
  if (c_eff > 0) {
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      hist[tid] = 0;
      __syncthreads();
      for (int i = tid; i < C; i += 256) {
        const uint32_t k = keys[i];
        if (k != 0u && (k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1);
      }
      __syncthreads();
      const int v = hist[255 - tid];
      int tot;
      const int excl = block_excl_scan<256>(v, sh, tot);
      if (excl < kk && excl + v >= kk) {
        sh_b = 255 - tid;
        sh_above = excl;
      }
      __syncthreads();
      kk -= sh_above;
      prefix |= (uint32_t)sh_b << shift;
      pmask |= 255u << shift;
      __syncthreads();
    }
  }
  // keys > prefix are all chosen; kk of the keys == prefix, lowest index first
  const int E = (C + 255) / 256;
  const int lo = tid * E;
  const int hi = min(C, lo + E);
  int neq = 0;
  if (c_eff > 0)
    for (int i = lo; i < hi; ++i) neq += keys[i] == prefix;
  int tot;
  int eqr = block_excl_scan<256>(neq, sh, tot);
  uint32_t selbits = 0u;
  int nsel = 0;
  if (c_eff > 0) {
    for (int i = lo; i < hi; ++i) {
      const uint32_t k = keys[i];
      bool s = false;
      if (k > prefix) {
        s = true;
      } else if (k == prefix) {
        s = eqr < kk;
        ++eqr;
      }
      if (s) {
        selbits |= 1u << (i - lo);
        ++nsel;
      }
    }
  }
  int r = block_excl_scan<256>(nsel, sh, tot);
  const int hq = U.kv_head * G + h;
  const int64_t row = (int64_t)U.seq * a.Hq + hq;
  for (int i = lo; i < hi; ++i) {
    int rank = -1;
    if ((selbits >> (i - lo)) & 1u) {
      rank = r++;
      atomicOr(&a.ws.cl_mask[U.cl_base + i], 1u << h);
      if (a.sel_c) a.sel_c[row * a.c_stride + rank] = i;
    }
    a.ws.cl_rank[(U.cl_base + i) * G + h] = rank;
  }
  if (a.sel_c)
    for (int j = c_eff + tid; j < a.c_stride; j += 256) a.sel_c[row * a.c_stride + j] = -1;
  if (a.sel_s) {
    const int64_t base = row * a.c_stride * a.s_stride;
    for (int j = c_eff * a.s_stride + tid; j < a.c_stride * a.s_stride; j += 256) a.sel_s[base + j] = -1;
  }
}

// ---------------------------------------------------------------------------
// 3. Subclusters and residual.  Grid (nb_chosen + nb_rest, units):
//    * block x < nb_chosen takes the x-th chosen cluster of its unit (in
//      cluster order; found by a block scan of the head masks): scores its S
//      subclusters for every head (one batch of row loads per wave), picks
//      the top-s of each head that chose the cluster, writes the subcluster
//      head masks and the cluster's exactly-read row count, and accumulates
//      the residual terms of the subclusters a choosing head left out;
//    * block nb_chosen + y covers clusters [16y, 16y+16) (4 per wave): the
//      residual terms of every head that left a cluster out, and a zero row
//      count for clusters no head chose.
//    Every block writes one residual record per head (slot = block index).
// ---------------------------------------------------------------------------
template <int D, int G>
__device__ inline void write_residual_record(float (*st)[G][D + 2], float* dst) {
  constexpr int RS = D + kPartPad;
  for (int idx = threadIdx.x; idx < G * D; idx += 256) {
    const int h = idx / D, e = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, st[w][h][D]);
    float l = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = st[w][h][D];
      const float f = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
      l += f * st[w][h][D + 1];
      o += f * st[w][h][e];
    }
    dst[h * RS + e] = o;
    if (e == 0) {
      dst[h * RS + D] = M;
      dst[h * RS + D + 1] = l;
    }
  }
}

template <int D, int G>
__global__ __launch_bounds__(256) void k_subclusters(DArgs a, BudgetArgs b, int nb_chosen) {
  constexpr int EPL = D / 32;
  constexpr int VPL = D / 64;
  constexpr int RS = D + kPartPad;
  constexpr int RPW = kMaxS / 4;   // subcluster rows per wave
  __shared__ float st[4][G][D + 2];
  __shared__ float lds_sc[kMaxS][G];
  __shared__ uint32_t lds_sm[kMaxS];
  __shared__ int sh[16];
  __shared__ int found;
  const int u = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const mog_unit U = a.L.units[u];
  const int S = U.S, C = U.C;
  const uint32_t all = (1u << G) - 1u;
  const int32_t* off = a.L.sub_off + U.off_base;
  float rm[G], rl[G], ro[G][VPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    rm[h] = -INFINITY;
    rl[h] = 0.f;
#pragma unroll
    for (int e = 0; e < VPL; ++e) ro[h][e] = 0.f;
  }
  float* dst = a.ws.res_part + ((int64_t)u * a.nb_res + blockIdx.x) * G * RS;

  if ((int)blockIdx.x < nb_chosen) {
    // -------- the x-th chosen cluster ---------------------------------------
    const int x = blockIdx.x;
    {
      constexpr int EM = kMaxC / 256;
      const int E = (C + 255) / 256;
      int cnt = 0;
#pragma unroll
      for (int k = 0; k < EM; ++k) {
        const int g = tid * E + k;
        if (k < E && g < C) cnt += a.ws.cl_mask[U.cl_base + g] != 0u;
      }
      if (tid == 0) found = -1;
      int total;
      int base = block_excl_scan<256>(cnt, sh, total);
      if (x >= base && x < base + cnt) {
        for (int k = 0; k < EM; ++k) {
          const int g = tid * E + k;
          if (k < E && g < C && a.ws.cl_mask[U.cl_base + g] != 0u) {
            if (base == x) found = g;
            ++base;
          }
        }
      }
      __syncthreads();
    }
    const int g = found;
    if (g >= 0) {
      const int64_t cg = U.cl_base + g;
      const int64_t sg0 = U.sub_base + (int64_t)g * S;
      const uint32_t mask = a.ws.cl_mask[cg];
      const float* qb = a.q + ((int64_t)U.seq * a.Hq + (int64_t)U.kv_head * G) * D;
      float coef[G][EPL];
      score_coefs<D, G>(a, qb, coef);
      // scores: wave w takes rows w, w+4, ...
      float xr[RPW][EPL];
#pragma unroll
      for (int k = 0; k < RPW; ++k) {
        const int i = min(wave + 4 * k, S - 1);
        load_floats<EPL>(a.L.sub_ms + (sg0 + i) * (2 * D) + lane * EPL, xr[k]);
      }
#pragma unroll
      for (int k = 0; k < RPW; ++k) {
        const int i = wave + 4 * k;
        if (i >= S) break;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float t = 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) t += coef[h][e] * xr[k][e];
          t = wave_sum_dpp(t);
          if (lane == 0) lds_sc[i][h] = t;
        }
      }
      if (tid < kMaxS) lds_sm[tid] = 0u;
      __syncthreads();
      // full scores (count term added; -inf for an empty subcluster)
      if (tid < S * G) {
        const int i = tid / G, h = tid % G;
        const int cnt = off[g * S + i + 1] - off[g * S + i];
        lds_sc[i][h] = cnt > 0 ? lds_sc[i][h] + log2f((float)cnt) : -INFINITY;
      }
      __syncthreads();
      // top-s of each choosing head: wave w handles heads w, w+4
      int my_cnt = 0;
      if (lane < S) my_cnt = off[g * S + lane + 1] - off[g * S + lane];
      const bool valid = lane < S && my_cnt > 0;
      int s_keep = b.top_s[U.seq];
      s_keep = s_keep < 0 ? 0 : s_keep;
      for (int h = wave; h < G; h += 4) {
        if (!((mask >> h) & 1u)) continue;
        const float my = valid ? lds_sc[lane][h] : -INFINITY;
        int rank = 0;
#pragma unroll
        for (int j = 0; j < kMaxS; ++j) {
          if (j >= S) break;
          const float o = lds_sc[j][h];
          if (o != -INFINITY && (o > my || (o == my && j < lane))) ++rank;
        }
        const bool sel = valid && rank < s_keep;
        if (sel) atomicOr(&lds_sm[lane], 1u << h);
        if (a.sel_s) {
          const unsigned long long bal = __ballot(sel);
          const int rc = a.ws.cl_rank[cg * G + h];
          const int hq = U.kv_head * G + h;
          const int64_t base = (((int64_t)U.seq * a.Hq + hq) * a.c_stride + rc) * a.s_stride;
          if (sel) a.sel_s[base + __popcll(bal & ((1ull << lane) - 1ull))] = lane;
          for (int j = __popcll(bal) + lane; j < a.s_stride; j += 64) a.sel_s[base + j] = -1;
        }
      }
      __syncthreads();
      if (tid < S) a.ws.sub_mask[sg0 + tid] = lds_sm[tid];
      if (wave == 0) {
        int rows = (lane < S && lds_sm[lane]) ? my_cnt : 0;
#pragma unroll
        for (int o2 = 1; o2 < 64; o2 <<= 1) rows += __shfl_xor(rows, o2, 64);
        if (lane == 0) a.ws.cl_rows[cg] = rows;
      }
      // residual of the subclusters a choosing head left out: wave w takes
      // subclusters w, w+4, ...
      if (a.residual) {
        float vb[RPW][VPL];
        uint32_t need[RPW];
#pragma unroll
        for (int k = 0; k < RPW; ++k) {
          const int i = wave + 4 * k;
          need[k] = 0u;
          if (i < S && off[g * S + i + 1] > off[g * S + i]) need[k] = mask & ~lds_sm[i];
          if (need[k]) load_floats<VPL>(a.L.sub_vbar + (sg0 + i) * D + lane * VPL, vb[k]);
        }
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
  } else {
    // -------- residual of clusters left out, 4 clusters per wave ------------
    const int y = blockIdx.x - nb_chosen;
    for (int k = 0; k < 4; ++k) {
      const int g = y * 16 + wave * 4 + k;
      if (g >= C) break;
      const int64_t cg = U.cl_base + g;
      const uint32_t mask = a.ws.cl_mask[cg];
      if (mask == 0u && lane == 0) a.ws.cl_rows[cg] = 0;
      const int n_g = off[(g + 1) * S] - off[g * S];
      const uint32_t unchosen = n_g > 0 ? (all & ~mask) : 0u;
      if (unchosen && a.residual) {
        float vb[VPL];
        load_floats<VPL>(a.L.cl_vbar + cg * D + lane * VPL, vb);
#pragma unroll
        for (int h = 0; h < G; ++h)
          if ((unchosen >> h) & 1u) add_group<VPL>(rm[h], rl[h], ro[h], a.ws.cl_score[cg * G + h], vb);
      }
    }
  }

#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int e = 0; e < VPL; ++e) st[wave][h][lane * VPL + e] = ro[h][e];
    if (lane == 0) {
      st[wave][h][D] = rm[h];
      st[wave][h][D + 1] = rl[h];
    }
  }
  __syncthreads();
  write_residual_record<D, G>(st, dst);
}

// ---------------------------------------------------------------------------
// 4. Exact split-K pass.  The rows a unit reads exactly are laid out
//    virtually as [sink anchors | recent anchors | rows of every cluster's
//    chosen subclusters, clusters in order]; wave w of the unit covers
//    virtual rows [w*T/NW, (w+1)*T/NW).  Every block first scans the
//    per-cluster row counts into LDS, then each wave locates its first
//    cluster by binary search and walks the chosen subclusters (adjacent
//    subclusters chosen by the same heads form one contiguous run).  The
//    block also folds the residual partials p, p+splits, ... of its unit
//    into its record.  Grid (splits, units).
// ---------------------------------------------------------------------------
template <int D, int G, typename Engine, typename T>
__global__ __launch_bounds__(256) void k_exact(DArgs a) {
  constexpr int RS = D + kPartPad;
  __shared__ u32x4 kvbuf[4][Engine::BUF];
  __shared__ float st[4 * G * (D + 2)];
  __shared__ int vpre[kMaxC + 1];
  __shared__ int sh[16];
  const int u = blockIdx.y, p = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const mog_unit U = a.L.units[u];
  const int C = U.C, S = U.S;
  const int A = a.n_sink + a.n_recent;
  {
    constexpr int EM = kMaxC / 256;
    const int E = (C + 255) / 256;
    int loc[EM];
    int sum = 0;
#pragma unroll
    for (int k = 0; k < EM; ++k) {
      const int g = tid * E + k;
      const int v = (k < E && g < C) ? a.ws.cl_rows[U.cl_base + g] : 0;
      loc[k] = v;
      sum += v;
    }
    int total;
    int base = block_excl_scan<256>(sum, sh, total);
#pragma unroll
    for (int k = 0; k < EM; ++k) {
      const int g = tid * E + k;
      if (k < E && g < C) vpre[g] = base;
      base += loc[k];
    }
    if (tid == 0) vpre[C] = total;
    __syncthreads();
  }
  const int64_t Tt = A + vpre[C];
  const int NW = a.splits * 4;
  const int w = p * 4 + wave;
  const int64_t r0 = (int64_t)w * Tt / NW;
  const int64_t r1 = (int64_t)(w + 1) * Tt / NW;
  Engine acc;
  acc.init(a.q + ((int64_t)U.seq * a.Hq + (int64_t)U.kv_head * G) * D, a.scale_l2);
  u32x4* buf = kvbuf[wave];
  const T* kc = static_cast<const T*>(a.kv.k);
  const T* vc = static_cast<const T*>(a.kv.v);
  const uint32_t all = (1u << G) - 1u;
  int64_t x = r0;
  if (x < r1 && x < A) {
    // anchors from the KV cache: virtual row x < n_sink is token x, else
    // token N - n_recent + (x - n_sink)
    const KVRef kv = a.kv;
    const int seq = U.seq, kvh = U.kv_head;
    const int64_t xe = r1 < A ? r1 : A;
    while (x < xe) {
      const bool sink = x < a.n_sink;
      const int tok = sink ? (int)x : U.N - a.n_recent + (int)(x - a.n_sink);
      const int64_t seg_end = sink ? (a.n_sink < xe ? a.n_sink : xe) : xe;
      const int nr = (int)((seg_end - x) < 32 ? (seg_end - x) : 32);
      if (!kv.paged) {
        const int64_t base = kv_row_offset(kv, seq, kvh, tok, D);
        acc.tile(buf, kc + base, vc + base, nr, all);
      } else {
        acc.tile_gather(buf, kc, vc, nr, all, [&](int i) { return kv_row_offset(kv, seq, kvh, tok + i, D); });
      }
      x += nr;
    }
  }
  if (x < r1) {
    const T* km = static_cast<const T*>(a.L.k_mid);
    const T* vm = static_cast<const T*>(a.L.v_mid);
    const int32_t* off = a.L.sub_off + U.off_base;
    int64_t y = x - A;
    const int64_t y1 = r1 - A;
    int lo = 0, hi = C;  // last cluster g with vpre[g] <= y
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (vpre[mid] <= y) lo = mid; else hi = mid;
    }
    int g = lo;
    while (y < y1 && g < C) {
      if (vpre[g + 1] == vpre[g]) {
        ++g;
        continue;
      }
      int skip = (int)(y - vpre[g]);
      // the S subclusters of cluster g, one per lane
      const int64_t sg0 = U.sub_base + (int64_t)g * S;
      uint32_t my_m = 0u;
      int my_st = 0, my_en = 0;
      if (lane < S) {
        my_m = a.ws.sub_mask[sg0 + lane];
        my_st = off[g * S + lane];
        my_en = off[g * S + lane + 1];
      }
      unsigned long long chosen = __ballot(my_m != 0u && my_en > my_st);
      while (chosen && y < y1) {
        const int i = __ffsll((long long)chosen) - 1;
        const uint32_t m = (uint32_t)__shfl((int)my_m, i, 64);
        const int st0 = __shfl(my_st, i, 64);
        int en = __shfl(my_en, i, 64);
        chosen &= chosen - 1ull;
        // absorb following subclusters chosen by the same heads
        while (chosen) {
          const int j = __ffsll((long long)chosen) - 1;
          if ((uint32_t)__shfl((int)my_m, j, 64) != m || __shfl(my_st, j, 64) != en) break;
          en = __shfl(my_en, j, 64);
          chosen &= chosen - 1ull;
        }
        const int len = en - st0;
        if (skip >= len) {
          skip -= len;
          continue;
        }
        const int take = (int)((int64_t)(len - skip) < y1 - y ? (len - skip) : (y1 - y));
        const int64_t base = (U.row_base + st0 + skip) * D;
        for (int t0 = 0; t0 < take; t0 += 32)
          acc.tile(buf, km + base + (int64_t)t0 * D, vm + base + (int64_t)t0 * D, min(32, take - t0), m);
        y += take;
        skip = 0;
      }
      ++g;
    }
  }
  acc.to_lds(st);
  __syncthreads();
  const int nres = a.residual ? a.nb_res : 0;
  const int n_extra = nres > p ? (nres - p + a.splits - 1) / a.splits : 0;
  const float* rp = a.ws.res_part + (int64_t)u * a.nb_res * G * RS;
  write_block_record<D, G>(st, n_extra, [&](int j) { return rp + (int64_t)(p + j * a.splits) * G * RS; },
                           a.ws.ex_part + ((int64_t)u * a.splits + p) * G * RS);
}

// ---------------------------------------------------------------------------
// 5. Merge: per query head, the records of the unit's splits: one max, one
//    weighted sum, one normalisation.  Grid (Hq, n_seq), 256 threads.
// ---------------------------------------------------------------------------
constexpr int kMaxParts = 1024;

template <int D>
__global__ __launch_bounds__(256) void k_merge(const float* part, int n_part, int G, int Hq, int Hkv, float* out,
                                               float* lse) {
  constexpr int RS = D + kPartPad;
  constexpr int NG = 256 / D;
  __shared__ float wts[kMaxParts];
  __shared__ float sh[8];
  __shared__ float acc[NG][D];
  const int hq = blockIdx.x, seq = blockIdx.y, tid = threadIdx.x;
  const int kvh = hq / G, h = hq % G;
  const int u = seq * Hkv + kvh;
  const float* base = part + ((int64_t)u * n_part * G + h) * RS;
  const int64_t stride = (int64_t)G * RS;
  float M = -INFINITY;
  for (int i = tid; i < n_part; i += 256) M = fmaxf(M, base[i * stride + D]);
  M = block_max<256>(M, sh);
  float den = 0.f;
  for (int i = tid; i < n_part; i += 256) {
    const float m = base[i * stride + D];
    const float f = (m == -INFINITY) ? 0.f : exp2f(m - M);
    wts[i] = f;
    den += f * base[i * stride + D + 1];
  }
  den = block_sum<256>(den, sh);
  const int d = tid % D, grp = tid / D;
  float num = 0.f;
#pragma unroll 8
  for (int i = grp; i < n_part; i += NG) num += wts[i] * base[i * stride + d];
  acc[grp][d] = num;
  __syncthreads();
  if (grp == 0) {
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < NG; ++k) t += acc[k][d];
    const int64_t orow = (int64_t)seq * Hq + hq;
    out[orow * D + d] = den > 0.f ? t / den : 0.f;
    if (lse && d == 0) lse[orow] = den > 0.f ? (M + log2f(den)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// Dense baseline: wave w of unit u covers tokens [w*N/NW, (w+1)*N/NW).
// ---------------------------------------------------------------------------
template <int D, int G, typename Engine, typename T>
__global__ __launch_bounds__(256) void k_dense(KVRef kv, const float* q, int Hq, int Hkv, int splits,
                                               float scale_l2, SeqArgs seq_args, float* ex_part) {
  constexpr int RS = D + kPartPad;
  __shared__ u32x4 kvbuf[4][Engine::BUF];
  __shared__ float st[4 * G * (D + 2)];
  const int u = blockIdx.y, p = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  const int seq = u / Hkv, kvh = u % Hkv;
  const int64_t N = seq_args.len[seq];
  const int NW = splits * 4;
  const int w = p * 4 + wave;
  const int t0 = (int)((int64_t)w * N / NW);
  const int t1 = (int)((int64_t)(w + 1) * N / NW);
  Engine acc;
  acc.init(q + ((int64_t)seq * Hq + (int64_t)kvh * G) * D, scale_l2);
  const T* kc = static_cast<const T*>(kv.k);
  const T* vc = static_cast<const T*>(kv.v);
  u32x4* buf = kvbuf[wave];
  if (!kv.paged) {
    const int64_t base = kv_row_offset(kv, seq, kvh, 0, D);
    for (int t = t0; t < t1; t += 32)
      acc.tile(buf, kc + base + (int64_t)t * D, vc + base + (int64_t)t * D, min(32, t1 - t), 0xffffffffu);
  } else {
    for (int t = t0; t < t1; t += 32)
      acc.tile_gather(buf, kc, vc, min(32, t1 - t), 0xffffffffu,
                      [&](int i) { return kv_row_offset(kv, seq, kvh, t + i, D); });
  }
  acc.to_lds(st);
  __syncthreads();
  write_block_record<D, G>(st, 0, [](int) { return (const float*)nullptr; },
                           ex_part + ((int64_t)u * splits + p) * G * RS);
}

// ---------------------------------------------------------------------------
// Unit table of a layout (same arithmetic as the host carving).
// ---------------------------------------------------------------------------
__global__ void k_layout_table(mog_unit* units, SeqArgs seq, int Hkv, int n_sink, int n_recent) {
  const int u = blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= seq.n_seq * Hkv) return;
  const int s = u / Hkv, kvh = u % Hkv;
  int64_t row = 0, cl = 0, sub = 0, offb = 0;
  for (int s2 = 0; s2 < s; ++s2) {
    const UnitSizes z = unit_sizes(seq.len[s2], n_sink, n_recent);
    row += (int64_t)Hkv * z.n_mid;
    cl += (int64_t)Hkv * z.C;
    sub += (int64_t)Hkv * z.C * z.S;
    offb += (int64_t)Hkv * (z.C * z.S + 1);
  }
  const UnitSizes z = unit_sizes(seq.len[s], n_sink, n_recent);
  mog_unit U;
  U.seq = s;
  U.kv_head = kvh;
  U.N = seq.len[s];
  U.n_mid = z.n_mid;
  U.C = z.C;
  U.S = z.S;
  U.reserved0 = U.reserved1 = 0;
  U.row_base = row + (int64_t)kvh * z.n_mid;
  U.cl_base = cl + (int64_t)kvh * z.C;
  U.sub_base = sub + (int64_t)kvh * z.C * z.S;
  U.off_base = offb + (int64_t)kvh * (z.C * z.S + 1);
  units[u] = U;
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_layout_table(const mog_layout& L, const SeqArgs& seq, hipStream_t s) {
  const int n = L.n_units;
  hipLaunchKernelGGL(k_layout_table, dim3((n + 255) / 256), dim3(256), 0, s, L.units, seq,
                     L.n_kv_heads, L.n_sink, L.n_recent);
  return hipGetLastError();
}

template <int D, int G>
static hipError_t decode_impl(const DecodeLaunch& x, const DArgs& a, const BudgetArgs& b, hipStream_t s) {
  const int nu = x.L.n_units;
  hipLaunchKernelGGL((k_score_clusters<D, G>), dim3((x.L.max_C + 15) / 16, nu), dim3(256), 0, s, a);
  hipLaunchKernelGGL(k_select_topc, dim3(G, nu), dim3(256), 0, s, a, b, G);
  hipLaunchKernelGGL((k_subclusters<D, G>), dim3(x.nb_res, nu), dim3(256), 0, s, a, b, x.nb_chosen);
  if (x.ev_begin) hipEventRecord(x.ev_begin, s);
  if (x.dtype == MOG_BF16) {
    hipLaunchKernelGGL((k_exact<D, G, MfmaTile<D, G>, uint16_t>), dim3(x.splits, nu), dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((k_exact<D, G, RowAcc<D, G>, float>), dim3(x.splits, nu), dim3(256), 0, s, a);
  }
  if (x.ev_end) hipEventRecord(x.ev_end, s);
  hipLaunchKernelGGL((k_merge<D>), dim3(x.Hq, x.L.n_seq), dim3(256), 0, s, a.ws.ex_part, x.splits, G, x.Hq,
                     x.L.n_kv_heads, x.out, x.lse);
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
  a.L.cl_ms = x.L.cl_ms;
  a.L.cl_vbar = x.L.cl_vbar;
  a.L.sub_ms = x.L.sub_ms;
  a.L.sub_vbar = x.L.sub_vbar;
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
  a.splits = x.splits;
  a.nb_res = x.nb_res;
  a.scale_l2 = x.scale * kLog2e;
  a.half_s2_l2 = 0.5f * x.scale * x.scale * kLog2e;
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
  if (x.ev_begin) hipEventRecord(x.ev_begin, s);
  if (x.dtype == MOG_BF16) {
    hipLaunchKernelGGL((k_dense<D, G, MfmaTile<D, G>, uint16_t>), dim3(x.splits, nu), dim3(256), 0, s, x.kv, x.q,
                       x.Hq, x.n_kv_heads, x.splits, x.scale * kLog2e, x.seq, x.ex_part);
  } else {
    hipLaunchKernelGGL((k_dense<D, G, RowAcc<D, G>, float>), dim3(x.splits, nu), dim3(256), 0, s, x.kv, x.q,
                       x.Hq, x.n_kv_heads, x.splits, x.scale * kLog2e, x.seq, x.ex_part);
  }
  if (x.ev_end) hipEventRecord(x.ev_end, s);
  hipLaunchKernelGGL((k_merge<D>), dim3(x.Hq, x.seq.n_seq), dim3(256), 0, s, x.ex_part, x.splits, G, x.Hq,
                     x.n_kv_heads, x.out, x.lse);
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
