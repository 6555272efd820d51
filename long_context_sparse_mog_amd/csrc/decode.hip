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
// Block-wide exclusive prefix sum over NT threads (NT a multiple of 64).
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

template <int D, int G>
__device__ inline void score_row(const float* row, const float (&coef)[G][D / 32], float (&s)[G]) {
  constexpr int EPL = D / 32;
  const int lane = threadIdx.x & 63;
  float x[EPL];
  load_floats<EPL>(row + lane * EPL, x);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float t = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) t += coef[h][e] * x[e];
    s[h] = wave_sum(t);
  }
}

// ---------------------------------------------------------------------------
// 1. Cluster scores: score[g][h] = log2 n_g + log2e (scale q_h.mu_g +
//    scale^2/2 sum_i q_{h,i}^2 var_{g,i}); -inf for an empty cluster.
//    Grid (ceil(maxC/64), units), 4 waves, each wave 16 clusters.
// ---------------------------------------------------------------------------
template <int D, int G>
__global__ __launch_bounds__(256) void k_score_clusters(DArgs a) {
  const int u = blockIdx.y;
  const mog_unit U = a.L.units[u];
  const int g_begin = blockIdx.x * 64;
  if (g_begin >= U.C) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* qb = a.q + ((int64_t)U.seq * a.Hq + (int64_t)U.kv_head * G) * D;
  float coef[G][D / 32];
  score_coefs<D, G>(a, qb, coef);
  const int32_t* off = a.L.sub_off + U.off_base;
  for (int k = 0; k < 16; ++k) {
    const int g = g_begin + wave + 4 * k;
    if (g >= U.C) break;
    const int64_t cg = U.cl_base + g;
    float s[G];
    score_row<D, G>(a.L.cl_ms + cg * (2 * D), coef, s);
    const int n = off[(g + 1) * U.S] - off[g * U.S];
    const float lg = n > 0 ? log2f((float)n) : -INFINITY;
    float mine = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h)
      if (lane == h) mine = s[h];
    if (lane < G) a.ws.cl_score[cg * G + lane] = n > 0 ? mine + lg : -INFINITY;
    if (lane == 0) a.ws.cl_mask[cg] = 0u;
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
// 3. Per cluster: the residual term of every head that left the cluster out;
//    for the heads that chose it, subcluster scores, top-s per head, and the
//    residual terms of the subclusters a head left out.  Writes the head
//    mask of every subcluster and one residual partial per (block, head).
//    Grid (ceil(maxC/16), units), 4 waves x 4 clusters.
// ---------------------------------------------------------------------------
template <int D, int G>
__global__ __launch_bounds__(256) void k_subclusters(DArgs a, BudgetArgs b) {
  constexpr int VPL = D / 64;
  constexpr int RS = D + kPartPad;
  const int u = blockIdx.y;
  const mog_unit U = a.L.units[u];
  const int g_begin = blockIdx.x * kResClustersPerBlock;
  if (g_begin >= U.C) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* qb = a.q + ((int64_t)U.seq * a.Hq + (int64_t)U.kv_head * G) * D;
  float coef[G][D / 32];
  score_coefs<D, G>(a, qb, coef);
  float rm[G], rl[G], ro[G][VPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    rm[h] = -INFINITY;
    rl[h] = 0.f;
#pragma unroll
    for (int e = 0; e < VPL; ++e) ro[h][e] = 0.f;
  }
  const int S = U.S;
  int s_keep = b.top_s[U.seq];
  s_keep = s_keep < 0 ? 0 : s_keep;
  const int32_t* off = a.L.sub_off + U.off_base;
  const uint32_t all = (1u << G) - 1u;

  for (int k = 0; k < kResClustersPerBlock / 4; ++k) {
    const int g = g_begin + wave * (kResClustersPerBlock / 4) + k;
    if (g >= U.C) break;
    const int64_t cg = U.cl_base + g;
    const int64_t sg0 = U.sub_base + (int64_t)g * S;
    const int n_g = off[(g + 1) * S] - off[g * S];
    if (n_g == 0) {
      if (lane < S) a.ws.sub_mask[sg0 + lane] = 0u;
      continue;
    }
    const uint32_t mask = a.ws.cl_mask[cg];
    const uint32_t unchosen = all & ~mask;
    if (unchosen && a.residual) {
      float vb[VPL];
      load_floats<VPL>(a.L.cl_vbar + cg * D + lane * VPL, vb);
#pragma unroll
      for (int h = 0; h < G; ++h)
        if ((unchosen >> h) & 1u) add_group<VPL>(rm[h], rl[h], ro[h], a.ws.cl_score[cg * G + h], vb);
    }
    uint32_t my_sm = 0u;
    if (mask) {
      int my_cnt = 0;
      if (lane < S) my_cnt = off[g * S + lane + 1] - off[g * S + lane];
      float my_ss[G];
#pragma unroll
      for (int h = 0; h < G; ++h) my_ss[h] = -INFINITY;
      for (int i = 0; i < S; ++i) {
        const int cnt_i = __shfl(my_cnt, i, 64);
        if (cnt_i == 0) continue;
        float s[G];
        score_row<D, G>(a.L.sub_ms + (sg0 + i) * (2 * D), coef, s);
        const float lg = log2f((float)cnt_i);
#pragma unroll
        for (int h = 0; h < G; ++h)
          if (lane == i) my_ss[h] = s[h] + lg;
      }
      const bool valid = lane < S && my_cnt > 0;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        if (!((mask >> h) & 1u)) continue;
        const float my = my_ss[h];
        int rank = 0;
        for (int j = 0; j < S; ++j) {
          const float o = __shfl(my, j, 64);
          const int vj = __shfl((int)valid, j, 64);
          if (vj && (o > my || (o == my && j < lane))) ++rank;
        }
        const bool sel = valid && rank < s_keep;
        if (sel) my_sm |= 1u << h;
        if (a.sel_s) {
          const unsigned long long bal = __ballot(sel);
          const int rc = a.ws.cl_rank[cg * G + h];
          const int hq = U.kv_head * G + h;
          const int64_t base = (((int64_t)U.seq * a.Hq + hq) * a.c_stride + rc) * a.s_stride;
          if (sel) a.sel_s[base + __popcll(bal & ((1ull << lane) - 1ull))] = lane;
          for (int j = __popcll(bal) + lane; j < a.s_stride; j += 64) a.sel_s[base + j] = -1;
        }
      }
      if (lane < S) a.ws.sub_mask[sg0 + lane] = my_sm;
      if (a.residual) {
        for (int i = 0; i < S; ++i) {
          const int cnt_i = __shfl(my_cnt, i, 64);
          const uint32_t sm_i = (uint32_t)__shfl((int)my_sm, i, 64);
          const uint32_t need = cnt_i > 0 ? (mask & ~sm_i) : 0u;
          if (!need) continue;
          float vb[VPL];
          load_floats<VPL>(a.L.sub_vbar + (sg0 + i) * D + lane * VPL, vb);
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const float w = __shfl(my_ss[h], i, 64);
            if ((need >> h) & 1u) add_group<VPL>(rm[h], rl[h], ro[h], w, vb);
          }
        }
      }
    } else {
      if (lane < S) a.ws.sub_mask[sg0 + lane] = 0u;
    }
  }

  // combine the four waves and write this block's residual partial per head
  __shared__ float st[4][G][D + 2];
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
  float* dst = a.ws.res_part + ((int64_t)u * a.nb_res + blockIdx.x) * G * RS;
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

// ---------------------------------------------------------------------------
// 4. Plan of the exact pass of one unit: the run list (two anchor runs read
//    from the KV cache, then every chosen subcluster as a run of layout rows
//    with the mask of the heads that chose it), its virtual row prefix, and
//    the first (run, offset) of each of the splits*4 wave ranges that divide
//    the rows evenly.  One block of 1024 threads per unit.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_plan(DArgs a, int G) {
  __shared__ int sh[16];
  const int u = blockIdx.x, tid = threadIdx.x;
  const mog_unit U = a.L.units[u];
  const int CS = U.C * U.S;
  const int64_t rb = U.sub_base + 2 * (int64_t)u;
  const uint32_t all = (1u << G) - 1u;
  const int32_t* off = a.L.sub_off + U.off_base;
  if (tid == 0) {
    a.ws.run_start[rb] = 0;
    a.ws.run_len[rb] = a.n_sink;
    a.ws.run_mask[rb] = all;
    a.ws.run_vstart[rb] = 0;
    a.ws.run_start[rb + 1] = U.N - a.n_recent;
    a.ws.run_len[rb + 1] = a.n_recent;
    a.ws.run_mask[rb + 1] = all;
    a.ws.run_vstart[rb + 1] = a.n_sink;
  }
  int cr = 2, crow = a.n_sink + a.n_recent;
  for (int base = 0; base < CS; base += 1024) {
    const int g = base + tid;
    uint32_t m = 0u;
    int st = 0, len = 0;
    if (g < CS) {
      m = a.ws.sub_mask[U.sub_base + g];
      if (m) {
        st = off[g];
        len = off[g + 1] - st;
      }
    }
    const int flag = (m != 0u && len > 0) ? 1 : 0;
    int tf, tl;
    const int ri = block_excl_scan<1024>(flag, sh, tf);
    const int vo = block_excl_scan<1024>(flag * len, sh, tl);
    if (flag) {
      const int64_t idx = rb + cr + ri;
      a.ws.run_start[idx] = st;
      a.ws.run_len[idx] = len;
      a.ws.run_mask[idx] = m;
      a.ws.run_vstart[idx] = crow + vo;
    }
    cr += tf;
    crow += tl;
  }
  const int R = cr, T = crow;
  if (tid == 0) {
    a.ws.unit_tot[2 * u] = R;
    a.ws.unit_tot[2 * u + 1] = T;
  }
  const int NW = a.splits * 4;
  int32_t* wst = a.ws.wstart + (int64_t)u * NW * 2;
  for (int w = tid; w < NW; w += 1024) {
    wst[2 * w] = R;
    wst[2 * w + 1] = 0;
  }
  __syncthreads();
  if (T > 0) {
    for (int r = tid; r < R; r += 1024) {
      const int64_t vs = a.ws.run_vstart[rb + r];
      const int64_t ve = vs + a.ws.run_len[rb + r];
      int64_t wlo = (vs * NW + T - 1) / T;
      const int64_t whi = (ve * NW + T - 1) / T;
      for (int64_t w = wlo; w < whi && w < NW; ++w) {
        wst[2 * w] = r;
        wst[2 * w + 1] = (int)(w * T / NW - vs);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Exact online-softmax accumulation shared by the MoG exact pass and the
// dense baseline.  A wave reads LPR = D/8 lanes per row (8 elements per lane,
// one 16-byte load per lane for bf16), RPI = 64/LPR rows per step; each lane
// keeps a (m, l, o[8]) state per head for its row slot.
// ---------------------------------------------------------------------------
template <int D, int G>
struct RowAcc {
  static constexpr int LPR = D / 8;
  static constexpr int RPI = 64 / LPR;
  float m[G], l[G], o[G][8];
  float qv[G][8];

  __device__ void init(const float* qb, float scale_l2) {
    const int sub = (threadIdx.x & 63) % LPR;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = -INFINITY;
      l[h] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        o[h][e] = 0.f;
        qv[h][e] = qb[h * D + sub * 8 + e] * scale_l2;
      }
    }
  }

  // rows given by a functor rowoff(i) -> element offset of row i, i < n
  template <typename T, typename RowOff>
  __device__ void rows(const T* kb, const T* vb, int n, uint32_t mask, RowOff rowoff) {
    const int lane = threadIdx.x & 63;
    const int sub = lane % LPR, slot = lane / LPR;
    for (int r = 0; r < n; r += RPI) {
      const int my = r + slot;
      const bool valid = my < n;
      float k8[8], v8[8];
      if (valid) {
        const int64_t ro = rowoff(my) + sub * 8;
        load8<T>(kb, ro, k8);
        load8<T>(vb, ro, v8);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) k8[e] = v8[e] = 0.f;
      }
      float s[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float t = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) t += qv[h][e] * k8[e];
#pragma unroll
        for (int o2 = 1; o2 < LPR; o2 <<= 1) t += __shfl_xor(t, o2, 64);
        s[h] = t;
      }
      if (valid) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          if (!((mask >> h) & 1u)) continue;
          const float mn = fmaxf(m[h], s[h]);
          const float al = exp2f(m[h] - mn);
          const float p = exp2f(s[h] - mn);
          l[h] = l[h] * al + p;
#pragma unroll
          for (int e = 0; e < 8; ++e) o[h][e] = o[h][e] * al + p * v8[e];
          m[h] = mn;
        }
      }
    }
  }

  // merge the RPI row slots of the wave, then the 4 waves of the block, and
  // write one partial record (o[D], m, l) per head to dst[h*RS].
  __device__ void finish(float* dst) {
    constexpr int RS = D + kPartPad;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int x = LPR; x < 64; x <<= 1) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float m2 = __shfl_xor(m[h], x, 64);
        const float l2 = __shfl_xor(l[h], x, 64);
        float a1, a2, mn;
        merge_scale(m[h], m2, a1, a2, mn);
        l[h] = a1 * l[h] + a2 * l2;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float o2 = __shfl_xor(o[h][e], x, 64);
          o[h][e] = a1 * o[h][e] + a2 * o2;
        }
        m[h] = mn;
      }
    }
    __shared__ float st[4][G][D + 2];
    if (lane < LPR) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int e = 0; e < 8; ++e) st[wave][h][lane * 8 + e] = o[h][e];
        if (lane == 0) {
          st[wave][h][D] = m[h];
          st[wave][h][D + 1] = l[h];
        }
      }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * D; idx += 256) {
      const int h = idx / D, e = idx % D;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < 4; ++w) M = fmaxf(M, st[w][h][D]);
      float l2 = 0.f, o2 = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float mw = st[w][h][D];
        const float f = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
        l2 += f * st[w][h][D + 1];
        o2 += f * st[w][h][e];
      }
      dst[h * RS + e] = o2;
      if (e == 0) {
        dst[h * RS + D] = M;
        dst[h * RS + D + 1] = l2;
      }
    }
  }
};

// ---------------------------------------------------------------------------
// 5. Exact split-K pass: wave w of unit u covers virtual rows
//    [w*T/NW, (w+1)*T/NW) of the unit's run list.  Grid (splits, units).
// ---------------------------------------------------------------------------
template <int D, int G, typename T>
__global__ __launch_bounds__(256) void k_exact(DArgs a) {
  constexpr int RS = D + kPartPad;
  const int u = blockIdx.y, p = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  const mog_unit U = a.L.units[u];
  const int R = a.ws.unit_tot[2 * u];
  const int64_t Tt = a.ws.unit_tot[2 * u + 1];
  const int NW = a.splits * 4;
  const int w = p * 4 + wave;
  const int64_t r0 = (int64_t)w * Tt / NW;
  const int64_t r1 = (int64_t)(w + 1) * Tt / NW;
  RowAcc<D, G> acc;
  acc.init(a.q + ((int64_t)U.seq * a.Hq + (int64_t)U.kv_head * G) * D, a.scale_l2);
  if (r0 < r1) {
    const int64_t rb = U.sub_base + 2 * (int64_t)u;
    const int32_t* wst = a.ws.wstart + ((int64_t)u * NW + w) * 2;
    int r = wst[0];
    int offr = wst[1];
    int64_t row = r0;
    const T* kc = static_cast<const T*>(a.kv.k);
    const T* vc = static_cast<const T*>(a.kv.v);
    const T* km = static_cast<const T*>(a.L.k_mid);
    const T* vm = static_cast<const T*>(a.L.v_mid);
    while (row < r1 && r < R) {
      const int st = a.ws.run_start[rb + r];
      const int ln = a.ws.run_len[rb + r];
      const uint32_t msk = a.ws.run_mask[rb + r];
      int take = ln - offr;
      if ((int64_t)take > r1 - row) take = (int)(r1 - row);
      if (take > 0) {
        if (r < 2) {
          const KVRef kv = a.kv;
          const int t0 = st + offr, seq = U.seq, kvh = U.kv_head;
          acc.template rows<T>(kc, vc, take, msk,
                               [&](int i) { return kv_row_offset(kv, seq, kvh, t0 + i, D); });
        } else {
          const int64_t base = (U.row_base + st + offr) * D;
          acc.template rows<T>(km, vm, take, msk, [&](int i) { return base + (int64_t)i * D; });
        }
      }
      row += take;
      ++r;
      offr = 0;
    }
  }
  acc.finish(a.ws.ex_part + ((int64_t)u * a.splits + p) * G * RS);
}

// ---------------------------------------------------------------------------
// 6. Merge: per query head, max over every partial (exact splits, then the
//    residual blocks), one normalisation.  Grid (Hq, n_seq), D threads.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(128) void k_merge(const float* ex_part, int n_ex, const float* res_part,
                                               int nb_res_stride, const mog_unit* units,
                                               int use_res, int G, int Hq, int Hkv, float* out,
                                               float* lse) {
  constexpr int RS = D + kPartPad;
  const int hq = blockIdx.x, seq = blockIdx.y, t = threadIdx.x;
  const int kvh = hq / G, h = hq % G;
  const int u = seq * Hkv + kvh;
  int n_res = 0;
  if (use_res) {
    const int C = units[u].C;
    n_res = (C + kResClustersPerBlock - 1) / kResClustersPerBlock;
  }
  const float* ex = ex_part + ((int64_t)u * n_ex * G + h) * RS;
  const float* rs = use_res ? res_part + ((int64_t)u * nb_res_stride * G + h) * RS : nullptr;
  float M = -INFINITY;
  for (int i = 0; i < n_ex; ++i) M = fmaxf(M, ex[(int64_t)i * G * RS + D]);
  for (int i = 0; i < n_res; ++i) M = fmaxf(M, rs[(int64_t)i * G * RS + D]);
  float den = 0.f, num = 0.f;
  for (int i = 0; i < n_ex; ++i) {
    const float* r = ex + (int64_t)i * G * RS;
    const float m = r[D];
    if (m == -INFINITY) continue;
    const float f = exp2f(m - M);
    den += f * r[D + 1];
    num += f * r[t];
  }
  for (int i = 0; i < n_res; ++i) {
    const float* r = rs + (int64_t)i * G * RS;
    const float m = r[D];
    if (m == -INFINITY) continue;
    const float f = exp2f(m - M);
    den += f * r[D + 1];
    num += f * r[t];
  }
  const int64_t orow = (int64_t)seq * Hq + hq;
  out[orow * D + t] = den > 0.f ? num / den : 0.f;
  if (lse && t == 0) lse[orow] = den > 0.f ? (M + log2f(den)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// Dense baseline: wave w of unit u covers tokens [w*N/NW, (w+1)*N/NW).
// ---------------------------------------------------------------------------
template <int D, int G, typename T>
__global__ __launch_bounds__(256) void k_dense(KVRef kv, const float* q, int Hq, int Hkv, int splits,
                                               float scale_l2, SeqArgs seq_args, float* ex_part) {
  constexpr int RS = D + kPartPad;
  const int u = blockIdx.y, p = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  const int seq = u / Hkv, kvh = u % Hkv;
  const int64_t N = seq_args.len[seq];
  const int NW = splits * 4;
  const int w = p * 4 + wave;
  const int t0 = (int)((int64_t)w * N / NW);
  const int t1 = (int)((int64_t)(w + 1) * N / NW);
  RowAcc<D, G> acc;
  acc.init(q + ((int64_t)seq * Hq + (int64_t)kvh * G) * D, scale_l2);
  if (t1 > t0) {
    const T* kc = static_cast<const T*>(kv.k);
    const T* vc = static_cast<const T*>(kv.v);
    if (!kv.paged) {
      const int64_t base = kv_row_offset(kv, seq, kvh, t0, D);
      acc.template rows<T>(kc, vc, t1 - t0, 0xffffffffu, [&](int i) { return base + (int64_t)i * D; });
    } else {
      acc.template rows<T>(kc, vc, t1 - t0, 0xffffffffu,
                           [&](int i) { return kv_row_offset(kv, seq, kvh, t0 + i, D); });
    }
  }
  acc.finish(ex_part + ((int64_t)u * splits + p) * G * RS);
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

template <int D, int G, typename T>
static hipError_t decode_impl(const DecodeLaunch& x, const DArgs& a, const BudgetArgs& b, hipStream_t s) {
  const int nu = x.L.n_units;
  hipLaunchKernelGGL((k_score_clusters<D, G>), dim3((x.L.max_C + 63) / 64, nu), dim3(256), 0, s, a);
  hipLaunchKernelGGL(k_select_topc, dim3(G, nu), dim3(256), 0, s, a, b, G);
  hipLaunchKernelGGL((k_subclusters<D, G>), dim3(x.nb_res, nu), dim3(256), 0, s, a, b);
  hipLaunchKernelGGL(k_plan, dim3(nu), dim3(1024), 0, s, a, G);
  hipLaunchKernelGGL((k_exact<D, G, T>), dim3(x.splits, nu), dim3(256), 0, s, a);
  hipLaunchKernelGGL((k_merge<D>), dim3(x.Hq, x.L.n_seq), dim3(D), 0, s, a.ws.ex_part, x.splits,
                     a.ws.res_part, x.nb_res, a.L.units, x.residual, G, x.Hq, x.L.n_kv_heads, x.out,
                     x.lse);
  return hipGetLastError();
}

template <int D, typename T>
static hipError_t decode_g(const DecodeLaunch& x, const DArgs& a, const BudgetArgs& b, hipStream_t s) {
  switch (x.G) {
    case 1: return decode_impl<D, 1, T>(x, a, b, s);
    case 2: return decode_impl<D, 2, T>(x, a, b, s);
    case 3: return decode_impl<D, 3, T>(x, a, b, s);
    case 4: return decode_impl<D, 4, T>(x, a, b, s);
    case 5: return decode_impl<D, 5, T>(x, a, b, s);
    case 6: return decode_impl<D, 6, T>(x, a, b, s);
    case 7: return decode_impl<D, 7, T>(x, a, b, s);
    case 8: return decode_impl<D, 8, T>(x, a, b, s);
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
  if (x.D == 128) {
    return x.dtype == MOG_BF16 ? decode_g<128, uint16_t>(x, a, b, s) : decode_g<128, float>(x, a, b, s);
  }
  return x.dtype == MOG_BF16 ? decode_g<64, uint16_t>(x, a, b, s) : decode_g<64, float>(x, a, b, s);
}

template <int D, int G, typename T>
static hipError_t dense_impl(const DenseLaunch& x, hipStream_t s) {
  const int nu = x.seq.n_seq * x.n_kv_heads;
  hipLaunchKernelGGL((k_dense<D, G, T>), dim3(x.splits, nu), dim3(256), 0, s, x.kv, x.q, x.Hq,
                     x.n_kv_heads, x.splits, x.scale * kLog2e, x.seq, x.ex_part);
  hipLaunchKernelGGL((k_merge<D>), dim3(x.Hq, x.seq.n_seq), dim3(D), 0, s, x.ex_part, x.splits,
                     (const float*)nullptr, 0, (const mog_unit*)nullptr, 0, G, x.Hq, x.n_kv_heads,
                     x.out, x.lse);
  return hipGetLastError();
}

template <int D, typename T>
static hipError_t dense_g(const DenseLaunch& x, hipStream_t s) {
  switch (x.G) {
    case 1: return dense_impl<D, 1, T>(x, s);
    case 2: return dense_impl<D, 2, T>(x, s);
    case 3: return dense_impl<D, 3, T>(x, s);
    case 4: return dense_impl<D, 4, T>(x, s);
    case 5: return dense_impl<D, 5, T>(x, s);
    case 6: return dense_impl<D, 6, T>(x, s);
    case 7: return dense_impl<D, 7, T>(x, s);
    case 8: return dense_impl<D, 8, T>(x, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_dense(const DenseLaunch& x, hipStream_t s) {
  if (x.D == 128) return x.dtype == MOG_BF16 ? dense_g<128, uint16_t>(x, s) : dense_g<128, float>(x, s);
  return x.dtype == MOG_BF16 ? dense_g<64, uint16_t>(x, s) : dense_g<64, float>(x, s);
}

}  // namespace mog
