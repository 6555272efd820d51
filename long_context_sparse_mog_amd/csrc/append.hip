// Incremental decode for libmog: the tokens that leave the recent window as a
// sequence grows join the partition built after prefill ("Iceberg Attention:
// Sublinear Long-Context Decoding with Mixture-of-Gaussians", abstract: the
// partition is built once and then serves every decode step).
//
// Per unit (sequence, KV head) and per folded token, oldest first:
//   1. the token's K/V rows are copied into the unit's fold area;
//   2. the nonempty cluster whose mean key is nearest (squared distance in
//      float64, ties to the lower id; float32 distances with their error
//      bound rule most clusters out first), then the nearest nonempty
//      subcluster of that cluster;
//   3. Welford's running formulas update both groups' mean key, population
//      variance and mean value (float64 from the stored float32, stored
//      float32, in the formulas' own operation order), and the fold counts.
// Tokens are taken one after the other (one launch each), since each
// decision sees the statistics the previous token left; the cluster scan of
// a token is spread over several blocks of the unit.
#include "attn_tile.h"
#include "mog_internal.h"

namespace mog {

struct AArgs {
  mog_unit* units;
  KVRef kv;
  const int32_t* sub_off;
  float* cl_ms;
  float* cl_vbar;
  float* sub_ms;
  float* sub_vbar;
  uint16_t* cl_ms16;  // bf16 copies, updated beside them
  uint16_t* cl_vbar16;
  uint16_t* sub_ms16;
  uint16_t* sub_vbar16;
  int32_t* cl_fold;
  int32_t* sub_fold;
  int32_t* fold_sub;
  int32_t* fold_pos;
  void* k_mid;
  void* v_mid;
  int64_t fold_row0;  // first fold-area row (unit u's start at fold_row0 + u * fold_cap)
  // feature-map summaries (fm_dim > 0): projection and per-group sums
  const float* fm_w;
  float* cl_fz;
  float* sub_fz;
  int32_t fm_dim;
  float fm_sqrt_scale;
  AppendSlot* slots;   // [n_units][kAppendMaxBlocks] per-block winners
  int32_t fold_cap, n_recent;
  AppendSeq seq[MOG_MAX_SEQ];
};

__device__ inline float to_f(float x) { return x; }
__device__ inline float to_f(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

// One member (k, v) joins a group of n: mean key mu, population variance
// var and mean value vbar of one dimension (the stored float32 values),
// updated by Welford's formulas in float64 and stored as float32.
__device__ inline void welford_add(float mu_f, float var_f, float vbar_f, int n, double k, double v, float* mu_o,
                                   float* var_o, float* vbar_o, uint16_t* mu_b, uint16_t* var_b, uint16_t* vbar_b) {
#pragma clang fp contract(off)
  const double n1 = (double)(n + 1);
  const double mu = mu_f, var = var_f, vbar = vbar_f;
  const double delta = k - mu;
  const double mu1 = mu + delta / n1;
  const double var1 = ((double)n * var + delta * (k - mu1)) / n1;
  const double vbar1 = vbar + (v - vbar) / n1;
  *mu_o = (float)mu1;
  *var_o = (float)var1;
  *vbar_o = (float)vbar1;
  // (the decode's bf16 copies, rounded from the stored float32 values)
  *mu_b = bf16_bits((float)mu1);
  *var_b = bf16_bits((float)var1);
  *vbar_b = bf16_bits((float)vbar1);
}

// (d2, id) lexicographic minimum over the lanes l of the wave that differ
// from each other in bits LO..32 (lanes that agree in the lower bits hold
// the same values): the smaller distance, on a tie the lower id; (n, nf)
// travel with the winner.
template <int LO>
__device__ inline void wave_argmin(double& d2, int& id, int& n, int& nf) {
#pragma unroll
  for (int o = 32; o >= LO; o >>= 1) {
    const double od = __shfl_xor(d2, o, 64);
    const int oi = __shfl_xor(id, o, 64);
    const int on = __shfl_xor(n, o, 64);
    const int of = __shfl_xor(nf, o, 64);
    if (od < d2 || (od == d2 && oi < id)) {
      d2 = od;
      id = oi;
      n = on;
      nf = of;
    }
  }
}

template <int CTRL>
__device__ inline double dpp_d(double x) {
  const long long b = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)((unsigned long long)b >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo));
}

// Sums over the LPC (8 or 16) lanes of a group row by DPP inside each row of
// 16 lanes; every lane of the group gets the same value.
template <int LPC>
__device__ inline float group_sum(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror
  if constexpr (LPC == 16) x += dpp<0x140>(x);  // row_mirror
  return x;
}

template <int LPC>
__device__ inline double group_sum(double x) {
  x += dpp_d<0xB1>(x);
  x += dpp_d<0x4E>(x);
  x += dpp_d<0x141>(x);
  if constexpr (LPC == 16) x += dpp_d<0x140>(x);
  return x;
}

// Squared distance of a group row to the key, float64: lane `part` of the
// LPC lanes of the row holds dimensions [8 part, 8 part + 8).
template <int LPC>
__device__ inline double row_dist2(const float (&m)[8], const double (&kd)[8]) {
  double d2 = 0.0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const double df = (double)m[e] - kd[e];
    d2 += df * df;
  }
  return group_sum<LPC>(d2);
}

__device__ inline void load_row8(const float* p, float (&m)[8]) {
  const float4 x0 = reinterpret_cast<const float4*>(p)[0], x1 = reinterpret_cast<const float4*>(p)[1];
  m[0] = x0.x; m[1] = x0.y; m[2] = x0.z; m[3] = x0.w;
  m[4] = x1.x; m[5] = x1.y; m[6] = x1.z; m[7] = x1.w;
}

template <typename T>
__device__ inline void load_key8(const T* p, float (&k)[8]);
template <>
__device__ inline void load_key8<float>(const float* p, float (&k)[8]) {
  load_row8(p, k);
}
template <>
__device__ inline void load_key8<uint16_t>(const uint16_t* p, float (&k)[8]) {
  const uint4 w = *reinterpret_cast<const uint4*>(p);
  k[0] = bf16_lo(w.x); k[1] = bf16_hi(w.x); k[2] = bf16_lo(w.y); k[3] = bf16_hi(w.y);
  k[4] = bf16_lo(w.z); k[5] = bf16_hi(w.z); k[6] = bf16_lo(w.w); k[7] = bf16_hi(w.w);
}

// Blocks per unit that share the cluster scan of one token: about
// kAppendRowsPerBlock clusters each, at most kAppendMaxBlocks.
__host__ __device__ inline int append_blocks(int C) {
  const int p = (C + kAppendRowsPerBlock - 1) / kAppendRowsPerBlock;
  return p < 1 ? 1 : (p > kAppendMaxBlocks ? kAppendMaxBlocks : p);
}

// The nearest nonempty cluster: float32 distances of every cluster row,
// and float64 distances of the rows the float32 ones cannot rule out.  For
// D nonnegative terms (m - k)^2, each from a rounded difference and a fused
// multiply-add, summed in any order, the float32 value d' satisfies
// |d' - d| <= gamma d, gamma = (D + 3) 2^-24 (plus an absolute error of a
// few 2^-149 D for results in the subnormal range).  Every group of LPC
// lanes walks its own ascending sequence of rows keeping the float32
// minimum r seen so far; a row with d' > r (1 + 2 gamma) / (1 - 2 gamma) +
// slack has a true distance above that of the row that set r, so it can be
// neither the nearest cluster nor a tie of it, and is skipped.  Every other
// row gets its float64 distance from the same registers, and the float64
// minimum (ties to the lower id) over all groups decides.
//
// Two launches per folded token (token index `it` of every sequence's new
// tokens).  k_append, grid (append_blocks(max C), units): block p of unit u
// scans clusters [p C / P, (p + 1) C / P) and writes its winner to the
// unit's slot p.  k_append_apply, one block per unit, then takes the
// winners' minimum, picks the subcluster, applies the running updates and
// writes the fold bookkeeping (the kernel boundary orders the slots before
// it; no fences or counters).
template <int D, typename T>
__global__ __launch_bounds__(kAppendThreads) void k_append(AArgs a, int it) {
  constexpr int NW = kAppendThreads / 64;
  constexpr int LPC = D / 8;       // lanes per group row: 8 dimensions each
  constexpr int CPW = 64 / LPC;    // group rows per wave and step
  constexpr int UNR = 4;           // steps whose loads are in flight together
  constexpr float kGamma = (D + 3) * 5.9604645e-8f;
  constexpr float kFactor = (1.0f + 2.0f * kGamma) / (1.0f - 2.0f * kGamma);
  constexpr float kSlack = 1e-30f;
  __shared__ double w_d2[NW];
  __shared__ int w_id[NW], w_n[NW], w_f[NW];
  const int u = blockIdx.y, p = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const mog_unit U = uni_unit(a.units + u);
  const AppendSeq sq = a.seq[U.seq];
  const int C = U.C, S = U.S, P = append_blocks(C);
  if (it >= sq.n_new || p >= P) return;
  const int32_t* off = a.sub_off + U.off_base;
  const int part = lane % LPC, row_in = lane / LPC;
  const T* kc = static_cast<const T*>(a.kv.k);
  const T* vc = static_cast<const T*>(a.kv.v);
  const int t = sq.len - a.n_recent + it;  // token position
  const int f = sq.f0 + it;                // its fold row
  const int64_t src = kv_row_offset(a.kv, U.seq, U.kv_head, t, D);
  // dimensions [8 part, 8 part + 8) of the key (their loads go out with the
  // first cluster rows')
  float kx[8];
  load_key8<T>(kc + src + part * 8, kx);
  double kd[8];
  bool have_kd = false;
  const int c_lo = (int)((int64_t)p * C / P), c_hi = (int)((int64_t)(p + 1) * C / P);
  double best = INFINITY;
  int bid = 0x7fffffff, bn = 0, bf = 0;
  float run = INFINITY;  // the group's float32 minimum so far
  for (int c0 = c_lo + wave * CPW; c0 < c_hi; c0 += NW * CPW * UNR) {
    float m[UNR][8];
    int cnt[UNR], fc[UNR];
#pragma unroll
    for (int r = 0; r < UNR; ++r) {
      const int c = min(c0 + r * NW * CPW + row_in, c_hi - 1);
      load_row8(a.cl_ms + (U.cl_base + c) * (2 * D) + part * 8, m[r]);
      fc[r] = a.cl_fold[U.cl_base + c];
      cnt[r] = off[(c + 1) * S] - off[c * S];
    }
    if (!have_kd) {
#pragma unroll
      for (int e = 0; e < 8; ++e) kd[e] = (double)kx[e];
      have_kd = true;
    }
#pragma unroll
    for (int r = 0; r < UNR; ++r) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float df = m[r][e] - kx[e];
        d = fmaf(df, df, d);
      }
      d = group_sum<LPC>(d);
      const int c = c0 + r * NW * CPW + row_in;
      // (uniform across the LPC lanes of a row)
      if (c < c_hi && cnt[r] + fc[r] > 0 && d <= run * kFactor + kSlack) {
        run = fminf(run, d);
        const double d2 = row_dist2<LPC>(m[r], kd);
        if (d2 < best) {  // ids grow along the group's sequence: ties keep the lower
          best = d2;
          bid = c;
          bn = cnt[r] + fc[r];
          bf = fc[r];
        }
      }
    }
  }
  wave_argmin<LPC>(best, bid, bn, bf);
  if (lane == 0) {
    w_d2[wave] = best;
    w_id[wave] = bid;
    w_n[wave] = bn;
    w_f[wave] = bf;
  }
  __syncthreads();
  AppendSlot* slots = a.slots + (int64_t)u * kAppendMaxBlocks;
  if (wave == 0) {
    double bd = lane < NW ? w_d2[lane] : INFINITY;
    int bj = lane < NW ? w_id[lane] : 0x7fffffff;
    int cn = lane < NW ? w_n[lane] : 0, cf = lane < NW ? w_f[lane] : 0;
    wave_argmin<1>(bd, bj, cn, cf);
    if (lane == 0) slots[p] = AppendSlot{bd, bj, cn, cf, 0};
  }
}

template <int D, typename T>
__global__ __launch_bounds__(256) void k_append_apply(AArgs a, int it) {
  constexpr int LPC = D / 8;
  constexpr int CPW = 64 / LPC;
  __shared__ int sel[4];   // (unused), subcluster, its size, its fold count
  __shared__ float xs[D];  // sqrt(scale) k for the feature map
  const int u = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const mog_unit U = uni_unit(a.units + u);
  const AppendSeq sq = a.seq[U.seq];
  const int C = U.C, S = U.S, P = append_blocks(C);
  if (it >= sq.n_new) return;
  const int32_t* off = a.sub_off + U.off_base;
  const int part = lane % LPC, row_in = lane / LPC;
  const T* kc = static_cast<const T*>(a.kv.k);
  const T* vc = static_cast<const T*>(a.kv.v);
  const int t = sq.len - a.n_recent + it;
  const int f = sq.f0 + it;
  const int64_t src = kv_row_offset(a.kv, U.seq, U.kv_head, t, D);
  float kx[8];
  load_key8<T>(kc + src + part * 8, kx);
  double kd[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) kd[e] = (double)kx[e];
  const bool have_kd = true;
  const AppendSlot* slots = a.slots + (int64_t)u * kAppendMaxBlocks;
  double bd = INFINITY;
  int bj = 0x7fffffff, cn = 0, cf = 0;
  if (lane < P) {
    const AppendSlot sl = slots[lane];
    bd = sl.d2;
    bj = sl.id;
    cn = sl.n;
    cf = sl.nf;
  }
  wave_argmin<1>(bd, bj, cn, cf);
  const int j = bj == 0x7fffffff ? 0 : bj;  // (a built layout has a nonempty cluster)
  const int64_t cg = U.cl_base + j, sg0 = U.sub_base + (int64_t)j * S;
  // the token's rows and the cluster's statistics for the running updates,
  // loaded while wave 0 looks for the subcluster
  T kx_t{}, vx_t{};
  float c_mu = 0.f, c_var = 0.f, c_vb = 0.f;
  if (tid < D) {
    kx_t = kc[src + tid];
    vx_t = vc[src + tid];
    c_mu = a.cl_ms[cg * (2 * D) + tid];
    c_var = a.cl_ms[cg * (2 * D) + D + tid];
    c_vb = a.cl_vbar[cg * D + tid];
  }
  if (!have_kd) {
#pragma unroll
    for (int e = 0; e < 8; ++e) kd[e] = (double)kx[e];
  }
  if (wave == 0) {
    // nearest nonempty subcluster of cluster j, in float64: every row's
    // loads at once
    constexpr int SST = (kMaxS + CPW - 1) / CPW;
    float m[SST][8];
    int scnt[SST], sfc[SST];
#pragma unroll
    for (int r = 0; r < SST; ++r) {
      const int is = min(r * CPW + row_in, S - 1);
      load_row8(a.sub_ms + (sg0 + is) * (2 * D) + part * 8, m[r]);
      sfc[r] = a.sub_fold[sg0 + is];
      scnt[r] = off[j * S + is + 1] - off[j * S + is];
    }
    double sb = INFINITY;
    int si = 0x7fffffff, sn = 0, sf = 0;
#pragma unroll
    for (int r = 0; r < SST; ++r) {
      if (r * CPW >= S) break;
      const double d2 = row_dist2<LPC>(m[r], kd);
      const int is = r * CPW + row_in;
      if (is < S && scnt[r] + sfc[r] > 0 && d2 < sb) {
        sb = d2;
        si = is;
        sn = scnt[r] + sfc[r];
        sf = sfc[r];
      }
    }
    wave_argmin<LPC>(sb, si, sn, sf);
    if (lane == 0) {
      sel[1] = si == 0x7fffffff ? 0 : si;
      sel[2] = sn;
      sel[3] = sf;
    }
  }
  __syncthreads();
  // running updates of both groups, and the fold bookkeeping
  const int is = sel[1];
  const int64_t sg = sg0 + is;
  if (tid < D) {
    T* kf = static_cast<T*>(a.k_mid) + (a.fold_row0 + (int64_t)u * a.fold_cap + f) * D;
    T* vf = static_cast<T*>(a.v_mid) + (a.fold_row0 + (int64_t)u * a.fold_cap + f) * D;
    kf[tid] = kx_t;
    vf[tid] = vx_t;
    const double k = (double)to_f(kx_t), v = (double)to_f(vx_t);
    welford_add(c_mu, c_var, c_vb, cn, k, v, a.cl_ms + cg * (2 * D) + tid, a.cl_ms + cg * (2 * D) + D + tid,
                a.cl_vbar + cg * D + tid, a.cl_ms16 + cg * (2 * D) + tid, a.cl_ms16 + cg * (2 * D) + D + tid,
                a.cl_vbar16 + cg * D + tid);
    welford_add(a.sub_ms[sg * (2 * D) + tid], a.sub_ms[sg * (2 * D) + D + tid], a.sub_vbar[sg * D + tid], sel[2], k,
                v, a.sub_ms + sg * (2 * D) + tid, a.sub_ms + sg * (2 * D) + D + tid, a.sub_vbar + sg * D + tid,
                a.sub_ms16 + sg * (2 * D) + tid, a.sub_ms16 + sg * (2 * D) + D + tid, a.sub_vbar16 + sg * D + tid);
  }
  if (a.fm_dim) {
    // the token's features join both groups' feature sums
    if (tid < D) xs[tid] = a.fm_sqrt_scale * to_f(kx_t);
    __syncthreads();
    const int m = a.fm_dim;
    if (tid < m) {
      const float* w = a.fm_w + (int64_t)tid * D;
      float t = 0.f, xx = 0.f;
#pragma unroll 8
      for (int e = 0; e < D; ++e) {
        t += w[e] * xs[e];
        xx += xs[e] * xs[e];
      }
      const float ph = expf(t - 0.5f * xx) * rsqrtf((float)m);
      a.cl_fz[cg * m + tid] += ph;
      a.sub_fz[sg * m + tid] += ph;
    }
  }
  if (tid == 0) {
    a.cl_fold[cg] = cf + 1;
    a.sub_fold[sg] = sel[3] + 1;
    a.fold_sub[(int64_t)u * a.fold_cap + f] = j * S + is;
    a.fold_pos[(int64_t)u * a.fold_cap + f] = t;
    a.units[u].N = sq.len + it + 1;
    a.units[u].n_fold = f + 1;
  }
}

template <int D, typename T>
static hipError_t append_impl(const AppendLaunch& x, const AArgs& a, hipStream_t s) {
  int max_new = 0;
  for (int i = 0; i < x.n_seq; ++i) max_new = max(max_new, (int)x.seq[i].n_new);
  const dim3 grid(append_blocks(x.L.max_C), x.L.n_units);
  for (int it = 0; it < max_new; ++it) {
    hipLaunchKernelGGL((k_append<D, T>), grid, dim3(kAppendThreads), 0, s, a, it);
    hipLaunchKernelGGL((k_append_apply<D, T>), dim3(x.L.n_units), dim3(256), 0, s, a, it);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_append(const AppendLaunch& x, hipStream_t s) {
  AArgs a;
  a.units = x.L.units;
  a.kv = x.kv;
  a.sub_off = x.L.sub_off;
  a.cl_ms = x.L.cl_ms;
  a.cl_vbar = x.L.cl_vbar;
  a.sub_ms = x.L.sub_ms;
  a.sub_vbar = x.L.sub_vbar;
  a.cl_ms16 = x.L.cl_ms16;
  a.cl_vbar16 = x.L.cl_vbar16;
  a.sub_ms16 = x.L.sub_ms16;
  a.sub_vbar16 = x.L.sub_vbar16;
  a.cl_fold = x.L.cl_fold;
  a.sub_fold = x.L.sub_fold;
  a.fold_sub = x.L.fold_sub;
  a.fold_pos = x.L.fold_pos;
  a.k_mid = x.L.k_mid;
  a.v_mid = x.L.v_mid;
  a.fold_row0 = x.L.total_mid;
  a.fold_cap = x.L.fold_capacity;
  a.n_recent = x.L.n_recent;
  a.fm_w = x.L.fm_w;
  a.cl_fz = x.L.cl_fz;
  a.sub_fz = x.L.sub_fz;
  a.fm_dim = x.L.fm_dim;
  a.fm_sqrt_scale = sqrtf(x.L.fm_scale);
  a.slots = static_cast<AppendSlot*>(x.L.append_scratch);
  for (int i = 0; i < MOG_MAX_SEQ; ++i) a.seq[i] = x.seq[i];
  const bool bf = x.L.dtype == MOG_BF16;
  if (x.L.head_dim == 128) return bf ? append_impl<128, uint16_t>(x, a, s) : append_impl<128, float>(x, a, s);
  return bf ? append_impl<64, uint16_t>(x, a, s) : append_impl<64, float>(x, a, s);
}

}  // namespace mog
