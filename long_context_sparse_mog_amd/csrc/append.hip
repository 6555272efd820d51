// Incremental decode for libmog: the tokens that leave the recent window as a
// sequence grows join the partition built after prefill ("Iceberg Attention:
// Sublinear Long-Context Decoding with Mixture-of-Gaussians", abstract: the
// partition is built once and then serves every decode step).
//
// Per unit (sequence, KV head) and per folded token, oldest first:
//   1. the token's K/V rows are copied into the unit's fold area;
//   2. the nonempty cluster whose mean key is nearest (squared distance in
//      float64, ties to the lower id), then the nearest nonempty subcluster
//      of that cluster;
//   3. Welford's running formulas update both groups' mean key, population
//      variance and mean value (float64 from the stored float32, stored
//      float32, in the formulas' own operation order), and the fold counts.
// One block per unit; its tokens are taken one after the other, since each
// decision sees the statistics the previous token left.
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
  int32_t* cl_fold;
  int32_t* sub_fold;
  int32_t* fold_sub;
  int32_t* fold_pos;
  void* k_mid;
  void* v_mid;
  int64_t fold_row0;  // first fold-area row (unit u's start at fold_row0 + u * fold_cap)
  int32_t fold_cap, n_recent;
  AppendSeq seq[MOG_MAX_SEQ];
};

__device__ inline float to_f(float x) { return x; }
__device__ inline float to_f(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

// One member (k, v) joins a group of n: mean key, population variance and
// mean value of dimension d, float64 from the stored float32 values.
__device__ inline void welford_add(float* ms, float* vb, int n, int d, int D, double k, double v) {
#pragma clang fp contract(off)
  const double n1 = (double)(n + 1);
  const double mu = ms[d], var = ms[D + d], vbar = vb[d];
  const double delta = k - mu;
  const double mu1 = mu + delta / n1;
  const double var1 = ((double)n * var + delta * (k - mu1)) / n1;
  const double vbar1 = vbar + (v - vbar) / n1;
  ms[d] = (float)mu1;
  ms[D + d] = (float)var1;
  vb[d] = (float)vbar1;
}

// (d2, id) lexicographic minimum over the wave: the smaller distance, on a
// tie the lower id.
__device__ inline void wave_argmin(double& d2, int& id) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const double od = __shfl_xor(d2, o, 64);
    const int oi = __shfl_xor(id, o, 64);
    if (od < d2 || (od == d2 && oi < id)) {
      d2 = od;
      id = oi;
    }
  }
}

constexpr int kAppendThreads = 512;

template <int D, typename T>
__global__ __launch_bounds__(kAppendThreads) void k_append(AArgs a) {
  constexpr int NW = kAppendThreads / 64;
  constexpr int LPC = D / 8;       // lanes per group row: 8 dimensions each
  constexpr int CPW = 64 / LPC;    // group rows per wave and step
  constexpr int UNR = 8;           // steps whose loads are in flight together
  __shared__ float sk[D], sv[D];
  __shared__ double w_d2[NW];
  __shared__ int w_id[NW];
  __shared__ int sel[6];  // cluster, subcluster, their sizes, their fold counts
  const int u = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const mog_unit U = uni_unit(a.units + u);
  const AppendSeq sq = a.seq[U.seq];
  const int n_new = sq.n_new;
  if (n_new == 0) return;
  const int C = U.C, S = U.S;
  const int32_t* off = a.sub_off + U.off_base;
  const int part = lane % LPC, row_in = lane / LPC;
  const T* kc = static_cast<const T*>(a.kv.k);
  const T* vc = static_cast<const T*>(a.kv.v);
  T* kf = static_cast<T*>(a.k_mid) + (a.fold_row0 + (int64_t)u * a.fold_cap) * D;
  T* vf = static_cast<T*>(a.v_mid) + (a.fold_row0 + (int64_t)u * a.fold_cap) * D;
  for (int i = 0; i < n_new; ++i) {
    const int t = sq.len - a.n_recent + i;  // token position
    const int f = sq.f0 + i;                // its fold row
    // 1. the token's rows: copied into the fold area, staged in LDS
    if (tid < D) {
      const int64_t src = kv_row_offset(a.kv, U.seq, U.kv_head, t, D) + tid;
      const T kx = kc[src], vx = vc[src];
      kf[(int64_t)f * D + tid] = kx;
      vf[(int64_t)f * D + tid] = vx;
      sk[tid] = to_f(kx);
      sv[tid] = to_f(vx);
    }
    __syncthreads();
    double kd[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) kd[e] = (double)sk[part * 8 + e];
    // 2a. nearest nonempty cluster: LPC lanes per cluster row, partial sums
    //     over 8 dimensions each, summed across the lanes
    double best = INFINITY;
    int bid = 0x7fffffff;
    for (int c0 = wave * CPW; c0 < C; c0 += NW * CPW * UNR) {
      float m[UNR][8];
      int cnt[UNR];
#pragma unroll
      for (int r = 0; r < UNR; ++r) {
        const int c = min(c0 + r * NW * CPW + row_in, C - 1);
        const float4* p = reinterpret_cast<const float4*>(a.cl_ms + (U.cl_base + c) * (2 * D) + part * 8);
        const float4 x0 = p[0], x1 = p[1];
        m[r][0] = x0.x; m[r][1] = x0.y; m[r][2] = x0.z; m[r][3] = x0.w;
        m[r][4] = x1.x; m[r][5] = x1.y; m[r][6] = x1.z; m[r][7] = x1.w;
        cnt[r] = off[(c + 1) * S] - off[c * S] + a.cl_fold[U.cl_base + c];
      }
#pragma unroll
      for (int r = 0; r < UNR; ++r) {
        double d2 = 0.0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const double df = (double)m[r][e] - kd[e];
          d2 += df * df;
        }
#pragma unroll
        for (int o = LPC / 2; o > 0; o >>= 1) d2 += __shfl_xor(d2, o, 64);
        const int c = c0 + r * NW * CPW + row_in;
        // ids grow with r, so a strict comparison keeps the lower id on a tie
        if (c < C && cnt[r] > 0 && d2 < best) {
          best = d2;
          bid = c;
        }
      }
    }
    wave_argmin(best, bid);
    if (lane == 0) {
      w_d2[wave] = best;
      w_id[wave] = bid;
    }
    __syncthreads();
    if (wave == 0) {
      double bd = lane < NW ? w_d2[lane] : INFINITY;
      int bj = lane < NW ? w_id[lane] : 0x7fffffff;
      wave_argmin(bd, bj);
      const int j = bj == 0x7fffffff ? 0 : bj;  // (a built layout has a nonempty cluster)
      // 2b. nearest nonempty subcluster of cluster j
      const int64_t sg0 = U.sub_base + (int64_t)j * S;
      double sb = INFINITY;
      int si = 0x7fffffff;
      for (int i0 = 0; i0 < S; i0 += CPW) {
        const int is = min(i0 + row_in, S - 1);
        const float4* p = reinterpret_cast<const float4*>(a.sub_ms + (sg0 + is) * (2 * D) + part * 8);
        const float4 x0 = p[0], x1 = p[1];
        const float m[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        const int cnt = off[j * S + is + 1] - off[j * S + is] + a.sub_fold[sg0 + is];
        double d2 = 0.0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const double df = (double)m[e] - kd[e];
          d2 += df * df;
        }
#pragma unroll
        for (int o = LPC / 2; o > 0; o >>= 1) d2 += __shfl_xor(d2, o, 64);
        if (i0 + row_in < S && cnt > 0 && d2 < sb) {
          sb = d2;
          si = i0 + row_in;
        }
      }
      wave_argmin(sb, si);
      const int is = si == 0x7fffffff ? 0 : si;
      if (lane == 0) {
        const int cf = a.cl_fold[U.cl_base + j];
        const int sf = a.sub_fold[sg0 + is];
        sel[0] = j;
        sel[1] = is;
        sel[2] = off[(j + 1) * S] - off[j * S] + cf;
        sel[3] = off[j * S + is + 1] - off[j * S + is] + sf;
        sel[4] = cf;
        sel[5] = sf;
      }
    }
    __syncthreads();
    // 3. running updates of both groups, and the fold bookkeeping
    const int j = sel[0], is = sel[1];
    const int64_t cg = U.cl_base + j, sg = U.sub_base + (int64_t)j * S + is;
    if (tid < D) {
      const double k = (double)sk[tid], v = (double)sv[tid];
      welford_add(a.cl_ms + cg * (2 * D), a.cl_vbar + cg * D, sel[2], tid, D, k, v);
      welford_add(a.sub_ms + sg * (2 * D), a.sub_vbar + sg * D, sel[3], tid, D, k, v);
    }
    if (tid == 0) {
      a.cl_fold[cg] = sel[4] + 1;
      a.sub_fold[sg] = sel[5] + 1;
      a.fold_sub[(int64_t)u * a.fold_cap + f] = j * S + is;
      a.fold_pos[(int64_t)u * a.fold_cap + f] = t;
    }
    __syncthreads();
  }
  if (tid == 0) {
    a.units[u].N = sq.len + n_new;
    a.units[u].n_fold = sq.f0 + n_new;
  }
}

template <int D, typename T>
static hipError_t append_impl(const AppendLaunch& x, const AArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((k_append<D, T>), dim3(x.L.n_units), dim3(kAppendThreads), 0, s, a);
  return hipGetLastError();
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
  a.cl_fold = x.L.cl_fold;
  a.sub_fold = x.L.sub_fold;
  a.fold_sub = x.L.fold_sub;
  a.fold_pos = x.L.fold_pos;
  a.k_mid = x.L.k_mid;
  a.v_mid = x.L.v_mid;
  a.fold_row0 = x.L.total_mid;
  a.fold_cap = x.L.fold_capacity;
  a.n_recent = x.L.n_recent;
  for (int i = 0; i < MOG_MAX_SEQ; ++i) a.seq[i] = x.seq[i];
  const bool bf = x.L.dtype == MOG_BF16;
  if (x.L.head_dim == 128) return bf ? append_impl<128, uint16_t>(x, a, s) : append_impl<128, float>(x, a, s);
  return bf ? append_impl<64, uint16_t>(x, a, s) : append_impl<64, float>(x, a, s);
}

}  // namespace mog
