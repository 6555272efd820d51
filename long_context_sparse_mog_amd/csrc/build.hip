// Prefill-side build of libmog ("Iceberg Attention" abstract: after prefill,
// partition the keys of each head into about sqrt(N) clusters and about
// log2(N) subclusters per cluster and represent every group by a Gaussian).
//
// Per unit (sequence, KV head), over the middle-region keys:
//   1. Forgy init: C distinct keys drawn by a partial Fisher-Yates shuffle
//      driven by SplitMix64 (Steele, Lea & Flood, OOPSLA 2014).
//   2. Lloyd rounds: nearest centroid by ||mu||^2 - 2 x.mu (lowest id wins a
//      tie), new centroid = mean of its keys (an empty cluster keeps its
//      centroid).  Sums are accumulated in 64-bit fixed point (keys scaled by
//      2^24), so the result does not depend on the order of the atomics.
//   3. Final assignment, stable grouping of the keys by cluster.
//   4. Per cluster, the same k-means with k = min(S, n) on its members,
//      then stable grouping by subcluster: rows ordered by (cluster,
//      subcluster, token position).
//   5. Copy of the K/V rows into that order, and per-group statistics: count
//      (offsets), mean key, population variance of the keys, mean value.
#include "mog_internal.h"

namespace mog {

constexpr unsigned long long kGamma = 0x9E3779B97F4A7C15ull;
constexpr unsigned long long kMix1 = 0xBF58476D1CE4E5B9ull;
constexpr unsigned long long kMix2 = 0x94D049BB133111EBull;
constexpr unsigned long long kSubStreamMul = 0xD1B54A32D192ED03ull;
constexpr float kFixScale = 16777216.0f;  // 2^24

__device__ inline unsigned long long splitmix_next(unsigned long long& state) {
  state += kGamma;
  unsigned long long z = state;
  z = (z ^ (z >> 30)) * kMix1;
  z = (z ^ (z >> 27)) * kMix2;
  return z ^ (z >> 31);
}

__device__ inline unsigned long long unit_prng_state(unsigned long long seed, int unit) {
  return seed ^ (kGamma * (unsigned long long)(1 + unit));
}

struct BArgs {
  const mog_unit* units;
  KVRef kv;
  int n_sink, D;
  float* cent;
  float* cent_norm;
  unsigned long long* sums;
  int32_t* counts;
  int32_t* labels;
  int32_t* cl_start;
  int32_t* members;
  int32_t* sublab;
  int32_t* perm;
  int32_t* sub_off;
  void* k_mid;
  void* v_mid;
  float* cl_ms;
  float* cl_vbar;
  float* sub_ms;
  float* sub_vbar;
  uint16_t* cl_ms16;  // bf16 copies of the four, written beside them
  uint16_t* cl_vbar16;
  uint16_t* sub_ms16;
  uint16_t* sub_vbar16;
  unsigned long long seed;
  // feature-map summaries
  const float* fm_w_in;
  float* fm_w;
  float* cl_fz;
  float* sub_fz;
  int fm_dim;
  float fm_sqrt_scale;
};

template <typename T>
__device__ inline float elem(const T* p, int64_t i);
template <>
__device__ inline float elem<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ inline float elem<uint16_t>(const uint16_t* p, int64_t i) {
  return __uint_as_float((uint32_t)p[i] << 16);
}

// ---------------------------------------------------------------------------
// 1a. Forgy draw of one unit: one thread runs the partial Fisher-Yates
//     shuffle of [0, n_mid) with an open-addressing map (in LDS) of the
//     positions already swapped.  The C drawn ids go to labels[row_base + i].
// ---------------------------------------------------------------------------
constexpr int kHashSize = 8192;  // >= 2 * (2 * kMaxC) entries: load <= 1/2

__device__ inline int hash_slot(int key) { return (int)(((uint32_t)key * 2654435761u) >> 19); }

__device__ inline int map_get(const int* hk, const int* hv, int key) {
  int s = hash_slot(key);
  while (true) {
    const int k = hk[s];
    if (k == key) return hv[s];
    if (k < 0) return key;
    s = (s + 1) & (kHashSize - 1);
  }
}

__device__ inline void map_put(int* hk, int* hv, int key, int val) {
  int s = hash_slot(key);
  while (hk[s] >= 0 && hk[s] != key) s = (s + 1) & (kHashSize - 1);
  hk[s] = key;
  hv[s] = val;
}

__global__ __launch_bounds__(256) void k_forgy(BArgs a) {
  __shared__ int hk[kHashSize];
  __shared__ int hv[kHashSize];
  const int u = blockIdx.x;
  const mog_unit U = a.units[u];
  for (int i = threadIdx.x; i < kHashSize; i += 256) hk[i] = -1;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long st = unit_prng_state(a.seed, u);
    const int n = U.n_mid;
    for (int i = 0; i < U.C; ++i) {
      const unsigned long long r = splitmix_next(st);
      const int j = i + (int)(r % (unsigned long long)(n - i));
      const int vi = map_get(hk, hv, i);
      const int vj = map_get(hk, hv, j);
      map_put(hk, hv, i, vj);
      map_put(hk, hv, j, vi);
      a.labels[U.row_base + i] = vj;
    }
  }
}

// 1b. Centroid i of unit u = key of middle position labels[row_base + i];
//     also zero the fixed-point sums and counts.  One wave per centroid.
template <int D, typename T>
__global__ __launch_bounds__(256) void k_init_centroids(BArgs a) {
  const int u = blockIdx.y;
  const mog_unit U = a.units[u];
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= U.C) return;
  const int id = a.labels[U.row_base + i];
  const T* kb = static_cast<const T*>(a.kv.k) + kv_row_offset(a.kv, U.seq, U.kv_head, a.n_sink + id, D);
  const int64_t cg = U.cl_base + i;
  float nrm = 0.f;
  for (int d = lane; d < D; d += 64) {
    const float x = elem<T>(kb, d);
    a.cent[cg * D + d] = x;
    nrm += x * x;
    a.sums[cg * D + d] = 0ull;
  }
  nrm = wave_sum(nrm);
  if (lane == 0) {
    a.cent_norm[cg] = nrm;
    a.counts[cg] = 0;
  }
}

// ---------------------------------------------------------------------------
// 2. Assignment of 64 keys per block against all centroids of the unit:
//    register-blocked 4x4 dot products from LDS tiles, running argmin of
//    ||mu||^2 - 2 x.mu; then (optionally) fixed-point sums of the key into
//    its cluster, and the cluster count.
// ---------------------------------------------------------------------------
template <int D, typename T>
__global__ __launch_bounds__(256) void k_assign(BArgs a, int accumulate) {
  __shared__ float xs[D * 64];   // [d][key]
  __shared__ float cs[D * 64];   // [d][centroid]
  __shared__ float cn[64];
  const int u = blockIdx.y;
  const mog_unit U = a.units[u];
  const int k0 = blockIdx.x * 64;
  if (k0 >= U.n_mid) return;
  const int tid = threadIdx.x;
  const int nk = min(64, U.n_mid - k0);
  const T* kbase = static_cast<const T*>(a.kv.k);
  // stage keys, transposed
  for (int idx = tid; idx < 64 * D; idx += 256) {
    const int kk = idx / D, d = idx % D;
    float x = 0.f;
    if (kk < nk) x = elem<T>(kbase, kv_row_offset(a.kv, U.seq, U.kv_head, a.n_sink + k0 + kk, D) + d);
    xs[d * 64 + kk] = x;
  }
  const int tk = tid & 15, tc = tid >> 4;   // keys tk*4.., centroids tc*4..
  float best[4];
  int bid[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    best[i] = INFINITY;
    bid[i] = 0x7fffffff;
  }
  for (int c0 = 0; c0 < U.C; c0 += 64) {
    __syncthreads();
    const int nc = min(64, U.C - c0);
    for (int idx = tid; idx < 64 * D; idx += 256) {
      const int cc = idx / D, d = idx % D;
      cs[d * 64 + cc] = cc < nc ? a.cent[(U.cl_base + c0 + cc) * D + d] : 0.f;
    }
    if (tid < 64) cn[tid] = tid < nc ? a.cent_norm[U.cl_base + c0 + tid] : INFINITY;
    __syncthreads();
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
#pragma unroll 8
    for (int d = 0; d < D; ++d) {
      const float4 xv = *reinterpret_cast<const float4*>(&xs[d * 64 + tk * 4]);
      const float4 cv = *reinterpret_cast<const float4*>(&cs[d * 64 + tc * 4]);
      const float xa[4] = {xv.x, xv.y, xv.z, xv.w};
      const float ca[4] = {cv.x, cv.y, cv.z, cv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += xa[i] * ca[j];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int cid = c0 + tc * 4 + j;
      const float nrm = cn[tc * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float dist = nrm - 2.f * acc[i][j];
        if (dist < best[i]) {  // centroids visited in increasing id: ties keep the lower id
          best[i] = dist;
          bid[i] = cid;
        }
      }
    }
  }
  __syncthreads();
  // reduce over the 16 centroid groups of each key
  float* rb = cs;                                   // [16][64] distances
  int* ri = reinterpret_cast<int*>(cs + 16 * 64);   // [16][64] ids
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    rb[tc * 64 + tk * 4 + i] = best[i];
    ri[tc * 64 + tk * 4 + i] = bid[i];
  }
  __syncthreads();
  __shared__ int lab[64];
  if (tid < 64) {
    float b = rb[tid];
    int id = ri[tid];
    for (int g = 1; g < 16; ++g) {
      const float v = rb[g * 64 + tid];
      const int vid = ri[g * 64 + tid];
      if (v < b || (v == b && vid < id)) {
        b = v;
        id = vid;
      }
    }
    if (id < 0 || id >= U.C) id = 0;  // only reachable for non-finite keys
    lab[tid] = id;
    if (tid < nk) {
      a.labels[U.row_base + k0 + tid] = id;
      atomicAdd(&a.counts[U.cl_base + id], 1);
    }
  }
  if (!accumulate) return;
  __syncthreads();
  for (int idx = tid; idx < nk * D; idx += 256) {
    const int kk = idx / D, d = idx % D;
    const long long fx = __float2ll_rn(xs[d * 64 + kk] * kFixScale);
    atomicAdd(&a.sums[(U.cl_base + lab[kk]) * D + d], (unsigned long long)fx);
  }
}

// ---------------------------------------------------------------------------
// 2'. The same assignment for bf16 keys on the matrix cores: the x.mu of 64
//     keys per wave against 64 centroids per stage are 16x16 tiles of
//     v_mfma_f32_16x16x32_bf16.  Keys are the A operand straight from their
//     rows (lane (g, n): key n of the tile, dimensions 32 s + 8 g .. + 7);
//     each centroid is split into bf16 high and low parts (hi + lo carries
//     about 16 mantissa bits) staged in LDS in B-operand order, and both
//     parts accumulate into one float32 tile, so a distance
//     ||mu||^2 - 2 x.mu differs from the float32 one by about 2^-16 of
//     |x||mu|.  Lane (g, n) of a result tile holds keys 4g .. 4g+3 against
//     centroid n; a running argmin per lane (centroids visited in increasing
//     id) and a 16-lane reduction (ties to the lower id) finish the key.
//     Stages are double-buffered.  256 keys per block.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ inline uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <int D>
__global__ __launch_bounds__(256) void k_assign_mfma(BArgs a, int accumulate) {
  constexpr int KS = D / 32;    // k-steps of 32 dimensions
  constexpr int RT = 4;         // 16-key row tiles per wave
  constexpr int KPB = 4 * 16 * RT;
  constexpr int CT = 4;         // 16-centroid column tiles per stage
  __shared__ uint4 cf[2][2][KS][CT][64];  // [buffer][hi, lo][k-step][column tile][lane]
  __shared__ float cn[2][16 * CT];
  __shared__ int lab[KPB];
  const int u = blockIdx.y;
  const mog_unit U = a.units[u];
  const int k0 = blockIdx.x * KPB;
  if (k0 >= U.n_mid) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, n = lane & 15;
  const int C = U.C;
  const uint16_t* kb = static_cast<const uint16_t*>(a.kv.k);
  // A fragments of the wave's 64 keys (zero past the middle region)
  uint4 af[RT][KS];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int key = k0 + wave * 16 * RT + rt * 16 + n;
    if (key < U.n_mid) {
      const int64_t off = kv_row_offset(a.kv, U.seq, U.kv_head, a.n_sink + key, D) + 8 * g;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) af[rt][ks] = *reinterpret_cast<const uint4*>(kb + off + 32 * ks);
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) af[rt][ks] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  // stage centroids [c0, c0 + 64) into buffer b: thread (c, q) converts
  // dimensions [q D/4, (q+1) D/4) of centroid c
  auto stage = [&](int b, int c0) {
    const int c = tid >> 2, q = tid & 3;
    const int cid = c0 + c;
#pragma unroll
    for (int d0 = q * (D / 4); d0 < (q + 1) * (D / 4); d0 += 8) {
      float x[8];
      if (cid < C) {
        const float4* p = reinterpret_cast<const float4*>(a.cent + (U.cl_base + cid) * D + d0);
        const float4 v0 = p[0], v1 = p[1];
        x[0] = v0.x; x[1] = v0.y; x[2] = v0.z; x[3] = v0.w;
        x[4] = v1.x; x[5] = v1.y; x[6] = v1.z; x[7] = v1.w;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = 0.f;
      }
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t h0 = bf16_rne(x[2 * e]), h1 = bf16_rne(x[2 * e + 1]);
        const uint32_t l0 = bf16_rne(x[2 * e] - __uint_as_float(h0 << 16));
        const uint32_t l1 = bf16_rne(x[2 * e + 1] - __uint_as_float(h1 << 16));
        hi[e] = h0 | (h1 << 16);
        lo[e] = l0 | (l1 << 16);
      }
      const int ks = d0 / 32, gg = (d0 % 32) / 8;
      const int ct = c / 16, ln = (c % 16) + 16 * gg;
      cf[b][0][ks][ct][ln] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      cf[b][1][ks][ct][ln] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    }
    if (tid < 16 * CT) cn[b][tid] = c0 + tid < C ? a.cent_norm[U.cl_base + c0 + tid] : INFINITY;
  };
  float best[RT][4];
  int bid[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      best[rt][i] = INFINITY;
      bid[rt][i] = 0x7fffffff;
    }
  const int nst = (C + 16 * CT - 1) / (16 * CT);
  stage(0, 0);
  __syncthreads();
  for (int t = 0; t < nst; ++t) {
    const int b = t & 1;
    if (t + 1 < nst) stage(b ^ 1, (t + 1) * 16 * CT);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      f32x4_t acc[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) acc[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8_t bh = __builtin_bit_cast(bf16x8_t, cf[b][0][ks][ct][lane]);
        const bf16x8_t bl = __builtin_bit_cast(bf16x8_t, cf[b][1][ks][ct][lane]);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const bf16x8_t av = __builtin_bit_cast(bf16x8_t, af[rt][ks]);
          acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bh, acc[rt], 0, 0, 0);
          acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bl, acc[rt], 0, 0, 0);
        }
      }
      const int cid = t * 16 * CT + ct * 16 + n;
      const float nrm = cn[b][ct * 16 + n];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float dist = nrm - 2.f * acc[rt][i];
          if (dist < best[rt][i]) {  // a lane's centroids come in increasing id
            best[rt][i] = dist;
            bid[rt][i] = cid;
          }
        }
    }
    __syncthreads();
  }
  // the 16 lanes of a row group hold the same keys against different
  // centroids: reduce (ties to the lower id)
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int o = 8; o > 0; o >>= 1) {
        const float od = __shfl_xor(best[rt][i], o, 64);
        const int oi = __shfl_xor(bid[rt][i], o, 64);
        if (od < best[rt][i] || (od == best[rt][i] && oi < bid[rt][i])) {
          best[rt][i] = od;
          bid[rt][i] = oi;
        }
      }
    }
  const int nk = min(KPB, U.n_mid - k0);
  if (n == 0) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kk = wave * 16 * RT + rt * 16 + 4 * g + i;
        int id = bid[rt][i];
        if (id < 0 || id >= C) id = 0;  // only reachable for non-finite keys
        lab[kk] = id;
        if (kk < nk) {
          a.labels[U.row_base + k0 + kk] = id;
          atomicAdd(&a.counts[U.cl_base + id], 1);
        }
      }
  }
  if (!accumulate) return;
  __syncthreads();
  // fixed-point sums of every key into its cluster: a wave per key, lanes
  // over the dimensions
  for (int kk = wave; kk < nk; kk += 4) {
    const int64_t off = kv_row_offset(a.kv, U.seq, U.kv_head, a.n_sink + k0 + kk, D);
    const int64_t dst = (U.cl_base + lab[kk]) * D;
    for (int d = lane; d < D; d += 64) {
      const long long fx = __float2ll_rn(elem<uint16_t>(kb, off + d) * kFixScale);
      atomicAdd(&a.sums[dst + d], (unsigned long long)fx);
    }
  }
}

// 2b. New centroid = fixed-point sum / count (empty keeps); zero the sums.
template <int D>
__global__ __launch_bounds__(256) void k_update(BArgs a) {
  const int u = blockIdx.y;
  const mog_unit U = a.units[u];
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (j >= U.C) return;
  const int64_t cg = U.cl_base + j;
  const int n = a.counts[cg];
  float nrm = 0.f;
  for (int d = lane; d < D; d += 64) {
    float c = a.cent[cg * D + d];
    if (n > 0) {
      const long long s = (long long)a.sums[cg * D + d];
      c = (float)((double)s / (double)kFixScale / (double)n);
      a.cent[cg * D + d] = c;
    }
    nrm += c * c;
    a.sums[cg * D + d] = 0ull;
  }
  nrm = wave_sum(nrm);
  if (lane == 0) {
    a.cent_norm[cg] = nrm;
    a.counts[cg] = 0;
  }
}

// ---------------------------------------------------------------------------
// 3a. Exclusive prefix of the final cluster counts -> first member slot.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_cluster_starts(BArgs a) {
  __shared__ int sh[16];
  __shared__ int carry;
  const int u = blockIdx.x, tid = threadIdx.x;
  const mog_unit U = a.units[u];
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < U.C; base += 1024) {
    const int j = base + tid;
    const int v = j < U.C ? a.counts[U.cl_base + j] : 0;
    int x = v;
    const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) sh[wave] = x;
    __syncthreads();
    int off = carry, tot = 0;
    for (int w = 0; w < 16; ++w) {
      off += (w < wave) ? sh[w] : 0;
      tot += sh[w];
    }
    if (j < U.C) a.cl_start[U.cl_base + j] = off + x - v;
    __syncthreads();
    if (tid == 0) carry += tot;
    __syncthreads();
  }
}

// 3b. Stable grouping: block (b, u) scans all middle keys of unit u in order
//     and appends those of clusters [8b, 8b+8) to their member lists.
__global__ __launch_bounds__(1024) void k_group_members(BArgs a) {
  __shared__ int cnt[16][8];
  __shared__ int run[8];
  __shared__ int start[8];
  const int u = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const mog_unit U = a.units[u];
  const int j0 = blockIdx.x * 8;
  if (j0 >= U.C) return;
  if (tid < 8) {
    run[tid] = 0;
    start[tid] = (j0 + tid < U.C) ? a.cl_start[U.cl_base + j0 + tid] : 0;
  }
  __syncthreads();
  const unsigned long long lt = (1ull << lane) - 1ull;
  for (int base = 0; base < U.n_mid; base += 1024) {
    const int i = base + tid;
    int slot = -1;
    if (i < U.n_mid) {
      const int lab = a.labels[U.row_base + i];
      if (lab >= j0 && lab < j0 + 8) slot = lab - j0;
    }
    int myrank = 0;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const unsigned long long b = __ballot(slot == s);
      if (slot == s) myrank = __popcll(b & lt);
      if (lane == 0) cnt[wave][s] = __popcll(b);
    }
    __syncthreads();
    if (slot >= 0) {
      int pos = run[slot] + myrank;
      for (int w = 0; w < wave; ++w) pos += cnt[w][slot];
      a.members[U.row_base + start[slot] + pos] = i;
    }
    __syncthreads();
    if (tid < 8) {
      int t = 0;
      for (int w = 0; w < 16; ++w) t += cnt[w][tid];
      run[tid] += t;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// 4. Subcluster k-means of one cluster per block, then the stable order of
//    its members by subcluster: writes perm and the cluster's S offsets.
// ---------------------------------------------------------------------------
template <int D, typename T>
__global__ __launch_bounds__(256) void k_subkmeans(BArgs a, int iters) {
  __shared__ float cen[kMaxS][D];
  __shared__ float cnorm[kMaxS];
  __shared__ unsigned long long accq[kMaxS][D];  // fixed-point sums of the members
  __shared__ int scount[kMaxS];
  __shared__ int sstart[kMaxS + 1];
  __shared__ int ids[kMaxS];
  __shared__ int wcnt[4][kMaxS];
  __shared__ int run[kMaxS];
  const int u = blockIdx.y, j = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const mog_unit U = a.units[u];
  if (j >= U.C) return;
  const int S = U.S;
  const int64_t cg = U.cl_base + j;
  const int cl0 = a.cl_start[cg];
  const int n = (j + 1 < U.C ? a.cl_start[cg + 1] : U.n_mid) - cl0;
  int32_t* off = a.sub_off + U.off_base;
  if (j == U.C - 1 && tid == 0) off[U.C * S] = U.n_mid;
  if (n == 0) {
    for (int i = tid; i < S; i += 256) off[j * S + i] = cl0;
    return;
  }
  const int k = n < S ? n : S;
  const int32_t* mem = a.members + U.row_base + cl0;
  int32_t* sl = a.sublab + U.row_base + cl0;
  const T* kb = static_cast<const T*>(a.kv.k);
  // Forgy draw over [0, n): k <= 32 steps, the swapped positions kept in a
  // short list (at most 2k entries)
  if (tid == 0) {
    unsigned long long st = unit_prng_state(a.seed, u) ^ (kSubStreamMul * (unsigned long long)(j + 1));
    int pk[2 * kMaxS], pv[2 * kMaxS], np = 0;
    auto get = [&](int key) {
      for (int e = 0; e < np; ++e)
        if (pk[e] == key) return pv[e];
      return key;
    };
    auto put = [&](int key, int val) {
      for (int e = 0; e < np; ++e)
        if (pk[e] == key) {
          pv[e] = val;
          return;
        }
      pk[np] = key;
      pv[np] = val;
      ++np;
    };
    for (int i = 0; i < k; ++i) {
      const unsigned long long r = splitmix_next(st);
      const int jj = i + (int)(r % (unsigned long long)(n - i));
      const int vi = get(i), vj = get(jj);
      put(i, vj);
      put(jj, vi);
      ids[i] = vj;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < k * D; idx += 256) {
    const int c = idx / D, d = idx % D;
    const int m = mem[ids[c]];
    cen[c][d] = elem<T>(kb, kv_row_offset(a.kv, U.seq, U.kv_head, a.n_sink + m, D) + d);
  }
  __syncthreads();
  for (int round = 0; round <= iters; ++round) {
    // norms of the current centroids
    if (tid < k) {
      float s = 0.f;
      for (int d = 0; d < D; ++d) s += cen[tid][d] * cen[tid][d];
      cnorm[tid] = s;
    }
    if (tid < kMaxS) scount[tid] = 0;
    if (round < iters)
      for (int idx = tid; idx < k * D; idx += 256) accq[idx / D][idx % D] = 0ull;
    __syncthreads();
    // assignment: one member per thread, which then adds the member into its
    // subcluster's fixed-point sums (integer adds: the order does not
    // matter)
    for (int m = tid; m < n; m += 256) {
      const int64_t ro = kv_row_offset(a.kv, U.seq, U.kv_head, a.n_sink + mem[m], D);
      // the whole row in registers (one batch of 16-byte loads)
      float x[D];
#pragma unroll
      for (int d0 = 0; d0 < D; d0 += 8) {
        float t8[8];
        load8<T>(kb, ro + d0, t8);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[d0 + e] = t8[e];
      }
      float dot[kMaxS];
#pragma unroll
      for (int c = 0; c < kMaxS; ++c) dot[c] = 0.f;
#pragma unroll
      for (int c = 0; c < kMaxS; ++c) {
        if (c < k) {
#pragma unroll
          for (int d = 0; d < D; ++d) dot[c] += x[d] * cen[c][d];
        }
      }
      float best = INFINITY;
      int bid = 0;
#pragma unroll
      for (int c = 0; c < kMaxS; ++c) {
        if (c < k) {
          const float dist = cnorm[c] - 2.f * dot[c];
          if (dist < best) {
            best = dist;
            bid = c;
          }
        }
      }
      sl[m] = bid;
      atomicAdd(&scount[bid], 1);
      if (round < iters) {
#pragma unroll
        for (int d = 0; d < D; ++d)
          atomicAdd(&accq[bid][d], (unsigned long long)__float2ll_rn(x[d] * kFixScale));
      }
    }
    __syncthreads();
    if (round == iters) break;
    // update: new centroid = sum / count (an empty subcluster keeps its own)
    for (int idx = tid; idx < k * D; idx += 256) {
      const int c = idx / D, dd = idx % D;
      if (scount[c] > 0)
        cen[c][dd] = (float)((double)(long long)accq[c][dd] / ((double)scount[c] * (double)kFixScale));
    }
    __syncthreads();
  }
  // offsets of the subclusters inside the cluster
  if (tid == 0) {
    int s = 0;
    for (int c = 0; c < S; ++c) {
      sstart[c] = s;
      run[c] = 0;
      s += c < k ? scount[c] : 0;
    }
    sstart[S] = s;
  }
  __syncthreads();
  for (int i = tid; i < S; i += 256) off[j * S + i] = cl0 + sstart[i];
  // stable scatter of the members by subcluster
  const unsigned long long lt = (1ull << lane) - 1ull;
  for (int base = 0; base < n; base += 256) {
    const int m = base + tid;
    const int lab = m < n ? sl[m] : -1;
    int myrank = 0;
    for (int c = 0; c < k; ++c) {
      const unsigned long long b = __ballot(lab == c);
      if (lab == c) myrank = __popcll(b & lt);
      if (lane == 0) wcnt[wave][c] = __popcll(b);
    }
    __syncthreads();
    if (lab >= 0) {
      int pos = sstart[lab] + run[lab] + myrank;
      for (int w = 0; w < wave; ++w) pos += wcnt[w][lab];
      a.perm[U.row_base + cl0 + pos] = a.n_sink + mem[m];
    }
    __syncthreads();
    if (tid < k) run[tid] += wcnt[0][tid] + wcnt[1][tid] + wcnt[2][tid] + wcnt[3][tid];
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// 5a. Copy K/V rows into (cluster, subcluster, position) order: 16-byte
//     pieces, rows spread over the wave.
// ---------------------------------------------------------------------------
template <int D, typename T>
__global__ __launch_bounds__(256) void k_gather_rows(BArgs a) {
  constexpr int EL = 16 / sizeof(T);      // elements per 16-byte piece
  constexpr int LPR = D / EL;             // lanes per row
  constexpr int RPW = 64 / LPR;           // rows per wave step
  const int u = blockIdx.y;
  const mog_unit U = a.units[u];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = (blockIdx.x * 4 + wave) * RPW + lane / LPR;
  if (r >= U.n_mid) return;
  const int t = a.perm[U.row_base + r];
  const int64_t src = kv_row_offset(a.kv, U.seq, U.kv_head, t, D) + (lane % LPR) * EL;
  const int64_t dst = (U.row_base + r) * D + (lane % LPR) * EL;
  const uint4* ks = reinterpret_cast<const uint4*>(static_cast<const T*>(a.kv.k) + src);
  const uint4* vs = reinterpret_cast<const uint4*>(static_cast<const T*>(a.kv.v) + src);
  *reinterpret_cast<uint4*>(static_cast<T*>(a.k_mid) + dst) = *ks;
  *reinterpret_cast<uint4*>(static_cast<T*>(a.v_mid) + dst) = *vs;
}

// 5b. Statistics of one cluster and its subclusters: two passes over the
//     reordered keys (means, then centred squares), one over the values,
//     accumulated in float64, stored in float32 and, rounded from that, in
//     bf16 for the decode.  Thread (d, phase) owns dimension d of every
//     NPH-th row.
template <int D, typename T>
__global__ __launch_bounds__(256) void k_group_stats(BArgs a) {
  constexpr int NPH = 256 / D;
  __shared__ double rk[NPH][D];
  __shared__ double rv[NPH][D];
  const int u = blockIdx.y, j = blockIdx.x, tid = threadIdx.x;
  const mog_unit U = a.units[u];
  if (j >= U.C) return;
  const int S = U.S;
  const int32_t* off = a.sub_off + U.off_base;
  const int64_t cg = U.cl_base + j;
  const T* km = static_cast<const T*>(a.k_mid);
  const T* vm = static_cast<const T*>(a.v_mid);
  const int d = tid % D, ph = tid / D;
  // g = -1 is the cluster itself, g >= 0 its subclusters
  for (int g = -1; g < S; ++g) {
    const int r0 = g < 0 ? off[j * S] : off[j * S + g];
    const int r1 = g < 0 ? off[(j + 1) * S] : off[j * S + g + 1];
    const int n = r1 - r0;
    const int64_t gi = g < 0 ? cg : U.sub_base + (int64_t)j * S + g;
    float* ms = (g < 0 ? a.cl_ms : a.sub_ms) + gi * 2 * D;
    float* vb = (g < 0 ? a.cl_vbar : a.sub_vbar) + gi * D;
    uint16_t* ms16 = (g < 0 ? a.cl_ms16 : a.sub_ms16) + gi * 2 * D;
    uint16_t* vb16 = (g < 0 ? a.cl_vbar16 : a.sub_vbar16) + gi * D;
    if (n == 0) {
      if (ph == 0) {
        ms[d] = 0.f;
        ms[D + d] = 0.f;
        vb[d] = 0.f;
        ms16[d] = ms16[D + d] = vb16[d] = 0;
      }
      continue;
    }
    double sk = 0.0, sv = 0.0;
    for (int r = r0 + ph; r < r1; r += NPH) {
      sk += (double)elem<T>(km, (U.row_base + r) * D + d);
      sv += (double)elem<T>(vm, (U.row_base + r) * D + d);
    }
    rk[ph][d] = sk;
    rv[ph][d] = sv;
    __syncthreads();
    double tk = 0.0, tv = 0.0;
#pragma unroll
    for (int p = 0; p < NPH; ++p) {
      tk += rk[p][d];
      tv += rv[p][d];
    }
    const double mean = tk / n, vmean = tv / n;
    __syncthreads();
    double sq = 0.0;
    for (int r = r0 + ph; r < r1; r += NPH) {
      const double x = (double)elem<T>(km, (U.row_base + r) * D + d) - mean;
      sq += x * x;
    }
    rk[ph][d] = sq;
    __syncthreads();
    if (ph == 0) {
      double t = 0.0;
#pragma unroll
      for (int p = 0; p < NPH; ++p) t += rk[p][d];
      ms[d] = (float)mean;
      ms[D + d] = (float)(t / n);
      vb[d] = (float)vmean;
      ms16[d] = bf16_bits((float)mean);
      ms16[D + d] = bf16_bits((float)(t / n));
      vb16[d] = bf16_bits((float)vmean);
    }
    __syncthreads();
  }
}

// 6. Feature-map summaries (retrieval-completion page, abstract: a
//    fixed-size feature-map summary of the keys, computed at prefill): per
//    group the sum over its members of phi(x) = exp(W x - |x|^2 / 2) /
//    sqrt(m), x = sqrt(s) k.  Thread (i, ph) holds row i of W in registers
//    and takes every NPH-th row of each subcluster (rows staged 32 at a time
//    in LDS with their |x|^2); sums are float32.  Block (0, 0) also copies W
//    into the layout.
template <int D, typename T>
__global__ __launch_bounds__(256) void k_fm_summaries(BArgs a) {
  constexpr int RB = 32;  // rows staged at once
  __shared__ float xs[RB][D];
  __shared__ float xx[RB];
  __shared__ float part[256];
  const int u = blockIdx.y, j = blockIdx.x, tid = threadIdx.x;
  const int m = a.fm_dim, NPH = 256 / m;
  if (u == 0 && j == 0)
    for (int e = tid; e < m * D; e += 256) a.fm_w[e] = a.fm_w_in[e];
  const mog_unit U = a.units[u];
  if (j >= U.C) return;
  const int S = U.S;
  const int fi = tid % m, ph = tid / m;
  float w[D];
#pragma unroll
  for (int e = 0; e < D; e += 4) {
    const float4 v = *reinterpret_cast<const float4*>(a.fm_w_in + (int64_t)fi * D + e);
    w[e] = v.x; w[e + 1] = v.y; w[e + 2] = v.z; w[e + 3] = v.w;
  }
  const int32_t* off = a.sub_off + U.off_base;
  const T* km = static_cast<const T*>(a.k_mid);
  const float sq = a.fm_sqrt_scale, inv_sqrt_m = rsqrtf((float)m);
  float zc = 0.f;
  for (int i = 0; i < S; ++i) {
    const int r0 = off[j * S + i], r1 = off[j * S + i + 1];
    float zs = 0.f;
    for (int rb = r0; rb < r1; rb += RB) {
      const int nr = min(RB, r1 - rb);
      __syncthreads();
      for (int e = tid; e < nr * D; e += 256)
        xs[e / D][e % D] = sq * elem<T>(km, (U.row_base + rb) * D + e);
      __syncthreads();
      if (tid < nr) {
        float t = 0.f;
#pragma unroll 8
        for (int e = 0; e < D; ++e) t += xs[tid][e] * xs[tid][e];
        xx[tid] = t;
      }
      __syncthreads();
      for (int r = ph; r < nr; r += NPH) {
        float t = 0.f;
#pragma unroll
        for (int e = 0; e < D; ++e) t += w[e] * xs[r][e];
        zs += expf(t - 0.5f * xx[r]);
      }
    }
    part[tid] = zs;
    __syncthreads();
    if (ph == 0) {
      float t = 0.f;
      for (int p = 0; p < NPH; ++p) t += part[p * m + fi];
      a.sub_fz[(U.sub_base + (int64_t)j * S + i) * m + fi] = t * inv_sqrt_m;
      zc += t;
    }
  }
  if (ph == 0) a.cl_fz[(U.cl_base + j) * m + fi] = zc * inv_sqrt_m;
}

// ---------------------------------------------------------------------------
// Unit table of a layout (same arithmetic as the host carving).
// ---------------------------------------------------------------------------
__global__ void k_layout_table(mog_unit* units, SeqArgs seq, int Hkv, int n_sink, int n_recent,
                               int32_t* cl_fold, int64_t n_cl, int32_t* sub_fold, int64_t n_sub) {
  // no folded tokens yet: zero the per-group fold counts
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_cl + n_sub; i += step) {
    if (i < n_cl) cl_fold[i] = 0;
    else sub_fold[i - n_cl] = 0;
  }
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
  U.n_fold = 0;
  U.reserved1 = 0;
  U.row_base = row + (int64_t)kvh * z.n_mid;
  U.cl_base = cl + (int64_t)kvh * z.C;
  U.sub_base = sub + (int64_t)kvh * z.C * z.S;
  U.off_base = offb + (int64_t)kvh * (z.C * z.S + 1);
  units[u] = U;
}

// The bf16 copies of the group statistics: element i of each float32
// array, rounded (grid-stride over the four arrays one after another).
__global__ __launch_bounds__(256) void k_stats16(const float* a0, uint16_t* b0, int64_t n0, const float* a1,
                                                 uint16_t* b1, int64_t n1, const float* a2, uint16_t* b2,
                                                 int64_t n2, const float* a3, uint16_t* b3, int64_t n3) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n0 + n1 + n2 + n3; i += stride) {
    int64_t j = i;
    if (j < n0) { b0[j] = bf16_bits(a0[j]); continue; }
    j -= n0;
    if (j < n1) { b1[j] = bf16_bits(a1[j]); continue; }
    j -= n1;
    if (j < n2) { b2[j] = bf16_bits(a2[j]); continue; }
    j -= n2;
    b3[j] = bf16_bits(a3[j]);
  }
}

hipError_t launch_stats16(const mog_layout& L, hipStream_t s) {
  const int64_t D = L.head_dim;
  const int64_t n0 = L.total_cl * 2 * D, n1 = L.total_cl * D, n2 = L.total_sub * 2 * D, n3 = L.total_sub * D;
  const int64_t nt = n0 + n1 + n2 + n3;
  const int64_t nb = nt <= 0 ? 1 : (nt + 255) / 256 < 4096 ? (nt + 255) / 256 : 4096;
  hipLaunchKernelGGL(k_stats16, dim3((unsigned)nb), dim3(256), 0, s, L.cl_ms, L.cl_ms16, n0, L.cl_vbar,
                     L.cl_vbar16, n1, L.sub_ms, L.sub_ms16, n2, L.sub_vbar, L.sub_vbar16, n3);
  return hipGetLastError();
}

hipError_t launch_layout_table(const mog_layout& L, const SeqArgs& seq, hipStream_t s) {
  const int n = L.n_units;
  const int64_t n_cnt = L.total_cl + L.total_sub;
  const int64_t nb = max((int64_t)(n + 255) / 256, min((n_cnt + 255) / 256, (int64_t)1024));
  hipLaunchKernelGGL(k_layout_table, dim3((unsigned)nb), dim3(256), 0, s, L.units, seq, L.n_kv_heads, L.n_sink,
                     L.n_recent, L.cl_fold, L.total_cl, L.sub_fold, L.total_sub);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Launcher
// ---------------------------------------------------------------------------
template <int D, typename T>
static hipError_t build_impl(const BuildLaunch& x, hipStream_t s) {
  BArgs a;
  a.units = x.L.units;
  a.kv = x.kv;
  a.n_sink = x.L.n_sink;
  a.D = D;
  a.cent = x.ws.cent;
  a.cent_norm = x.ws.cent_norm;
  a.sums = x.ws.sums;
  a.counts = x.ws.counts;
  a.labels = x.ws.labels;
  a.cl_start = x.ws.cl_start;
  a.members = x.ws.members;
  a.sublab = x.ws.sublab;
  a.perm = x.L.perm;
  a.sub_off = x.L.sub_off;
  a.k_mid = x.L.k_mid;
  a.v_mid = x.L.v_mid;
  a.cl_ms = x.L.cl_ms;
  a.cl_vbar = x.L.cl_vbar;
  a.sub_ms = x.L.sub_ms;
  a.sub_vbar = x.L.sub_vbar;
  a.cl_ms16 = x.L.cl_ms16;
  a.cl_vbar16 = x.L.cl_vbar16;
  a.sub_ms16 = x.L.sub_ms16;
  a.sub_vbar16 = x.L.sub_vbar16;
  a.seed = x.seed;
  const int nu = x.L.n_units;
  int max_mid = 0;
  for (int si = 0; si < x.seq.n_seq; ++si) {
    const UnitSizes z = unit_sizes(x.seq.len[si], x.L.n_sink, x.L.n_recent);
    max_mid = z.n_mid > max_mid ? z.n_mid : max_mid;
  }
  const int maxC = x.L.max_C;
  hipLaunchKernelGGL(k_forgy, dim3(nu), dim3(256), 0, s, a);
  hipLaunchKernelGGL((k_init_centroids<D, T>), dim3((maxC + 3) / 4, nu), dim3(256), 0, s, a);
  // bf16 keys: the matrix-core assignment; float32 keys: the float32 one
  auto assign = [&](int accumulate) {
    if constexpr (sizeof(T) == 2)
      hipLaunchKernelGGL((k_assign_mfma<D>), dim3((max_mid + 255) / 256, nu), dim3(256), 0, s, a, accumulate);
    else
      hipLaunchKernelGGL((k_assign<D, T>), dim3((max_mid + 63) / 64, nu), dim3(256), 0, s, a, accumulate);
  };
  for (int it = 0; it < x.iters; ++it) {
    assign(1);
    hipLaunchKernelGGL((k_update<D>), dim3((maxC + 3) / 4, nu), dim3(256), 0, s, a);
  }
  assign(0);
  hipLaunchKernelGGL(k_cluster_starts, dim3(nu), dim3(1024), 0, s, a);
  hipLaunchKernelGGL(k_group_members, dim3((maxC + 7) / 8, nu), dim3(1024), 0, s, a);
  hipLaunchKernelGGL((k_subkmeans<D, T>), dim3(maxC, nu), dim3(256), 0, s, a, x.iters);
  constexpr int RPB = 4 * (64 / (D / (16 / (int)sizeof(T))));
  hipLaunchKernelGGL((k_gather_rows<D, T>), dim3((max_mid + RPB - 1) / RPB, nu), dim3(256), 0, s, a);
  hipLaunchKernelGGL((k_group_stats<D, T>), dim3(maxC, nu), dim3(256), 0, s, a);
  if (x.L.fm_dim) {
    a.fm_w_in = x.fm_w;
    a.fm_w = x.L.fm_w;
    a.cl_fz = x.L.cl_fz;
    a.sub_fz = x.L.sub_fz;
    a.fm_dim = x.L.fm_dim;
    a.fm_sqrt_scale = sqrtf(x.L.fm_scale);
    hipLaunchKernelGGL((k_fm_summaries<D, T>), dim3(maxC, nu), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_build(const BuildLaunch& x, hipStream_t s) {
  if (x.D == 128) return x.dtype == MOG_BF16 ? build_impl<128, uint16_t>(x, s) : build_impl<128, float>(x, s);
  return x.dtype == MOG_BF16 ? build_impl<64, uint16_t>(x, s) : build_impl<64, float>(x, s);
}

}  // namespace mog
