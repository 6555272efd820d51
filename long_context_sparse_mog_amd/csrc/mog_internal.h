// Internal declarations of libmog: geometry shared by the host API and the
// kernels, the argument blocks handed to the launchers, and small device
// helpers.  gfx950 only (64-wide wavefronts).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mog.h"

namespace mog {

constexpr int kWave = 64;
constexpr int kMaxG = 8;        // query heads per KV head
constexpr int kMaxS = 32;       // subclusters per cluster (N <= 2^22 gives S <= 22)
constexpr int kMaxC = 2048;     // clusters per unit (N <= 2^22 gives C <= 2048)
constexpr int kWaveListMax = 256;  // chosen clusters per unit an exact wave lists on its own (4 per lane)
// subcluster rows the decode kernels hold per cluster: S = ceil(log2 n) <= 22
// for n <= 2^22, rounded up to a multiple of 4 (one row per wave and step)
constexpr int kDecodeSubRows = 24;
static_assert(MOG_MAX_LEN <= (1 << 22) && kDecodeSubRows >= 22 && kDecodeSubRows % 4 == 0,
              "every subcluster of a cluster fits the decode kernels' rows");
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// Geometry: one unit = one (sequence, KV head).  The same arithmetic runs on
// the host (sizes, carving) and in the layout-table kernel.
// ---------------------------------------------------------------------------

__host__ __device__ inline int ceil_sqrt_i(int64_t n) {
  if (n <= 0) return 0;
  int64_t r = (int64_t)sqrt((double)n);
  while (r * r > n) --r;
  while (r * r < n) ++r;
  return (int)r;
}

__host__ __device__ inline int ceil_log2_i(int64_t n) {
  int e = 0;
  while (((int64_t)1 << e) < n) ++e;
  return e;
}

struct UnitSizes {
  int n_mid, C, S;
};

__host__ __device__ inline UnitSizes unit_sizes(int N, int n_sink, int n_recent) {
  UnitSizes s;
  s.n_mid = N - n_sink - n_recent;
  int c = ceil_sqrt_i(N);
  s.C = c < s.n_mid ? c : s.n_mid;
  int S = ceil_log2_i(N);
  s.S = S < 1 ? 1 : S;
  return s;
}

// Per-sequence numbers passed by value to kernels.
struct SeqArgs {
  int32_t n_seq;
  int32_t len[MOG_MAX_SEQ];
  int16_t top_c[MOG_MAX_SEQ];
  int8_t top_s[MOG_MAX_SEQ];
};

// ---------------------------------------------------------------------------
// KV cache addressing (contiguous or paged) for kernels.
// ---------------------------------------------------------------------------
struct KVRef {
  const void* k;
  const void* v;
  const int32_t* block_table;
  int32_t paged;
  int32_t n_kv_heads;
  int32_t max_len;      // contiguous
  int32_t page_shift;   // paged: log2(page_size)
  int32_t max_blocks;   // paged
};

// Element offset of token t of (seq, kvh) in the K (or V) array.
__device__ inline int64_t kv_row_offset(const KVRef& kv, int seq, int kvh, int t, int D) {
  if (!kv.paged) {
    return ((int64_t)(seq * kv.n_kv_heads + kvh) * kv.max_len + t) * D;
  }
  const int blk = t >> kv.page_shift;
  const int slot = t & ((1 << kv.page_shift) - 1);
  const int page = kv.block_table[(int64_t)seq * kv.max_blocks + blk];
  const int64_t row = (((int64_t)page * kv.n_kv_heads + kvh) << kv.page_shift) + slot;
  return row * D;
}

// ---------------------------------------------------------------------------
// Decode launch block.
// ---------------------------------------------------------------------------
// One exact tile (16 bytes): element offset of its first row (in the layout
// rows, or in the KV cache when the src bit is set), row count (<= 32) with
// the src bit in bit 31, and the mask of the query heads that read it.
struct TileRec {
  int64_t off;
  int32_t nrows_src;
  uint32_t mask;
};

// Tile slots of a unit start here.  A chosen cluster of n reordered rows and
// f folded rows yields at most ceil(n/32) + S + f tiles (one partial tile
// per run, at most S runs; a folded row in a tile of its own at worst), so
// n_mid/32 + C (S + 1) + 1 + fold_cap slots per unit suffice; the base below
// grows by at least that much from one unit to the next.
__host__ __device__ inline int64_t tile_unit_base(int64_t row_base, int64_t cl_base, int u, int fold_cap) {
  return cl_base * (kMaxS + 1) + (row_base >> 5) + (int64_t)u * (1 + fold_cap);
}

// Per-cluster entries of unit u start at u * max_C (the largest C of the
// layout), so a kernel can address them from the unit index alone.
struct DecodeWS {
  float* cl_score;      // [n_units][G][max_C]  log2-domain scores (head-major: a head's scores are contiguous)
  float* cl_lse;        // [n_units][G]          shared selection: log2 of each head's total estimated mass
  uint32_t* cl_mask;    // [n_units * max_C]     heads that chose the cluster
  int32_t* cl_tiles;    // [n_units * max_C]     tile slots the cluster needs at most if chosen
                        //                       (whole-cluster steps: its reordered rows)
  int32_t* cl_row0;     // [n_units * max_C]     whole-cluster steps: the cluster's first row in the unit
  int32_t* cl_rank;     // [n_units * max_C][G]  rank among a head's chosen clusters, or -1
                        //                       (written only when sel_s is requested)
  int32_t* unit_rows;   // [n_units]             rows of chosen subclusters per unit
  int32_t* cl_list;     // [n_units * max_C]     per unit: chosen clusters, ascending
  int32_t* n_chosen;    // [n_units]             length of the unit's list
  int32_t* uinfo;       // [n_units][2]          first exact block of the unit, its blocks
  int32_t* ch_tbase;    // [n_units * max_C]     per unit: tile-slot base of the x-th chosen cluster
  int32_t* ch_ntiles;   // [n_units * max_C]     per unit: tiles of the x-th chosen cluster
  int32_t* ch_row0;     // [n_units * max_C]     whole-cluster steps, per unit: first row of the x-th
                        //                       chosen cluster in the unit
  uint32_t* ch_nm;      // [n_units * max_C]     whole-cluster steps: its rows | head mask << 24
  TileRec* tiles;       // [tile slots]          exact tiles, per unit at tile_unit_base()
  float* res_part;      // [n_units][nb_res][G][D+4] residual partials: one per chosen
                        //                       cluster, then one per rest block
  float* ex_part;       // [nblk][G][D+4]        exact-attention block records
  float* fq;            // [n_units][G][fm_dim]  feature-map residual: log2 of each head's features
};

struct DecodeLaunch {
  mog_layout L;
  KVRef kv;
  SeqArgs seq;
  const float* q;
  float* out;
  float* lse;
  int32_t* sel_c;
  int32_t* sel_s;
  int32_t c_stride, s_stride;
  int32_t Hq, G, D, dtype;
  int32_t residual;     // 0 none, 1 Gaussian, 2 feature map
  int32_t shared;       // one selection per KV head
  int32_t splits;       // target exact blocks in total (balanced over units)
  int32_t nblk;         // exact blocks launched: splits + n_units
  int32_t nb_res;       // residual record slots per unit: nb_chosen + ceil(max_C / kRestClustersSmall)
  int32_t nb_chosen;    // chosen-cluster blocks per unit (max G * top_c)
  int32_t half;         // exact blocks in halves of 2 waves, each with a unit share of its own
  int32_t whole;        // whole-cluster step: every sequence's top_s reaches its S, no folded
                        // rows, Gaussian residual or none, no subcluster output, at most
                        // kWaveListMax chosen clusters per unit.  The top-c kernel writes each
                        // chosen cluster's rows and head mask, the exact kernel cuts them into
                        // tiles, the residual of the clusters left out runs in blocks after the
                        // exact ones, and the subcluster kernel is skipped.
  float scale;
  hipEvent_t ev_begin, ev_end;  // optional, around the exact kernel
  int32_t repeat;               // exact-kernel launches between the events (>= 1)
  DecodeWS ws;
};

struct DenseLaunch {
  KVRef kv;
  SeqArgs seq;
  const float* q;
  float* out;
  float* lse;
  int32_t Hq, G, D, dtype, n_kv_heads;
  int32_t splits;
  float scale;
  hipEvent_t ev_begin, ev_end;  // optional, around the dense kernel
  int32_t repeat;               // dense-kernel launches between the events (>= 1)
  float* ex_part;       // [n_units][splits][G][D+4]
};

// Residual-only blocks (the clusters some head left out) take
// kRestClustersPerBlock clusters (16 per wave), or kRestClustersSmall (4 per
// wave) when that makes at most kRestSmallMaxBlocks of them in all: few
// small blocks fit in the spread of the exact blocks' end times, many queue
// behind them.  The feature-map residual always takes the large blocks.
constexpr int kRestClustersPerBlock = 64;
constexpr int kRestClustersSmall = 16;
constexpr int kRestSmallMaxBlocks = 1024;
__host__ __device__ inline int rest_clusters_per_block(int residual, int n_units, int max_C) {
  if (residual == 2) return kRestClustersPerBlock;
  const int64_t small = (int64_t)n_units * ((max_C + kRestClustersSmall - 1) / kRestClustersSmall);
  return small <= kRestSmallMaxBlocks ? kRestClustersSmall : kRestClustersPerBlock;
}
constexpr int kPartPad = 4;
// blocks of the exact-attention kernel resident at once on the chip: 256
// compute units x 2 (its registers allow 2 waves per SIMD)
constexpr int kExactResidentBlocks = 512;   // partial record = o[D], m, l, pad

hipError_t launch_layout_table(const mog_layout& L, const SeqArgs& seq, hipStream_t s);
// the bf16 copies of every group statistic, rewritten from the float32 ones
hipError_t launch_stats16(const mog_layout& L, hipStream_t s);

// ---------------------------------------------------------------------------
// Append (incremental decode) launch block.
// ---------------------------------------------------------------------------
struct AppendSeq {
  int32_t len;     // sequence length before the append
  uint16_t n_new;  // tokens to fold
  uint16_t f0;     // tokens folded before (first fold row to write)
};

// mog_append: a token's cluster scan is shared by up to kAppendMaxBlocks
// blocks per unit (about kAppendRowsPerBlock clusters each); each leaves
// its winner in a slot of the layout buffer (mog_layout.append_scratch),
// which the next kernel reads.
constexpr int kAppendThreads = 512;
constexpr int kAppendRowsPerBlock = 128;
constexpr int kAppendMaxBlocks = 16;
struct AppendSlot {
  double d2;
  int32_t id, n, nf, pad;
};
__host__ __device__ inline size_t append_scratch_bytes(int64_t n_units) {
  return (size_t)n_units * kAppendMaxBlocks * sizeof(AppendSlot);
}

struct AppendLaunch {
  mog_layout L;
  KVRef kv;
  int32_t n_seq;
  AppendSeq seq[MOG_MAX_SEQ];
};

hipError_t launch_append(const AppendLaunch& a, hipStream_t s);
hipError_t launch_decode(const DecodeLaunch& a, hipStream_t s);
hipError_t launch_dense(const DenseLaunch& a, hipStream_t s);

// ---------------------------------------------------------------------------
// Build launch block.
// ---------------------------------------------------------------------------
struct BuildWS {
  float* cent;          // [total_cl][D]  centroids
  float* cent_norm;     // [total_cl]     ||mu||^2
  unsigned long long* sums;  // [total_cl][D] fixed-point sums
  int32_t* counts;      // [total_cl]
  int32_t* labels;      // [total_mid]    cluster of every middle key
  int32_t* cl_start;    // [total_cl]     first member slot of each cluster
  int32_t* members;     // [total_mid]    middle-local ids grouped by cluster, ascending
  int32_t* sublab;      // [total_mid]    subcluster of every member slot
};

struct BuildLaunch {
  mog_layout L;
  KVRef kv;
  SeqArgs seq;
  int32_t D, dtype, iters;
  uint64_t seed;
  const float* fm_w;  // feature-map projection to summarise with (fm_dim > 0)
  BuildWS ws;
};

hipError_t launch_build(const BuildLaunch& a, hipStream_t s);

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
#if defined(__HIP_DEVICE_COMPILE__) || defined(__HIPCC__)
// Wave-uniform copies (scalar registers) of values every lane holds alike.
__device__ inline int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ inline int64_t uni(int64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ inline mog_unit uni_unit(const mog_unit* p) {
  const mog_unit x = *p;
  mog_unit U;
  U.seq = uni(x.seq);
  U.kv_head = uni(x.kv_head);
  U.N = uni(x.N);
  U.n_mid = uni(x.n_mid);
  U.C = uni(x.C);
  U.S = uni(x.S);
  U.n_fold = uni(x.n_fold);
  U.reserved1 = 0;
  U.row_base = uni(x.row_base);
  U.cl_base = uni(x.cl_base);
  U.sub_base = uni(x.sub_base);
  U.off_base = uni(x.off_base);
  return U;
}

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
// float32 -> bf16 bits, rounded to nearest, ties to even (NaN stays NaN)
__device__ inline uint16_t bf16_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 8 consecutive elements starting at element offset `off` as float32.
template <typename T>
__device__ inline void load8(const T* base, int64_t off, float (&x)[8]);

template <>
__device__ inline void load8<float>(const float* base, int64_t off, float (&x)[8]) {
  const float4* p = reinterpret_cast<const float4*>(base + off);
  float4 a = p[0], b = p[1];
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

template <>
__device__ inline void load8<uint16_t>(const uint16_t* base, int64_t off, float (&x)[8]) {
  uint4 w = *reinterpret_cast<const uint4*>(base + off);
  x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x);
  x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
  x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z);
  x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// Merge partial softmax state (m2, l2, o2) into (m1, l1, o1); log2 domain.
__device__ inline void merge_scale(float m1, float m2, float& a1, float& a2, float& mnew) {
  mnew = fmaxf(m1, m2);
  a1 = (m1 == -INFINITY) ? 0.f : exp2f(m1 - mnew);
  a2 = (m2 == -INFINITY) ? 0.f : exp2f(m2 - mnew);
}

// Order-preserving map of a float to uint32 (larger float -> larger key).
__device__ inline uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
#endif

}  // namespace mog
