// Exact online-softmax accumulation over rows of K/V, shared by the MoG exact
// pass and the dense baseline.  One wave accumulates, for the G query heads
// of one KV head, the running (m, l, o) of softmax attention in the base-2
// log domain (logits carry a factor log2(e), folded into the query).
//
//  * MfmaTile (bf16 K/V): 32-row tiles.  Rows are read with coalesced 16-byte
//    loads and staged row-major in a wave-private LDS buffer whose rows are
//    padded by 16 bytes, so the writes and the 16-row fragment reads are
//    bank-conflict free and every LDS access is one base plus an immediate.  Scores are S^T = K Q^T on the 16x16x32 bf16
//    matrix cores, with Q split into bf16 high and low parts placed in
//    columns h and h+8 (so scores carry ~16 mantissa bits of the fp32
//    query).  The probabilities of a lane's 8 tokens come out of the score
//    accumulator in exactly the layout the P^T operand needs, split into
//    high/low parts the same way, and O^T += V^T P^T takes V^T fragments
//    from LDS with transpose reads.
//  * RowAcc (fp32 K/V, or bf16 widened on load): plain VALU, 16 (D=128) or
//    8 (D=64) lanes per row.
#pragma once

#include "mog_internal.h"

namespace mog {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

template <int CTRL>
__device__ inline float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// sum over the 16 lanes of each row (every lane gets the row sum)
__device__ inline float row16_sum(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror
  x += dpp<0x140>(x);  // row_mirror
  return x;
}

// Sum over the wave, returned as a wave-uniform value: row sums by DPP, then
// the row broadcasts 15 and 31 carry rows 0..2 into row 3, and lane 63's
// total is read out.  No LDS traffic, unlike a shuffle-based reduction.
__device__ inline float wave_sum_uniform(float x) {
  x = row16_sum(x);
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x142, 0xA, 0xF, false));  // row_bcast:15
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x143, 0xC, 0xF, false));  // row_bcast:31
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

// Reduction of a 32-bit value over the wave with an associative op,
// returned wave-uniform (same DPP pattern as wave_sum_uniform; `identity`
// fills the rows the broadcasts leave out).
template <typename Op>
__device__ inline uint32_t wave_reduce_uniform(uint32_t x, Op op, uint32_t identity) {
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xF, 0xF, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x140, 0xF, 0xF, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)identity, (int)x, 0x142, 0xA, 0xF, false));
  x = op(x, (uint32_t)__builtin_amdgcn_update_dpp((int)identity, (int)x, 0x143, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// Inclusive prefix sum over lanes 0..63 (lane l gets x_0 + ... + x_l): three
// row shifts give each lane the sum of up to 4 lanes, shifts by 4 and 8 on
// the banks that have a full source finish every row of 16, and the row
// broadcasts 15 and 31 carry the row totals forward.
__device__ inline int wave_incl_scan(int x) {
  int s = x;
  s += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  s += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  s += __builtin_amdgcn_update_dpp(0, x, 0x113, 0xF, 0xF, false);  // row_shr:3
  s += __builtin_amdgcn_update_dpp(0, s, 0x114, 0xF, 0xE, false);  // row_shr:4, lanes 4..15 of a row
  s += __builtin_amdgcn_update_dpp(0, s, 0x118, 0xF, 0xC, false);  // row_shr:8, lanes 8..15 of a row
  s += __builtin_amdgcn_update_dpp(0, s, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  s += __builtin_amdgcn_update_dpp(0, s, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
  return s;
}

__device__ inline float wave_sum_dpp(float x) {
  x = row16_sum(x);
  x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}

// value of lane (lane ^ 8) inside each row of 16 lanes
__device__ inline float swap8(float x) { return dpp<0x128>(x); }  // row_ror:8

// ---------------------------------------------------------------------------
// Reduce-scatter over the wave: every lane holds V partial values (V <= 64);
// afterwards lane l holds the wave sum of value rs_index<V>(l).  Six lane
// exchanges are taken in turn: row mirror (partner l ^ 15 in its row of 16),
// half-row mirror (l ^ 7 in its 8), l ^ 2, l ^ 1 (DPP), l ^ 16 (swizzle) and
// l ^ 32 (permute).  In each of the first H = ceil(log2 V) of them a lane keeps
// the half of its values its lane bit selects (b3, b2, b1, b0, b4, b5 in that
// order) and adds the partner's copy of that half, which the partner sends
// because it keeps the other half; partners always agree on the bits of the
// earlier exchanges, so they hold the same values.  The remaining exchanges
// add the last value.  This takes about 3V lane operations where V separate
// wave sums take about 7V.  When V < 64, 64 / 2^H lanes hold each sum.
// ---------------------------------------------------------------------------
template <int V>
struct RsSteps {
  static_assert(V >= 1 && V <= 64, "reduce-scatter of up to 64 values");
  static constexpr int H = V <= 1 ? 0 : V <= 2 ? 1 : V <= 4 ? 2 : V <= 8 ? 3 : V <= 16 ? 4 : V <= 32 ? 5 : 6;
  static constexpr int P = 1 << H;  // values after padding with zeros
};

// one exchange on the first N values of w: halve them when N > 1, else add
template <int N, typename X>
__device__ inline void rs_exchange(float* w, bool upper, X partner) {
  if constexpr (N > 1) {
#pragma unroll
    for (int j = 0; j < N / 2; ++j) {
      const float lo = w[j], hi = w[j + N / 2];
      const float keep = upper ? hi : lo, send = upper ? lo : hi;
      w[j] = keep + partner(send);
    }
  } else {
    w[0] += partner(w[0]);
  }
}

__device__ inline float lane_xor16(float x) {
  // ds_swizzle bit mode: and 0x1f, or 0, xor 0x10 (lane ^ 16 in each 32)
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));
}

template <int V>
__device__ inline float wave_reduce_scatter(const float (&v)[V]) {
  constexpr int P = RsSteps<V>::P;
  const int lane = threadIdx.x & 63;
  float w[P];
#pragma unroll
  for (int j = 0; j < P; ++j) w[j] = j < V ? v[j] : 0.f;
  constexpr int N0 = P, N1 = N0 > 1 ? N0 / 2 : 1, N2 = N1 > 1 ? N1 / 2 : 1, N3 = N2 > 1 ? N2 / 2 : 1,
                N4 = N3 > 1 ? N3 / 2 : 1, N5 = N4 > 1 ? N4 / 2 : 1;
  rs_exchange<N0>(w, (lane >> 3) & 1, [](float x) { return dpp<0x140>(x); });  // row mirror
  rs_exchange<N1>(w, (lane >> 2) & 1, [](float x) { return dpp<0x141>(x); });  // half-row mirror
  rs_exchange<N2>(w, (lane >> 1) & 1, [](float x) { return dpp<0x4E>(x); });   // l ^ 2
  rs_exchange<N3>(w, lane & 1, [](float x) { return dpp<0xB1>(x); });          // l ^ 1
  rs_exchange<N4>(w, (lane >> 4) & 1, [](float x) { return lane_xor16(x); });
  rs_exchange<N5>(w, (lane >> 5) & 1, [](float x) { return __shfl_xor(x, 32, 64); });
  return w[0];
}

// index of the value whose sum wave_reduce_scatter<V> leaves in lane l
template <int V>
__device__ inline int rs_index(int l) {
  constexpr int H = RsSteps<V>::H;
  const int bits[6] = {(l >> 3) & 1, (l >> 2) & 1, (l >> 1) & 1, l & 1, (l >> 4) & 1, (l >> 5) & 1};
  int j = 0;
#pragma unroll
  for (int s = 0; s < H; ++s) j = 2 * j + bits[s];
  return j;
}

// whether lane l reports its sum: lanes that differ only in the bits of the
// plain-add exchanges hold the same index; the one with those bits clear
// reports it (if the index is below V)
template <int V>
__device__ inline bool rs_owner(int l) {
  constexpr int H = RsSteps<V>::H;
  constexpr int order[6] = {3, 2, 1, 0, 4, 5};  // lane bit decided by each exchange
  int undecided = 0;
#pragma unroll
  for (int s = H; s < 6; ++s) undecided |= 1 << order[s];
  return (l & undecided) == 0 && rs_index<V>(l) < V;
}

// the lane that reports value j of wave_reduce_scatter<V> (the inverse of
// rs_index over the rs_owner lanes: the bit each exchange decided, undecided
// bits clear)
template <int V>
__host__ __device__ constexpr int rs_lane(int j) {
  constexpr int H = RsSteps<V>::H;
  constexpr int order[6] = {3, 2, 1, 0, 4, 5};
  int l = 0;
  for (int s = 0; s < H; ++s) l |= ((j >> (H - 1 - s)) & 1) << order[s];
  return l;
}

// ---------------------------------------------------------------------------
// MFMA tile engine (bf16)
// ---------------------------------------------------------------------------
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Third word of a raw buffer resource on gfx9-family chips: 32-bit data
// format (a zero format makes untyped loads return zero), no swizzle.
constexpr int kBufferWord3 = 0x00020000;

template <int D, int G>
struct MfmaTile {
  static constexpr int PPR = D / 8;      // 16-byte pieces per row
  static constexpr int RPI = 64 / PPR;   // rows per wave-wide 16-byte load
  static constexpr int NLI = 32 / RPI;   // loads per 32-row tile (per K or V)
  static constexpr int NC = D / 32;      // k-chunks of the score product
  static constexpr int NB = D / 16;      // 16-wide d blocks of the output
  static constexpr int RSB = D * 2 + 16; // LDS row stride in bytes (one 16-byte pad)
  static constexpr int VBUF = 32 * RSB / 16;  // u32x4 of the V staging rows
  static constexpr int BUF = VBUF + NC * 64;   // + the query fragments

  static constexpr bool PIPELINED = true;
  struct Regs {
    u32x4 k[NLI], v[NLI];
  };

  f32x4 o[NB];
  float m, l;
  const u32x4* qf;  // LDS: query fragment c of lane l at qf[64 c + l]

  // The query fragments live in the wave's LDS buffer (after the V rows),
  // read back once per tile: registers go to the tile pipeline instead.
  __device__ void init(const float* qb, float scale_l2, u32x4* buf) {
    const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15, h = n & 7;
    // every lane loads (heads past G read head 0 and are zeroed): no
    // divergent loads, all 2 * NC vector loads in flight together
    const float4* src = reinterpret_cast<const float4*>(qb + (h < G ? h : 0) * D + 8 * g);
    float4 raw[NC][2];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      raw[c][0] = src[8 * c];
      raw[c][1] = src[8 * c + 1];
    }
    const float sc = h < G ? scale_l2 : 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const float v8[8] = {raw[c][0].x, raw[c][0].y, raw[c][0].z, raw[c][0].w,
                           raw[c][1].x, raw[c][1].y, raw[c][1].z, raw[c][1].w};
      bf16x8 f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float qv = v8[j] * sc;
        const __bf16 hi = (__bf16)qv;
        f[j] = n < 8 ? hi : (__bf16)(qv - (float)hi);
      }
      buf[VBUF + 64 * c + lane] = __builtin_bit_cast(u32x4, f);
    }
    qf = buf + VBUF + lane;
#pragma unroll
    for (int b = 0; b < NB; ++b) o[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    m = -INFINITY;
    l = 0.f;
  }

  // 16-byte piece of this lane for load i of a tile of rows r0 + RPI*i:
  // lane = (row r0 = lane / PPR, piece p = lane % PPR).  Rows at or past
  // nrows re-read the last row: their probability is exactly zero.
  __device__ static int load_row(int i, int nrows) {
    const int r = (threadIdx.x & 63) / PPR + RPI * i;
    return r < nrows ? r : nrows - 1;
  }

  // Cache policy of the K/V stream loads: non-temporal (bit 1 of the buffer
  // instruction's cache-policy operand, "nt" on gfx94x/gfx950).  Each row is
  // read once per step, and without the hint the stream displaces the decode
  // kernels' code and their small per-unit arrays from the L2 every step, so
  // the short kernels of the next step start cold.
  static constexpr int kStreamPolicy = 2;

  // Raw buffer resource over `bytes` bytes at p: a lane whose offset is at
  // or past `bytes` reads zeros and touches no memory.
  __device__ static __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, kBufferWord3);
  }

  // Register layouts of a 32-row tile (lane = 16 g + n):
  //  K: kr[NC t + c] holds row 16t + n, elements 32c + 8g .. +7: exactly the
  //     A fragment of the score product, so K never passes through LDS;
  //  V: vr[i] holds row lane / PPR + RPI i, elements 8 (lane % PPR) .. +7
  //     (whole rows per load), staged row-major in LDS for transpose reads.
  static_assert(2 * NC == NLI, "K and V tiles take the same registers");

  // Load a tile of contiguous rows (row i at kp + i*D elements) with buffer
  // loads over exactly nrows rows.  A lane's row offset is its row clamped
  // to the tile's last row (row 0 of an empty tile), so every address lies
  // in the tile whatever the range check covers; the row goes in the
  // per-lane offset, column steps in the instruction's immediate, and the
  // scalar offset is zero.  The descriptor's range (nrows rows) makes an
  // empty tile's loads return zeros without a memory access.  Rows at or
  // past nrows get probability zero in compute(), by position.
  __device__ static void load(const uint16_t* kp, const uint16_t* vp, int nrows, u32x4 (&kr)[NLI],
                              u32x4 (&vr)[NLI]) {
    const int lane = threadIdx.x & 63;
    const int last = nrows > 0 ? nrows - 1 : 0;
    const uint32_t bytes = (uint32_t)nrows * (D * 2);
    const __amdgpu_buffer_rsrc_t rk = rsrc(kp, bytes), rv = rsrc(vp, bytes);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int kb = min((lane & 15) + 16 * t, last) * (D * 2) + (lane >> 4) * 16;
#pragma unroll
      for (int c = 0; c < NC; ++c)
        kr[NC * t + c] = __builtin_amdgcn_raw_buffer_load_b128(rk, kb + c * 64, 0, kStreamPolicy);
    }
#pragma unroll
    for (int i = 0; i < NLI; ++i) {
      const int vb = min(lane / PPR + RPI * i, last) * (D * 2) + (lane % PPR) * 16;
      vr[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, vb, 0, kStreamPolicy);
    }
  }

  // Contiguous rows: row i of the tile at kp + i*D (elements).
  __device__ void tile(u32x4* buf, const uint16_t* kp, const uint16_t* vp, int nrows, uint32_t mask) {
    u32x4 kr[NLI], vr[NLI];
    load(kp, vp, nrows, kr, vr);
    compute(buf, kr, vr, nrows, mask);
  }

  // Rows anywhere: row i of the tile at element offset rowoff(i); rows at or
  // past nrows re-read row nrows - 1 (their probability is zero).
  template <typename RowOff>
  __device__ void tile_gather(u32x4* buf, const uint16_t* kb, const uint16_t* vb, int nrows, uint32_t mask,
                              RowOff rowoff) {
    const int lane = threadIdx.x & 63;
    u32x4 kr[NLI], vr[NLI];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int r = 16 * t + (lane & 15);
      const int64_t off = rowoff(r < nrows ? r : nrows - 1) + (lane >> 4) * 8;
#pragma unroll
      for (int c = 0; c < NC; ++c)
        kr[NC * t + c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + off + 32 * c));
    }
#pragma unroll
    for (int i = 0; i < NLI; ++i) {
      const int r = lane / PPR + RPI * i;
      const int64_t off = rowoff(r < nrows ? r : nrows - 1) + (lane % PPR) * 8;
      vr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vb + off));  // (the stream policy)
    }
    compute(buf, kr, vr, nrows, mask);
  }

  __device__ void compute(u32x4* buf, const u32x4 (&kr)[NLI], const u32x4 (&vr)[NLI], int nrows,
                          uint32_t mask) {
    const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15, h = n & 7;
    char* lds = reinterpret_cast<char*>(buf);
    // S^T = K Q^T for the two 16-token halves, K straight from registers
    f32x4 s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      s[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c)
        s[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[NC * t + c]),
                                                       __builtin_bit_cast(bf16x8, qf[64 * c]), s[t], 0, 0, 0);
    }
    const bool hv = h < G && ((mask >> h) & 1u);
    // token 16t + 4g + j of the tile exists when 16t + j < nrows - 4g (one
    // per-lane register instead of eight row constants)
    const int lim = nrows - 4 * g;
    float mt = -INFINITY;
    float sv[8];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float x = s[t][j] + swap8(s[t][j]);
        const bool ok = hv && (16 * t + j) < lim;
        x = ok ? x : -INFINITY;
        sv[4 * t + j] = x;
        mt = fmaxf(mt, x);
      }
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float mn = fmaxf(m, mt);
    const float alpha = (m == -INFINITY) ? 0.f : fast_exp2(m - mn);
    bf16x8 pf;
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float pj = sv[j] == -INFINITY ? 0.f : fast_exp2(sv[j] - mn);
      ps += pj;
      const __bf16 hi = (__bf16)pj;
      pf[j] = n < 8 ? hi : (__bf16)(pj - (float)hi);
    }
    l = l * alpha + ps;
    m = mn;
#pragma unroll
    for (int b = 0; b < NB; ++b) o[b] *= alpha;
    // values: row-major in the wave's LDS buffer, then V^T fragments by
    // transpose reads: src lane (g, s) of each 16-lane group points at row
    // 4g + s/4 (+16), columns 16b + 4(s%4) .. +3.  The previous tile's reads
    // of this buffer were issued before these writes, and LDS executes a
    // wave's operations in order.
    char* wr = lds + (lane / PPR) * RSB + (lane % PPR) * 16;
    __asm__ volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < NLI; ++i) *reinterpret_cast<u32x4*>(wr + i * RPI * RSB) = vr[i];
    auto* tr = (__attribute__((address_space(3))) char*)(lds) + (4 * g + (n >> 2)) * RSB + (n & 3) * 8;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const bf16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(tr + 32 * b));
      const bf16x4 vc = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(tr + 32 * b + 16 * RSB));
      const bf16x8 vf = {va[0], va[1], va[2], va[3], vc[0], vc[1], vc[2], vc[3]};
      o[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, o[b], 0, 0, 0);
    }
  }

  // Combine the lanes of the wave and store its state (o[D], m, l) per head
  // in st[wave][h][0..D+1] (rows of D + 4 floats).
  __device__ void to_lds(float* st) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, n = lane & 15;
    float lt = l;
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int j = 0; j < 4; ++j) o[b][j] += swap8(o[b][j]);
    }
    if (n < G) {
      float* w = st + (wave * G + n) * (D + kPartPad);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
#pragma unroll
        for (int j = 0; j < 4; ++j) w[16 * b + 4 * g + j] = o[b][j];
      }
      if (g == 0) {
        w[D] = m;
        w[D + 1] = lt;
      }
    }
  }
};

// ---------------------------------------------------------------------------
// VALU row engine (fp32 K/V): LPR = D/8 lanes per row, 8 elements per lane.
// ---------------------------------------------------------------------------
template <int D, int G, typename T = float>
struct RowAcc {
  static constexpr int LPR = D / 8;
  static constexpr int RPI = 64 / LPR;
  float m[G], l[G], o[G][8];
  float qv[G][8];

  __device__ void init(const float* qb, float scale_l2, u32x4*) {
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

  static constexpr int BUF = 1;
  static constexpr bool PIPELINED = false;
  struct Regs {
    u32x4 k[1], v[1];
  };
  __device__ static void load(const T*, const T*, int, u32x4 (&)[1], u32x4 (&)[1]) {}
  __device__ void compute(u32x4*, const u32x4 (&)[1], const u32x4 (&)[1], int, uint32_t) {}

  __device__ void tile(u32x4*, const T* kp, const T* vp, int nrows, uint32_t mask) {
    rows(kp, vp, nrows, mask, [](int i) { return (int64_t)i * D; });
  }

  template <typename RowOff>
  __device__ void tile_gather(u32x4*, const T* kb, const T* vb, int nrows, uint32_t mask, RowOff rowoff) {
    rows(kb, vb, nrows, mask, rowoff);
  }

  template <typename RowOff>
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

  __device__ void to_lds(float* st) {
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
    if (lane < LPR) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float* w = st + (wave * G + h) * (D + kPartPad);
#pragma unroll
        for (int e = 0; e < 8; ++e) w[lane * 8 + e] = o[h][e];
        if (lane == 0) {
          w[D] = m[h];
          w[D + 1] = l[h];
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------
// exp2(m - M) of a record with max m under the common max M; 0 for an
// empty record (m = -inf)
__device__ inline float exp2_or_zero(float m, float M) { return m == -INFINITY ? 0.f : exp2f(m - M); }

// Epilogue: merge NWS wave states in st, rows (w0 + w) G + h for w < NWS
// (st is [4][G][D+4]: o[D], m, l, two pad words, so every row starts 16-byte
// aligned), into one record per head, dst[h][0..D) = o, dst[h][D] = m,
// dst[h][D+1] = l (G x (D+4) floats).  One float4 of o per thread; thread t
// of the nt threads that write this record.  Called after a barrier that
// made st visible.
template <int D, int G, int NWS>
__device__ inline void write_record(const float* st, int w0, float* dst, int t, int nt) {
  constexpr int RS = D + kPartPad;
  constexpr int Q = D / 4;
  for (int idx = t; idx < G * Q; idx += nt) {
    const int h = idx / Q, e4 = idx % Q;
    float mw[NWS], lw[NWS];
    float4 ow[NWS];
#pragma unroll
    for (int w = 0; w < NWS; ++w) {
      const float* r = st + ((w0 + w) * G + h) * RS;
      const float2 ml = *reinterpret_cast<const float2*>(r + D);
      mw[w] = ml.x;
      lw[w] = ml.y;
      ow[w] = reinterpret_cast<const float4*>(r)[e4];
    }
    float M = mw[0];
#pragma unroll
    for (int w = 1; w < NWS; ++w) M = fmaxf(M, mw[w]);
    float L = 0.f;
    float4 O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NWS; ++w) {
      const float f = exp2_or_zero(mw[w], M);
      L += f * lw[w];
      O.x += f * ow[w].x;
      O.y += f * ow[w].y;
      O.z += f * ow[w].z;
      O.w += f * ow[w].w;
    }
    reinterpret_cast<float4*>(dst + h * RS)[e4] = O;
    if (e4 == 0) *reinterpret_cast<float2*>(dst + h * RS + D) = float2{M, L};
  }
}

// Block epilogue: the 4 wave states of a block, all 256 threads.
template <int D, int G>
__device__ inline void write_block_record(const float* st, float* dst) {
  write_record<D, G, 4>(st, 0, dst, threadIdx.x, 256);
}

}  // namespace mog
