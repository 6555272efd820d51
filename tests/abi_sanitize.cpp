// Host-side checks of the libmog C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer (host code only) together with the library's
// argument validation (api.cpp).  Nothing here needs a GPU: every call either
// computes sizes on the host or is rejected before anything is enqueued.
// Exit status 0 when every expectation holds and no sanitizer fired.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "mog.h"

static int g_fails = 0;
#define EXPECT(cond)                                                        \
  do {                                                                      \
    if (!(cond)) {                                                          \
      std::fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
      ++g_fails;                                                            \
    }                                                                       \
  } while (0)

static void* fake(uintptr_t a) { return reinterpret_cast<void*>(a); }  // never dereferenced

static mog_dims dims(const std::vector<int32_t>& lens, int hkv = 8, int d = 128, int dtype = MOG_BF16) {
  mog_dims x;
  std::memset(&x, 0, sizeof(x));
  x.n_seq = (int32_t)lens.size();
  x.n_kv_heads = hkv;
  x.head_dim = d;
  x.dtype = dtype;
  x.n_sink = 64;
  x.n_recent = 256;
  x.seq_lens = lens.data();
  return x;
}

static mog_kv kv_of(const std::vector<int32_t>& lens) {
  mog_kv kv;
  std::memset(&kv, 0, sizeof(kv));
  kv.format = MOG_KV_CONTIGUOUS;
  kv.dtype = MOG_BF16;
  kv.n_seq = (int32_t)lens.size();
  kv.n_kv_heads = 8;
  kv.head_dim = 128;
  int mx = 0;
  for (int x : lens) mx = x > mx ? x : mx;
  kv.max_len = mx;
  kv.seq_lens = lens.data();
  kv.k = fake(0x100000);
  kv.v = fake(0x200000);
  return kv;
}

static mog_layout host_layout(const std::vector<int32_t>& lens, int cap, const std::vector<int32_t>& folded) {
  mog_layout L;
  std::memset(&L, 0, sizeof(L));
  L.n_seq = (int32_t)lens.size();
  L.n_kv_heads = 8;
  L.head_dim = 128;
  L.dtype = MOG_BF16;
  L.n_sink = 64;
  L.n_recent = 256;
  L.n_units = 8 * L.n_seq;
  L.fold_capacity = cap;
  for (size_t i = 0; i < lens.size(); ++i) {
    L.seq_lens[i] = lens[i];
    L.fold_count[i] = folded[i];
  }
  void* p = fake(0x10000);
  L.units = static_cast<mog_unit*>(p);
  L.k_mid = L.v_mid = p;
  L.perm = L.sub_off = L.fold_sub = L.fold_pos = L.cl_fold = L.sub_fold = static_cast<int32_t*>(p);
  L.cl_ms = L.cl_vbar = L.sub_ms = L.sub_vbar = static_cast<float*>(p);
  L.cl_ms16 = L.cl_vbar16 = L.sub_ms16 = L.sub_vbar16 = static_cast<uint16_t*>(p);
  L.append_scratch = p;
  return L;
}

int main() {
  // status texts, including codes outside the enum
  for (int s = -3; s < 12; ++s) {
    const char* t = mog_status_string(static_cast<mog_status>(s));
    EXPECT(t != nullptr && std::strlen(t) > 0);
  }
  EXPECT(mog_last_error() != nullptr);

  // layout sizes and rows
  std::vector<int32_t> one_m = {1 << 20};
  mog_dims d = dims(one_m);
  size_t bytes = 0, bytes2 = 0;
  EXPECT(mog_layout_size(&d, &bytes) == MOG_OK && bytes > 0);
  int64_t rows = 0;
  EXPECT(mog_layout_rows(&d, &rows) == MOG_OK && rows == 8LL * ((1 << 20) - 320));
  d.fold_capacity = 1000;
  EXPECT(mog_layout_size(&d, &bytes2) == MOG_OK && bytes2 > bytes);
  d.fm_dim = 128;
  EXPECT(mog_layout_size(&d, &bytes2) == MOG_OK);
  d.rows_external = 1;
  EXPECT(mog_layout_size(&d, &bytes2) == MOG_OK && bytes2 < bytes);
  std::vector<int32_t> ragged = {8192, 262143, 1000, 4096, 330};
  mog_dims r = dims(ragged, 2, 64, MOG_F32);
  EXPECT(mog_layout_size(&r, &bytes) == MOG_OK);
  EXPECT(mog_layout_rows(&r, &rows) == MOG_OK);

  // layout size rejections
  std::vector<int32_t> short_len = {300}, ok_len = {5000}, too_long = {(1 << 22) + 1};
  mog_dims b = dims(short_len);
  EXPECT(mog_layout_size(&b, &bytes) == MOG_ERR_INVALID_ARG);
  b = dims(ok_len, 8, 96);
  EXPECT(mog_layout_size(&b, &bytes) == MOG_ERR_UNSUPPORTED);
  b = dims(too_long);
  EXPECT(mog_layout_size(&b, &bytes) == MOG_ERR_UNSUPPORTED);
  b = dims(ok_len);
  b.n_sink = -1;
  EXPECT(mog_layout_size(&b, &bytes) == MOG_ERR_INVALID_ARG);
  b = dims(ok_len, 8, 128, 7);
  EXPECT(mog_layout_size(&b, &bytes) == MOG_ERR_UNSUPPORTED);
  b = dims(ok_len);
  b.n_seq = 0;
  EXPECT(mog_layout_size(&b, &bytes) == MOG_ERR_INVALID_ARG);
  b = dims(ok_len);
  b.n_seq = MOG_MAX_SEQ + 1;
  EXPECT(mog_layout_size(&b, &bytes) != MOG_OK);
  b = dims(ok_len);
  b.seq_lens = nullptr;
  EXPECT(mog_layout_size(&b, &bytes) == MOG_ERR_INVALID_ARG);
  b = dims(ok_len);
  b.fold_capacity = -1;
  EXPECT(mog_layout_size(&b, &bytes) == MOG_ERR_INVALID_ARG);
  b.fold_capacity = MOG_MAX_FOLD + 1;
  EXPECT(mog_layout_size(&b, &bytes) == MOG_ERR_INVALID_ARG);
  b = dims(ok_len);
  b.fm_dim = 100;
  EXPECT(mog_layout_size(&b, &bytes) == MOG_ERR_UNSUPPORTED);
  EXPECT(mog_layout_size(nullptr, &bytes) != MOG_OK);
  EXPECT(mog_layout_size(&d, nullptr) != MOG_OK);
  EXPECT(std::strlen(mog_last_error()) > 0);

  // per-unit geometry of a host descriptor
  std::vector<int32_t> three = {4096, 20000, 777};
  mog_layout g = host_layout(three, 0, {0, 0, 0});
  g.n_kv_heads = 2;
  g.n_units = 6;
  int64_t row = 0;
  for (int u = 0; u < 6; ++u) {
    mog_unit U;
    EXPECT(mog_layout_unit(&g, u, &U) == MOG_OK);
    EXPECT(U.seq == u / 2 && U.kv_head == u % 2 && U.row_base == row);
    row += U.n_mid;
  }
  mog_unit U;
  EXPECT(mog_layout_unit(&g, 6, &U) == MOG_ERR_INVALID_ARG);
  EXPECT(mog_layout_unit(&g, -1, &U) == MOG_ERR_INVALID_ARG);
  // the statistics copy: rejected before any launch
  EXPECT(mog_layout_sync_stats(nullptr, nullptr) == MOG_ERR_INVALID_ARG);
  mog_layout bad = g;
  bad.head_dim = 96;
  EXPECT(mog_layout_sync_stats(&bad, nullptr) == MOG_ERR_INVALID_ARG);

  // workspace sizes and parameter rejections
  mog_kv kv = kv_of(ok_len);
  mog_decode_params p;
  std::memset(&p, 0, sizeof(p));
  p.n_q_heads = 32;
  p.top_c = 4;
  p.top_s = 2;
  p.residual = 1;
  EXPECT(mog_workspace_size(MOG_OP_DENSE, &kv, nullptr, nullptr, &p, &bytes) == MOG_OK && bytes > 0);
  p.n_q_heads = 12;
  EXPECT(mog_workspace_size(MOG_OP_DENSE, &kv, nullptr, nullptr, &p, &bytes) == MOG_ERR_INVALID_ARG);
  p.n_q_heads = 72;
  EXPECT(mog_workspace_size(MOG_OP_DENSE, &kv, nullptr, nullptr, &p, &bytes) == MOG_ERR_UNSUPPORTED);
  p.n_q_heads = 32;
  p.splits = 9000;
  EXPECT(mog_workspace_size(MOG_OP_DENSE, &kv, nullptr, nullptr, &p, &bytes) == MOG_ERR_INVALID_ARG);
  p.splits = 0;
  p.exact_repeat = 65;
  EXPECT(mog_workspace_size(MOG_OP_DENSE, &kv, nullptr, nullptr, &p, &bytes) == MOG_ERR_INVALID_ARG);
  p.exact_repeat = 0;
  p.residual = 3;
  EXPECT(mog_workspace_size(MOG_OP_DENSE, &kv, nullptr, nullptr, &p, &bytes) == MOG_ERR_INVALID_ARG);
  p.residual = 1;
  p.top_c = -1;
  EXPECT(mog_workspace_size(MOG_OP_DENSE, &kv, nullptr, nullptr, &p, &bytes) == MOG_ERR_INVALID_ARG);
  p.top_c = 4;
  EXPECT(mog_workspace_size(static_cast<mog_op>(9), &kv, nullptr, nullptr, &p, &bytes) != MOG_OK);
  mog_layout hl = host_layout(ok_len, 0, {0});
  EXPECT(mog_workspace_size(MOG_OP_DECODE, nullptr, &hl, nullptr, &p, &bytes) == MOG_OK && bytes > 0);
  std::vector<int32_t> per_c = {40};
  p.top_c_per_seq = per_c.data();
  EXPECT(mog_workspace_size(MOG_OP_DECODE, nullptr, &hl, nullptr, &p, &bytes2) == MOG_OK && bytes2 >= bytes);
  p.top_c_per_seq = nullptr;

  mog_build_params bp;
  std::memset(&bp, 0, sizeof(bp));
  bp.kmeans_iters = 10;
  bp.n_sink = 64;
  bp.n_recent = 256;
  bp.seed = 7;
  EXPECT(mog_workspace_size(MOG_OP_BUILD, &kv, nullptr, &bp, nullptr, &bytes) == MOG_OK);
  bp.kmeans_iters = -1;
  EXPECT(mog_workspace_size(MOG_OP_BUILD, &kv, nullptr, &bp, nullptr, &bytes) == MOG_ERR_INVALID_ARG);
  bp.kmeans_iters = 10;
  bp.fm_dim = 128;
  EXPECT(mog_workspace_size(MOG_OP_BUILD, &kv, nullptr, &bp, nullptr, &bytes) == MOG_ERR_INVALID_ARG);
  bp.fm_dim = 0;
  bp.rows_k = fake(0x50000);
  EXPECT(mog_workspace_size(MOG_OP_BUILD, &kv, nullptr, &bp, nullptr, &bytes) == MOG_ERR_INVALID_ARG);
  bp.rows_k = nullptr;

  // entry points that enqueue work: rejected before anything is enqueued
  mog_layout out_layout;
  EXPECT(mog_build(&kv, &bp, fake(0x1001), size_t(1) << 40, fake(0x1000), size_t(1) << 40, &out_layout, nullptr) ==
         MOG_ERR_INVALID_ARG);
  EXPECT(mog_build(&kv, &bp, fake(0x1000), 64, fake(0x1000), size_t(1) << 40, &out_layout, nullptr) ==
         MOG_ERR_WORKSPACE);
  EXPECT(mog_build(nullptr, &bp, fake(0x1000), 64, fake(0x1000), 64, &out_layout, nullptr) == MOG_ERR_INVALID_ARG);
  float* q = static_cast<float*>(fake(0x1000));
  EXPECT(mog_decode(nullptr, &kv, q, &p, q, nullptr, nullptr, nullptr, fake(0x1000), size_t(1) << 30, nullptr) ==
         MOG_ERR_INVALID_ARG);
  mog_layout mism = host_layout(ok_len, 0, {0});
  mism.n_kv_heads = 4;
  EXPECT(mog_decode(&mism, &kv, q, &p, q, nullptr, nullptr, nullptr, fake(0x1000), size_t(1) << 30, nullptr) ==
         MOG_ERR_INVALID_ARG);
  EXPECT(mog_decode(&hl, &kv, q, &p, q, nullptr, nullptr, nullptr, fake(0x1000), 16, nullptr) == MOG_ERR_WORKSPACE);
  EXPECT(mog_decode(&hl, &kv, nullptr, &p, q, nullptr, nullptr, nullptr, fake(0x1000), size_t(1) << 30, nullptr) ==
         MOG_ERR_INVALID_ARG);
  p.residual = 2;
  EXPECT(mog_decode(&hl, &kv, q, &p, q, nullptr, nullptr, nullptr, fake(0x1000), size_t(1) << 40, nullptr) ==
         MOG_ERR_INVALID_ARG);
  p.residual = 1;
  EXPECT(mog_dense_decode(&kv, nullptr, &p, q, nullptr, fake(0x1000), size_t(1) << 30, nullptr) ==
         MOG_ERR_INVALID_ARG);
  EXPECT(mog_dense_decode(&kv, q, &p, q, nullptr, fake(0x1000), 16, nullptr) == MOG_ERR_WORKSPACE);
  mog_kv misaligned = kv;
  misaligned.k = fake(0x100004);
  EXPECT(mog_dense_decode(&misaligned, q, &p, q, nullptr, fake(0x1000), size_t(1) << 30, nullptr) ==
         MOG_ERR_INVALID_ARG);

  // appends: nothing grew (nothing enqueued), shorter, over capacity
  std::vector<int32_t> two = {5000, 6000}, grown = {5008, 6001}, shorter = {4999, 6000};
  mog_layout al = host_layout(two, 10, {3, 0});
  mog_kv kv2 = kv_of(two);
  EXPECT(mog_append(&kv2, &al, nullptr) == MOG_OK);
  mog_kv kv3 = kv_of(shorter);
  EXPECT(mog_append(&kv3, &al, nullptr) == MOG_ERR_INVALID_ARG);
  mog_kv kv4 = kv_of(grown);
  EXPECT(mog_append(&kv4, &al, nullptr) == MOG_ERR_CAPACITY);
  EXPECT(al.seq_lens[0] == 5000 && al.fold_count[0] == 3);
  EXPECT(mog_append(&kv2, nullptr, nullptr) == MOG_ERR_INVALID_ARG);

  if (g_fails) std::fprintf(stderr, "%d expectation(s) failed\n", g_fails);
  else std::printf("abi_sanitize: all host checks passed\n");
  return g_fails ? 1 : 0;
}
