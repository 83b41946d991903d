// Host-side argument validation and size queries of the C ABI, built with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host code (no GPU:
// every call below is refused, or answered, before anything is launched).
// Exit status 0 when every expectation holds; a sanitizer report aborts.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ts.h"

static int g_fail = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++g_fail;                                                        \
    }                                                                  \
  } while (0)

// Never dereferenced: every call that receives it fails validation first.
static void* const FAKE = reinterpret_cast<void*>(uintptr_t{0x1000});
static const int32_t* const FAKE_I = reinterpret_cast<const int32_t*>(uintptr_t{0x1000});

static void sizes() {
  EXPECT(ts_hash_capacity(0, 2.0) == 64);
  EXPECT(ts_hash_capacity(102835, 2.0) == 262144);
  EXPECT(ts_hash_capacity(10, 0.5) == -1);
  EXPECT(ts_hash_capacity(-1, 2.0) == -1);
  EXPECT(ts_hash_table_bytes(0) == 0);
  EXPECT(ts_hash_table_bytes(1024) > 1024 * 8);
  EXPECT(ts_hash_table_bytes(int64_t{1} << 25) > 0);
  const size_t b = ts_kmap_bytes(1000, 1000, 3, 3, 1, 0);
  EXPECT(b > 1000 * 27 * 4);
  EXPECT(ts_kmap_bytes(1000, 1000, 3, 3, 1, TS_KMAP_PAIRS) > b);
  EXPECT(ts_kmap_bytes(1000, 1000, 3, 3, 1, TS_KMAP_GROUPS | TS_KMAP_NO_TABLE) > 0);
  EXPECT(ts_kmap_bytes(10, 10, 4, 3, 1, 0) == 0);
  EXPECT(ts_kmap_bytes(10, 10, 3, 5, 1, 0) == 0);
  EXPECT(ts_kmap_bytes(-1, 10, 3, 3, 1, 0) == 0);
  EXPECT(ts_kmap_bytes(80000000, 80000000, 3, 3, 1, TS_KMAP_PAIRS) == 0);  // int32 positions
  EXPECT(ts_kmap_bytes(INT64_MAX, 10, 3, 3, 1, 0) == 0);
  EXPECT(ts_generative_scratch_bytes(100, 3, 3) >= 3 * 100 * 27 * 4);
  EXPECT(ts_generative_scratch_bytes(-1, 3, 3) == 0);
  EXPECT(ts_generative_scratch_bytes(INT64_MAX / 2, 3, 3) == 0);
  EXPECT(ts_generative_scratch_bytes(int64_t{1} << 27, 3, 3) == 0);  // 27 * 2^27 candidates
  EXPECT(ts_support_scratch_bytes(INT64_MAX) == 0);
  EXPECT(ts_voxelize_scratch_bytes(INT64_MAX) == 0);
  EXPECT(ts_support_scratch_bytes(-5) == 0);
  EXPECT(ts_voxelize_scratch_bytes(100) >= 4 * 100 * 4);
  EXPECT(ts_voxelize_scratch_bytes(-1) == 0);
  EXPECT(strcmp(ts_status_string(TS_OK), "ok") == 0);
  EXPECT(ts_status_string(static_cast<ts_status>(99)) != nullptr);
  EXPECT(ts_status_string(static_cast<ts_status>(-7)) != nullptr);
  EXPECT(strstr(ts_version(), "gfx950") != nullptr);
  EXPECT(ts_debug_violations(nullptr) == TS_ERR_UNSUPPORTED);  // the regular build has no checks
}

static void hash() {
  EXPECT(ts_hash_build(nullptr, 10, 3, FAKE, 64, nullptr, nullptr) == TS_ERR_INVALID_ARG);
  EXPECT(ts_hash_build(FAKE_I, 10, 3, nullptr, 64, nullptr, nullptr) == TS_ERR_INVALID_ARG);
  EXPECT(ts_hash_build(FAKE_I, -1, 3, FAKE, 64, nullptr, nullptr) == TS_ERR_INVALID_ARG);
  EXPECT(ts_hash_build(FAKE_I, 10, 4, FAKE, 64, nullptr, nullptr) == TS_ERR_INVALID_ARG);
  EXPECT(ts_hash_build(FAKE_I, 10, 3, FAKE, 48, nullptr, nullptr) == TS_ERR_INVALID_ARG);
  EXPECT(ts_hash_build(FAKE_I, 100, 3, FAKE, 64, nullptr, nullptr) == TS_ERR_INVALID_ARG);
  EXPECT(ts_hash_build(FAKE_I, 10, 3, FAKE, int64_t{1} << 26, nullptr, nullptr) == TS_ERR_UNSUPPORTED);
  int32_t rows[1];
  EXPECT(ts_hash_query(nullptr, 64, 3, FAKE_I, 5, rows, nullptr) == TS_ERR_INVALID_ARG);
  EXPECT(ts_hash_query(FAKE, 63, 3, FAKE_I, 5, rows, nullptr) == TS_ERR_INVALID_ARG);
  EXPECT(ts_hash_query(FAKE, 64, 1, FAKE_I, 5, rows, nullptr) == TS_ERR_INVALID_ARG);
}

static void kmap_build() {
  ts_kmap km;
  memset(&km, 0, sizeof km);
  const size_t need = ts_kmap_bytes(100, 100, 3, 3, 1, 0);
  auto call = [&](int64_t n_in, const void* in_table, int64_t in_cap, int ndim, int ksize, int stride,
                  uint32_t flags, size_t bytes) {
    return ts_kmap_build(FAKE_I, n_in, in_table, in_cap, nullptr, 0, nullptr, nullptr, 0, ndim, ksize, stride, flags,
                         FAKE, bytes, &km, nullptr);
  };
  EXPECT(call(100, FAKE, 256, 3, 3, 1, 0, need - 1) == TS_ERR_INVALID_ARG);
  EXPECT(call(100, FAKE, 256, 3, 2, 1, 0, need) == TS_ERR_UNSUPPORTED);
  EXPECT(call(100, FAKE, 256, 3, 5, 1, 0, need) == TS_ERR_UNSUPPORTED);
  EXPECT(call(100, FAKE, 256, 1, 3, 1, 0, need) == TS_ERR_INVALID_ARG);
  EXPECT(call(100, FAKE, 256, 3, 3, 0, 0, need) == TS_ERR_INVALID_ARG);
  EXPECT(call(100, nullptr, 256, 3, 3, 1, 0, need) == TS_ERR_INVALID_ARG);
  EXPECT(call(100, FAKE, 100, 3, 3, 1, 0, need) == TS_ERR_INVALID_ARG);
  EXPECT(call(100, FAKE, 256, 3, 3, 1, TS_KMAP_NO_TABLE, need) == TS_ERR_INVALID_ARG);
  EXPECT(call(80000000, FAKE, int64_t{1} << 25, 3, 3, 1, TS_KMAP_PAIRS, need) == TS_ERR_UNSUPPORTED);
  const size_t sneed = ts_kmap_bytes(100, 100, 3, 2, 2, TS_KMAP_BWD);
  EXPECT(ts_kmap_build(FAKE_I, 100, FAKE, 256, nullptr, 100, nullptr, nullptr, 0, 3, 2, 2, 0, FAKE, sneed, &km,
                       nullptr) == TS_ERR_INVALID_ARG);
}

// A map that looks built (fields only; nothing behind the pointers is read).
static ts_kmap fake_map() {
  ts_kmap km;
  memset(&km, 0, sizeof km);
  km.kvol = 27;
  km.stride = 1;
  km.n_in = km.n_out_cap = 100;
  km.fwd.n_dest_cap = 100;
  km.fwd.tile_mask = reinterpret_cast<uint64_t*>(uintptr_t{0x2000});
  km.fwd.row_mask = reinterpret_cast<uint64_t*>(uintptr_t{0x3000});
  km.fwd.n_tiles = 7;
  return km;
}

static void conv() {
  ts_kmap empty;
  memset(&empty, 0, sizeof empty);
  EXPECT(ts_conv_fwd(&empty, FAKE, 16, FAKE, 16, FAKE, TS_F16, TS_F16, TS_DATAFLOW_AUTO, nullptr, 0, nullptr) ==
         TS_ERR_INVALID_ARG);
  ts_kmap km = fake_map();
  EXPECT(ts_conv_fwd(&km, FAKE, 0, FAKE, 16, FAKE, TS_F16, TS_F16, TS_DATAFLOW_AUTO, nullptr, 0, nullptr) ==
         TS_ERR_INVALID_ARG);
  EXPECT(ts_conv_fwd(&km, FAKE, 16, FAKE, 16, FAKE, static_cast<ts_dtype>(7), TS_F16, TS_DATAFLOW_AUTO, nullptr, 0,
                     nullptr) == TS_ERR_INVALID_ARG);
  EXPECT(ts_conv_fwd(&km, FAKE, 16, FAKE, 16, FAKE, static_cast<ts_dtype>(-1), TS_F16, TS_DATAFLOW_AUTO, nullptr, 0,
                     nullptr) == TS_ERR_INVALID_ARG);
  EXPECT(ts_conv_fwd(&km, FAKE, 16, FAKE, 16, FAKE, TS_F16, TS_F16, static_cast<ts_dataflow>(-3), nullptr, 0,
                     nullptr) == TS_ERR_INVALID_ARG);
  EXPECT(ts_conv_fwd(&km, FAKE, 16, FAKE, 16, FAKE, TS_F16, TS_BF16, TS_DATAFLOW_AUTO, nullptr, 0, nullptr) ==
         TS_ERR_UNSUPPORTED);
  EXPECT(ts_conv_fwd(&km, nullptr, 64, FAKE, 64, FAKE, TS_F16, TS_F16, TS_DATAFLOW_AUTO, nullptr, 0, nullptr) ==
         TS_ERR_INVALID_ARG);
  EXPECT(ts_conv_fwd(&km, FAKE, 64, FAKE, 64, nullptr, TS_F16, TS_F16, TS_DATAFLOW_AUTO, nullptr, 0, nullptr) ==
         TS_ERR_INVALID_ARG);
  EXPECT(ts_conv_fwd(&km, FAKE, 64, FAKE, 64, FAKE, TS_F16, TS_F16, TS_DATAFLOW_GATHER_SCATTER, FAKE, size_t{1} << 30,
                     nullptr) == TS_ERR_INVALID_ARG);
  EXPECT(ts_conv_fwd(&km, FAKE, 16, FAKE, 16, FAKE, TS_F16, TS_F16, static_cast<ts_dataflow>(9), nullptr, 0,
                     nullptr) == TS_ERR_INVALID_ARG);
  EXPECT(ts_conv_fwd(&km, FAKE, 64, FAKE, 64, FAKE, TS_F16, TS_F16, TS_DATAFLOW_FETCH_ON_DEMAND, nullptr, 0,
                     nullptr) == TS_ERR_INVALID_ARG);
  // groups without a table
  km.fwd.tile_mask = nullptr;
  km.fwd.gcount = reinterpret_cast<int32_t*>(uintptr_t{0x4000});
  km.fwd.n_gtiles = 1;
  EXPECT(ts_conv_fwd(&km, FAKE, 64, FAKE, 64, FAKE, TS_F32, TS_F32, TS_DATAFLOW_FETCH_ON_DEMAND, nullptr, 0,
                     nullptr) == TS_ERR_UNSUPPORTED);
  EXPECT(ts_conv_fwd(&km, FAKE, 64, FAKE, 64, FAKE, TS_F16, TS_F16, TS_DATAFLOW_IMPLICIT_GEMM, nullptr, 0,
                     nullptr) == TS_ERR_INVALID_ARG);
  EXPECT(ts_pool_fwd(&km, FAKE, 16, FAKE, TS_F16, TS_F16, TS_POOL_MAX, nullptr) == TS_ERR_INVALID_ARG);
  km = fake_map();
  EXPECT(ts_conv_bwd_wgrad(&km, FAKE, 16, FAKE, 16, TS_F16, reinterpret_cast<float*>(FAKE), FAKE, size_t{1} << 30,
                           nullptr) == TS_ERR_INVALID_ARG);
  km.stride = 2;
  EXPECT(ts_conv_bwd_dgrad(&km, FAKE, 16, FAKE, 16, FAKE, TS_F16, TS_F16, TS_DATAFLOW_AUTO, nullptr, 0, nullptr) ==
         TS_ERR_INVALID_ARG);
  km.stride = 1;
  EXPECT(ts_subm_conv_fwd(&km, FAKE, 16, FAKE, 16, FAKE, static_cast<ts_dtype>(9), TS_F16, TS_DATAFLOW_AUTO, nullptr,
                          0, nullptr) == TS_ERR_INVALID_ARG);
  // weight packing and workspace sizes
  km.mirror_bwd = 1;
  const size_t need = ts_conv_workspace_bytes(&km, 64, 64, TS_OP_FWD, TS_F16, TS_DATAFLOW_IMPLICIT_GEMM);
  EXPECT(need == size_t{27} * 64 * 64 * 2);
  EXPECT(ts_conv_pack_weights(&km, nullptr, 64, 64, TS_OP_FWD, TS_F16, FAKE, need, nullptr) == TS_ERR_INVALID_ARG);
  EXPECT(ts_conv_pack_weights(&km, FAKE, 64, 64, TS_OP_FWD, TS_F16, FAKE, need - 1, nullptr) == TS_ERR_INVALID_ARG);
  EXPECT(ts_conv_pack_weights(&km, FAKE, 48, 64, TS_OP_FWD, TS_F16, FAKE, need, nullptr) == TS_ERR_UNSUPPORTED);
  EXPECT(ts_conv_pack_weights(&km, FAKE, 64, 64, 7, TS_F16, FAKE, need, nullptr) == TS_ERR_INVALID_ARG);
  EXPECT(ts_conv_workspace_bytes(&km, 16, 16, TS_OP_FWD, TS_F32, TS_DATAFLOW_AUTO) == 0);
  EXPECT(ts_conv_workspace_bytes(&km, 64, 64, TS_OP_WGRAD, TS_F16, TS_DATAFLOW_AUTO) >= size_t{27} * 64 * 64 * 4);
}

static void supports() {
  const size_t sb = ts_generative_scratch_bytes(100, 3, 3);
  int64_t n_out = 0;
  EXPECT(ts_generative_support(FAKE_I, 100, 3, 3, reinterpret_cast<int32_t*>(FAKE), 2700, nullptr, FAKE, 1024, FAKE,
                               sb, nullptr, nullptr) == TS_ERR_INVALID_ARG);
  EXPECT(ts_generative_support(FAKE_I, 100, 3, 3, reinterpret_cast<int32_t*>(FAKE), 2700, &n_out, FAKE, 1000, FAKE,
                               sb, nullptr, nullptr) == TS_ERR_INVALID_ARG);
  EXPECT(ts_generative_support(FAKE_I, 100, 3, 3, reinterpret_cast<int32_t*>(FAKE), 2700, &n_out, FAKE, 1024, FAKE,
                               sb - 1, nullptr, nullptr) == TS_ERR_INVALID_ARG);
  EXPECT(ts_generative_support(FAKE_I, 100, 3, 5, reinterpret_cast<int32_t*>(FAKE), 2700, &n_out, FAKE, 1024, FAKE,
                               sb, nullptr, nullptr) == TS_ERR_INVALID_ARG);
  const size_t tb = ts_generative_scratch_bytes(100, 3, 2);
  EXPECT(ts_transposed_support(FAKE_I, 100, 3, 2, 0, reinterpret_cast<int32_t*>(FAKE), 800, &n_out, FAKE, 1024, FAKE,
                               tb, nullptr, nullptr) == TS_ERR_INVALID_ARG);
  EXPECT(ts_strided_support(FAKE_I, 100, 3, 2, reinterpret_cast<int32_t*>(FAKE), &n_out, FAKE, 64, FAKE,
                            ts_support_scratch_bytes(100), nullptr, nullptr) == TS_ERR_INVALID_ARG);  // cap < n
  const float sz[3] = {0.1f, 0.1f, 0.1f}, og[3] = {0.f, 0.f, 0.f}, bad[3] = {0.1f, 0.f, 0.1f};
  const size_t vb = ts_voxelize_scratch_bytes(100);
  EXPECT(ts_voxelize(nullptr, reinterpret_cast<const float*>(FAKE), 100, 3, bad, og, nullptr, 0,
                     reinterpret_cast<int32_t*>(FAKE), &n_out, FAKE, 256, reinterpret_cast<int32_t*>(FAKE), nullptr,
                     FAKE, vb, nullptr, nullptr) == TS_ERR_INVALID_ARG);
  EXPECT(ts_voxelize(nullptr, reinterpret_cast<const float*>(FAKE), 100, 3, sz, og, nullptr, 0,
                     reinterpret_cast<int32_t*>(FAKE), &n_out, FAKE, 256, reinterpret_cast<int32_t*>(FAKE), nullptr,
                     FAKE, vb - 1, nullptr, nullptr) == TS_ERR_INVALID_ARG);
}

static void fused_and_others() {
  // strided forward with support generation: every argument is checked
  // before the first launch
  ts_kmap km;
  memset(&km, 0, sizeof km);
  const size_t kb = ts_kmap_bytes(100, 100, 3, 2, 2, 0) + ts_support_scratch_bytes(100);
  auto strided = [&](int stride, size_t bytes, int cin, void* y, ts_dtype in, ts_dtype out, ts_dataflow df) {
    return ts_conv_fwd_strided(FAKE_I, 100, 3, FAKE, 256, 2, stride, 0, reinterpret_cast<int32_t*>(FAKE),
                               reinterpret_cast<int64_t*>(FAKE), FAKE, 256, nullptr, FAKE, bytes, &km, FAKE, cin, FAKE,
                               64, y, in, out, df, FAKE, size_t{1} << 30, nullptr);
  };
  EXPECT(strided(1, kb, 64, FAKE, TS_F16, TS_F16, TS_DATAFLOW_AUTO) == TS_ERR_INVALID_ARG);      // stride 1
  EXPECT(strided(2, kb - 1, 64, FAKE, TS_F16, TS_F16, TS_DATAFLOW_AUTO) == TS_ERR_INVALID_ARG);  // short map buffer
  EXPECT(strided(2, kb, 0, FAKE, TS_F16, TS_F16, TS_DATAFLOW_AUTO) == TS_ERR_INVALID_ARG);       // no channels
  EXPECT(strided(2, kb, 64, nullptr, TS_F16, TS_F16, TS_DATAFLOW_AUTO) == TS_ERR_INVALID_ARG);   // no output
  EXPECT(strided(2, kb, 64, FAKE, TS_F16, TS_BF16, TS_DATAFLOW_AUTO) == TS_ERR_UNSUPPORTED);     // f16 -> bf16
  EXPECT(strided(2, kb, 64, FAKE, TS_F16, TS_F16, TS_DATAFLOW_GATHER_SCATTER) == TS_ERR_INVALID_ARG);  // no pairs
  // ConvTranspose over a strided relation needs its transposed relation
  ts_kmap t;
  memset(&t, 0, sizeof t);
  t.kvol = 8;
  t.stride = 2;
  t.n_in = 100;
  t.n_out_cap = 60;
  t.fwd.n_dest_cap = 60;
  t.fwd.tile_mask = reinterpret_cast<uint64_t*>(uintptr_t{0x2000});
  t.fwd.row_mask = reinterpret_cast<uint64_t*>(uintptr_t{0x3000});
  t.fwd.n_tiles = 4;
  EXPECT(ts_conv_transpose_fwd(&t, FAKE, 16, FAKE, 16, FAKE, TS_F32, TS_F32, TS_DATAFLOW_AUTO, nullptr, 0, nullptr) ==
         TS_ERR_INVALID_ARG);
  // graph convolution
  const int64_t* ip = reinterpret_cast<const int64_t*>(FAKE);
  EXPECT(ts_graph_conv_fwd(ip, FAKE_I, FAKE_I, 10, 10, 0, FAKE, 8, FAKE, 8, FAKE, TS_F16, TS_F16, nullptr, nullptr) ==
         TS_ERR_INVALID_ARG);  // no relations
  EXPECT(ts_graph_conv_fwd(nullptr, FAKE_I, FAKE_I, 10, 10, 3, FAKE, 8, FAKE, 8, FAKE, TS_F16, TS_F16, nullptr,
                           nullptr) == TS_ERR_INVALID_ARG);  // no CSR offsets
  EXPECT(ts_graph_conv_fwd(ip, FAKE_I, FAKE_I, -1, 10, 3, FAKE, 8, FAKE, 8, FAKE, TS_F16, TS_F16, nullptr, nullptr) ==
         TS_ERR_INVALID_ARG);
  EXPECT(ts_graph_conv_fwd(ip, FAKE_I, FAKE_I, 10, 10, 3, FAKE, 8, FAKE, 8, FAKE, TS_BF16, TS_F16, nullptr, nullptr) ==
         TS_ERR_UNSUPPORTED);
  EXPECT(ts_graph_conv_fwd(ip, FAKE_I, FAKE_I, 10, 10, 3, FAKE, 8, FAKE, 8, FAKE, static_cast<ts_dtype>(5), TS_F16,
                           nullptr, nullptr) == TS_ERR_INVALID_ARG);
  // devoxelization and pooling
  EXPECT(ts_devoxelize(FAKE_I, 10, FAKE, 0, FAKE, TS_F32, nullptr) == TS_ERR_INVALID_ARG);
  EXPECT(ts_devoxelize(nullptr, 10, FAKE, 4, FAKE, TS_F32, nullptr) == TS_ERR_INVALID_ARG);
  EXPECT(ts_devoxelize(FAKE_I, 10, FAKE, 4, FAKE, static_cast<ts_dtype>(-2), nullptr) == TS_ERR_INVALID_ARG);
  EXPECT(ts_pool_fwd(&t, FAKE, 8, FAKE, TS_F16, TS_F16, 2, nullptr) == TS_ERR_INVALID_ARG);  // mode
  EXPECT(ts_pool_fwd(&t, FAKE, 0, FAKE, TS_F16, TS_F16, TS_POOL_MAX, nullptr) == TS_ERR_INVALID_ARG);
  EXPECT(ts_pool_fwd(&t, FAKE, 8, FAKE, TS_F16, TS_BF16, TS_POOL_MAX, nullptr) == TS_ERR_UNSUPPORTED);
}

int main() {
  sizes();
  hash();
  kmap_build();
  conv();
  supports();
  fused_and_others();
  if (g_fail) fprintf(stderr, "%d expectation(s) failed\n", g_fail);
  else printf("abi host checks: all passed\n");
  return g_fail ? 1 : 0;
}
