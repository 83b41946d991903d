// Host-side launchers of the library's kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ts.h"

namespace ts {

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// small fill kernels (graph-capturable replacements for memset); scan.hip
hipError_t fill_i64(int64_t* p, int64_t n, int64_t v, hipStream_t s);
hipError_t fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s);
hipError_t fill_f32(float* p, int64_t n, float v, hipStream_t s);

// scan.hip
size_t scan_tmp_bytes(int64_t n);
// out[i] = sum_{k<i} in[k] (in and out may alias); *total (device, may be
// NULL) = sum of all.  `tmp` holds scan_tmp_bytes(n) bytes.
hipError_t scan_exclusive_i32(const int32_t* in, int32_t* out, int64_t n, int64_t* total, void* tmp,
                              hipStream_t s);

// hash.hip
hipError_t launch_hash_build(const int32_t* coords, int64_t n, int ndim, void* table, int64_t cap, uint32_t* flags,
                             hipStream_t s);
hipError_t launch_hash_query(const void* table, int64_t cap, int ndim, const int32_t* q, int64_t m, int32_t* rows,
                             hipStream_t s);
size_t support_scratch_bytes(int64_t n);
hipError_t launch_strided_support(const int32_t* coords, int64_t n, int ndim, int stride, int32_t* out_coords,
                                  int64_t* n_out, void* out_table, int64_t out_cap, void* scratch, uint32_t* flags,
                                  hipStream_t s);

size_t generative_scratch_bytes(int64_t n_cand);
// site of candidate (i, o) = scale * c_i + sign * delta_o
hipError_t launch_generative_support(const int32_t* coords, int64_t n, int ndim, int ksize, int scale, int sign,
                                     int32_t* out_coords, int64_t n_out_cap, int64_t* n_out, void* out_table,
                                     int64_t out_cap, void* scratch, uint32_t* flags, hipStream_t s);

size_t voxelize_scratch_bytes(int64_t n);
hipError_t launch_voxelize(const int32_t* batch, const float* pos, int64_t n, int ndim, const float* size,
                           const float* origin, const float* feats, int c, int32_t* out_coords, int64_t* n_out,
                           void* out_table, int64_t out_cap, int32_t* vox_of, float* out_feats, void* scratch,
                           uint32_t* flags, hipStream_t s);
hipError_t launch_devoxelize(const int32_t* vox_of, int64_t n, const void* vf, int c, void* pf, ts_dtype dt,
                             hipStream_t s);

// kmap.hip
enum RelMode { kModeSubm = 0, kModeDown = 1, kModeUp = 2 };

struct RelBuild {
  int mode;
  const int32_t* dest_coords;  // [n_dest_cap][ndim+1]
  int64_t n_dest_cap;
  const int64_t* n_dest;       // device count (may be NULL: = n_dest_cap)
  int ndim, ksize, stride, kvol;
  const void* src_table;       // table probed for neighbours
  int64_t src_cap;
  const void* own_table;       // kModeUp: input table for the ownership test
  int64_t own_cap;
};

size_t rel_scratch_bytes(int64_t n_dest_cap, int kvol);
// True when the probe of this relation writes its pair groups itself (so the
// relation needs no neighbour table for them).
bool rel_probe_emits_groups(int mode, int ndim, int ksize);
// n_out_fill (device, may be NULL): receives n_dest_cap (the submanifold output count)
hipError_t launch_rel_build(const RelBuild& b, const ts_rel& rel, bool natural, int64_t* n_out_fill, hipStream_t s);
size_t pairs_scratch_bytes(int64_t n_dest_cap, int kvol);
// Pair lists of capacity pair_cap: entries past it are dropped and the
// starts clamped to it, so a short capacity can never write out of bounds.
hipError_t launch_pairs_build(const RelBuild& b, const ts_rel& rel, int64_t pair_cap, int64_t* pair_start,
                              int32_t* pair_in, int32_t* pair_out, void* scratch, hipStream_t s);

// conv.hip
struct ConvArgs {
  const ts_rel* rel;  // relation walked (destination tiles)
  int kvol;
  const void* src;    // source features [n_src][c_src]
  int64_t n_src;
  int c_src;
  void* dst;          // destination features [n_dest][c_dst]
  int c_dst;
  const void* w;      // weights [kvol][cin][cout] of the layer
  int w_cin, w_cout;
  bool transpose;     // dgrad: contract over the layer's cout
  bool mirror;        // dgrad of a submanifold map: use W[kvol-1-o]
  bool rows_in_order; // tiles keep rows in index order (no grouping by mask)
  ts_dtype in_dtype, out_dtype;
  bool prepacked = false;  // implicit GEMM: ws already holds the packed weights
};

size_t igemm_workspace_bytes(int kvol, int c_src, int c_dst);
bool igemm_supported(int kvol, int64_t n_src, int c_src, int c_dst, ts_dtype in_dtype);
hipError_t launch_wpack(const ConvArgs& a, void* ws, hipStream_t s);
hipError_t launch_igemm(const ConvArgs& a, void* ws, hipStream_t s);
hipError_t launch_direct(const ConvArgs& a, hipStream_t s);
hipError_t launch_graph_conv(const int64_t* indptr, const int32_t* src, const int32_t* rel, int64_t n_dst,
                             int64_t n_src, int n_rel, const void* x, int cin, const void* w, int cout, void* y,
                             ts_dtype in, ts_dtype out, uint32_t* flags, hipStream_t s);
hipError_t launch_pool(const ts_rel& rel, int kvol, const void* x, int64_t n_src, int c, void* y, ts_dtype in,
                       ts_dtype out, int mode, hipStream_t s);

// fod.hip: the fetch-on-demand dataflow over a relation's pair groups
bool fod_supported(int kvol, int64_t n_src, int c_src, int c_dst, ts_dtype in_dtype);
hipError_t launch_fod(const ConvArgs& a, hipStream_t s);

size_t gs_workspace_bytes(int64_t n_dest_cap, int c_dst, ts_dtype out_dtype);
hipError_t launch_gather_scatter(const ts_kmap* map, const ConvArgs& a, bool backward, int64_t n_dest_cap,
                                 void* ws, hipStream_t s);

// bounds-check build: each checking translation unit's violation word
// (read and cleared); defined only under TS_DEBUG_CHECKS
hipError_t debug_take_conv(uint32_t* v);
hipError_t debug_take_igemm(uint32_t* v);
hipError_t debug_take_fod(uint32_t* v);
hipError_t debug_take_wgrad(uint32_t* v);

// wgrad.hip
size_t wgrad_workspace_bytes(const ts_kmap* map, int cin, int cout);
hipError_t launch_wgrad(const ts_kmap* map, const void* x, int cin, const void* dy, int cout, ts_dtype dt, float* dw,
                        void* ws, hipStream_t s);

}  // namespace ts
