// C entry points: host-side validation, buffer layout and kernel dispatch.
// Every check that the host can make happens here, before any launch.
#include <string.h>

#include <cmath>

#include "common.h"
#include "launch.h"

using namespace ts;

namespace {

#define TS_TRY(expr)                                  \
  do {                                                \
    hipError_t e_ = (expr);                           \
    if (e_ != hipSuccess) return TS_ERR_HIP;          \
  } while (0)

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
bool dtype_ok(int d) { return d == TS_F32 || d == TS_F16 || d == TS_BF16; }
int ipow(int b, int e) {
  int v = 1;
  for (int i = 0; i < e; ++i) v *= b;
  return v;
}
bool shape_ok(int ndim, int ksize, int stride) {
  if (ndim != 2 && ndim != 3) return false;
  if (ksize < 1 || ksize > 64 || stride < 1 || stride > 65535) return false;
  return ipow(ksize, ndim) <= TS_MAX_KVOL;
}

constexpr int64_t kMaxRows = (int64_t{1} << 31) - 1;
constexpr int64_t kMaxCap = int64_t{1} << 25;  // block slots (cell indices stay int32)
constexpr int kMaxChannels = 1 << 16;

// Layout of the kernel-map buffer: every region starts on a 256-byte boundary.
struct Carver {
  char* base;
  size_t off = 0;
  template <typename T>
  T* take(size_t count) {
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off = align_up(off + count * sizeof(T), 256);
    return p;
  }
};

// Pairs a map can hold.  Forward maps: at most kvol per output row; with
// distinct outputs (submanifold, or a support from ts_strided_support) also
// at most ceil(k/s)^D per input row.  Caller targets may repeat a coordinate,
// so a target map takes the first bound alone.  A transposed map swaps the
// roles: at most ceil(k/s)^D per (fine) output row and kvol per input row.
int64_t pair_capacity(int64_t n_in, int64_t n_out_cap, int ndim, int ksize, int stride, uint32_t flags) {
  const int kvol = ipow(ksize, ndim);
  const int64_t per_row = ipow((ksize + stride - 1) / stride, ndim);
  if (flags & TS_KMAP_TRANSPOSED) {
    const int64_t a = n_out_cap * per_row, b = n_in * kvol;
    return a < b ? a : b;
  }
  const int64_t a = n_out_cap * kvol;
  const int64_t b = n_in * per_row;
  return ((flags & TS_KMAP_TARGET) || a < b) ? a : b;
}

// One relation: the neighbour table and tile lists (`table`), the row
// masks, and the pair groups (`groups`).
void carve_rel(Carver& c, ts_rel* r, int64_t n_dest_cap, int kvol, bool table, bool groups) {
  r->n_dest_cap = n_dest_cap;
  r->n_tiles = ceil_div<int64_t>(n_dest_cap, kTile);
  r->tile_mask = table ? c.take<uint64_t>(static_cast<size_t>(r->n_tiles)) : nullptr;
  r->tile_rows = table ? c.take<int32_t>(static_cast<size_t>(r->n_tiles) * kTile) : nullptr;
  r->nbr = table ? c.take<int32_t>(static_cast<size_t>(n_dest_cap) * kvol) : nullptr;
  r->row_mask = c.take<uint64_t>(static_cast<size_t>(n_dest_cap));
  r->n_dest = nullptr;
  r->n_gtiles = groups ? ceil_div<int64_t>(n_dest_cap, TS_GTILE) : 0;
  const size_t entries = static_cast<size_t>(r->n_gtiles) * kvol * TS_GTILE;
  r->gcount = groups ? c.take<int32_t>(static_cast<size_t>(r->n_gtiles) * kvol) : nullptr;
  r->gsrc = groups ? c.take<int32_t>(entries) : nullptr;
  r->gslot = groups ? c.take<uint8_t>(entries) : nullptr;
}

// Probe mode of a map's forward relation (see ts_kmap_build).
int fwd_mode(int stride, uint32_t flags) {
  if (flags & TS_KMAP_TRANSPOSED) return kModeUp;
  return (stride == 1 && !(flags & TS_KMAP_TARGET)) ? kModeSubm : kModeDown;
}

// Lays out a map; with base == NULL only the size is computed.
size_t layout_kmap(char* base, ts_kmap* m, int64_t n_in, int64_t n_out_cap, int ndim, int ksize, int stride,
                   uint32_t flags) {
  Carver c{base};
  memset(m, 0, sizeof(*m));
  m->ndim = ndim;
  m->ksize = ksize;
  m->stride = stride;
  m->kvol = ipow(ksize, ndim);
  m->flags = flags;
  // a target map's outputs are not its inputs, so its transposed relation is
  // a map of its own, as for a strided one
  const bool own_bwd = stride > 1 || (flags & (TS_KMAP_TARGET | TS_KMAP_TRANSPOSED));
  m->mirror_bwd = own_bwd ? 0 : 1;
  m->n_in = n_in;
  m->n_out_cap = n_out_cap;
  m->n_out = c.take<int64_t>(1);
  const bool groups = (flags & TS_KMAP_GROUPS) != 0;
  const bool fwd_table =
      !(groups && (flags & TS_KMAP_NO_TABLE) && rel_probe_emits_groups(fwd_mode(stride, flags), ndim, ksize));
  carve_rel(c, &m->fwd, n_out_cap, m->kvol, fwd_table, groups);
  if (own_bwd && (flags & TS_KMAP_BWD)) carve_rel(c, &m->bwd, n_in, m->kvol, true, groups);
  size_t scratch = rel_scratch_bytes(n_out_cap, m->kvol);
  if (flags & TS_KMAP_PAIRS) {
    m->pair_cap = pair_capacity(n_in, n_out_cap, ndim, ksize, stride, flags);
    m->pair_start = c.take<int64_t>(static_cast<size_t>(m->kvol) + 1);
    m->pair_in = c.take<int32_t>(static_cast<size_t>(m->pair_cap));
    m->pair_out = c.take<int32_t>(static_cast<size_t>(m->pair_cap));
    const size_t ps = pairs_scratch_bytes(n_out_cap, m->kvol);
    if (ps > scratch) scratch = ps;
  }
  if (own_bwd && (flags & TS_KMAP_BWD)) {
    const size_t rs = rel_scratch_bytes(n_in, m->kvol);
    if (rs > scratch) scratch = rs;
  }
  m->scratch_bytes = scratch;
  m->scratch = c.take<char>(scratch);
  return c.off;
}

ts_status check_conv(const ts_kmap* map, int cin, int cout, ts_dtype in, ts_dtype out) {
  if (!map || map->kvol < 1 || map->kvol > TS_MAX_KVOL || !map->fwd.row_mask) return TS_ERR_INVALID_ARG;
  if (!map->fwd.tile_mask && !map->fwd.gcount) return TS_ERR_INVALID_ARG;
  if (cin < 1 || cout < 1 || cin > kMaxChannels || cout > kMaxChannels) return TS_ERR_INVALID_ARG;
  if (!dtype_ok(in) || !dtype_ok(out)) return TS_ERR_INVALID_ARG;
  if (out != TS_F32 && out != in) return TS_ERR_UNSUPPORTED;
  return TS_OK;
}

bool use_igemm(ts_dataflow df, int kvol, int64_t n_src, int c_src, int c_dst, ts_dtype in) {
  return (df == TS_DATAFLOW_AUTO || df == TS_DATAFLOW_IMPLICIT_GEMM || df == TS_DATAFLOW_IMPLICIT_GEMM_PACKED) &&
         igemm_supported(kvol, n_src, c_src, c_dst, in);
}

// Dataflow in range; the weights are needed unless they come packed.
ts_status check_dataflow(ts_dataflow df, const void* w) {
  if (df < TS_DATAFLOW_AUTO || df > TS_DATAFLOW_FETCH_ON_DEMAND) return TS_ERR_INVALID_ARG;
  if (!w && df != TS_DATAFLOW_IMPLICIT_GEMM_PACKED) return TS_ERR_INVALID_ARG;
  return TS_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Which kernel runs a contraction over relation `rel` (the forward's, dgrad's
// or the transposed convolution's): the fetch-on-demand dataflow when asked
// for, or by default when the relation has pair groups and the shape has a
// kernel; the implicit GEMM or the direct kernel over the neighbour table
// otherwise.  Returns TS_OK and sets *kind, or the error to report.
enum Kind { kFod, kIgemm, kDirect };
ts_status pick_kernel(ts_dataflow df, const ts_rel& rel, int kvol, int64_t n_src, int c_src, int c_dst,
                      ts_dtype in, const void* src, Kind* kind) {
  const bool fod_ok = rel.gcount && aligned16(src) && fod_supported(kvol, n_src, c_src, c_dst, in);
  if (df == TS_DATAFLOW_FETCH_ON_DEMAND) {
    if (!rel.gcount) return TS_ERR_INVALID_ARG;  // the map has no pair groups
    if (!fod_ok) return TS_ERR_UNSUPPORTED;
    *kind = kFod;
    return TS_OK;
  }
  if (df == TS_DATAFLOW_AUTO && fod_ok) {
    *kind = kFod;
    return TS_OK;
  }
  if (!rel.tile_mask) return TS_ERR_INVALID_ARG;  // the other kernels walk the neighbour table
  const bool ig = (df == TS_DATAFLOW_AUTO || df == TS_DATAFLOW_IMPLICIT_GEMM || df == TS_DATAFLOW_IMPLICIT_GEMM_PACKED) &&
                  igemm_supported(kvol, n_src, c_src, c_dst, in) && aligned16(src);
  if (df == TS_DATAFLOW_IMPLICIT_GEMM_PACKED && !ig) return TS_ERR_UNSUPPORTED;
  *kind = ig ? kIgemm : kDirect;
  return TS_OK;
}

hipError_t run_kernel(Kind kind, const ConvArgs& a, void* ws, hipStream_t s) {
  switch (kind) {
    case kFod: return launch_fod(a, s);
    case kIgemm: return launch_igemm(a, ws, s);
    default: return launch_direct(a, s);
  }
}

size_t conv_ws(const ts_kmap* map, int c_src, int c_dst, ts_dtype in, ts_dtype out, ts_dataflow df, int64_t n_dest,
               int64_t n_src) {
  if (df == TS_DATAFLOW_GATHER_SCATTER) return gs_workspace_bytes(n_dest, c_dst, out);
  if (use_igemm(df, map->kvol, n_src, c_src, c_dst, in)) return igemm_workspace_bytes(map->kvol, c_src, c_dst);
  return 0;
}

}  // namespace

extern "C" {

const char* ts_status_string(ts_status s) {
  switch (s) {
    case TS_OK: return "ok";
    case TS_ERR_INVALID_ARG: return "invalid argument";
    case TS_ERR_UNSUPPORTED: return "unsupported";
    case TS_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

#ifdef TS_DEBUG_CHECKS
const char* ts_version(void) { return "ts 0.1.0 (gfx950, bounds checks)"; }
#else
const char* ts_version(void) { return "ts 0.1.0 (gfx950)"; }
#endif

ts_status ts_debug_violations(uint32_t* bits) {
#ifdef TS_DEBUG_CHECKS
  if (!bits) return TS_ERR_INVALID_ARG;
  if (hipDeviceSynchronize() != hipSuccess) return TS_ERR_HIP;
  hipError_t (*const take[])(uint32_t*) = {debug_take_conv, debug_take_igemm, debug_take_fod, debug_take_wgrad};
  for (auto f : take) {
    uint32_t v = 0;
    if (f(&v) != hipSuccess) return TS_ERR_HIP;
    *bits |= v;
  }
  return TS_OK;
#else
  (void)bits;
  return TS_ERR_UNSUPPORTED;
#endif
}

int64_t ts_hash_capacity(int64_t n, double rsv_ratio) {
  if (n < 0 || !(rsv_ratio >= 1.0)) return -1;
  double want = rsv_ratio * static_cast<double>(n);
  int64_t cap = 64;
  while (static_cast<double>(cap) < want) cap <<= 1;
  return cap;
}

size_t ts_hash_table_bytes(int64_t cap) {
  return cap > 0 ? table_keys_bytes(cap) + static_cast<size_t>(cap) * kCells * sizeof(int32_t) : 0;
}

ts_status ts_hash_build(const int32_t* coords, int64_t n, int ndim, void* table, int64_t cap, uint32_t* err_flags,
                        hipStream_t stream) {
  if (n < 0 || n > kMaxRows || (n > 0 && !coords) || !table) return TS_ERR_INVALID_ARG;
  if ((ndim != 2 && ndim != 3) || !is_pow2(cap) || cap < n) return TS_ERR_INVALID_ARG;
  if (cap > kMaxCap) return TS_ERR_UNSUPPORTED;
  TS_TRY(launch_hash_build(coords, n, ndim, table, cap, err_flags, stream));
  return TS_OK;
}

ts_status ts_hash_query(const void* table, int64_t cap, int ndim, const int32_t* q, int64_t m, int32_t* rows,
                        hipStream_t stream) {
  if (!table || m < 0 || m > kMaxRows || (m > 0 && (!q || !rows))) return TS_ERR_INVALID_ARG;
  if ((ndim != 2 && ndim != 3) || !is_pow2(cap) || cap > kMaxCap) return TS_ERR_INVALID_ARG;
  TS_TRY(launch_hash_query(table, cap, ndim, q, m, rows, stream));
  return TS_OK;
}

size_t ts_support_scratch_bytes(int64_t n_in) {
  return n_in < 0 || n_in > kMaxRows ? 0 : support_scratch_bytes(n_in);
}

ts_status ts_strided_support(const int32_t* in_coords, int64_t n_in, int ndim, int stride, int32_t* out_coords,
                             int64_t* n_out, void* out_table, int64_t out_cap, void* scratch, size_t scratch_bytes,
                             uint32_t* err_flags, hipStream_t stream) {
  if (n_in < 0 || n_in > kMaxRows || (n_in > 0 && (!in_coords || !out_coords)) || !n_out || !out_table)
    return TS_ERR_INVALID_ARG;
  if ((ndim != 2 && ndim != 3) || stride < 1 || stride > 65535) return TS_ERR_INVALID_ARG;
  if (!is_pow2(out_cap) || out_cap < n_in) return TS_ERR_INVALID_ARG;
  if (out_cap > kMaxCap) return TS_ERR_UNSUPPORTED;
  if (!scratch || scratch_bytes < support_scratch_bytes(n_in)) return TS_ERR_INVALID_ARG;
  TS_TRY(launch_strided_support(in_coords, n_in, ndim, stride, out_coords, n_out, out_table, out_cap, scratch,
                                err_flags, stream));
  return TS_OK;
}

size_t ts_generative_scratch_bytes(int64_t n_in, int ndim, int ksize) {
  if (n_in < 0 || n_in > kMaxRows || !shape_ok(ndim, ksize, 1)) return 0;
  const int64_t n_cand = n_in * ipow(ksize, ndim);  // kvol <= 64: no overflow
  return n_cand > kMaxRows ? 0 : generative_scratch_bytes(n_cand);
}

namespace {
// Shared checks and launch of the two generated supports (site = scale * c +
// sign * delta).
ts_status generated_support(const int32_t* in_coords, int64_t n_in, int ndim, int ksize, int stride, int scale,
                            int sign, int32_t* out_coords, int64_t n_out_cap, int64_t* n_out, void* out_table,
                            int64_t out_cap, void* scratch, size_t scratch_bytes, uint32_t* err_flags,
                            hipStream_t stream) {
  if (!shape_ok(ndim, ksize, stride)) return TS_ERR_INVALID_ARG;
  if (n_in < 0 || n_in > kMaxRows || (n_in > 0 && !in_coords) || !n_out || !out_table) return TS_ERR_INVALID_ARG;
  if (n_out_cap < 0 || n_out_cap > kMaxRows || (n_out_cap > 0 && !out_coords)) return TS_ERR_INVALID_ARG;
  if (n_in * ipow(ksize, ndim) > kMaxRows) return TS_ERR_UNSUPPORTED;
  if (!is_pow2(out_cap)) return TS_ERR_INVALID_ARG;
  if (out_cap > kMaxCap) return TS_ERR_UNSUPPORTED;
  if (!scratch || scratch_bytes < ts_generative_scratch_bytes(n_in, ndim, ksize)) return TS_ERR_INVALID_ARG;
  TS_TRY(launch_generative_support(in_coords, n_in, ndim, ksize, scale, sign, out_coords, n_out_cap, n_out, out_table,
                                   out_cap, scratch, err_flags, stream));
  return TS_OK;
}
}  // namespace

ts_status ts_generative_support(const int32_t* in_coords, int64_t n_in, int ndim, int ksize, int32_t* out_coords,
                                int64_t n_out_cap, int64_t* n_out, void* out_table, int64_t out_cap, void* scratch,
                                size_t scratch_bytes, uint32_t* err_flags, hipStream_t stream) {
  return generated_support(in_coords, n_in, ndim, ksize, 1, 1, -1, out_coords, n_out_cap, n_out, out_table, out_cap,
                           scratch, scratch_bytes, err_flags, stream);
}

ts_status ts_transposed_support(const int32_t* in_coords, int64_t n_in, int ndim, int ksize, int stride,
                                int32_t* out_coords, int64_t n_out_cap, int64_t* n_out, void* out_table,
                                int64_t out_cap, void* scratch, size_t scratch_bytes, uint32_t* err_flags,
                                hipStream_t stream) {
  if (stride < 1) return TS_ERR_INVALID_ARG;
  return generated_support(in_coords, n_in, ndim, ksize, stride, stride, 1, out_coords, n_out_cap, n_out, out_table,
                           out_cap, scratch, scratch_bytes, err_flags, stream);
}

size_t ts_voxelize_scratch_bytes(int64_t n_points) {
  return n_points < 0 || n_points > kMaxRows ? 0 : voxelize_scratch_bytes(n_points);
}

ts_status ts_voxelize(const int32_t* batch, const float* pos, int64_t n, int ndim, const float* size,
                      const float* origin, const float* feats, int c, int32_t* out_coords, int64_t* n_out,
                      void* out_table, int64_t out_cap, int32_t* vox_of, float* out_feats, void* scratch,
                      size_t scratch_bytes, uint32_t* err_flags, hipStream_t stream) {
  if (ndim != 2 && ndim != 3) return TS_ERR_INVALID_ARG;
  if (n < 0 || n > kMaxRows || !n_out || !out_table || !size || !origin) return TS_ERR_INVALID_ARG;
  if (n > 0 && (!pos || !out_coords || !vox_of)) return TS_ERR_INVALID_ARG;
  for (int d = 0; d < ndim; ++d)
    if (!(size[d] > 0.f) || !std::isfinite(size[d]) || !std::isfinite(origin[d])) return TS_ERR_INVALID_ARG;
  if (feats && (c < 1 || c > kMaxChannels || (n > 0 && !out_feats))) return TS_ERR_INVALID_ARG;
  if (!is_pow2(out_cap)) return TS_ERR_INVALID_ARG;
  if (out_cap > kMaxCap) return TS_ERR_UNSUPPORTED;
  if (!scratch || scratch_bytes < voxelize_scratch_bytes(n)) return TS_ERR_INVALID_ARG;
  TS_TRY(launch_voxelize(batch, pos, n, ndim, size, origin, feats, feats ? c : 0, out_coords, n_out, out_table,
                         out_cap, vox_of, out_feats, scratch, err_flags, stream));
  return TS_OK;
}

ts_status ts_devoxelize(const int32_t* vox_of, int64_t n, const void* vox_feats, int c, void* point_feats,
                        ts_dtype dtype, hipStream_t stream) {
  if (n < 0 || n > kMaxRows || c < 1 || c > kMaxChannels || !dtype_ok(dtype)) return TS_ERR_INVALID_ARG;
  if (n > 0 && (!vox_of || !vox_feats || !point_feats)) return TS_ERR_INVALID_ARG;
  TS_TRY(launch_devoxelize(vox_of, n, vox_feats, c, point_feats, dtype, stream));
  return TS_OK;
}

size_t ts_kmap_bytes(int64_t n_in, int64_t n_out_cap, int ndim, int ksize, int stride, uint32_t flags) {
  if (n_in < 0 || n_out_cap < 0 || n_in > kMaxRows || n_out_cap > kMaxRows || !shape_ok(ndim, ksize, stride)) return 0;
  const int kvol = ipow(ksize, ndim);
  if (n_out_cap * kvol > kMaxRows || n_in * kvol > kMaxRows) return 0;  // ts_kmap_build refuses these shapes
  ts_kmap tmp;
  return layout_kmap(nullptr, &tmp, n_in, n_out_cap, ndim, ksize, stride, flags);
}

ts_status ts_kmap_build(const int32_t* in_coords, int64_t n_in, const void* in_table, int64_t in_cap,
                        const int32_t* out_coords, int64_t n_out_cap, const int64_t* n_out, const void* out_table,
                        int64_t out_cap, int ndim, int ksize, int stride, uint32_t flags, void* buf,
                        size_t buf_bytes, ts_kmap* map, hipStream_t stream) {
  if (!map || !buf || !in_table) return TS_ERR_INVALID_ARG;
  if (!shape_ok(ndim, ksize, stride)) {
    if ((ndim == 2 || ndim == 3) && ksize >= 1 && stride >= 1) return TS_ERR_UNSUPPORTED;
    return TS_ERR_INVALID_ARG;
  }
  if (n_in < 0 || n_in > kMaxRows || (n_in > 0 && !in_coords) || !is_pow2(in_cap) || in_cap > kMaxCap)
    return TS_ERR_INVALID_ARG;
  if (flags & ~(TS_KMAP_PAIRS | TS_KMAP_BWD | TS_KMAP_NATURAL | TS_KMAP_TARGET | TS_KMAP_TRANSPOSED | TS_KMAP_GROUPS |
                TS_KMAP_NO_TABLE))
    return TS_ERR_INVALID_ARG;
  if ((flags & TS_KMAP_NO_TABLE) && !(flags & TS_KMAP_GROUPS)) return TS_ERR_INVALID_ARG;
  const int kvol = ipow(ksize, ndim);
  const bool target = (flags & TS_KMAP_TARGET) != 0;
  const bool transposed = (flags & TS_KMAP_TRANSPOSED) != 0;
  if (target && transposed) return TS_ERR_INVALID_ARG;
  const bool subm = stride == 1 && !target && !transposed;
  if (subm) {
    if (ksize % 2 == 0) return TS_ERR_UNSUPPORTED;  // submanifold needs a centred kernel
    out_coords = in_coords;
    n_out_cap = n_in;
  } else {
    if (n_out_cap < 0 || n_out_cap > kMaxRows || (n_out_cap > 0 && !out_coords) || !n_out) return TS_ERR_INVALID_ARG;
    if (((flags & TS_KMAP_BWD) || transposed) && (!out_table || !is_pow2(out_cap) || out_cap > kMaxCap))
      return TS_ERR_INVALID_ARG;
  }
  // Neighbour-table entries, pair-list positions and their scans are int32:
  // a map with more than 2^31 - 1 (row, offset) slots on either side, or a
  // pair capacity past that, is refused before anything is laid out.
  if (n_out_cap * kvol > kMaxRows || n_in * kvol > kMaxRows) return TS_ERR_UNSUPPORTED;
  if ((flags & TS_KMAP_PAIRS) && pair_capacity(n_in, n_out_cap, ndim, ksize, stride, flags) > kMaxRows)
    return TS_ERR_UNSUPPORTED;
  ts_kmap m;
  const size_t need = layout_kmap(static_cast<char*>(buf), &m, n_in, n_out_cap, ndim, ksize, stride, flags);
  if (buf_bytes < need) return TS_ERR_INVALID_ARG;
  const bool natural = (flags & TS_KMAP_NATURAL) != 0;

  RelBuild f;
  // targets and strided outputs take the inputs at s*q + delta (s = 1 for a
  // target map); only a submanifold output must also own its coordinate.  A
  // transposed map reads the strided relation the other way: fine output p
  // takes the coarse input at (p - delta)/s, and owns p in out_table.
  f.mode = subm ? kModeSubm : (transposed ? kModeUp : kModeDown);
  f.dest_coords = out_coords;
  f.n_dest_cap = n_out_cap;
  f.ndim = ndim;
  f.ksize = ksize;
  f.stride = stride;
  f.kvol = kvol;
  f.src_table = in_table;
  f.src_cap = in_cap;
  f.own_table = transposed ? out_table : nullptr;
  f.own_cap = transposed ? out_cap : 0;
  int64_t* n_out_fill = nullptr;
  if (subm) {
    n_out_fill = m.n_out;  // written by the map kernel: outputs = inputs
    f.n_dest = nullptr;
  } else {
    m.n_out = const_cast<int64_t*>(n_out);
    f.n_dest = n_out;
  }
  m.fwd.n_dest = m.n_out;
  TS_TRY(launch_rel_build(f, m.fwd, natural, n_out_fill, stream));

  if (!subm && (flags & TS_KMAP_BWD)) {
    RelBuild b = f;
    b.mode = transposed ? kModeDown : kModeUp;
    b.dest_coords = in_coords;
    b.n_dest_cap = n_in;
    b.n_dest = nullptr;
    b.src_table = out_table;
    b.src_cap = out_cap;
    b.own_table = transposed ? nullptr : in_table;
    b.own_cap = transposed ? 0 : in_cap;
    TS_TRY(launch_rel_build(b, m.bwd, natural, nullptr, stream));
  }
  if (flags & TS_KMAP_PAIRS)
    TS_TRY(launch_pairs_build(f, m.fwd, m.pair_cap, m.pair_start, m.pair_in, m.pair_out, m.scratch, stream));
  *map = m;
  return TS_OK;
}

size_t ts_conv_workspace_bytes(const ts_kmap* map, int cin, int cout, int op, ts_dtype in_dtype,
                               ts_dataflow dataflow) {
  if (!map || cin < 1 || cout < 1) return 0;
  switch (op) {
    case TS_OP_FWD: return conv_ws(map, cin, cout, in_dtype, TS_BF16, dataflow, map->n_out_cap, map->n_in);
    case TS_OP_DGRAD: return conv_ws(map, cout, cin, in_dtype, TS_BF16, dataflow, map->n_in, map->n_out_cap);
    case TS_OP_WGRAD: return wgrad_workspace_bytes(map, cin, cout);
    case TS_OP_TRANSPOSE: return conv_ws(map, cin, cout, in_dtype, TS_BF16, dataflow, map->n_in, map->n_out_cap);
  }
  return 0;
}

ts_status ts_conv_pack_weights(const ts_kmap* map, const void* w, int cin, int cout, int op, ts_dtype in_dtype,
                               void* ws, size_t ws_bytes, hipStream_t stream) {
  ts_status st = check_conv(map, cin, cout, in_dtype, in_dtype);
  if (st != TS_OK) return st;
  if (!w || !ws) return TS_ERR_INVALID_ARG;
  ConvArgs a;
  a.kvol = map->kvol;
  a.w = w;
  a.w_cin = cin;
  a.w_cout = cout;
  a.in_dtype = a.out_dtype = in_dtype;
  int64_t n_src = 0;
  switch (op) {
    case TS_OP_FWD:  // the forward contracts over cin, mirror-free
      a.c_src = cin, a.c_dst = cout, a.transpose = false, a.mirror = false, n_src = map->n_in;
      break;
    case TS_OP_DGRAD:  // contracts over cout; mirrored offsets on a submanifold map
      a.c_src = cout, a.c_dst = cin, a.transpose = true, a.mirror = map->mirror_bwd != 0, n_src = map->n_out_cap;
      break;
    case TS_OP_TRANSPOSE:  // the forward's weights over the dgrad relation
      a.c_src = cin, a.c_dst = cout, a.transpose = false, a.mirror = map->mirror_bwd != 0, n_src = map->n_out_cap;
      break;
    default:
      return TS_ERR_INVALID_ARG;
  }
  if (!igemm_supported(a.kvol, n_src, a.c_src, a.c_dst, in_dtype)) return TS_ERR_UNSUPPORTED;
  if (ws_bytes < igemm_workspace_bytes(a.kvol, a.c_src, a.c_dst)) return TS_ERR_INVALID_ARG;
  TS_TRY(launch_wpack(a, ws, stream));
  return TS_OK;
}

ts_status ts_conv_fwd(const ts_kmap* map, const void* x, int cin, const void* w, int cout, void* y,
                      ts_dtype in_dtype, ts_dtype out_dtype, ts_dataflow dataflow, void* ws, size_t ws_bytes,
                      hipStream_t stream) {
  ts_status st = check_conv(map, cin, cout, in_dtype, out_dtype);
  if (st != TS_OK) return st;
  if ((st = check_dataflow(dataflow, w)) != TS_OK) return st;
  if ((map->n_in > 0 && !x) || (map->n_out_cap > 0 && !y)) return TS_ERR_INVALID_ARG;
  const size_t need = conv_ws(map, cin, cout, in_dtype, out_dtype, dataflow, map->n_out_cap, map->n_in);
  if (need > 0 && (!ws || ws_bytes < need)) return TS_ERR_INVALID_ARG;
  ConvArgs a;
  a.rows_in_order = (map->flags & TS_KMAP_NATURAL) != 0;
  a.rel = &map->fwd;
  a.kvol = map->kvol;
  a.src = x;
  a.n_src = map->n_in;
  a.c_src = cin;
  a.dst = y;
  a.c_dst = cout;
  a.w = w;
  a.w_cin = cin;
  a.w_cout = cout;
  a.transpose = false;
  a.mirror = false;
  a.in_dtype = in_dtype;
  a.out_dtype = out_dtype;
  a.prepacked = dataflow == TS_DATAFLOW_IMPLICIT_GEMM_PACKED;
  if (dataflow == TS_DATAFLOW_GATHER_SCATTER) {
    if (!(map->flags & TS_KMAP_PAIRS)) return TS_ERR_INVALID_ARG;
    TS_TRY(launch_gather_scatter(map, a, false, map->n_out_cap, ws, stream));
    return TS_OK;
  }
  Kind kind;
  if ((st = pick_kernel(dataflow, map->fwd, map->kvol, map->n_in, cin, cout, in_dtype, x, &kind)) != TS_OK) return st;
  TS_TRY(run_kernel(kind, a, ws, stream));
  return TS_OK;
}

ts_status ts_subm_conv_fwd(const ts_kmap* map, const void* x, int cin, const void* w, int cout, void* y,
                           ts_dtype in_dtype, ts_dtype out_dtype, ts_dataflow dataflow, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  if (!map || map->stride != 1 || (map->flags & (TS_KMAP_TARGET | TS_KMAP_TRANSPOSED))) return TS_ERR_INVALID_ARG;
  return ts_conv_fwd(map, x, cin, w, cout, y, in_dtype, out_dtype, dataflow, ws, ws_bytes, stream);
}

ts_status ts_conv_fwd_strided(const int32_t* in_coords, int64_t n_in, int ndim, const void* in_table, int64_t in_cap,
                              int ksize, int stride, uint32_t kmap_flags, int32_t* out_coords, int64_t* n_out,
                              void* out_table, int64_t out_cap, uint32_t* err_flags, void* map_buf, size_t map_bytes,
                              ts_kmap* map, const void* x, int cin, const void* w, int cout, void* y,
                              ts_dtype in_dtype, ts_dtype out_dtype, ts_dataflow dataflow, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  if (stride < 2 || !map_buf || !map) return TS_ERR_INVALID_ARG;
  if (!shape_ok(ndim, ksize, stride)) return TS_ERR_INVALID_ARG;
  if (n_in < 0 || n_in > kMaxRows) return TS_ERR_INVALID_ARG;
  const size_t kb = ts_kmap_bytes(n_in, n_in, ndim, ksize, stride, kmap_flags);
  const size_t sb = support_scratch_bytes(n_in);
  if (kb == 0 || map_bytes < kb + sb) return TS_ERR_INVALID_ARG;
  // validate the convolution arguments before launching anything
  {
    const int kvol = ipow(ksize, ndim);
    if (cin < 1 || cout < 1 || cin > kMaxChannels || cout > kMaxChannels || !w) return TS_ERR_INVALID_ARG;
    if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return TS_ERR_INVALID_ARG;
    if (out_dtype != TS_F32 && out_dtype != in_dtype) return TS_ERR_UNSUPPORTED;
    if (n_in > 0 && (!x || !y)) return TS_ERR_INVALID_ARG;
    if (dataflow == TS_DATAFLOW_GATHER_SCATTER && !(kmap_flags & TS_KMAP_PAIRS)) return TS_ERR_INVALID_ARG;
    ts_kmap probe;
    layout_kmap(nullptr, &probe, n_in, n_in, ndim, ksize, stride, kmap_flags);
    const size_t need = conv_ws(&probe, cin, cout, in_dtype, out_dtype, dataflow, n_in, n_in);
    if (need > 0 && (!ws || ws_bytes < need)) return TS_ERR_INVALID_ARG;
    (void)kvol;
  }
  void* scratch = static_cast<char*>(map_buf) + kb;
  ts_status st = ts_strided_support(in_coords, n_in, ndim, stride, out_coords, n_out, out_table, out_cap, scratch, sb,
                                    err_flags, stream);
  if (st != TS_OK) return st;
  st = ts_kmap_build(in_coords, n_in, in_table, in_cap, out_coords, n_in, n_out, out_table, out_cap, ndim, ksize,
                     stride, kmap_flags, map_buf, kb, map, stream);
  if (st != TS_OK) return st;
  return ts_conv_fwd(map, x, cin, w, cout, y, in_dtype, out_dtype, dataflow, ws, ws_bytes, stream);
}

ts_status ts_conv_fwd_generative(const int32_t* in_coords, int64_t n_in, int ndim, const void* in_table,
                                 int64_t in_cap, int ksize, uint32_t kmap_flags, int32_t* out_coords,
                                 int64_t n_out_cap, int64_t* n_out, void* out_table, int64_t out_cap,
                                 uint32_t* err_flags, void* map_buf, size_t map_bytes, ts_kmap* map, const void* x,
                                 int cin, const void* w, int cout, void* y, ts_dtype in_dtype, ts_dtype out_dtype,
                                 ts_dataflow dataflow, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!map_buf || !map) return TS_ERR_INVALID_ARG;
  if (!shape_ok(ndim, ksize, 1)) return TS_ERR_INVALID_ARG;
  if (n_in < 0 || n_in > kMaxRows || n_out_cap < 0 || n_out_cap > kMaxRows) return TS_ERR_INVALID_ARG;
  const uint32_t flags = kmap_flags | TS_KMAP_TARGET;
  const size_t kb = ts_kmap_bytes(n_in, n_out_cap, ndim, ksize, 1, flags);
  const size_t sb = ts_generative_scratch_bytes(n_in, ndim, ksize);
  if (kb == 0 || map_bytes < kb + sb) return TS_ERR_INVALID_ARG;
  // validate the convolution arguments before launching anything
  if (cin < 1 || cout < 1 || cin > kMaxChannels || cout > kMaxChannels || !w) return TS_ERR_INVALID_ARG;
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return TS_ERR_INVALID_ARG;
  if (out_dtype != TS_F32 && out_dtype != in_dtype) return TS_ERR_UNSUPPORTED;
  if ((n_in > 0 && !x) || (n_out_cap > 0 && !y)) return TS_ERR_INVALID_ARG;
  if (dataflow == TS_DATAFLOW_GATHER_SCATTER && !(flags & TS_KMAP_PAIRS)) return TS_ERR_INVALID_ARG;
  {
    ts_kmap probe;
    layout_kmap(nullptr, &probe, n_in, n_out_cap, ndim, ksize, 1, flags);
    const size_t need = conv_ws(&probe, cin, cout, in_dtype, out_dtype, dataflow, n_out_cap, n_in);
    if (need > 0 && (!ws || ws_bytes < need)) return TS_ERR_INVALID_ARG;
  }
  void* scratch = static_cast<char*>(map_buf) + kb;
  ts_status st = ts_generative_support(in_coords, n_in, ndim, ksize, out_coords, n_out_cap, n_out, out_table, out_cap,
                                       scratch, sb, err_flags, stream);
  if (st != TS_OK) return st;
  st = ts_kmap_build(in_coords, n_in, in_table, in_cap, out_coords, n_out_cap, n_out, out_table, out_cap, ndim, ksize,
                     1, flags, map_buf, kb, map, stream);
  if (st != TS_OK) return st;
  return ts_conv_fwd(map, x, cin, w, cout, y, in_dtype, out_dtype, dataflow, ws, ws_bytes, stream);
}

ts_status ts_conv_bwd_dgrad(const ts_kmap* map, const void* dy, int cout, const void* w, int cin, void* dx,
                            ts_dtype in_dtype, ts_dtype out_dtype, ts_dataflow dataflow, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  ts_status st = check_conv(map, cin, cout, in_dtype, out_dtype);
  if (st != TS_OK) return st;
  if ((st = check_dataflow(dataflow, w)) != TS_OK) return st;
  if ((map->n_out_cap > 0 && !dy) || (map->n_in > 0 && !dx)) return TS_ERR_INVALID_ARG;
  const size_t need = conv_ws(map, cout, cin, in_dtype, out_dtype, dataflow, map->n_in, map->n_out_cap);
  if (need > 0 && (!ws || ws_bytes < need)) return TS_ERR_INVALID_ARG;
  ConvArgs a;
  a.rows_in_order = (map->flags & TS_KMAP_NATURAL) != 0;
  a.kvol = map->kvol;
  a.src = dy;
  a.n_src = map->n_out_cap;
  a.c_src = cout;
  a.dst = dx;
  a.c_dst = cin;
  a.w = w;
  a.w_cin = cin;
  a.w_cout = cout;
  a.transpose = true;
  a.in_dtype = in_dtype;
  a.out_dtype = out_dtype;
  a.prepacked = dataflow == TS_DATAFLOW_IMPLICIT_GEMM_PACKED;
  if (dataflow == TS_DATAFLOW_GATHER_SCATTER) {
    if (!(map->flags & TS_KMAP_PAIRS)) return TS_ERR_INVALID_ARG;
    a.rel = &map->fwd;
    a.mirror = false;
    TS_TRY(launch_gather_scatter(map, a, true, map->n_in, ws, stream));
    return TS_OK;
  }
  if (map->mirror_bwd) {
    a.rel = &map->fwd;
    a.mirror = true;
  } else {
    if (!(map->flags & TS_KMAP_BWD) || !map->bwd.row_mask) return TS_ERR_INVALID_ARG;
    a.rel = &map->bwd;
    a.mirror = false;
  }
  Kind kind;
  if ((st = pick_kernel(dataflow, *a.rel, map->kvol, map->n_out_cap, cout, cin, in_dtype, dy, &kind)) != TS_OK) return st;
  TS_TRY(run_kernel(kind, a, ws, stream));
  return TS_OK;
}

ts_status ts_conv_transpose_fwd(const ts_kmap* map, const void* x, int cin, const void* w, int cout, void* y,
                                ts_dtype in_dtype, ts_dtype out_dtype, ts_dataflow dataflow, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
  ts_status st = check_conv(map, cin, cout, in_dtype, out_dtype);
  if (st != TS_OK) return st;
  if ((st = check_dataflow(dataflow, w)) != TS_OK) return st;
  if ((map->n_out_cap > 0 && !x) || (map->n_in > 0 && !y)) return TS_ERR_INVALID_ARG;
  const size_t need = conv_ws(map, cin, cout, in_dtype, out_dtype, dataflow, map->n_in, map->n_out_cap);
  if (need > 0 && (!ws || ws_bytes < need)) return TS_ERR_INVALID_ARG;
  // the relation of dgrad, the weights as the forward reads them
  ConvArgs a;
  a.rows_in_order = (map->flags & TS_KMAP_NATURAL) != 0;
  a.kvol = map->kvol;
  a.src = x;
  a.n_src = map->n_out_cap;
  a.c_src = cin;
  a.dst = y;
  a.c_dst = cout;
  a.w = w;
  a.w_cin = cin;
  a.w_cout = cout;
  a.transpose = false;
  a.in_dtype = in_dtype;
  a.out_dtype = out_dtype;
  a.prepacked = dataflow == TS_DATAFLOW_IMPLICIT_GEMM_PACKED;
  if (dataflow == TS_DATAFLOW_GATHER_SCATTER) {
    if (!(map->flags & TS_KMAP_PAIRS)) return TS_ERR_INVALID_ARG;
    a.rel = &map->fwd;
    a.mirror = false;
    TS_TRY(launch_gather_scatter(map, a, true, map->n_in, ws, stream));
    return TS_OK;
  }
  if (map->mirror_bwd) {
    a.rel = &map->fwd;
    a.mirror = true;
  } else {
    if (!(map->flags & TS_KMAP_BWD) || !map->bwd.row_mask) return TS_ERR_INVALID_ARG;
    a.rel = &map->bwd;
    a.mirror = false;
  }
  Kind kind;
  if ((st = pick_kernel(dataflow, *a.rel, map->kvol, map->n_out_cap, cin, cout, in_dtype, x, &kind)) != TS_OK) return st;
  TS_TRY(run_kernel(kind, a, ws, stream));
  return TS_OK;
}

ts_status ts_pool_fwd(const ts_kmap* map, const void* x, int c, void* y, ts_dtype in_dtype, ts_dtype out_dtype,
                      int mode, hipStream_t stream) {
  if (!map || map->kvol < 1 || map->kvol > TS_MAX_KVOL || !map->fwd.tile_mask) return TS_ERR_INVALID_ARG;
  if (c < 1 || c > kMaxChannels || (mode != TS_POOL_MAX && mode != TS_POOL_AVG)) return TS_ERR_INVALID_ARG;
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return TS_ERR_INVALID_ARG;
  if (out_dtype != TS_F32 && out_dtype != in_dtype) return TS_ERR_UNSUPPORTED;
  if ((map->n_in > 0 && !x) || (map->n_out_cap > 0 && !y)) return TS_ERR_INVALID_ARG;
  TS_TRY(launch_pool(map->fwd, map->kvol, x, map->n_in, c, y, in_dtype, out_dtype, mode, stream));
  return TS_OK;
}

ts_status ts_graph_conv_fwd(const int64_t* indptr, const int32_t* src, const int32_t* rel, int64_t n_dst,
                            int64_t n_src, int n_rel, const void* x, int cin, const void* w, int cout, void* y,
                            ts_dtype in_dtype, ts_dtype out_dtype, uint32_t* err_flags, hipStream_t stream) {
  if (n_dst < 0 || n_dst > kMaxRows || n_src < 0 || n_src > kMaxRows || n_rel < 1) return TS_ERR_INVALID_ARG;
  if (cin < 1 || cout < 1 || cin > kMaxChannels || cout > kMaxChannels) return TS_ERR_INVALID_ARG;
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return TS_ERR_INVALID_ARG;
  if (out_dtype != TS_F32 && out_dtype != in_dtype) return TS_ERR_UNSUPPORTED;
  if (n_dst > 0 && (!indptr || !src || !rel || !w || !y)) return TS_ERR_INVALID_ARG;
  if (n_dst > 0 && n_src > 0 && !x) return TS_ERR_INVALID_ARG;
  TS_TRY(launch_graph_conv(indptr, src, rel, n_dst, n_src, n_rel, x, cin, w, cout, y, in_dtype, out_dtype, err_flags,
                           stream));
  return TS_OK;
}

ts_status ts_conv_bwd_wgrad(const ts_kmap* map, const void* x, int cin, const void* dy, int cout, ts_dtype in_dtype,
                            float* dw, void* ws, size_t ws_bytes, hipStream_t stream) {
  ts_status st = check_conv(map, cin, cout, in_dtype, TS_F32);
  if (st != TS_OK) return st;
  if (!(map->flags & TS_KMAP_PAIRS) || !dw || (map->n_in > 0 && !x) || (map->n_out_cap > 0 && !dy))
    return TS_ERR_INVALID_ARG;
  if (!ws || ws_bytes < wgrad_workspace_bytes(map, cin, cout)) return TS_ERR_INVALID_ARG;
  TS_TRY(launch_wgrad(map, x, cin, dy, cout, in_dtype, dw, ws, stream));
  return TS_OK;
}

}  // extern "C"
