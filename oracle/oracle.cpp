// CPU oracle for sparse convolution over coordinate/feature sparse tensors.
//
// TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct
// reference that the GPU library is checked against.  Only the test suite,
// the smoke check and the benchmark's CPU-baseline leg load it; the product
// path never does.  It shares no code, header, table or constant with the GPU
// library.
//
// What it computes (torch-lattice "Migrating from TorchSparse" page, sections
// "Sparse tensor expectations", "Convolution mapping" and "Backend and
// configuration differences"):
//   * a sparse tensor is integer coordinate rows (batch, x, y[, z]) with one
//     dense feature row per coordinate row; the batch id lives in column 0;
//   * SubmConv3d keeps the input coordinate set as the output set;
//   * a strided Conv3d creates a downsampled output set;
//   * a stride-1 Conv3d with a kernel wider than one cell generates its output
//     set (section "What is intentionally different", row on convolution
//     intent);
//   * TargetConv3d computes at output coordinates the caller gives (same
//     table, and the "Convolution mapping" table);
//   * a transposed convolution either reuses an existing relation
//     (ConvTranspose3d) or generates its output support
//     (GenerativeConvTranspose3d) ("Convolution mapping" table);
//   * pooling runs over the same kernel maps as convolution (torch-lattice
//     "What remains familiar": CUDA kernels cover pooling);
//   * voxelization turns points into a sparse tensor and devoxelization
//     carries voxel features back to the points (same list);
//   * graph convolution (TorchSparse++ abstract: the library also runs graph
//     convolutions): a relational sum over incoming edges, of which sparse
//     convolution is the case "edges = map triples, relations = offsets";
//   * every dataflow must give the same result for a fixed relation
//     (input row, output row, kernel offset) and weight tensor.
//
// Readings taken where the pages are silent (all of them are also listed in
// the design notes):
//   * key = the full coordinate tuple; a repeated coordinate keeps the
//     lowest row and raises the DUP flag;
//   * batch must lie in [0, 65534] and every spatial value in
//     [-32768, 32767]; a row outside is not inserted and raises RANGE;
//   * a row that is out of range, or repeats the coordinate of a lower row,
//     takes no part in the convolution: it is never found as a neighbour
//     and, as a submanifold output row, it has no neighbours (zero output);
//   * kernel offsets delta_d in {-r, ..., K-1-r} with r = (K-1)/2, enumerated
//     with the first spatial axis slowest; no cross-batch neighbours;
//   * submanifold: output row j reads input q_j + delta;
//     strided: outputs are unique(floor(c/s)) in first-occurrence order and
//     output j reads input s*q_j + delta;
//     target: output row j (any caller coordinate, repeats allowed) reads
//     input s*q_j + delta, s = 1 included, with no ownership condition;
//     generative stride 1: outputs are every q = c_i - delta (the sites some
//     input reaches), in first-occurrence order over (i, then offset), and
//     are then used as targets;
//     transposed: the relation of a stride-s convolution read the other way
//     (fine output p takes coarse input q where p = s*q + delta); its
//     generated support is every s*c_j + delta, first occurrence over
//     (j, then offset); the contraction over it is the forward formula;
//   * cross-correlation (no kernel flip), W laid out [offset][cin][cout];
//   * all arithmetic in fp64.
//
// Parity pins: tests/test_oracle_*.py check every function here against dense
// convolution (torch CPU, fp64), brute-force searches, closed forms and the
// page's two-voxel example.
#include <algorithm>
#include <array>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <unordered_map>
#include <vector>

namespace {

using Key = std::array<int64_t, 4>;

struct KeyHash {
  size_t operator()(const Key& k) const {
    size_t h = 1469598103934665603ull;
    for (int64_t v : k) {
      h ^= static_cast<size_t>(v) + 0x9e3779b97f4a7c15ull + (h << 6) + (h >> 2);
    }
    return h;
  }
};

using Map = std::unordered_map<Key, int64_t, KeyHash>;

const uint32_t FLAG_DUP = 1u, FLAG_RANGE = 2u;

bool in_range(const int32_t* row, int ndim) {
  if (row[0] < 0 || row[0] > 65534) return false;
  for (int d = 1; d <= ndim; ++d)
    if (row[d] < -32768 || row[d] > 32767) return false;
  return true;
}

Key key_of(const int32_t* row, int ndim) {
  Key k{0, 0, 0, 0};
  for (int d = 0; d <= ndim; ++d) k[d] = row[d];
  return k;
}

// Insert rows in index order; first insertion of a coordinate wins.
Map build_map(const int32_t* coords, int64_t n, int ndim, uint32_t* flags) {
  Map m;
  m.reserve(static_cast<size_t>(n) * 2 + 1);
  for (int64_t i = 0; i < n; ++i) {
    const int32_t* row = coords + i * (ndim + 1);
    if (!in_range(row, ndim)) {
      if (flags) *flags |= FLAG_RANGE;
      continue;
    }
    auto ins = m.emplace(key_of(row, ndim), i);
    if (!ins.second && flags) *flags |= FLAG_DUP;
  }
  return m;
}

int64_t lookup(const Map& m, const Key& k) {
  auto it = m.find(k);
  return it == m.end() ? -1 : it->second;
}

int64_t floor_div(int64_t a, int64_t b) {
  int64_t q = a / b;
  if ((a % b != 0) && ((a < 0) != (b < 0))) --q;
  return q;
}

// Offset o -> spatial displacement, first spatial axis slowest.
void offset_delta(int o, int ndim, int ksize, int64_t* delta) {
  const int r = (ksize - 1) / 2;
  for (int d = ndim - 1; d >= 0; --d) {
    delta[d] = (o % ksize) - r;
    o /= ksize;
  }
}

int ipow(int b, int e) {
  int v = 1;
  for (int i = 0; i < e; ++i) v *= b;
  return v;
}

}  // namespace

extern "C" {

// Key -> row lookup of every query row (batch, spatial...) after inserting
// `coords` in row order.  rows[i] = owning input row or -1.  Returns 0.
int64_t oracle_hash_query(const int32_t* coords, int64_t n, int ndim, const int32_t* q, int64_t m,
                          int32_t* rows, uint32_t* flags) {
  uint32_t f = 0;
  Map map = build_map(coords, n, ndim, &f);
  for (int64_t i = 0; i < m; ++i) {
    const int32_t* row = q + i * (ndim + 1);
    rows[i] = static_cast<int32_t>(lookup(map, key_of(row, ndim)));
  }
  if (flags) *flags = f;
  return 0;
}

// Downsampled output coordinates of a stride-s convolution: for each input
// row in order, (b, floor(x/s), ...) appended when first seen.  Rows outside
// the coordinate range take no part.  Returns the number of output rows.
int64_t oracle_strided_support(const int32_t* coords, int64_t n, int ndim, int stride,
                               int32_t* out_coords) {
  Map seen;
  int64_t n_out = 0;
  for (int64_t i = 0; i < n; ++i) {
    const int32_t* row = coords + i * (ndim + 1);
    if (!in_range(row, ndim)) continue;
    Key k{0, 0, 0, 0};
    k[0] = row[0];
    for (int d = 1; d <= ndim; ++d) k[d] = floor_div(row[d], stride);
    if (seen.emplace(k, n_out).second) {
      for (int d = 0; d <= ndim; ++d) out_coords[n_out * (ndim + 1) + d] = static_cast<int32_t>(k[d]);
      ++n_out;
    }
  }
  return n_out;
}

// Generated output set of a stride-1 convolution: for each input row i in
// order that owns its coordinate, and each offset o in order, the site
// q = c_i - delta_o (the output whose window holds c_i at offset o) is
// appended when first seen; a site outside the coordinate range is skipped.
// Writes up to `cap` rows and returns how many sites exist.
int64_t oracle_generative_support(const int32_t* coords, int64_t n, int ndim, int ksize, int32_t* out_coords,
                                  int64_t cap) {
  Map owner = build_map(coords, n, ndim, nullptr);
  Map seen;
  const int kvol = ipow(ksize, ndim);
  int64_t n_out = 0;
  int64_t delta[3];
  for (int64_t i = 0; i < n; ++i) {
    const int32_t* row = coords + i * (ndim + 1);
    if (!in_range(row, ndim) || lookup(owner, key_of(row, ndim)) != i) continue;
    for (int o = 0; o < kvol; ++o) {
      offset_delta(o, ndim, ksize, delta);
      int32_t q[4] = {row[0], 0, 0, 0};
      bool ok = true;
      for (int d = 0; d < ndim; ++d) {
        const int64_t v = static_cast<int64_t>(row[d + 1]) - delta[d];
        if (v < -32768 || v > 32767) ok = false;
        q[d + 1] = static_cast<int32_t>(v);
      }
      if (!ok) continue;
      if (seen.emplace(key_of(q, ndim), n_out).second) {
        if (n_out < cap)
          for (int d = 0; d <= ndim; ++d) out_coords[n_out * (ndim + 1) + d] = q[d];
        ++n_out;
      }
    }
  }
  return n_out;
}

// Generated output set of a transposed convolution of stride s: for each input
// row j in order that owns its coordinate, and each offset o in order, the
// site s*c_j + delta_o is appended when first seen; a site outside the
// coordinate range is skipped.  Writes up to `cap` rows and returns how many
// sites exist.
int64_t oracle_transposed_support(const int32_t* coords, int64_t n, int ndim, int ksize, int stride,
                                  int32_t* out_coords, int64_t cap) {
  Map owner = build_map(coords, n, ndim, nullptr);
  Map seen;
  const int kvol = ipow(ksize, ndim);
  int64_t n_out = 0;
  int64_t delta[3];
  for (int64_t j = 0; j < n; ++j) {
    const int32_t* row = coords + j * (ndim + 1);
    if (!in_range(row, ndim) || lookup(owner, key_of(row, ndim)) != j) continue;
    for (int o = 0; o < kvol; ++o) {
      offset_delta(o, ndim, ksize, delta);
      int32_t p[4] = {row[0], 0, 0, 0};
      bool ok = true;
      for (int d = 0; d < ndim; ++d) {
        const int64_t v = static_cast<int64_t>(stride) * row[d + 1] + delta[d];
        if (v < -32768 || v > 32767) ok = false;
        p[d + 1] = static_cast<int32_t>(v);
      }
      if (!ok) continue;
      if (seen.emplace(key_of(p, ndim), n_out).second) {
        if (n_out < cap)
          for (int d = 0; d <= ndim; ++d) out_coords[n_out * (ndim + 1) + d] = p[d];
        ++n_out;
      }
    }
  }
  return n_out;
}

// Transposed kernel map: for every fine output row j (in order) that owns its
// coordinate among the outputs, and every offset o (in order), the coarse
// input row i with s*q_i + delta_o = p_j, when p_j - delta_o is divisible by
// s on every axis and that coarse site exists.  Triples (in = coarse row,
// out = fine row, offset); returns how many exist (writes up to `cap`).
int64_t oracle_kmap_transposed(const int32_t* in_coords, int64_t n_in, const int32_t* out_coords, int64_t n_out,
                               int ndim, int ksize, int stride, int32_t* t_in, int32_t* t_out, int32_t* t_off,
                               int64_t cap) {
  Map coarse = build_map(in_coords, n_in, ndim, nullptr);
  Map fine = build_map(out_coords, n_out, ndim, nullptr);
  const int kvol = ipow(ksize, ndim);
  int64_t count = 0;
  int64_t delta[3];
  for (int64_t j = 0; j < n_out; ++j) {
    const int32_t* p = out_coords + j * (ndim + 1);
    if (!in_range(p, ndim) || lookup(fine, key_of(p, ndim)) != j) continue;
    for (int o = 0; o < kvol; ++o) {
      offset_delta(o, ndim, ksize, delta);
      Key q{0, 0, 0, 0};
      q[0] = p[0];
      bool whole = true;
      for (int d = 0; d < ndim; ++d) {
        const int64_t t = static_cast<int64_t>(p[d + 1]) - delta[d];
        if (t % stride != 0) whole = false;
        q[d + 1] = floor_div(t, stride);
      }
      if (!whole) continue;
      const int64_t i = lookup(coarse, q);
      if (i < 0) continue;
      if (count < cap) {
        t_in[count] = static_cast<int32_t>(i);
        t_out[count] = static_cast<int32_t>(j);
        t_off[count] = o;
      }
      ++count;
    }
  }
  return count;
}

// Kernel map: for every output row j (in order) and offset o (in order), the
// input row i at s*q_j + delta_o (s = 1: q_j + delta_o) if it exists.  With
// `target` == 0 and s = 1 the outputs are the inputs themselves (submanifold)
// and a row takes part only if it owns its coordinate; with `target` != 0
// every in-range output row takes part.  Writes up to `cap` triples
// (in, out, offset) and returns how many exist.
int64_t oracle_kmap(const int32_t* in_coords, int64_t n_in, const int32_t* out_coords, int64_t n_out,
                    int ndim, int ksize, int stride, int target, int32_t* t_in, int32_t* t_out,
                    int32_t* t_off, int64_t cap) {
  Map map = build_map(in_coords, n_in, ndim, nullptr);
  const int kvol = ipow(ksize, ndim);
  int64_t count = 0;
  int64_t delta[3];
  for (int64_t j = 0; j < n_out; ++j) {
    const int32_t* q = out_coords + j * (ndim + 1);
    if (!in_range(q, ndim)) continue;
    // submanifold outputs are the input rows: only the owner of a coordinate
    // takes part
    if (stride == 1 && !target && lookup(map, key_of(q, ndim)) != j) continue;
    for (int o = 0; o < kvol; ++o) {
      offset_delta(o, ndim, ksize, delta);
      Key p{0, 0, 0, 0};
      p[0] = q[0];
      for (int d = 0; d < ndim; ++d) p[d + 1] = static_cast<int64_t>(stride) * q[d + 1] + delta[d];
      const int64_t i = lookup(map, p);
      if (i < 0) continue;
      if (count < cap) {
        t_in[count] = static_cast<int32_t>(i);
        t_out[count] = static_cast<int32_t>(j);
        t_off[count] = o;
      }
      ++count;
    }
  }
  return count;
}

// y[j][co] = sum over triples (i, j, o) and ci of x[i][ci] * w[o][ci][co].
void oracle_conv_fwd(const int32_t* t_in, const int32_t* t_out, const int32_t* t_off, int64_t n_pairs,
                     const double* x, int cin, const double* w, int cout, double* y, int64_t n_out) {
  std::fill_n(y, static_cast<size_t>(n_out) * cout, 0.0);
  for (int64_t p = 0; p < n_pairs; ++p) {
    const double* xi = x + static_cast<int64_t>(t_in[p]) * cin;
    const double* wo = w + static_cast<int64_t>(t_off[p]) * cin * cout;
    double* yj = y + static_cast<int64_t>(t_out[p]) * cout;
    for (int ci = 0; ci < cin; ++ci)
      for (int co = 0; co < cout; ++co) yj[co] += xi[ci] * wo[ci * cout + co];
  }
}

// dx[i][ci] = sum over triples (i, j, o) and co of dy[j][co] * w[o][ci][co].
void oracle_conv_dgrad(const int32_t* t_in, const int32_t* t_out, const int32_t* t_off, int64_t n_pairs,
                       const double* dy, int cout, const double* w, int cin, double* dx, int64_t n_in) {
  std::fill_n(dx, static_cast<size_t>(n_in) * cin, 0.0);
  for (int64_t p = 0; p < n_pairs; ++p) {
    const double* g = dy + static_cast<int64_t>(t_out[p]) * cout;
    const double* wo = w + static_cast<int64_t>(t_off[p]) * cin * cout;
    double* d = dx + static_cast<int64_t>(t_in[p]) * cin;
    for (int ci = 0; ci < cin; ++ci)
      for (int co = 0; co < cout; ++co) d[ci] += g[co] * wo[ci * cout + co];
  }
}

// Pooling over a relation: y[j][c] = the maximum (mode 0) or the mean
// (mode 1) of x[i][c] over the triples (i, j, o) of output row j -- over the
// inputs present in its window, not over K^D -- and 0 for an output with
// none.
void oracle_pool(const int32_t* t_in, const int32_t* t_out, int64_t n_pairs, const double* x, int c, int mode,
                 double* y, int64_t n_out) {
  std::vector<int64_t> count(static_cast<size_t>(n_out), 0);
  for (int64_t k = 0; k < n_out * c; ++k) y[k] = 0.0;
  for (int64_t p = 0; p < n_pairs; ++p) {
    const double* xi = x + static_cast<int64_t>(t_in[p]) * c;
    double* yj = y + static_cast<int64_t>(t_out[p]) * c;
    const bool first = count[t_out[p]]++ == 0;
    for (int ch = 0; ch < c; ++ch) {
      if (mode == 0) yj[ch] = first ? xi[ch] : (xi[ch] > yj[ch] ? xi[ch] : yj[ch]);
      else yj[ch] += xi[ch];
    }
  }
  if (mode == 1)
    for (int64_t j = 0; j < n_out; ++j)
      if (count[j] > 0)
        for (int ch = 0; ch < c; ++ch) y[j * c + ch] /= static_cast<double>(count[j]);
}

// Voxelization of points (batch b_i, position p_i in float32): voxel
// coordinate v_i = floor((p_i - origin) / size) per axis, computed in float32
// exactly as written (one rounded subtraction, one rounded division), then
// floored.  Voxels are numbered in order of first occurrence over the points;
// a point whose voxel leaves the coordinate range (or whose batch is out of
// range) is dropped (voxel -1).  Voxel features are the mean of the features
// of their points.  Writes out_coords (up to n rows), vox_of[n], feats
// [n][c] (the first n_vox rows) and returns n_vox.
int64_t oracle_voxelize(const int32_t* batch, const float* pos, int64_t n, int ndim, const float* size,
                        const float* origin, const double* f, int c, int32_t* out_coords, int32_t* vox_of,
                        double* feats) {
  Map seen;
  int64_t n_vox = 0;
  std::vector<int64_t> count;
  for (int64_t i = 0; i < n; ++i) {
    int32_t q[4] = {batch ? batch[i] : 0, 0, 0, 0};
    for (int d = 0; d < ndim; ++d) {
      const float rel = pos[i * ndim + d] - origin[d];
      const float v = std::floor(rel / size[d]);
      q[d + 1] = (v >= -32768.0f && v <= 32767.0f) ? static_cast<int32_t>(v) : 40000;
    }
    if (!in_range(q, ndim)) {
      vox_of[i] = -1;
      continue;
    }
    auto ins = seen.emplace(key_of(q, ndim), n_vox);
    if (ins.second) {
      for (int d = 0; d <= ndim; ++d) out_coords[n_vox * (ndim + 1) + d] = q[d];
      for (int ch = 0; ch < c; ++ch) feats[n_vox * c + ch] = 0.0;
      count.push_back(0);
      ++n_vox;
    }
    const int64_t j = ins.first->second;
    vox_of[i] = static_cast<int32_t>(j);
    ++count[j];
    for (int ch = 0; ch < c; ++ch) feats[j * c + ch] += f[i * c + ch];
  }
  for (int64_t j = 0; j < n_vox; ++j)
    for (int ch = 0; ch < c; ++ch) feats[j * c + ch] /= static_cast<double>(count[j]);
  return n_vox;
}

// Graph convolution over edges grouped by destination (CSR): for destination
// v, edges e in [indptr[v], indptr[v+1]) carry source src[e] and relation
// rel[e], and y[v][co] = sum over them of sum_ci x[src[e]][ci] *
// w[rel[e]][ci][co] (no normalisation; 0 for a node without edges).
void oracle_graph_conv(const int64_t* indptr, const int32_t* src, const int32_t* rel, int64_t n_dst,
                       const double* x, int cin, const double* w, int cout, double* y) {
  for (int64_t v = 0; v < n_dst; ++v) {
    double* yv = y + v * cout;
    for (int co = 0; co < cout; ++co) yv[co] = 0.0;
    for (int64_t e = indptr[v]; e < indptr[v + 1]; ++e) {
      const double* xs = x + static_cast<int64_t>(src[e]) * cin;
      const double* wr = w + static_cast<int64_t>(rel[e]) * cin * cout;
      for (int ci = 0; ci < cin; ++ci)
        for (int co = 0; co < cout; ++co) yv[co] += xs[ci] * wr[ci * cout + co];
    }
  }
}

// dw[o][ci][co] = sum over triples (i, j, o) of x[i][ci] * dy[j][co].
void oracle_conv_wgrad(const int32_t* t_in, const int32_t* t_out, const int32_t* t_off, int64_t n_pairs,
                       const double* x, int cin, const double* dy, int cout, double* dw, int kvol) {
  std::fill_n(dw, static_cast<size_t>(kvol) * cin * cout, 0.0);
  for (int64_t p = 0; p < n_pairs; ++p) {
    const double* xi = x + static_cast<int64_t>(t_in[p]) * cin;
    const double* g = dy + static_cast<int64_t>(t_out[p]) * cout;
    double* d = dw + static_cast<int64_t>(t_off[p]) * cin * cout;
    for (int ci = 0; ci < cin; ++ci)
      for (int co = 0; co < cout; ++co) d[ci * cout + co] += xi[ci] * g[co];
  }
}

}  // extern "C"
