// Coordinate hash table (build / query) and the downsampled support of a
// strided convolution.  The torch-lattice page "Migrating from TorchSparse"
// lists hashing and coordinate query among the library's kernels (section
// "What remains familiar") and says a strided convolution creates a
// downsampled support (section "Convolution mapping").
//
// Stored encodings (slots hold NOT key, cells NOT row) make an all-zero
// buffer an empty table.  A table buffer starts zero-filled and every build
// returns it to that state before filling it:
//   1. clear: each slot the previous build occupied gets its 64 cells and its
//      key zeroed (slots never occupied are zero already);
//   2. insert: each voxel claims the slot of its block (CAS of the zero key,
//      linear probing) unless the previous lane holds a voxel of the same
//      block, in which case it takes that lane's slot; then it atomicMax's
//      NOT row into its cell, so a repeated coordinate keeps the lowest row
//      (and raises TS_FLAG_DUP).
// Cells are zero before any insert starts (a kernel boundary apart), so a
// claim needs no reset and no insert can be overwritten.
#include "common.h"
#include "launch.h"

namespace ts {

// One lane per slot; the wave then zeroes the cells of its occupied slots
// together, 16 lanes per slot (16 bytes each), four slots per store.
__global__ __launch_bounds__(256) void k_table_clear(Table t, int64_t cap) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int lane = threadIdx.x & 63;
  const bool occ = i < cap && t.keys[i] != 0;
  if (occ) t.keys[i] = 0;
  uint64_t pend = __ballot(occ);  // wave-uniform
  const int64_t first = i - lane;
  const int q = lane >> 4, c = lane & 15;
  const uint4 z = make_uint4(0u, 0u, 0u, 0u);
  while (pend) {
    int sl = -1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int b = pend ? __builtin_ctzll(pend) : -1;
      pend &= pend - 1;
      sl = (q == j) ? b : sl;
    }
    if (sl >= 0) reinterpret_cast<uint4*>(t.cells + (first + sl) * kCells)[c] = z;
  }
}

// Slot of block `bkey`, claiming an empty one.  Returns -1 when the table is
// full.
// Each round reads the aligned group of kSlotGroup slots with a plain load
// and takes the first slot that holds the key or is empty, with a CAS only
// on an empty one; a CAS lost to another key moves on to the next slot.  So
// a key still lands in the first empty slot of its probe order, and most
// claims cost one atomic instead of one per occupied slot passed (keys that
// share a group start there, so first-slot CASes collide often).
__device__ __forceinline__ int64_t block_claim(const Table& t, uint64_t bkey, uint32_t* flags) {
  uint64_t group = first_slot(t, bkey);
  for (uint64_t round = 0; round * kSlotGroup <= t.mask; ++round) {
    const uint4* p = reinterpret_cast<const uint4*>(t.keys + group);
    const uint4 a = p[0], b = p[1];
    const uint64_t k4[4] = {(static_cast<uint64_t>(a.y) << 32) | a.x, (static_cast<uint64_t>(a.w) << 32) | a.z,
                            (static_cast<uint64_t>(b.y) << 32) | b.x, (static_cast<uint64_t>(b.w) << 32) | b.z};
    for (int j = 0; j < static_cast<int>(kSlotGroup); ++j) {
      if (k4[j] != 0) {
        if (~k4[j] == bkey) return static_cast<int64_t>(group + j);
        continue;
      }
      const uint64_t k = atomicCAS(reinterpret_cast<unsigned long long*>(t.keys + group + j), 0ull, ~bkey);
      if (k == 0 || ~k == bkey) return static_cast<int64_t>(group + j);
    }
    group = (group + kSlotGroup) & t.mask;
  }
  if (flags) atomicOr(flags, TS_FLAG_FULL);
  return -1;
}

// True when the previous lane holds a valid key of the same block: that lane
// claims (or finds) the block's slot, so this one need not touch it.  Rows in
// index order are often neighbours in space, so runs of equal block keys are
// common and most of a run's atomics are saved.  Every lane must call this.
__device__ __forceinline__ bool same_block_as_prev_lane(uint64_t bkey, bool valid) {
  const int lane = threadIdx.x & 63;
  const uint32_t lo = __shfl_up(static_cast<uint32_t>(bkey), 1, 64);
  const uint32_t hi = __shfl_up(static_cast<uint32_t>(bkey >> 32), 1, 64);
  const int pv = __shfl_up(valid ? 1 : 0, 1, 64);
  return valid && lane > 0 && pv && ((static_cast<uint64_t>(hi) << 32) | lo) == bkey;
}

// Slot of this lane's block: the first lane of a run of equal block keys
// claims it, the others take it from that lane.  Every lane must call this.
__device__ __forceinline__ int32_t run_slot(const Table& t, uint64_t bkey, bool valid, uint32_t* flags) {
  const int lane = threadIdx.x & 63;
  const bool follow = same_block_as_prev_lane(bkey, valid);
  const int64_t slot = (valid && !follow) ? block_claim(t, bkey, flags) : -1;
  const uint64_t heads = __ballot(!follow) & ((2ull << lane) - 1);  // lanes <= this one that start a run
  const int head = 63 - __builtin_clzll(heads);
  return __shfl(static_cast<int32_t>(slot), head, 64);
}

__global__ __launch_bounds__(256) void k_hash_insert(const int32_t* __restrict__ coords, int64_t n, Table t,
                                                     uint32_t* flags) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  uint64_t key = 0;
  const bool in = i < n;
  const bool valid = in && row_key(coords, i, t.nd, &key);
  const int32_t s = run_slot(t, block_key(key, t.nd), valid, flags);
  if (!valid) {
    if (in && flags) atomicOr(flags, TS_FLAG_RANGE);
    return;
  }
  if (s < 0) return;  // only when the table was full
  unsigned* cell = reinterpret_cast<unsigned*>(t.cells) + static_cast<int64_t>(s) * kCells + cell_of(key, t.nd);
  const unsigned old = atomicMax(cell, cell_enc(i));
  if (old != kNoCell && flags) atomicOr(flags, TS_FLAG_DUP);
}

__global__ __launch_bounds__(256) void k_hash_query(Table t, const int32_t* __restrict__ q, int64_t m,
                                                    int32_t* __restrict__ rows) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= m) return;
  uint64_t key;
  rows[i] = row_key(q, i, t.nd, &key) ? table_find(t, key) : -1;
}

hipError_t launch_hash_build(const int32_t* coords, int64_t n, int ndim, void* table, int64_t cap, uint32_t* flags,
                             hipStream_t s) {
  Table t = table_view(table, cap, ndim);
  k_table_clear<<<static_cast<unsigned>(ceil_div<int64_t>(cap, 256)), 256, 0, s>>>(t, cap);
  if (n > 0) k_hash_insert<<<static_cast<unsigned>(ceil_div<int64_t>(n, 256)), 256, 0, s>>>(coords, n, t, flags);
  return hipGetLastError();
}

hipError_t launch_hash_query(const void* table, int64_t cap, int ndim, const int32_t* q, int64_t m, int32_t* rows,
                             hipStream_t s) {
  if (m == 0) return hipSuccess;
  Table t = table_view(table, cap, ndim);
  k_hash_query<<<static_cast<unsigned>(ceil_div<int64_t>(m, 256)), 256, 0, s>>>(t, q, m, rows);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Strided support: unique(floor(c / s)) per batch, in first-occurrence order.
//   0. the output table is cleared as in a build;
//   1. every in-range input claims (or shares) the block of its downsampled
//      key;
//   2. it atomicMax's NOT row into the key's cell (the cell keeps the lowest
//      input row = the first occurrence) and remembers the cell (steps 1-2
//      are one kernel);
//   3. an input is "first" when its cell holds its own row;
//   4. an exclusive scan over the first-flags numbers the outputs;
//   5. each first input writes its output coordinate and stores NOT its
//      output row into the cell, so the table then maps coordinate -> output
//      row.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool down_key(const int32_t* coords, int64_t i, int ndim, int stride, uint64_t* key) {
  const int32_t* c = coords + i * (ndim + 1);
  int64_t full[3] = {0, 0, 0};
  for (int d = 0; d < ndim; ++d) full[d] = c[1 + d];
  uint64_t k0;
  if (!make_key(ndim, c[0], full, &k0)) return false;  // the input row itself must be valid
  int64_t q[3] = {0, 0, 0};
  for (int d = 0; d < ndim; ++d) q[d] = floor_div(full[d], stride);
  return make_key(ndim, c[0], q, key);
}

// Steps 1-2 in one pass (the table's cells are zero before it starts): the
// first lane of a run of equal block keys claims the slot, the run shares
// it, and each input atomicMax's NOT its row into its cell and remembers the
// cell.
__global__ __launch_bounds__(256) void k_down_insert(const int32_t* __restrict__ coords, int64_t n, int stride,
                                                     Table t, uint32_t* flags, int32_t* __restrict__ cell_at) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  uint64_t key = 0;
  const bool in = i < n;
  const bool valid = in && down_key(coords, i, t.nd, stride, &key);
  const int32_t sl = run_slot(t, block_key(key, t.nd), valid, flags);
  if (!in) return;
  int32_t at = -1;
  if (!valid) {
    if (flags) atomicOr(flags, TS_FLAG_RANGE);
  } else if (sl >= 0) {
    at = sl * kCells + cell_of(key, t.nd);
    atomicMax(reinterpret_cast<unsigned*>(t.cells) + at, cell_enc(i));
  }
  cell_at[i] = at;
}

__global__ __launch_bounds__(256) void k_down_flag(const int32_t* __restrict__ cell_at, int64_t n, Table t,
                                                   int32_t* __restrict__ first) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int32_t at = cell_at[i];
  first[i] = (at >= 0 && static_cast<uint32_t>(t.cells[at]) == cell_enc(i)) ? 1 : 0;
}

__global__ __launch_bounds__(256) void k_down_emit(const int32_t* __restrict__ coords, int64_t n, int ndim,
                                                   int stride, const int32_t* __restrict__ cell_at,
                                                   const int32_t* __restrict__ first,
                                                   const int32_t* __restrict__ index, Table t,
                                                   int32_t* __restrict__ out_coords) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n || !first[i]) return;
  const int32_t j = index[i];
  const int32_t* c = coords + i * (ndim + 1);
  int32_t* o = out_coords + static_cast<int64_t>(j) * (ndim + 1);
  o[0] = c[0];
  for (int d = 0; d < ndim; ++d) o[1 + d] = static_cast<int32_t>(floor_div(c[1 + d], stride));
  t.cells[cell_at[i]] = static_cast<int32_t>(cell_enc(j));
}

size_t support_scratch_bytes(int64_t n) {
  const size_t a = align_up(static_cast<size_t>(n) * 4, 256);
  return 3 * a + scan_tmp_bytes(n);
}

hipError_t launch_strided_support(const int32_t* coords, int64_t n, int ndim, int stride, int32_t* out_coords,
                                  int64_t* n_out, void* out_table, int64_t out_cap, void* scratch,
                                  uint32_t* flags, hipStream_t s) {
  Table t = table_view(out_table, out_cap, ndim);
  const size_t a = align_up(static_cast<size_t>(n) * 4, 256);
  char* p = static_cast<char*>(scratch);
  int32_t* cell_at = reinterpret_cast<int32_t*>(p);
  int32_t* first = reinterpret_cast<int32_t*>(p + a);
  int32_t* index = reinterpret_cast<int32_t*>(p + 2 * a);
  void* tmp = p + 3 * a;
  k_table_clear<<<static_cast<unsigned>(ceil_div<int64_t>(out_cap, 256)), 256, 0, s>>>(t, out_cap);
  if (n == 0) return fill_i64(n_out, 1, 0, s);
  const unsigned g = static_cast<unsigned>(ceil_div<int64_t>(n, 256));
  k_down_insert<<<g, 256, 0, s>>>(coords, n, stride, t, flags, cell_at);
  k_down_flag<<<g, 256, 0, s>>>(cell_at, n, t, first);
  hipError_t e = scan_exclusive_i32(first, index, n, n_out, tmp, s);
  if (e != hipSuccess) return e;
  k_down_emit<<<g, 256, 0, s>>>(coords, n, ndim, stride, cell_at, first, index, t, out_coords);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Generated supports.  Candidate m = i*kvol + o is the site scale*c_i +
// sign*delta_o: c_i - delta_o for a stride-1 convolution (the output whose
// window holds input i at offset o), s*c_i + delta_o for a transposed
// convolution of stride s (the fine site input i reaches at offset o).  The
// smallest candidate of each site owns it (cells keep NOT of the candidate,
// raised with atomicMax), so the outputs come out in first-occurrence order
// over (input row, offset) after the same flag / scan / emit steps as the
// strided support.  Sites outside the packable range are not generated; an
// out-of-range input raises RANGE.  Outputs past n_out_cap are dropped (their
// cells emptied) and raise FULL.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool gen_key(const int32_t* coords, int64_t m, int ndim, int kvol, const Offsets& offs,
                                        int scale, int sign, bool* input_ok, uint64_t* key) {
  const int64_t i = m / kvol;
  const int o = static_cast<int>(m - i * kvol);
  const int32_t* c = coords + i * (ndim + 1);
  int64_t full[3] = {0, 0, 0};
  for (int d = 0; d < ndim; ++d) full[d] = c[1 + d];
  uint64_t k0;
  *input_ok = make_key(ndim, c[0], full, &k0);
  if (!*input_ok) return false;
  int64_t q[3] = {0, 0, 0};
  for (int d = 0; d < ndim; ++d) q[d] = scale * full[d] + sign * offs.d[o][d];
  return make_key(ndim, c[0], q, key);
}

__global__ __launch_bounds__(256) void k_gen_insert(const int32_t* __restrict__ coords, int64_t n_cand, int kvol,
                                                    Offsets offs, int scale, int sign, Table t, uint32_t* flags,
                                                    int32_t* __restrict__ cell_at) {
  const int64_t m = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  uint64_t key = 0;
  bool input_ok = true;
  const bool in = m < n_cand;
  const bool valid = in && gen_key(coords, m, t.nd, kvol, offs, scale, sign, &input_ok, &key);
  const int32_t sl = run_slot(t, block_key(key, t.nd), valid, flags);
  // The candidate kvol + 1 lanes earlier is input i - 1 at offset o - 1: for
  // a stride-1 generation and inputs that are neighbours along the last
  // axis, the same site.  A candidate whose site an earlier lane also has
  // cannot own it (the smallest candidate does), so it skips the atomic; the
  // cell still ends up holding the owner, and first occurrences are read
  // from the cells afterwards as before.
  const int back = kvol + 1;
  const uint32_t plo = __shfl_up(static_cast<uint32_t>(key), back, 64);
  const uint32_t phi = __shfl_up(static_cast<uint32_t>(key >> 32), back, 64);
  const int pvalid = __shfl_up(valid ? 1 : 0, back, 64);
  const bool shadowed = scale == 1 && back < 64 && static_cast<int>(threadIdx.x & 63) >= back && pvalid &&
                        ((static_cast<uint64_t>(phi) << 32) | plo) == key;
  if (!in) return;
  int32_t at = -1;
  if (!input_ok) {
    if (flags && m % kvol == 0) atomicOr(flags, TS_FLAG_RANGE);
  } else if (valid && sl >= 0) {
    at = sl * kCells + cell_of(key, t.nd);
    if (!shadowed) atomicMax(reinterpret_cast<unsigned*>(t.cells) + at, cell_enc(m));
  }
  cell_at[m] = at;
}

__global__ __launch_bounds__(256) void k_gen_emit(const int32_t* __restrict__ coords, int64_t n_cand, int ndim,
                                                  int kvol, Offsets offs, int scale, int sign,
                                                  const int32_t* __restrict__ cell_at,
                                                  const int32_t* __restrict__ first,
                                                  const int32_t* __restrict__ index, int64_t n_out_cap,
                                                  int64_t* n_out, Table t, uint32_t* flags,
                                                  int32_t* __restrict__ out_coords) {
  const int64_t m = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (m == 0 && *n_out > n_out_cap) *n_out = n_out_cap;  // n_out is read by no other lane
  if (m >= n_cand || !first[m]) return;
  const int32_t j = index[m];
  if (j >= n_out_cap) {
    t.cells[cell_at[m]] = static_cast<int32_t>(kNoCell);
    if (flags) atomicOr(flags, TS_FLAG_FULL);
    return;
  }
  const int64_t i = m / kvol;
  const int o = static_cast<int>(m - i * kvol);
  const int32_t* c = coords + i * (ndim + 1);
  int32_t* q = out_coords + static_cast<int64_t>(j) * (ndim + 1);
  q[0] = c[0];
  for (int d = 0; d < ndim; ++d) q[1 + d] = scale * c[1 + d] + sign * offs.d[o][d];
  t.cells[cell_at[m]] = static_cast<int32_t>(cell_enc(j));
}

size_t generative_scratch_bytes(int64_t n_cand) {
  const size_t a = align_up(static_cast<size_t>(n_cand) * 4, 256);
  return 3 * a + scan_tmp_bytes(n_cand);
}

hipError_t launch_generative_support(const int32_t* coords, int64_t n, int ndim, int ksize, int scale, int sign,
                                     int32_t* out_coords, int64_t n_out_cap, int64_t* n_out, void* out_table,
                                     int64_t out_cap, void* scratch, uint32_t* flags, hipStream_t s) {
  Table t = table_view(out_table, out_cap, ndim);
  const Offsets offs = make_offsets(ndim, ksize);
  int kvol = 1;
  for (int d = 0; d < ndim; ++d) kvol *= ksize;
  const int64_t n_cand = n * kvol;
  const size_t a = align_up(static_cast<size_t>(n_cand) * 4, 256);
  char* p = static_cast<char*>(scratch);
  int32_t* cell_at = reinterpret_cast<int32_t*>(p);
  int32_t* first = reinterpret_cast<int32_t*>(p + a);
  int32_t* index = reinterpret_cast<int32_t*>(p + 2 * a);
  void* tmp = p + 3 * a;
  k_table_clear<<<static_cast<unsigned>(ceil_div<int64_t>(out_cap, 256)), 256, 0, s>>>(t, out_cap);
  if (n_cand == 0) return fill_i64(n_out, 1, 0, s);
  const unsigned g = static_cast<unsigned>(ceil_div<int64_t>(n_cand, 256));
  k_gen_insert<<<g, 256, 0, s>>>(coords, n_cand, kvol, offs, scale, sign, t, flags, cell_at);
  k_down_flag<<<g, 256, 0, s>>>(cell_at, n_cand, t, first);
  hipError_t e = scan_exclusive_i32(first, index, n_cand, n_out, tmp, s);
  if (e != hipSuccess) return e;
  k_gen_emit<<<g, 256, 0, s>>>(coords, n_cand, ndim, kvol, offs, scale, sign, cell_at, first, index, n_out_cap, n_out,
                               t, flags, out_coords);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Voxelization: point i goes to voxel floor((p_i - origin) / size) per axis,
// decided in float32 (a rounded subtraction, a division rounded to nearest
// even, a floor).  The smallest point index owns each voxel (NOT of it raised
// with atomicMax in the voxel's cell), voxels are numbered in that order by
// the flag / scan / emit steps of the strided support, and the table is left
// mapping each voxel to its row.  Each point then reads its voxel row back,
// and the features are summed per voxel with float atomics (the order of the
// additions is not fixed) and divided by the point count.
// ---------------------------------------------------------------------------
struct VoxGeo {
  float size[3];
  float origin[3];
};

__device__ __forceinline__ bool vox_cell(const int32_t* batch, const float* pos, int64_t i, int ndim,
                                         const VoxGeo& g, int64_t* b, int64_t* q) {
  *b = batch ? batch[i] : 0;
  q[0] = q[1] = q[2] = 0;
  for (int d = 0; d < ndim; ++d) {
    const float rel = pos[i * ndim + d] - g.origin[d];
    const float v = floorf(__fdiv_rn(rel, g.size[d]));
    if (!(v >= -32768.f && v <= 32767.f)) return false;  // NaN fails too
    q[d] = static_cast<int64_t>(v);
  }
  return true;
}

__global__ __launch_bounds__(256) void k_vox_insert(const int32_t* __restrict__ batch, const float* __restrict__ pos,
                                                    int64_t n, VoxGeo g, Table t, uint32_t* flags,
                                                    int32_t* __restrict__ cell_at) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  uint64_t key = 0;
  const bool in = i < n;
  bool valid = false;
  if (in) {
    int64_t b, q[3];
    valid = vox_cell(batch, pos, i, t.nd, g, &b, q) && make_key(t.nd, b, q, &key);
  }
  const int32_t sl = run_slot(t, block_key(key, t.nd), valid, flags);
  if (!in) return;
  int32_t at = -1;
  if (!valid) {
    if (flags) atomicOr(flags, TS_FLAG_RANGE);
  } else if (sl >= 0) {
    at = sl * kCells + cell_of(key, t.nd);
    atomicMax(reinterpret_cast<unsigned*>(t.cells) + at, cell_enc(i));
  }
  cell_at[i] = at;
}

__global__ __launch_bounds__(256) void k_vox_emit(const int32_t* __restrict__ batch, const float* __restrict__ pos,
                                                  int64_t n, int ndim, VoxGeo g, const int32_t* __restrict__ cell_at,
                                                  const int32_t* __restrict__ first, const int32_t* __restrict__ index,
                                                  Table t, int32_t* __restrict__ out_coords) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n || !first[i]) return;
  const int32_t j = index[i];
  int64_t b, q[3];
  vox_cell(batch, pos, i, ndim, g, &b, q);
  int32_t* o = out_coords + static_cast<int64_t>(j) * (ndim + 1);
  o[0] = static_cast<int32_t>(b);
  for (int d = 0; d < ndim; ++d) o[1 + d] = static_cast<int32_t>(q[d]);
  t.cells[cell_at[i]] = static_cast<int32_t>(cell_enc(j));
}

// Voxel row of every point (-1 when dropped); with features, their sum and
// count per voxel (out_feats and counts start at zero).
__global__ __launch_bounds__(256) void k_vox_assign(const int32_t* __restrict__ cell_at, int64_t n, Table t,
                                                    int32_t* __restrict__ vox_of, const float* __restrict__ f,
                                                    int c, float* __restrict__ out_feats, int32_t* __restrict__ counts) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int32_t at = cell_at[i];
  const int32_t v = at >= 0 ? cell_row(static_cast<uint32_t>(t.cells[at])) : -1;
  vox_of[i] = v;
  if (v < 0 || !f) return;
  atomicAdd(counts + v, 1);
  for (int ch = 0; ch < c; ++ch) atomicAdd(out_feats + static_cast<int64_t>(v) * c + ch, f[i * c + ch]);
}

__global__ __launch_bounds__(256) void k_vox_mean(float* __restrict__ out_feats, const int32_t* __restrict__ counts,
                                                  int64_t n_cap, const int64_t* n_out, int c) {
  const int64_t k = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t n = *n_out < n_cap ? *n_out : n_cap;
  if (k >= n * c) return;
  const int32_t cnt = counts[k / c];
  out_feats[k] = cnt > 0 ? out_feats[k] / static_cast<float>(cnt) : 0.f;
}

__global__ __launch_bounds__(256) void k_zero_f32(float* __restrict__ p, int64_t n) {
  const int64_t k = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (k < n) p[k] = 0.f;
}

size_t voxelize_scratch_bytes(int64_t n) {
  const size_t a = align_up(static_cast<size_t>(n) * 4, 256);
  return 4 * a + scan_tmp_bytes(n);
}

hipError_t launch_voxelize(const int32_t* batch, const float* pos, int64_t n, int ndim, const float* size,
                           const float* origin, const float* feats, int c, int32_t* out_coords, int64_t* n_out,
                           void* out_table, int64_t out_cap, int32_t* vox_of, float* out_feats, void* scratch,
                           uint32_t* flags, hipStream_t s) {
  Table t = table_view(out_table, out_cap, ndim);
  VoxGeo g{};
  for (int d = 0; d < ndim; ++d) {
    g.size[d] = size[d];
    g.origin[d] = origin[d];
  }
  const size_t a = align_up(static_cast<size_t>(n) * 4, 256);
  char* p = static_cast<char*>(scratch);
  int32_t* cell_at = reinterpret_cast<int32_t*>(p);
  int32_t* first = reinterpret_cast<int32_t*>(p + a);
  int32_t* index = reinterpret_cast<int32_t*>(p + 2 * a);
  int32_t* counts = reinterpret_cast<int32_t*>(p + 3 * a);
  void* tmp = p + 4 * a;
  k_table_clear<<<static_cast<unsigned>(ceil_div<int64_t>(out_cap, 256)), 256, 0, s>>>(t, out_cap);
  if (n == 0) return fill_i64(n_out, 1, 0, s);
  const unsigned g1 = static_cast<unsigned>(ceil_div<int64_t>(n, 256));
  if (feats) {
    k_zero_f32<<<static_cast<unsigned>(ceil_div<int64_t>(n * c, 256)), 256, 0, s>>>(out_feats, n * c);
    k_zero_f32<<<g1, 256, 0, s>>>(reinterpret_cast<float*>(counts), n);  // zero bits: int 0
  }
  k_vox_insert<<<g1, 256, 0, s>>>(batch, pos, n, g, t, flags, cell_at);
  k_down_flag<<<g1, 256, 0, s>>>(cell_at, n, t, first);
  hipError_t e = scan_exclusive_i32(first, index, n, n_out, tmp, s);
  if (e != hipSuccess) return e;
  k_vox_emit<<<g1, 256, 0, s>>>(batch, pos, n, ndim, g, cell_at, first, index, t, out_coords);
  k_vox_assign<<<g1, 256, 0, s>>>(cell_at, n, t, vox_of, feats, c, out_feats, counts);
  if (feats)
    k_vox_mean<<<static_cast<unsigned>(ceil_div<int64_t>(n * c, 256)), 256, 0, s>>>(out_feats, counts, n, n_out, c);
  return hipGetLastError();
}

// Devoxelization: every point takes its voxel's features (0 when dropped).
template <typename T>
__global__ __launch_bounds__(256) void k_devox(const int32_t* __restrict__ vox_of, int64_t n, const T* __restrict__ vf,
                                               int c, T* __restrict__ pf) {
  const int64_t k = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (k >= n * c) return;
  const int64_t i = k / c;
  const int32_t v = vox_of[i];
  pf[k] = v >= 0 ? vf[static_cast<int64_t>(v) * c + (k - i * c)] : T(0);
}

hipError_t launch_devoxelize(const int32_t* vox_of, int64_t n, const void* vf, int c, void* pf, ts_dtype dt,
                             hipStream_t s) {
  if (n == 0) return hipSuccess;
  const unsigned g = static_cast<unsigned>(ceil_div<int64_t>(n * c, 256));
  switch (dt) {
    case TS_F32: k_devox<float><<<g, 256, 0, s>>>(vox_of, n, static_cast<const float*>(vf), c, static_cast<float*>(pf)); break;
    case TS_F16:
      k_devox<_Float16><<<g, 256, 0, s>>>(vox_of, n, static_cast<const _Float16*>(vf), c, static_cast<_Float16*>(pf));
      break;
    default: k_devox<__bf16><<<g, 256, 0, s>>>(vox_of, n, static_cast<const __bf16*>(vf), c, static_cast<__bf16*>(pf)); break;
  }
  return hipGetLastError();
}

}  // namespace ts
