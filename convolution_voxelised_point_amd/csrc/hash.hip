// Coordinate hash table (build / query) and the downsampled support of a
// strided convolution.  The torch-lattice page "Migrating from TorchSparse"
// lists hashing and coordinate query among the library's kernels (section
// "What remains familiar") and says a strided convolution creates a
// downsampled support (section "Convolution mapping").
#include "common.h"
#include "launch.h"

namespace ts {

// Fill every slot with the empty key and the "no row" value.  A plain fill
// kernel (not a memset node) so the call can be captured in a graph.
__global__ __launch_bounds__(256) void k_table_clear(uint64_t* __restrict__ keys, int32_t* __restrict__ vals,
                                                     int64_t cap) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < cap) {
    keys[i] = kEmptyKey;
    vals[i] = 0x7fffffff;
  }
}

// Insert `key` -> `row`: claim the first empty slot of the probe sequence or
// join the slot already holding the key; the row value is the minimum over
// all inserters (lowest row wins).  Returns the slot or -1 when full.
__device__ __forceinline__ int64_t table_insert(const Table& t, uint64_t key, int32_t row, uint32_t* flags) {
  uint64_t slot = hash64(key) & t.mask;
  for (uint64_t probe = 0; probe <= t.mask; ++probe) {
    uint64_t k = t.keys[slot];
    if (k == kEmptyKey) {
      k = atomicCAS(reinterpret_cast<unsigned long long*>(t.keys + slot), kEmptyKey, key);
      if (k == kEmptyKey) {
        atomicMin(t.vals + slot, row);
        return static_cast<int64_t>(slot);
      }
    }
    if (k == key) {
      atomicMin(t.vals + slot, row);
      if (flags) atomicOr(flags, TS_FLAG_DUP);
      return static_cast<int64_t>(slot);
    }
    slot = (slot + 1) & t.mask;
  }
  if (flags) atomicOr(flags, TS_FLAG_FULL);
  return -1;
}

__global__ __launch_bounds__(256) void k_hash_insert(const int32_t* __restrict__ coords, int64_t n, int ndim,
                                                     Table t, uint32_t* flags) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  uint64_t key;
  if (!row_key(coords, i, ndim, &key)) {
    if (flags) atomicOr(flags, TS_FLAG_RANGE);
    return;
  }
  table_insert(t, key, static_cast<int32_t>(i), flags);
}

__global__ __launch_bounds__(256) void k_hash_query(Table t, int ndim, const int32_t* __restrict__ q, int64_t m,
                                                    int32_t* __restrict__ rows) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= m) return;
  uint64_t key;
  rows[i] = row_key(q, i, ndim, &key) ? table_find(t, key) : -1;
}

hipError_t launch_hash_build(const int32_t* coords, int64_t n, int ndim, void* table, int64_t cap, uint32_t* flags,
                             hipStream_t s) {
  Table t = table_view(table, cap);
  k_table_clear<<<static_cast<unsigned>(ceil_div<int64_t>(cap, 256)), 256, 0, s>>>(t.keys, t.vals, cap);
  if (n > 0)
    k_hash_insert<<<static_cast<unsigned>(ceil_div<int64_t>(n, 256)), 256, 0, s>>>(coords, n, ndim, t, flags);
  return hipGetLastError();
}

hipError_t launch_hash_query(const void* table, int64_t cap, int ndim, const int32_t* q, int64_t m, int32_t* rows,
                             hipStream_t s) {
  if (m == 0) return hipSuccess;
  Table t = table_view(table, cap);
  k_hash_query<<<static_cast<unsigned>(ceil_div<int64_t>(m, 256)), 256, 0, s>>>(t, ndim, q, m, rows);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Strided support: unique(floor(c / s)) per batch, in first-occurrence order.
//   1. every in-range input inserts its downsampled key, the table value
//      keeping the lowest input row (= the first occurrence);
//   2. an input is "first" when the slot's value is its own row;
//   3. an exclusive scan over the first-flags numbers the outputs;
//   4. each first input writes its output coordinate and stores its output
//      row into the slot, so the table then maps coordinate -> output row.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool down_key(const int32_t* coords, int64_t i, int ndim, int stride, int64_t* b,
                                         int64_t* s, uint64_t* key) {
  const int32_t* c = coords + i * (ndim + 1);
  int64_t full[3] = {0, 0, 0};
  for (int d = 0; d < ndim; ++d) full[d] = c[1 + d];
  *b = c[0];
  uint64_t k0;
  if (!make_key(ndim, *b, full, &k0)) return false;  // the input row itself must be valid
  s[0] = s[1] = s[2] = 0;
  for (int d = 0; d < ndim; ++d) s[d] = floor_div(full[d], stride);
  return make_key(ndim, *b, s, key);
}

__global__ __launch_bounds__(256) void k_down_insert(const int32_t* __restrict__ coords, int64_t n, int ndim,
                                                     int stride, Table t, int32_t* __restrict__ slot_of,
                                                     uint32_t* flags) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  int64_t b, s[3];
  uint64_t key;
  int64_t slot = -1;
  if (down_key(coords, i, ndim, stride, &b, s, &key)) {
    slot = table_insert(t, key, static_cast<int32_t>(i), nullptr);
    if (slot < 0 && flags) atomicOr(flags, TS_FLAG_FULL);
  } else if (flags) {
    atomicOr(flags, TS_FLAG_RANGE);
  }
  slot_of[i] = static_cast<int32_t>(slot);
}

__global__ __launch_bounds__(256) void k_down_flag(const int32_t* __restrict__ slot_of, int64_t n, Table t,
                                                   int32_t* __restrict__ first) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int32_t slot = slot_of[i];
  first[i] = (slot >= 0 && t.vals[slot] == static_cast<int32_t>(i)) ? 1 : 0;
}

__global__ __launch_bounds__(256) void k_down_emit(const int32_t* __restrict__ coords, int64_t n, int ndim,
                                                   int stride, const int32_t* __restrict__ slot_of,
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
  t.vals[slot_of[i]] = j;
}

size_t support_scratch_bytes(int64_t n) {
  const size_t a = align_up(static_cast<size_t>(n) * 4, 256);
  return 3 * a + scan_tmp_bytes(n);
}

hipError_t launch_strided_support(const int32_t* coords, int64_t n, int ndim, int stride, int32_t* out_coords,
                                  int64_t* n_out, void* out_table, int64_t out_cap, void* scratch,
                                  uint32_t* flags, hipStream_t s) {
  Table t = table_view(out_table, out_cap);
  const size_t a = align_up(static_cast<size_t>(n) * 4, 256);
  char* p = static_cast<char*>(scratch);
  int32_t* slot_of = reinterpret_cast<int32_t*>(p);
  int32_t* first = reinterpret_cast<int32_t*>(p + a);
  int32_t* index = reinterpret_cast<int32_t*>(p + 2 * a);
  void* tmp = p + 3 * a;
  k_table_clear<<<static_cast<unsigned>(ceil_div<int64_t>(out_cap, 256)), 256, 0, s>>>(t.keys, t.vals, out_cap);
  if (n == 0) {
    return fill_i64(n_out, 1, 0, s);
  }
  const unsigned g = static_cast<unsigned>(ceil_div<int64_t>(n, 256));
  k_down_insert<<<g, 256, 0, s>>>(coords, n, ndim, stride, t, slot_of, flags);
  k_down_flag<<<g, 256, 0, s>>>(slot_of, n, t, first);
  hipError_t e = scan_exclusive_i32(first, index, n, n_out, tmp, s);
  if (e != hipSuccess) return e;
  k_down_emit<<<g, 256, 0, s>>>(coords, n, ndim, stride, slot_of, first, index, t, out_coords);
  return hipGetLastError();
}

}  // namespace ts
