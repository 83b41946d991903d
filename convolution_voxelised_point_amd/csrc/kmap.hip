// Kernel-map construction (the "kernel-map construction" that the
// torch-lattice page "Migrating from TorchSparse" names in section "Sparse
// tensor expectations"): for each destination row and kernel offset, the
// source row at the displaced coordinate, stored as a tiled relation with
// per-tile offset masks so that the contraction skips empty offsets.
//
// Three relations share one kernel, differing only in how the probed
// coordinate is formed from the destination coordinate c and offset delta:
//   submanifold  (dest = outputs = inputs):  c + delta       in the input table
//   downsampling (dest = strided outputs):   s*c + delta     in the input table
//   transposed   (dest = inputs):            (c - delta)/s   in the output table,
//                                            only when s divides c - delta
#include "common.h"
#include "launch.h"

namespace ts {

namespace {

struct RelK {
  const int32_t* dc;
  int64_t n_dest_cap;
  const int64_t* n_dest;
  int ndim, stride, kvol, centre;
  Offsets offs;
  Table src;
  Table own;
  int64_t n_tiles;
  uint64_t* tile_mask;
  int32_t* tile_rows;
  int32_t* pool;
  uint64_t* row_mask;
};

__device__ __forceinline__ int64_t dest_count(const int64_t* n_dest, int64_t cap) {
  if (!n_dest) return cap;
  const int64_t n = *n_dest;
  return n < cap ? n : cap;
}

// Destination coordinate of `row`; false when the row takes no part.
template <int MODE>
__device__ __forceinline__ bool dest_load(const RelK& a, int64_t row, int64_t* b, int64_t* s) {
  const int32_t* c = a.dc + row * (a.ndim + 1);
  *b = c[0];
  s[0] = s[1] = s[2] = 0;
  for (int d = 0; d < a.ndim; ++d) s[d] = c[1 + d];
  uint64_t key;
  if (!make_key(a.ndim, *b, s, &key)) return false;
  if (MODE == kModeUp) return table_find(a.own, key) == static_cast<int32_t>(row);
  return true;
}

template <int MODE>
__device__ __forceinline__ int32_t probe(const RelK& a, const int8_t* offs, int64_t b, const int64_t* s, int o) {
  int64_t p[3] = {0, 0, 0};
  for (int d = 0; d < a.ndim; ++d) {
    const int64_t dd = offs[o * 3 + d];
    if (MODE == kModeSubm) {
      p[d] = s[d] + dd;
    } else if (MODE == kModeDown) {
      p[d] = static_cast<int64_t>(a.stride) * s[d] + dd;
    } else {
      const int64_t t = s[d] - dd;
      if (t % a.stride != 0) return -1;
      p[d] = t / a.stride;
    }
  }
  uint64_t key;
  if (!make_key(a.ndim, b, p, &key)) return -1;
  return table_find(a.src, key);
}

__device__ __forceinline__ uint64_t group16_or(uint64_t v) {
  uint32_t lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(v >> 32);
#pragma unroll
  for (int sh = 8; sh >= 1; sh >>= 1) {
    lo |= __shfl_xor(lo, sh, 64);
    hi |= __shfl_xor(hi, sh, 64);
  }
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// One 16-lane group per tile of destination rows in index order: probe every
// offset, keep the neighbours in LDS, then write the row masks, the tile mask
// and the tile's neighbour blocks for the offsets present in the tile.
template <int MODE>
__global__ __launch_bounds__(256) void k_rel_natural(RelK a) {
  extern __shared__ int32_t nbr_lds[];  // [256][kvol]
  __shared__ int8_t offs[TS_MAX_KVOL * 3];
  const int8_t* src_offs = &a.offs.d[0][0];
  for (int i = threadIdx.x; i < a.kvol * 3; i += blockDim.x) offs[i] = src_offs[i];
  __syncthreads();

  const int64_t t = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) / kTile;
  const int r = threadIdx.x & (kTile - 1);
  if (t >= a.n_tiles) return;  // whole 16-lane groups leave together
  const int64_t n_dest = dest_count(a.n_dest, a.n_dest_cap);
  const int64_t row = t * kTile + r;

  int64_t b, s[3];
  const bool valid = row < n_dest && dest_load<MODE>(a, row, &b, s);
  int32_t* my = nbr_lds + threadIdx.x * a.kvol;
  uint64_t mask = 0;
  if (valid) {
    for (int o = 0; o < a.kvol; ++o) {
      const int32_t n = probe<MODE>(a, offs, b, s, o);
      my[o] = n;
      if (n >= 0) mask |= 1ull << o;
    }
    // a submanifold output takes part only when it owns its coordinate
    if (MODE == kModeSubm && my[a.centre] != static_cast<int32_t>(row)) mask = 0;
  }
  if (row < a.n_dest_cap) a.row_mask[row] = mask;
  const uint64_t tmask = group16_or(mask);
  if (r == 0) a.tile_mask[t] = tmask;
  a.tile_rows[t * kTile + r] = row < n_dest ? static_cast<int32_t>(row) : -1;
  int k = 0;
  for (uint64_t m = tmask; m; m &= m - 1, ++k) {
    const int o = __builtin_ctzll(m);
    a.pool[(t * a.kvol + k) * kTile + r] = ((mask >> o) & 1) ? my[o] : -1;
  }
}

// Per-offset pair lists, destination rows in index order.  Blocks of 256
// destination rows count their pairs per offset; an exclusive scan over the
// (offset, block) counts gives each block its write positions.
__global__ __launch_bounds__(256) void k_pairs_count(const uint64_t* __restrict__ row_mask, int64_t n_dest_cap,
                                                     const int64_t* n_dest_p, int kvol, int64_t nblk,
                                                     int32_t* __restrict__ cnt) {
  __shared__ int wave_cnt[4][TS_MAX_KVOL];
  const int64_t n_dest = dest_count(n_dest_p, n_dest_cap);
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const uint64_t mask = row < n_dest ? row_mask[row] : 0;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int o = 0; o < kvol; ++o) {
    const uint64_t bal = __ballot((mask >> o) & 1);
    if (lane == 0) wave_cnt[wave][o] = __popcll(bal);
  }
  __syncthreads();
  if (threadIdx.x < kvol) {
    const int o = threadIdx.x;
    cnt[o * nblk + blockIdx.x] = wave_cnt[0][o] + wave_cnt[1][o] + wave_cnt[2][o] + wave_cnt[3][o];
  }
}

__global__ void k_pairs_start(const int32_t* __restrict__ base, int kvol, int64_t nblk, const int64_t* total,
                              int64_t* __restrict__ pair_start) {
  const int o = threadIdx.x;
  if (o < kvol) pair_start[o] = base[o * nblk];
  if (o == kvol) pair_start[kvol] = *total;
}

template <int MODE>
__global__ __launch_bounds__(256) void k_pairs_fill(RelK a, int64_t nblk, const int32_t* __restrict__ base,
                                                    int32_t* __restrict__ pair_in, int32_t* __restrict__ pair_out) {
  __shared__ int wave_cnt[4][TS_MAX_KVOL];
  __shared__ int8_t offs[TS_MAX_KVOL * 3];
  const int8_t* src_offs = &a.offs.d[0][0];
  for (int i = threadIdx.x; i < a.kvol * 3; i += blockDim.x) offs[i] = src_offs[i];
  const int64_t n_dest = dest_count(a.n_dest, a.n_dest_cap);
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const uint64_t mask = row < n_dest ? a.row_mask[row] : 0;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint64_t below = (1ull << lane) - 1;
  for (int o = 0; o < a.kvol; ++o) {
    const uint64_t bal = __ballot((mask >> o) & 1);
    if (lane == 0) wave_cnt[wave][o] = __popcll(bal);
  }
  __syncthreads();
  int64_t b = 0, s[3] = {0, 0, 0};
  if (mask) dest_load<MODE>(a, row, &b, s);
  for (int o = 0; o < a.kvol; ++o) {
    const bool has = (mask >> o) & 1;
    const uint64_t bal = __ballot(has);  // every lane takes part
    if (!has) continue;
    int pos = base[o * nblk + blockIdx.x] + __popcll(bal & below);
    for (int w = 0; w < wave; ++w) pos += wave_cnt[w][o];
    pair_out[pos] = static_cast<int32_t>(row);
    pair_in[pos] = probe<MODE>(a, offs, b, s, o);
  }
}

RelK make_relk(const RelBuild& bld, const ts_rel& rel) {
  RelK a;
  a.dc = bld.dest_coords;
  a.n_dest_cap = bld.n_dest_cap;
  a.n_dest = bld.n_dest;
  a.ndim = bld.ndim;
  a.stride = bld.stride;
  a.kvol = bld.kvol;
  a.centre = (bld.kvol - 1) / 2;
  a.offs = make_offsets(bld.ndim, bld.ksize);
  a.src = table_view(bld.src_table, bld.src_cap);
  a.own = bld.own_table ? table_view(bld.own_table, bld.own_cap) : a.src;
  a.n_tiles = rel.n_tiles;
  a.tile_mask = rel.tile_mask;
  a.tile_rows = rel.tile_rows;
  a.pool = rel.pool;
  a.row_mask = rel.row_mask;
  return a;
}

}  // namespace

size_t rel_scratch_bytes(int64_t n_dest_cap, int kvol) {
  (void)n_dest_cap;
  (void)kvol;
  return 0;
}

hipError_t launch_rel_build(const RelBuild& bld, const ts_rel& rel, bool natural, void* scratch, hipStream_t s) {
  (void)natural;
  (void)scratch;
  if (rel.n_tiles == 0) return hipSuccess;
  RelK a = make_relk(bld, rel);
  const unsigned grid = static_cast<unsigned>(ceil_div<int64_t>(rel.n_tiles * kTile, 256));
  const size_t lds = static_cast<size_t>(256) * bld.kvol * sizeof(int32_t);
  switch (bld.mode) {
    case kModeSubm: k_rel_natural<kModeSubm><<<grid, 256, lds, s>>>(a); break;
    case kModeDown: k_rel_natural<kModeDown><<<grid, 256, lds, s>>>(a); break;
    default: k_rel_natural<kModeUp><<<grid, 256, lds, s>>>(a); break;
  }
  return hipGetLastError();
}

size_t pairs_scratch_bytes(int64_t n_dest_cap, int kvol) {
  const int64_t nblk = ceil_div<int64_t>(n_dest_cap, 256);
  const int64_t n = nblk * kvol;
  return align_up(static_cast<size_t>(n > 0 ? n : 1) * 4, 256) + scan_tmp_bytes(n);
}

hipError_t launch_pairs_build(const RelBuild& bld, const ts_rel& rel, int64_t* pair_start, int32_t* pair_in,
                              int32_t* pair_out, void* scratch, hipStream_t s) {
  const int64_t nblk = ceil_div<int64_t>(bld.n_dest_cap, 256);
  if (nblk == 0) return fill_i64(pair_start, bld.kvol + 1, 0, s);
  const int64_t n = nblk * bld.kvol;
  int32_t* cnt = static_cast<int32_t*>(scratch);
  void* tmp = static_cast<char*>(scratch) + align_up(static_cast<size_t>(n) * 4, 256);
  k_pairs_count<<<static_cast<unsigned>(nblk), 256, 0, s>>>(rel.row_mask, bld.n_dest_cap, bld.n_dest, bld.kvol,
                                                              nblk, cnt);
  hipError_t e = scan_exclusive_i32(cnt, cnt, n, pair_start + bld.kvol, tmp, s);
  if (e != hipSuccess) return e;
  k_pairs_start<<<1, 128, 0, s>>>(cnt, bld.kvol, nblk, pair_start + bld.kvol, pair_start);
  RelK a = make_relk(bld, rel);
  switch (bld.mode) {
    case kModeSubm: k_pairs_fill<kModeSubm><<<static_cast<unsigned>(nblk), 256, 0, s>>>(a, nblk, cnt, pair_in, pair_out); break;
    case kModeDown: k_pairs_fill<kModeDown><<<static_cast<unsigned>(nblk), 256, 0, s>>>(a, nblk, cnt, pair_in, pair_out); break;
    default: k_pairs_fill<kModeUp><<<static_cast<unsigned>(nblk), 256, 0, s>>>(a, nblk, cnt, pair_in, pair_out); break;
  }
  return hipGetLastError();
}

}  // namespace ts
