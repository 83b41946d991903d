// Internal device helpers shared by the library's HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ts.h"

namespace ts {

constexpr uint64_t kEmptyKey = ~0ull;  // key read from an empty slot; batch 65535 is out of range, so no key equals it
constexpr int kTile = TS_TILE;
constexpr int kWave = 64;

// Kernel-offset displacements, passed by value to kernels.
struct Offsets {
  int8_t d[TS_MAX_KVOL][3];
};

inline Offsets make_offsets(int ndim, int ksize) {
  Offsets o{};
  int kvol = 1;
  for (int i = 0; i < ndim; ++i) kvol *= ksize;
  const int r = (ksize - 1) / 2;
  for (int k = 0; k < kvol; ++k) {
    int rem = k;
    for (int d = ndim - 1; d >= 0; --d) {
      o.d[k][d] = static_cast<int8_t>(rem % ksize - r);
      rem /= ksize;
    }
  }
  return o;
}

// Two-level coordinate table.  Voxels are grouped in blocks (4x4x4 in 3-D,
// 8x8 in 2-D, 64 cells either way).  An open-addressing table (linear
// probing) maps a block key to a block slot; each slot owns a dense array of
// 64 cells holding the row of each voxel of the block (encodings below).
// The neighbourhood of a voxel then needs a few block lookups and direct
// cell loads instead of one hashed probe per neighbour.
//   buffer: keys [cap] u64 | (256-byte aligned) cells [cap][64] int32
constexpr int kCells = 64;
// Stored encodings: a slot holds the bitwise NOT of its block key and a cell
// the bitwise NOT of its row, so an all-zero buffer is an empty table (no
// valid key is all ones: batch 65535 is out of range) and, with unsigned
// atomicMax on cells, the lowest row wins.
constexpr uint32_t kNoCell = 0;
__device__ __forceinline__ uint32_t cell_enc(int64_t row) { return ~static_cast<uint32_t>(row); }
__device__ __forceinline__ int32_t cell_row(uint32_t c) { return c == kNoCell ? -1 : static_cast<int32_t>(~c); }

struct Table {
  uint64_t* keys;
  int32_t* cells;
  uint64_t mask;  // cap - 1
  int nd;         // 2 or 3
};

inline size_t table_keys_bytes(int64_t cap) { return (static_cast<size_t>(cap) * 8 + 255) / 256 * 256; }

inline Table table_view(const void* base, int64_t cap, int ndim) {
  Table t;
  char* p = reinterpret_cast<char*>(const_cast<void*>(base));
  t.keys = reinterpret_cast<uint64_t*>(p);
  t.cells = reinterpret_cast<int32_t*>(p + table_keys_bytes(cap));
  t.mask = static_cast<uint64_t>(cap - 1);
  t.nd = ndim;
  return t;
}

__device__ __forceinline__ bool batch_ok(int64_t b) { return b >= 0 && b <= 65534; }
__device__ __forceinline__ bool axis_ok(int64_t v) { return v >= -32768 && v <= 32767; }

// Pack (b, s0, s1[, s2]) into 16-bit fields; 2-D keys fill the last field
// with the bias.  Returns false when a value is outside the packable range.
__device__ __forceinline__ bool make_key(int ndim, int64_t b, const int64_t* s, uint64_t* key) {
  if (!batch_ok(b)) return false;
  uint64_t k = static_cast<uint64_t>(b);
  for (int d = 0; d < 3; ++d) {
    int64_t v = d < ndim ? s[d] : 0;
    if (!axis_ok(v)) return false;
    k = (k << 16) | static_cast<uint64_t>(v + 32768);
  }
  *key = k;
  return true;
}

// Key of stored coordinate row `row` (int32 [ndim+1]).
__device__ __forceinline__ bool row_key(const int32_t* coords, int64_t row, int ndim, uint64_t* key) {
  const int32_t* c = coords + row * (ndim + 1);
  int64_t s[3] = {0, 0, 0};
  for (int d = 0; d < ndim; ++d) s[d] = c[1 + d];
  return make_key(ndim, c[0], s, key);
}

// Slot hash of a block key: the two 32-bit halves folded with a golden-ratio
// multiply, then the 32-bit finaliser of MurmurHash3 (xor-shift-multiply
// with its published constants).  32-bit multiplies only: the probe hashes
// up to eight corner blocks per row.
__device__ __forceinline__ uint32_t hash_key(uint64_t k) {
  uint32_t h = static_cast<uint32_t>(k) ^ (static_cast<uint32_t>(k >> 32) * 0x9e3779b1u);
  h ^= h >> 16;
  h *= 0x85ebca6bu;
  h ^= h >> 13;
  h *= 0xc2b2ae35u;
  h ^= h >> 16;
  return h;
}

// Key layout: [batch:16][f0:16][f1:16][f2:16] with f = value + 2^15 (a
// 2-D key keeps f2 = 2^15).  Block key: the fields divided by the block side
// (4 in 3-D, 8 in 2-D; 2-D keeps f2).  Cell: the remainders, row-major.
__device__ __forceinline__ uint64_t block_key(uint64_t key, int nd) {
  const uint64_t b = key >> 48, f0 = (key >> 32) & 0xffff, f1 = (key >> 16) & 0xffff, f2 = key & 0xffff;
  if (nd == 3) return (b << 48) | ((f0 >> 2) << 32) | ((f1 >> 2) << 16) | (f2 >> 2);
  return (b << 48) | ((f0 >> 3) << 32) | ((f1 >> 3) << 16) | f2;
}
__device__ __forceinline__ int cell_of(uint64_t key, int nd) {
  const uint32_t f0 = (key >> 32) & 0xffff, f1 = (key >> 16) & 0xffff, f2 = key & 0xffff;
  if (nd == 3) return static_cast<int>(((f0 & 3) << 4) | ((f1 & 3) << 2) | (f2 & 3));
  return static_cast<int>(((f0 & 7) << 3) | (f1 & 7));
}

// Linear probing starts at the hashed slot rounded down to a multiple of
// kSlotGroup, so a lookup may read several consecutive slots of an aligned
// group per round and check those probe positions at once.  On the
// ring-scan table (load 0.16), reading two slots per round, a wavefront's
// 8-corner lookups finish in about 2.3 rounds on average (at most 6) instead
// of 3.8 (at most 11); a claim reads the whole group of four.
constexpr uint64_t kSlotGroup = 4;
__device__ __forceinline__ uint64_t first_slot(const Table& t, uint64_t bkey) {
  return static_cast<uint64_t>(hash_key(bkey)) & t.mask & ~(kSlotGroup - 1);
}

// Slot of a block key or -1 (linear probing from its first slot).
__device__ __forceinline__ int64_t block_find(const Table& t, uint64_t bkey) {
  uint64_t slot = first_slot(t, bkey);
  for (uint64_t probe = 0; probe <= t.mask; ++probe) {
    const uint64_t k = ~t.keys[slot];
    if (k == bkey) return static_cast<int64_t>(slot);
    if (k == kEmptyKey) return -1;
    slot = (slot + 1) & t.mask;
  }
  return -1;
}

// Lookup of a voxel key: its row or -1.
__device__ __forceinline__ int32_t table_find(const Table& t, uint64_t key) {
  const int64_t s = block_find(t, block_key(key, t.nd));
  if (s < 0) return -1;
  return cell_row(static_cast<uint32_t>(t.cells[s * kCells + cell_of(key, t.nd)]));
}

__device__ __forceinline__ int64_t floor_div(int64_t a, int64_t b) {
  int64_t q = a / b;
  if ((a % b != 0) && ((a < 0) != (b < 0))) --q;
  return q;
}

template <typename T>
__host__ __device__ __forceinline__ T ceil_div(T a, T b) {
  return (a + b - 1) / b;
}

// ---------------------------------------------------------------- bounds-check build
// Compiled with TS_DEBUG_CHECKS (the separate bounds-check build of the
// library), the contraction, pooling and weight-gradient kernels check every
// row index they read from a map -- neighbour entries, tile rows, pairs,
// group entries and slots -- against the matrix it indexes before using it.
// An index out of range is replaced by one inside (an absent neighbour where
// the kernel knows absence, else row 0), so no access leaves the buffers, and
// ORs a TS_DEBUG_* bit into the violation word of its translation unit; the
// results of such a call are then meaningless, and ts_debug_violations reports
// the bits.  In the regular build the checks are the identity.
#ifdef TS_DEBUG_CHECKS
constexpr bool kDebugChecks = true;
static __device__ uint32_t g_debug_word;
#else
constexpr bool kDebugChecks = false;
#endif

// An optional row index (-1 = absent): r for -1 <= r < n, else -1.
__device__ __forceinline__ int32_t dbg_opt(int32_t r, int64_t n, uint32_t bit) {
#ifdef TS_DEBUG_CHECKS
  if (r < -1 || r >= n) {
    atomicOr(&g_debug_word, bit);
    return -1;
  }
#endif
  return r;
}

// A required row index: r for 0 <= r < n, else 0.
__device__ __forceinline__ int32_t dbg_req(int32_t r, int64_t n, uint32_t bit) {
#ifdef TS_DEBUG_CHECKS
  if (r < 0 || r >= n) {
    atomicOr(&g_debug_word, bit);
    return 0;
  }
#endif
  return r;
}

#ifdef TS_DEBUG_CHECKS
// This translation unit's violation word on the current device: read into
// *v, then cleared (synchronous copies).
static hipError_t debug_take_local(uint32_t* v) {
  hipError_t e = hipMemcpyFromSymbol(v, HIP_SYMBOL(g_debug_word), sizeof(uint32_t), 0, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return e;
  const uint32_t zero = 0;
  return hipMemcpyToSymbol(HIP_SYMBOL(g_debug_word), &zero, sizeof zero, 0, hipMemcpyHostToDevice);
}
#define TS_DEBUG_TU(name) \
  namespace ts {          \
  hipError_t debug_take_##name(uint32_t* v) { return debug_take_local(v); } \
  }
#else
#define TS_DEBUG_TU(name)
#endif

}  // namespace ts
