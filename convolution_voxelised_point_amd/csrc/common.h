// Internal device helpers shared by the library's HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ts.h"

namespace ts {

constexpr uint64_t kEmptyKey = ~0ull;  // batch 65535 is outside the valid range, so no key equals it
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

// Open-addressing table view: keys[cap] (u64) followed by vals[cap] (i32).
struct Table {
  uint64_t* keys;
  int32_t* vals;
  uint64_t mask;  // cap - 1
};

inline Table table_view(const void* base, int64_t cap) {
  Table t;
  t.keys = reinterpret_cast<uint64_t*>(const_cast<void*>(base));
  t.vals = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(const_cast<void*>(base)) + cap * 8);
  t.mask = static_cast<uint64_t>(cap - 1);
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

// 64-bit finaliser (xor-shift-multiply, constants of Stafford's "Mix13").
__device__ __forceinline__ uint64_t hash64(uint64_t k) {
  k ^= k >> 30;
  k *= 0xbf58476d1ce4e5b9ull;
  k ^= k >> 27;
  k *= 0x94d049bb133111ebull;
  k ^= k >> 31;
  return k;
}

// Lookup: linear probing from hash(key); returns the row or -1.
__device__ __forceinline__ int32_t table_find(const Table& t, uint64_t key) {
  uint64_t slot = hash64(key) & t.mask;
  for (uint64_t probe = 0; probe <= t.mask; ++probe) {
    const uint64_t k = t.keys[slot];
    if (k == key) return t.vals[slot];
    if (k == kEmptyKey) return -1;
    slot = (slot + 1) & t.mask;
  }
  return -1;
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

}  // namespace ts
