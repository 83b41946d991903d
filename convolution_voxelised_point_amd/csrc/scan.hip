// Device-wide exclusive prefix sum of int32 counts and small fill kernels.
// Blocks of 256 threads scan 2048 items each.  Up to kMaxDirect blocks, a
// second pass lets every block sum the block totals before it (one wave) and
// add that prefix; beyond that a single block first scans the per-block sums
// (in chunks of 2048 with a running carry).
#include "common.h"
#include "launch.h"

namespace ts {

namespace {

constexpr int kThreads = 256;
constexpr int kItems = 8;
constexpr int kPerBlock = kThreads * kItems;

// Exclusive prefix of `v` over the block; *total = block sum.
__device__ __forceinline__ int block_exclusive(int v, int* lds_wave, int* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) lds_wave[wave] = x;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {
    const int s = lds_wave[w];
    if (w < wave) before += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return before + x - v;
}

// Scans the 2048-item chunk starting at `base` with `carry` added; returns
// the chunk sum.
__device__ __forceinline__ int scan_chunk(const int32_t* in, int32_t* out, int64_t n, int64_t base, int carry,
                                          int* lds_wave) {
  const int64_t first = base + static_cast<int64_t>(threadIdx.x) * kItems;
  int v[kItems];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < kItems; ++i) {
    v[i] = (first + i < n) ? in[first + i] : 0;
    sum += v[i];
  }
  int tot;
  int run = carry + block_exclusive(sum, lds_wave, &tot);
#pragma unroll
  for (int i = 0; i < kItems; ++i) {
    if (first + i < n) out[first + i] = run;
    run += v[i];
  }
  return tot;
}

__global__ __launch_bounds__(kThreads) void k_scan_local(const int32_t* in, int32_t* out, int64_t n,
                                                         int32_t* block_sums, int64_t* total) {
  __shared__ int lw[kThreads / 64];
  const int tot = scan_chunk(in, out, n, static_cast<int64_t>(blockIdx.x) * kPerBlock, 0, lw);
  if (threadIdx.x == 0) {
    if (block_sums) block_sums[blockIdx.x] = tot;
    if (total) *total = tot;
  }
}

__global__ __launch_bounds__(kThreads) void k_scan_sums(int32_t* sums, int64_t nb, int64_t* total) {
  __shared__ int lw[kThreads / 64];
  int carry = 0;
  for (int64_t base = 0; base < nb; base += kPerBlock) carry += scan_chunk(sums, sums, nb, base, carry, lw);
  if (threadIdx.x == 0 && total) *total = carry;
}

__global__ __launch_bounds__(kThreads) void k_scan_add(int32_t* out, int64_t n, const int32_t* sums) {
  const int add = sums[blockIdx.x];
  const int64_t first = static_cast<int64_t>(blockIdx.x) * kPerBlock;
  for (int i = threadIdx.x; i < kPerBlock; i += kThreads)
    if (first + i < n) out[first + i] += add;
}

// Adds to block b's items the sum of the totals of blocks 0..b-1, summed by
// the first wave; the last block also writes the grand total.
constexpr int64_t kMaxDirect = 4096;
__global__ __launch_bounds__(kThreads) void k_scan_add_direct(int32_t* out, int64_t n, const int32_t* sums,
                                                              int64_t nb, int64_t* total) {
  __shared__ int pre;
  const int64_t b = blockIdx.x;
  if (threadIdx.x < 64) {
    int v = 0;
    for (int64_t i = threadIdx.x; i < b; i += 64) v += sums[i];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    if (threadIdx.x == 0) {
      pre = v;
      if (total && b == nb - 1) *total = static_cast<int64_t>(v) + sums[b];
    }
  }
  __syncthreads();
  const int add = pre;
  const int64_t first = b * kPerBlock;
  for (int i = threadIdx.x; i < kPerBlock; i += kThreads)
    if (first + i < n) out[first + i] += add;
}

__global__ __launch_bounds__(256) void k_fill_i64(int64_t* p, int64_t n, int64_t v) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}
__global__ __launch_bounds__(256) void k_fill_i32(int32_t* p, int64_t n, int32_t v) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}
__global__ __launch_bounds__(256) void k_fill_f32(float* p, int64_t n, float v) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace

size_t scan_tmp_bytes(int64_t n) {
  const int64_t nb = ceil_div<int64_t>(n, kPerBlock);
  return align_up(static_cast<size_t>(nb > 0 ? nb : 1) * 4, 256);
}

hipError_t scan_exclusive_i32(const int32_t* in, int32_t* out, int64_t n, int64_t* total, void* tmp,
                              hipStream_t s) {
  if (n <= 0) {
    if (total) return fill_i64(total, 1, 0, s);
    return hipSuccess;
  }
  const int64_t nb = ceil_div<int64_t>(n, kPerBlock);
  if (nb == 1) {
    k_scan_local<<<1, kThreads, 0, s>>>(in, out, n, nullptr, total);
    return hipGetLastError();
  }
  int32_t* sums = static_cast<int32_t*>(tmp);
  k_scan_local<<<static_cast<unsigned>(nb), kThreads, 0, s>>>(in, out, n, sums, nullptr);
  if (nb <= kMaxDirect) {
    k_scan_add_direct<<<static_cast<unsigned>(nb), kThreads, 0, s>>>(out, n, sums, nb, total);
    return hipGetLastError();
  }
  k_scan_sums<<<1, kThreads, 0, s>>>(sums, nb, total);
  k_scan_add<<<static_cast<unsigned>(nb), kThreads, 0, s>>>(out, n, sums);
  return hipGetLastError();
}

hipError_t fill_i64(int64_t* p, int64_t n, int64_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  k_fill_i64<<<static_cast<unsigned>(ceil_div<int64_t>(n, 256)), 256, 0, s>>>(p, n, v);
  return hipGetLastError();
}
hipError_t fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  k_fill_i32<<<static_cast<unsigned>(ceil_div<int64_t>(n, 256)), 256, 0, s>>>(p, n, v);
  return hipGetLastError();
}
hipError_t fill_f32(float* p, int64_t n, float v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  k_fill_f32<<<static_cast<unsigned>(ceil_div<int64_t>(n, 256)), 256, 0, s>>>(p, n, v);
  return hipGetLastError();
}

}  // namespace ts
