// Weight gradient: dW[o] = sum over the pairs (i, j) of offset o of
// x[i]^T dy[j]  -- one (Cin x M_o) . (M_o x Cout) product per offset, needed
// for the mixed-precision training the TorchSparse++ abstract reports.
//
// The pairs of each offset are cut into chunks of kChunk pairs.  A block
// reduces one chunk for one (Cin, Cout) tile into a private fp32 partial;
// k_wgrad_reduce then sums the partials of each offset in chunk order, so
// the result does not depend on scheduling (no atomics).
//
// fp16/bf16 with channel counts that are multiples of 16 use MFMA: per step
// of 32 pairs the block gathers 32 rows of x and of dy and stores them
// transposed in LDS (channel-major), so that each lane's A fragment (8
// consecutive pairs of one input channel) and B fragment (8 pairs of one
// output channel) are single 16-byte LDS reads.
#include "common.h"
#include "launch.h"

namespace ts {

namespace {

constexpr int kChunk = 4096;  // pairs per partial
constexpr int kBT = 64;       // channel tile (both dims) of one block
constexpr int kLdsStride = 40;  // 32 pairs + 8 pad (halves), keeps 16-byte rows aligned

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct WMfma;
template <>
struct WMfma<_Float16> {
  typedef f16x8 frag;
  static __device__ __forceinline__ f32x4 run(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};
template <>
struct WMfma<__bf16> {
  typedef bf16x8 frag;
  static __device__ __forceinline__ f32x4 run(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

// chunk_base[o] = number of chunks of offsets < o; chunk_base[kvol] = total.
__global__ void k_wgrad_chunks(const int64_t* __restrict__ pair_start, int kvol, int32_t* __restrict__ chunk_base) {
  if (threadIdx.x != 0) return;
  int32_t acc = 0;
  for (int o = 0; o < kvol; ++o) {
    chunk_base[o] = acc;
    const int64_t cnt = pair_start[o + 1] - pair_start[o];
    acc += static_cast<int32_t>((cnt + kChunk - 1) / kChunk);
  }
  chunk_base[kvol] = acc;
}

// Which offset / pair range block `c` covers; false for blocks past the end.
__device__ __forceinline__ bool chunk_range(const int32_t* chunk_base, const int64_t* pair_start, int kvol, int c,
                                            int* o_out, int64_t* p0, int64_t* p1) {
  if (c >= chunk_base[kvol]) return false;
  int o = 0;
  while (o + 1 < kvol && chunk_base[o + 1] <= c) ++o;
  const int64_t begin = pair_start[o] + static_cast<int64_t>(c - chunk_base[o]) * kChunk;
  const int64_t end = pair_start[o + 1];
  *o_out = o;
  *p0 = begin;
  *p1 = begin + kChunk < end ? begin + kChunk : end;
  return true;
}

template <typename T>
__global__ __launch_bounds__(256) void k_wgrad_mfma(const int32_t* __restrict__ chunk_base,
                                                    const int64_t* __restrict__ pair_start, int kvol,
                                                    const int32_t* __restrict__ pair_in,
                                                    const int32_t* __restrict__ pair_out, const T* __restrict__ x,
                                                    int cin, const T* __restrict__ dy, int cout,
                                                    float* __restrict__ partial) {
  typedef typename WMfma<T>::frag Frag;
  __shared__ __attribute__((aligned(16))) T xt[kBT * kLdsStride];
  __shared__ __attribute__((aligned(16))) T yt[kBT * kLdsStride];
  const int c = blockIdx.x;
  int o;
  int64_t p0, p1;
  if (!chunk_range(chunk_base, pair_start, kvol, c, &o, &p0, &p1)) return;
  const int ci0 = blockIdx.y * kBT, co0 = blockIdx.z * kBT;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;  // 2 x 2 waves, 32 x 32 channels each
  // staging: thread -> (pair sp, 8-channel group sg)
  const int sp = threadIdx.x >> 3, sg = threadIdx.x & 7;
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int64_t base = p0; base < p1; base += 32) {
    const int64_t p = base + sp;
    const bool live = p < p1;
    const int ci = ci0 + sg * 8, co = co0 + sg * 8;
    uint4 xv = make_uint4(0, 0, 0, 0), yv = make_uint4(0, 0, 0, 0);
    if (live && ci < cin) xv = *reinterpret_cast<const uint4*>(x + static_cast<int64_t>(pair_in[p]) * cin + ci);
    if (live && co < cout) yv = *reinterpret_cast<const uint4*>(dy + static_cast<int64_t>(pair_out[p]) * cout + co);
    const T* xe = reinterpret_cast<const T*>(&xv);
    const T* ye = reinterpret_cast<const T*>(&yv);
    __syncthreads();  // previous step's fragments are consumed
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      xt[(sg * 8 + e) * kLdsStride + sp] = xe[e];
      yt[(sg * 8 + e) * kLdsStride + sp] = ye[e];
    }
    __syncthreads();
    Frag af[2], bf[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = wm * 32 + i * 16 + (lane & 15);
      af[i] = __builtin_bit_cast(Frag, *reinterpret_cast<const uint4*>(&xt[row * kLdsStride + (lane >> 4) * 8]));
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int row = wn * 32 + j * 16 + (lane & 15);
      bf[j] = __builtin_bit_cast(Frag, *reinterpret_cast<const uint4*>(&yt[row * kLdsStride + (lane >> 4) * 8]));
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = WMfma<T>::run(af[i], bf[j], acc[i][j]);
  }
  // D[m][n]: lane holds n = lane%16, m = 4*(lane/16) + e
  float* part = partial + static_cast<int64_t>(c) * cin * cout;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int co = co0 + wn * 32 + j * 16 + (lane & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ci = ci0 + wm * 32 + i * 16 + (lane >> 4) * 4 + e;
        if (ci < cin && co < cout) part[static_cast<int64_t>(ci) * cout + co] = acc[i][j][e];
      }
    }
}

// FMA fallback: thread = one (ci, co) element of a 256-element tile.
template <typename T>
__global__ __launch_bounds__(256) void k_wgrad_fma(const int32_t* __restrict__ chunk_base,
                                                   const int64_t* __restrict__ pair_start, int kvol,
                                                   const int32_t* __restrict__ pair_in,
                                                   const int32_t* __restrict__ pair_out, const T* __restrict__ x,
                                                   int cin, const T* __restrict__ dy, int cout,
                                                   float* __restrict__ partial) {
  const int c = blockIdx.x;
  int o;
  int64_t p0, p1;
  if (!chunk_range(chunk_base, pair_start, kvol, c, &o, &p0, &p1)) return;
  const int64_t e = static_cast<int64_t>(blockIdx.y) * 256 + threadIdx.x;
  if (e >= static_cast<int64_t>(cin) * cout) return;
  const int ci = static_cast<int>(e / cout), co = static_cast<int>(e % cout);
  float acc = 0.f;
  for (int64_t p = p0; p < p1; ++p)
    acc = fmaf(static_cast<float>(x[static_cast<int64_t>(pair_in[p]) * cin + ci]),
               static_cast<float>(dy[static_cast<int64_t>(pair_out[p]) * cout + co]), acc);
  partial[static_cast<int64_t>(c) * cin * cout + e] = acc;
}

// dw[o][e] = sum of the partials of offset o in chunk order.
__global__ __launch_bounds__(256) void k_wgrad_reduce(const int32_t* __restrict__ chunk_base, int kvol,
                                                      const float* __restrict__ partial, int64_t elems,
                                                      float* __restrict__ dw) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= elems * kvol) return;
  const int o = static_cast<int>(i / elems);
  const int64_t e = i % elems;
  float s = 0.f;
  for (int c = chunk_base[o]; c < chunk_base[o + 1]; ++c) s += partial[static_cast<int64_t>(c) * elems + e];
  dw[i] = s;
}

int64_t max_chunks(const ts_kmap* map) { return map->pair_cap / kChunk + map->kvol + 1; }

}  // namespace

size_t wgrad_workspace_bytes(const ts_kmap* map, int cin, int cout) {
  return align_up(static_cast<size_t>(map->kvol + 1) * 4, 256) +
         static_cast<size_t>(max_chunks(map)) * cin * cout * 4;
}

hipError_t launch_wgrad(const ts_kmap* map, const void* x, int cin, const void* dy, int cout, ts_dtype dt, float* dw,
                        void* ws, hipStream_t s) {
  int32_t* chunk_base = static_cast<int32_t*>(ws);
  float* partial = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up(static_cast<size_t>(map->kvol + 1) * 4, 256));
  const int64_t elems = static_cast<int64_t>(cin) * cout;
  k_wgrad_chunks<<<1, 64, 0, s>>>(map->pair_start, map->kvol, chunk_base);
  const unsigned nch = static_cast<unsigned>(max_chunks(map));
  const bool mfma = dt != TS_F32 && cin % 16 == 0 && cout % 16 == 0;
  if (mfma) {
    dim3 grid(nch, static_cast<unsigned>(ceil_div(cin, kBT)), static_cast<unsigned>(ceil_div(cout, kBT)));
    if (dt == TS_F16)
      k_wgrad_mfma<_Float16><<<grid, 256, 0, s>>>(chunk_base, map->pair_start, map->kvol, map->pair_in, map->pair_out,
                                                   static_cast<const _Float16*>(x), cin,
                                                   static_cast<const _Float16*>(dy), cout, partial);
    else
      k_wgrad_mfma<__bf16><<<grid, 256, 0, s>>>(chunk_base, map->pair_start, map->kvol, map->pair_in, map->pair_out,
                                                 static_cast<const __bf16*>(x), cin, static_cast<const __bf16*>(dy),
                                                 cout, partial);
  } else {
    dim3 grid(nch, static_cast<unsigned>(ceil_div<int64_t>(elems, 256)));
    switch (dt) {
      case TS_F32:
        k_wgrad_fma<float><<<grid, 256, 0, s>>>(chunk_base, map->pair_start, map->kvol, map->pair_in, map->pair_out,
                                                 static_cast<const float*>(x), cin, static_cast<const float*>(dy), cout,
                                                 partial);
        break;
      case TS_F16:
        k_wgrad_fma<_Float16><<<grid, 256, 0, s>>>(chunk_base, map->pair_start, map->kvol, map->pair_in,
                                                    map->pair_out, static_cast<const _Float16*>(x), cin,
                                                    static_cast<const _Float16*>(dy), cout, partial);
        break;
      default:
        k_wgrad_fma<__bf16><<<grid, 256, 0, s>>>(chunk_base, map->pair_start, map->kvol, map->pair_in, map->pair_out,
                                                  static_cast<const __bf16*>(x), cin, static_cast<const __bf16*>(dy),
                                                  cout, partial);
        break;
    }
  }
  const int64_t total = elems * map->kvol;
  k_wgrad_reduce<<<static_cast<unsigned>(ceil_div<int64_t>(total, 256)), 256, 0, s>>>(chunk_base, map->kvol, partial,
                                                                                     elems, dw);
  return hipGetLastError();
}

}  // namespace ts
