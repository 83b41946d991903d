// Map-driven contraction: y[j] = sum_o x[nbr(j, o)] . W[o]  (forward) and the
// same walk with W[o]^T for dgrad.  The TorchSparse++ abstract names the
// implicit-GEMM and gather-GEMM-scatter dataflows; the torch-lattice page
// "Migrating from TorchSparse" (section "Backend and configuration
// differences") requires every dataflow to give the same result for a fixed
// relation and weight tensor.
//
// Dataflows here (the fp16/bf16 MFMA implicit GEMM lives in igemm.hip):
//  * direct: the implicit-GEMM walk over the tiles -- on the fp32 matrix
//    cores (k_mfma_f32) for fp32 features with channels in multiples of 16,
//    with FMA (k_direct) for the other shapes the MFMA kernels do not fit.
//  * gather-scatter (k_gs_offset): offsets one after another in fixed order;
//    per offset, gather the source rows of its pairs, multiply by W[o] and add
//    into an fp32 accumulator at the destination rows.  Within one offset the
//    destination rows are distinct, so no atomics are needed.
#include "common.h"
#include "launch.h"

namespace ts {

namespace {

template <typename T>
__device__ __forceinline__ float to_f32(T v) {
  return static_cast<float>(v);
}

template <typename T>
__device__ __forceinline__ T from_f32(float v) {
  return static_cast<T>(v);
}

// ---------------------------------------------------------------- direct (FMA)
struct DirectK {
  const uint64_t* tile_mask;
  const int32_t* tile_rows;
  const int32_t* nbr;  // [rows][kvol]
  int64_t n_tiles;
  int kvol;
  const void* src;
  int64_t n_src;       // rows of src and of dst (bounds-check build)
  int64_t n_dest;
  int c_src;
  const void* w;
  int w_cin, w_cout;
  bool transpose, mirror;
  void* dst;
  int c_dst;
};

// 256 threads = 16 tiles x 16 rows; each thread owns 8 destination channels
// (grid.y walks the 8-channel chunks).  With STAGE, the block first converts
// the 8-channel weight slice of every offset to fp32 in LDS ([o][ci][8]), so
// the inner loop reads weights as LDS broadcasts instead of global loads.
constexpr int kDirectLdsFloats = 12288;  // 48 KiB

template <typename T, typename OT, bool STAGE>
__global__ __launch_bounds__(256) void k_direct(DirectK a) {
  extern __shared__ __attribute__((aligned(16))) float wsh[];  // STAGE: kvol * c_src * 8 floats
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 16 + (threadIdx.x >> 4);
  const int r = threadIdx.x & 15;
  const int c0 = blockIdx.y * 8;
  const T* src = static_cast<const T*>(a.src);
  const T* w = static_cast<const T*>(a.w);
  const int c_src = a.c_src, kvol = a.kvol;
  if (STAGE) {
    const int total = kvol * c_src * 8;
    for (int i = threadIdx.x; i < total; i += 256) {
      const int e = i & 7;
      const int ci = (i >> 3) % c_src;
      const int o = (i >> 3) / c_src;
      const int os = a.mirror ? kvol - 1 - o : o;
      const int c = c0 + e;
      const T* wo = w + static_cast<int64_t>(os) * a.w_cin * a.w_cout;
      float v = 0.f;
      if (c < a.c_dst) v = to_f32(a.transpose ? wo[static_cast<int64_t>(c) * a.w_cout + ci] : wo[static_cast<int64_t>(ci) * a.w_cout + c]);
      wsh[i] = v;
    }
    __syncthreads();
  }
  if (t >= a.n_tiles) return;
  const uint64_t tm = a.tile_mask[t];
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int32_t row = dbg_opt(a.tile_rows[t * kTile + r], a.n_dest, TS_DEBUG_DST_ROW);
  for (uint64_t mm = row >= 0 ? tm : 0ull; mm; mm &= mm - 1) {
    const int o = __builtin_ctzll(mm);
    const int32_t nb = dbg_opt(a.nbr[static_cast<int64_t>(row) * kvol + o], a.n_src, TS_DEBUG_SRC_ROW);
    if (nb < 0) continue;
    const T* xs = src + static_cast<int64_t>(nb) * c_src;
    if (STAGE) {
      const float* wo = wsh + o * c_src * 8;
      for (int ci = 0; ci < c_src; ++ci) {
        const float xv = to_f32(xs[ci]);
        const float4 w0 = *reinterpret_cast<const float4*>(wo + ci * 8);
        const float4 w1 = *reinterpret_cast<const float4*>(wo + ci * 8 + 4);
        acc[0] = fmaf(xv, w0.x, acc[0]);
        acc[1] = fmaf(xv, w0.y, acc[1]);
        acc[2] = fmaf(xv, w0.z, acc[2]);
        acc[3] = fmaf(xv, w0.w, acc[3]);
        acc[4] = fmaf(xv, w1.x, acc[4]);
        acc[5] = fmaf(xv, w1.y, acc[5]);
        acc[6] = fmaf(xv, w1.z, acc[6]);
        acc[7] = fmaf(xv, w1.w, acc[7]);
      }
    } else {
      const int os = a.mirror ? kvol - 1 - o : o;
      const T* wo = w + static_cast<int64_t>(os) * a.w_cin * a.w_cout;
      for (int ci = 0; ci < c_src; ++ci) {
        const float xv = to_f32(xs[ci]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int c = c0 + e;
          if (c < a.c_dst) {
            const T wv = a.transpose ? wo[static_cast<int64_t>(c) * a.w_cout + ci] : wo[static_cast<int64_t>(ci) * a.w_cout + c];
            acc[e] = fmaf(xv, to_f32(wv), acc[e]);
          }
        }
      }
    }
  }
  if (row < 0) return;
  OT* out = static_cast<OT*>(a.dst) + static_cast<int64_t>(row) * a.c_dst;
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (c0 + e < a.c_dst) out[c0 + e] = from_f32<OT>(acc[e]);
}

// ---------------------------------------------------------------- gather-scatter
// One launch per offset o: thread = (pair, 8-channel chunk).  acc (fp32
// [n_dest][c_dst]) += src[src_row] . W[o] at dst_row.  With STAGE the offset's
// weights are first converted to fp32 in LDS ([ci][c_dst]) and read from
// there (broadcasts), instead of once per multiply from global memory.
template <typename T, bool STAGE>
__global__ __launch_bounds__(256) void k_gs_offset(const int64_t* __restrict__ pair_start, int o,
                                                   const int32_t* __restrict__ src_rows,
                                                   const int32_t* __restrict__ dst_rows, const T* __restrict__ src,
                                                   int64_t n_src, int c_src, const T* __restrict__ w, int w_cin,
                                                   int w_cout, bool transpose, float* __restrict__ acc,
                                                   int64_t n_dest, int c_dst) {
  extern __shared__ __attribute__((aligned(16))) float wsh[];  // STAGE: c_src * c_dst floats
  const int nchunk = (c_dst + 7) / 8;
  const T* wo = w + static_cast<int64_t>(o) * w_cin * w_cout;
  // blocks past this offset's pairs leave before staging (block-uniform)
  if (pair_start[o] + static_cast<int64_t>(blockIdx.x) * blockDim.x / nchunk >= pair_start[o + 1]) return;
  if (STAGE) {
    for (int i = threadIdx.x; i < c_src * c_dst; i += blockDim.x) {
      const int ci = i / c_dst, c = i % c_dst;
      wsh[i] = to_f32(transpose ? wo[static_cast<int64_t>(c) * w_cout + ci] : wo[static_cast<int64_t>(ci) * w_cout + c]);
    }
    __syncthreads();
  }
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t p = pair_start[o] + i / nchunk;
  if (p >= pair_start[o + 1]) return;
  const int c0 = static_cast<int>(i % nchunk) * 8;
  const T* xs = src + static_cast<int64_t>(dbg_req(src_rows[p], n_src, TS_DEBUG_SRC_ROW)) * c_src;
  float sum[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int ci = 0; ci < c_src; ++ci) {
    const float xv = to_f32(xs[ci]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = c0 + e;
      if (c < c_dst) {
        const float wv = STAGE ? wsh[ci * c_dst + c]
                               : to_f32(transpose ? wo[static_cast<int64_t>(c) * w_cout + ci]
                                                  : wo[static_cast<int64_t>(ci) * w_cout + c]);
        sum[e] = fmaf(xv, wv, sum[e]);
      }
    }
  }
  float* out = acc + static_cast<int64_t>(dbg_req(dst_rows[p], n_dest, TS_DEBUG_DST_ROW)) * c_dst;
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (c0 + e < c_dst) out[c0 + e] += sum[e];
}

template <typename OT>
__global__ __launch_bounds__(256) void k_cast_rows(const float* __restrict__ acc, int64_t n_elems,
                                                   const int64_t* n_rows, int c, OT* __restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t lim = n_rows ? (*n_rows) * c : n_elems;
  if (i < n_elems && i < lim) out[i] = from_f32<OT>(acc[i]);
}

// ---------------------------------------------------------------- fp32 on the matrix cores
// The same walk for fp32 features on v_mfma_f32_16x16x4_f32 (D[16][16] +=
// A[16][4] B[4][16] in fp32).  A wave owns one tile of 16 destination rows
// and one block of 16 destination channels:
//   A[m][k] = W[o][ci][co0 + m]   (the weights; dgrad: W[o][co0 + m][ci]),
//   B[k][n] = x[nbr(row n, o)][ci] (the gathered source rows, 0 if absent),
//   D[m][n] = y[row n][co0 + m],
// with lane l supplying A[l % 16][l / 16] and B[l / 16][l % 16] and holding
// D[4 (l / 16) + r][l % 16], r < 4.  For a block of 16 source channels ci0,
// lane l loads the 16 bytes x[nb][ci0 + 4 (l / 16) .. + 3] once; MFMA s of the
// block then contracts channel ci0 + 4 (l / 16) + s on both operands.  Each
// output row is written once, as 16-byte stores of 4 channels.
// Needs c_src and c_dst multiples of 16 and 16-byte aligned src and dst.
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_mfma_f32(DirectK a) {
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= a.n_tiles) return;  // wave-uniform
  const int n = lane & 15, g = lane >> 4;
  const int co0 = blockIdx.y * 16;
  const int kvol = a.kvol, c_src = a.c_src;
  const float* src = static_cast<const float*>(a.src);
  const float* w = static_cast<const float*>(a.w);
  const int32_t row = dbg_opt(a.tile_rows[t * kTile + n], a.n_dest, TS_DEBUG_DST_ROW);
  const uint64_t tm = a.tile_mask[t];
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (uint64_t mm = tm; mm; mm &= mm - 1) {  // wave-uniform
    const int o = __builtin_ctzll(mm);
    const int32_t nb = row >= 0 ? dbg_opt(a.nbr[static_cast<int64_t>(row) * kvol + o], a.n_src, TS_DEBUG_SRC_ROW) : -1;
    const int os = a.mirror ? kvol - 1 - o : o;
    const float* wo = w + static_cast<int64_t>(os) * a.w_cin * a.w_cout;
    const float* xs = src + static_cast<int64_t>(nb) * c_src;
    for (int ci0 = 0; ci0 < c_src; ci0 += 16) {
      const int ci = ci0 + 4 * g;
      f32x4_t xv = {0.f, 0.f, 0.f, 0.f};
      if (nb >= 0) xv = *reinterpret_cast<const f32x4_t*>(xs + ci);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float av = a.transpose ? wo[static_cast<int64_t>(co0 + n) * a.w_cout + ci + q]
                                     : wo[static_cast<int64_t>(ci + q) * a.w_cout + co0 + n];
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av, xv[q], acc, 0, 0, 0);
      }
    }
  }
  if (row < 0) return;
  *reinterpret_cast<f32x4_t*>(static_cast<float*>(a.dst) + static_cast<int64_t>(row) * a.c_dst + co0 + 4 * g) = acc;
}

bool mfma_f32_fits(const DirectK& k) {
  const uintptr_t s = reinterpret_cast<uintptr_t>(k.src), d = reinterpret_cast<uintptr_t>(k.dst);
  return k.c_src % 16 == 0 && k.c_dst % 16 == 0 && (s & 15) == 0 && (d & 15) == 0;
}

// ---------------------------------------------------------------- dispatch helpers
template <typename T, typename OT>
hipError_t direct_launch(const DirectK& k, hipStream_t s) {
  dim3 grid(static_cast<unsigned>(ceil_div<int64_t>(k.n_tiles, 16)), static_cast<unsigned>(ceil_div(k.c_dst, 8)));
  const int64_t floats = static_cast<int64_t>(k.kvol) * k.c_src * 8;
  if (floats <= kDirectLdsFloats)
    k_direct<T, OT, true><<<grid, 256, static_cast<size_t>(floats) * sizeof(float), s>>>(k);
  else
    k_direct<T, OT, false><<<grid, 256, 0, s>>>(k);
  return hipGetLastError();
}

template <typename T>
hipError_t direct_dispatch_out(const DirectK& k, ts_dtype out, hipStream_t s) {
  switch (out) {
    case TS_F32: return direct_launch<T, float>(k, s);
    case TS_F16: return direct_launch<T, _Float16>(k, s);
    default: return direct_launch<T, __bf16>(k, s);
  }
}

template <typename OT>
hipError_t cast_launch(const float* acc, int64_t n_rows_cap, const int64_t* n_rows, int c, void* out, hipStream_t s) {
  const int64_t n = n_rows_cap * c;
  if (n == 0) return hipSuccess;
  k_cast_rows<OT><<<static_cast<unsigned>(ceil_div<int64_t>(n, 256)), 256, 0, s>>>(acc, n, n_rows, c,
                                                                                    static_cast<OT*>(out));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_direct(const ConvArgs& a, hipStream_t s) {
  const ts_rel& rel = *a.rel;
  if (rel.n_tiles == 0) return hipSuccess;
  DirectK k;
  k.tile_mask = rel.tile_mask;
  k.tile_rows = rel.tile_rows;
  k.nbr = rel.nbr;
  k.n_tiles = rel.n_tiles;
  k.kvol = a.kvol;
  k.src = a.src;
  k.n_src = a.n_src;
  k.n_dest = rel.n_dest_cap;
  k.c_src = a.c_src;
  k.w = a.w;
  k.w_cin = a.w_cin;
  k.w_cout = a.w_cout;
  k.transpose = a.transpose;
  k.mirror = a.mirror;
  k.dst = a.dst;
  k.c_dst = a.c_dst;
  if (a.in_dtype == TS_F32 && mfma_f32_fits(k)) {  // fp32 in means fp32 out
    const dim3 grid(static_cast<unsigned>(ceil_div<int64_t>(k.n_tiles, 4)), static_cast<unsigned>(k.c_dst / 16));
    k_mfma_f32<<<grid, 256, 0, s>>>(k);
    return hipGetLastError();
  }
  switch (a.in_dtype) {
    case TS_F32: return direct_dispatch_out<float>(k, a.out_dtype, s);
    case TS_F16: return direct_dispatch_out<_Float16>(k, a.out_dtype, s);
    default: return direct_dispatch_out<__bf16>(k, a.out_dtype, s);
  }
}

// ---------------------------------------------------------------- pooling
// Thread = (destination slot, 8-channel chunk).  It walks the row's offsets
// in its mask and keeps the maximum, or the sum and the count, of the
// neighbours' channels in fp32 (the maximum of stored values is exact in any
// output type); an output with no neighbour gets 0.
struct PoolK {
  const int32_t* tile_rows;
  const uint64_t* row_mask;
  const int32_t* nbr;
  int64_t slots;
  int64_t n_src, n_dest;  // rows of src and of dst (bounds-check build)
  int kvol, c, nchunk;
  const void* src;
  void* dst;
  bool vec;  // channels a multiple of 8 and both buffers aligned to a whole vector
};

// Eight consecutive channels as one vector (16 bytes of fp16/bf16, 32 of
// fp32), for rows whose channel count is a multiple of 8.
template <typename T>
struct Vec8 {
  typedef T v __attribute__((ext_vector_type(8)));
};

template <typename T, typename OT, int MODE, bool VEC>
__global__ __launch_bounds__(256) void k_pool(PoolK a) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= a.slots * a.nchunk) return;
  const int64_t slot = i / a.nchunk;
  const int c0 = static_cast<int>(i - slot * a.nchunk) * 8;
  const int32_t row = dbg_opt(a.tile_rows[slot], a.n_dest, TS_DEBUG_DST_ROW);
  if (row < 0) return;
  const T* src = static_cast<const T*>(a.src);
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = MODE == TS_POOL_MAX ? -__builtin_inff() : 0.f;
  int count = 0;
  for (uint64_t mm = a.row_mask[row]; mm; mm &= mm - 1) {
    const int o = __builtin_ctzll(mm);
    const int32_t nb = dbg_opt(a.nbr[static_cast<int64_t>(row) * a.kvol + o], a.n_src, TS_DEBUG_SRC_ROW);
    if (nb < 0) continue;
    const T* xs = src + static_cast<int64_t>(nb) * a.c + c0;
    ++count;
    if (VEC) {
      const typename Vec8<T>::v v8 = *reinterpret_cast<const typename Vec8<T>::v*>(xs);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = to_f32(v8[e]);
        acc[e] = MODE == TS_POOL_MAX ? fmaxf(acc[e], v) : acc[e] + v;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (c0 + e >= a.c) break;
        const float v = to_f32(xs[e]);
        acc[e] = MODE == TS_POOL_MAX ? fmaxf(acc[e], v) : acc[e] + v;
      }
    }
  }
  OT* out = static_cast<OT*>(a.dst) + static_cast<int64_t>(row) * a.c + c0;
  const float inv = count > 0 ? 1.f / static_cast<float>(count) : 0.f;
  if (VEC) {
    typename Vec8<OT>::v o8;
#pragma unroll
    for (int e = 0; e < 8; ++e) o8[e] = from_f32<OT>(count == 0 ? 0.f : (MODE == TS_POOL_MAX ? acc[e] : acc[e] * inv));
    *reinterpret_cast<typename Vec8<OT>::v*>(out) = o8;
    return;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (c0 + e >= a.c) break;
    const float v = count == 0 ? 0.f : (MODE == TS_POOL_MAX ? acc[e] : acc[e] * inv);
    out[e] = from_f32<OT>(v);
  }
}

template <typename T, typename OT>
static hipError_t pool_mode(const PoolK& k, int mode, hipStream_t s) {
  const unsigned grid = static_cast<unsigned>(ceil_div<int64_t>(k.slots * k.nchunk, 256));
  if (mode == TS_POOL_MAX) {
    if (k.vec) k_pool<T, OT, TS_POOL_MAX, true><<<grid, 256, 0, s>>>(k);
    else k_pool<T, OT, TS_POOL_MAX, false><<<grid, 256, 0, s>>>(k);
  } else {
    if (k.vec) k_pool<T, OT, TS_POOL_AVG, true><<<grid, 256, 0, s>>>(k);
    else k_pool<T, OT, TS_POOL_AVG, false><<<grid, 256, 0, s>>>(k);
  }
  return hipGetLastError();
}

template <typename T>
static hipError_t pool_out(const PoolK& k, ts_dtype out, int mode, hipStream_t s) {
  switch (out) {
    case TS_F32: return pool_mode<T, float>(k, mode, s);
    case TS_F16: return pool_mode<T, _Float16>(k, mode, s);
    default: return pool_mode<T, __bf16>(k, mode, s);
  }
}

hipError_t launch_pool(const ts_rel& rel, int kvol, const void* x, int64_t n_src, int c, void* y, ts_dtype in,
                       ts_dtype out, int mode, hipStream_t s) {
  if (rel.n_tiles == 0) return hipSuccess;
  PoolK k;
  k.tile_rows = rel.tile_rows;
  k.row_mask = rel.row_mask;
  k.nbr = rel.nbr;
  k.slots = rel.n_tiles * kTile;
  k.n_src = n_src;
  k.n_dest = rel.n_dest_cap;
  k.kvol = kvol;
  k.c = c;
  k.nchunk = (c + 7) / 8;
  k.src = x;
  k.dst = y;
  const uintptr_t in_vec = 8 * (in == TS_F32 ? 4 : 2), out_vec = 8 * (out == TS_F32 ? 4 : 2);
  k.vec = c % 8 == 0 && reinterpret_cast<uintptr_t>(x) % in_vec == 0 && reinterpret_cast<uintptr_t>(y) % out_vec == 0;
  switch (in) {
    case TS_F32: return pool_out<float>(k, out, mode, s);
    case TS_F16: return pool_out<_Float16>(k, out, mode, s);
    default: return pool_out<__bf16>(k, out, mode, s);
  }
}

// ---------------------------------------------------------------- graph convolution
// Thread = (destination node, 8 output channels).  It walks the node's CSR
// edges in order (so the sum order is fixed) and accumulates x[src] . W[rel]
// in fp32.  An edge whose source or relation is out of range is skipped and
// raises TS_FLAG_RANGE.
struct GraphK {
  const int64_t* indptr;
  const int32_t* src;
  const int32_t* rel;
  int64_t n_dst, n_src;
  int n_rel;
  const void* x;
  int cin;
  const void* w;
  int cout, nchunk;
  void* y;
  uint32_t* flags;
};

template <typename T, typename OT>
__global__ __launch_bounds__(256) void k_graph(GraphK a) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= a.n_dst * a.nchunk) return;
  const int64_t v = i / a.nchunk;
  const int c0 = static_cast<int>(i - v * a.nchunk) * 8;
  const T* x = static_cast<const T*>(a.x);
  const T* w = static_cast<const T*>(a.w);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int64_t e1 = a.indptr[v + 1];
  bool bad = false;
  for (int64_t e = a.indptr[v]; e < e1; ++e) {
    const int32_t s = a.src[e], r = a.rel[e];
    if (s < 0 || s >= a.n_src || r < 0 || r >= a.n_rel) {
      bad = true;
      continue;
    }
    const T* xs = x + static_cast<int64_t>(s) * a.cin;
    const T* wr = w + static_cast<int64_t>(r) * a.cin * a.cout + c0;
    for (int ci = 0; ci < a.cin; ++ci) {
      const float xv = to_f32(xs[ci]);
      const T* wc = wr + static_cast<int64_t>(ci) * a.cout;
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8)
        if (c0 + e8 < a.cout) acc[e8] = fmaf(xv, to_f32(wc[e8]), acc[e8]);
    }
  }
  if (bad && a.flags) atomicOr(a.flags, TS_FLAG_RANGE);
  OT* out = static_cast<OT*>(a.y) + v * a.cout + c0;
#pragma unroll
  for (int e8 = 0; e8 < 8; ++e8)
    if (c0 + e8 < a.cout) out[e8] = from_f32<OT>(acc[e8]);
}

template <typename T>
static hipError_t graph_out(const GraphK& k, ts_dtype out, hipStream_t s) {
  const unsigned grid = static_cast<unsigned>(ceil_div<int64_t>(k.n_dst * k.nchunk, 256));
  switch (out) {
    case TS_F32: k_graph<T, float><<<grid, 256, 0, s>>>(k); break;
    case TS_F16: k_graph<T, _Float16><<<grid, 256, 0, s>>>(k); break;
    default: k_graph<T, __bf16><<<grid, 256, 0, s>>>(k); break;
  }
  return hipGetLastError();
}

hipError_t launch_graph_conv(const int64_t* indptr, const int32_t* src, const int32_t* rel, int64_t n_dst,
                             int64_t n_src, int n_rel, const void* x, int cin, const void* w, int cout, void* y,
                             ts_dtype in, ts_dtype out, uint32_t* flags, hipStream_t s) {
  if (n_dst == 0) return hipSuccess;
  GraphK k{indptr, src, rel, n_dst, n_src, n_rel, x, cin, w, cout, (cout + 7) / 8, y, flags};
  switch (in) {
    case TS_F32: return graph_out<float>(k, out, s);
    case TS_F16: return graph_out<_Float16>(k, out, s);
    default: return graph_out<__bf16>(k, out, s);
  }
}

size_t gs_workspace_bytes(int64_t n_dest_cap, int c_dst, ts_dtype out_dtype) {
  if (out_dtype == TS_F32) return 0;
  return align_up(static_cast<size_t>(n_dest_cap) * c_dst * 4, 256);
}

template <typename T>
static hipError_t gs_offsets(const ts_kmap* map, const ConvArgs& a, bool backward, int64_t n_dest_cap, float* acc,
                             hipStream_t s) {
  const int nchunk = (a.c_dst + 7) / 8;
  // pairs per offset never exceed the destination rows
  const int64_t threads = n_dest_cap * nchunk;
  if (threads == 0) return hipSuccess;
  const unsigned grid = static_cast<unsigned>(ceil_div<int64_t>(threads, 256));
  const int32_t* src_rows = backward ? map->pair_out : map->pair_in;
  const int32_t* dst_rows = backward ? map->pair_in : map->pair_out;
  const size_t lds = static_cast<size_t>(a.c_src) * a.c_dst * sizeof(float);
  const bool stage = lds <= 48 * 1024;
  for (int o = 0; o < a.kvol; ++o) {
    if (stage)
      k_gs_offset<T, true><<<grid, 256, lds, s>>>(map->pair_start, o, src_rows, dst_rows, static_cast<const T*>(a.src),
                                                  a.n_src, a.c_src, static_cast<const T*>(a.w), a.w_cin, a.w_cout,
                                                  a.transpose, acc, n_dest_cap, a.c_dst);
    else
      k_gs_offset<T, false><<<grid, 256, 0, s>>>(map->pair_start, o, src_rows, dst_rows, static_cast<const T*>(a.src),
                                                 a.n_src, a.c_src, static_cast<const T*>(a.w), a.w_cin, a.w_cout,
                                                 a.transpose, acc, n_dest_cap, a.c_dst);
  }
  return hipGetLastError();
}

hipError_t launch_gather_scatter(const ts_kmap* map, const ConvArgs& a, bool backward, int64_t n_dest_cap, void* ws,
                                 hipStream_t s) {
  float* acc = a.out_dtype == TS_F32 ? static_cast<float*>(a.dst) : static_cast<float*>(ws);
  const int64_t* n_rows = backward ? nullptr : map->n_out;
  hipError_t e = fill_f32(acc, n_dest_cap * a.c_dst, 0.f, s);
  if (e != hipSuccess) return e;
  switch (a.in_dtype) {
    case TS_F32: e = gs_offsets<float>(map, a, backward, n_dest_cap, acc, s); break;
    case TS_F16: e = gs_offsets<_Float16>(map, a, backward, n_dest_cap, acc, s); break;
    default: e = gs_offsets<__bf16>(map, a, backward, n_dest_cap, acc, s); break;
  }
  if (e != hipSuccess) return e;
  switch (a.out_dtype) {
    case TS_F32: return hipSuccess;
    case TS_F16: return cast_launch<_Float16>(acc, n_dest_cap, n_rows, a.c_dst, a.dst, s);
    default: return cast_launch<__bf16>(acc, n_dest_cap, n_rows, a.c_dst, a.dst, s);
  }
}

}  // namespace ts

TS_DEBUG_TU(conv)
