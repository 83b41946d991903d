// Map-driven contraction: y[j] = sum_o x[nbr(j, o)] . W[o]  (forward) and the
// same walk with W[o]^T for dgrad.  The TorchSparse++ abstract names the
// implicit-GEMM and gather-GEMM-scatter dataflows; the torch-lattice page
// "Migrating from TorchSparse" (section "Backend and configuration
// differences") requires every dataflow to give the same result for a fixed
// relation and weight tensor.
//
// Dataflows here:
//  * implicit GEMM (k_igemm): one wave owns G tiles of 16 destination rows
//    and walks the offsets present in their tile masks.  Per offset it
//    gathers the 16 source rows straight from HBM/L2 into MFMA B fragments
//    (16 bytes per lane) and multiplies them with the packed weight slice
//    (A fragments).  D = W^T . X^T, so each lane ends holding 4 consecutive
//    output channels of one row and every output row is written once.
//  * direct (k_direct): the same output-stationary walk with FMA, for fp32
//    and for channel counts the MFMA shapes do not fit.
//  * gather-scatter (k_gs_offset): offsets one after another in fixed order;
//    per offset, gather the source rows of its pairs, multiply by W[o] and add
//    into an fp32 accumulator at the destination rows.  Within one offset the
//    destination rows are distinct, so no atomics are needed.
#include <stdlib.h>

#include "common.h"
#include "launch.h"

namespace ts {

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct Mfma;

template <>
struct Mfma<_Float16> {
  typedef f16x8 frag;
  static __device__ __forceinline__ f32x4 run(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Mfma<__bf16> {
  typedef bf16x8 frag;
  static __device__ __forceinline__ f32x4 run(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <typename F>
__device__ __forceinline__ F load_frag(const void* p) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  return __builtin_bit_cast(F, v);
}

template <typename T>
__device__ __forceinline__ float to_f32(T v) {
  return static_cast<float>(v);
}

template <typename T>
__device__ __forceinline__ T from_f32(float v) {
  return static_cast<T>(v);
}

// ---------------------------------------------------------------- weights
// wpack[o][mb][kb][lane][8] = A[m][k] with m = mb*16 + lane%16 (destination
// channel), k = kb*32 + (lane/16)*8 + e (source channel), where
//   forward: A[m][k] = W[o][k][m]
//   dgrad:   A[m][k] = W[o'][m][k],  o' = kvol-1-o for a submanifold map.
template <typename T>
__global__ __launch_bounds__(256) void k_pack_w(const T* __restrict__ w, int w_cin, int w_cout, int kvol, int c_src,
                                                int c_dst, bool transpose, bool mirror, T* __restrict__ wpack) {
  const int mbt = c_dst / 16, kbt = c_src / 32;
  const int64_t total = static_cast<int64_t>(kvol) * mbt * kbt * 512;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int e = static_cast<int>(i & 7);
  const int lane = static_cast<int>((i >> 3) & 63);
  int64_t rest = i >> 9;
  const int kb = static_cast<int>(rest % kbt);
  rest /= kbt;
  const int mb = static_cast<int>(rest % mbt);
  const int o = static_cast<int>(rest / mbt);
  const int m = mb * 16 + (lane & 15);
  const int k = kb * 32 + (lane >> 4) * 8 + e;
  const int os = mirror ? kvol - 1 - o : o;
  const int64_t base = static_cast<int64_t>(os) * w_cin * w_cout;
  wpack[i] = transpose ? w[base + static_cast<int64_t>(m) * w_cout + k] : w[base + static_cast<int64_t>(k) * w_cout + m];
}

// ---------------------------------------------------------------- implicit GEMM
// Where the A fragments (weights) come from:
//   kWPacked:  wpack[o][mb][kb][lane][8], one 16-byte load per fragment;
//   kWContig:  dgrad, A[m][k] = W[o'][m][k]: the 8 k values are contiguous in
//              the layer's [kvol][cin][cout] weights, one 16-byte load;
//   kWStrided: forward, A[m][k] = W[o][k][m]: 8 two-byte loads, one per k,
//              each coalesced over the 16 lanes that share k.
enum WMode { kWPacked = 0, kWContig = 1, kWStrided = 2 };

struct IgemmK {
  const uint64_t* tile_mask;
  const int32_t* tile_rows;
  const int32_t* pool;
  int64_t n_tiles;
  int kvol;
  const void* src;
  int c_src;
  const void* wpack;  // kWPacked
  const void* w;      // the layer's weights [kvol][w_cin][w_cout]
  int w_cout;
  int mirror;
  void* dst;
  int c_dst;
  int mbt, kbt;
};

template <typename T, typename Frag, int WM>
__device__ __forceinline__ Frag load_a(const IgemmK& a, int o, int mb, int kb, int lane) {
  if (WM == kWPacked) {
    const T* wp = static_cast<const T*>(a.wpack);
    return load_frag<Frag>(wp + ((static_cast<int64_t>(o) * a.mbt + mb) * a.kbt + kb) * 512 + lane * 8);
  }
  const T* w = static_cast<const T*>(a.w);
  const int m = mb * 16 + (lane & 15);
  const int k = kb * 32 + (lane >> 4) * 8;
  if (WM == kWContig) {
    const int os = a.mirror ? a.kvol - 1 - o : o;
    // A[m][k] = W[os][m][k]: row m of the slice has w_cout = c_src entries
    return load_frag<Frag>(w + (static_cast<int64_t>(os) * a.c_dst + m) * a.c_src + k);
  }
  // A[m][k] = W[o][k][m]: rows of length w_cout = c_dst
  const T* base = w + (static_cast<int64_t>(o) * a.c_src + k) * a.c_dst + m;
  Frag f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = base[static_cast<int64_t>(e) * a.c_dst];
  return f;
}

template <typename T, typename OT, int MB, int G, int WM>
__global__ __launch_bounds__(256) void k_igemm(IgemmK a) {
  typedef typename Mfma<T>::frag Frag;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15;  // tile slot this lane gathers / writes
  const int kq = lane >> 4;   // which 8-wide k group of the fragment
  const int64_t tbase = (static_cast<int64_t>(blockIdx.x) * 4 + wave) * G;
  const int mb0 = blockIdx.y * MB;

  uint64_t m[G];
  uint64_t uni = 0;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = (tbase + g < a.n_tiles) ? a.tile_mask[tbase + g] : 0ull;
    uni |= m[g];
  }
  f32x4 acc[G][MB];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[g][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const T* src = static_cast<const T*>(a.src);
  for (uint64_t mm = uni; mm; mm &= mm - 1) {
    const int o = __builtin_ctzll(mm);
    const uint64_t below = (1ull << o) - 1;
    int32_t nb[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      nb[g] = -1;
      if ((m[g] >> o) & 1) {
        const int k = __popcll(m[g] & below);
        nb[g] = a.pool[((tbase + g) * a.kvol + k) * kTile + col];
      }
    }
    for (int kb = 0; kb < a.kbt; ++kb) {
      Frag af[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int mbg = mb0 + mb < a.mbt ? mb0 + mb : a.mbt - 1;
        af[mb] = load_a<T, Frag, WM>(a, o, mbg, kb, lane);
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if (!((m[g] >> o) & 1)) continue;  // wave-uniform
        Frag bf;
        if (nb[g] >= 0) {
          bf = load_frag<Frag>(src + static_cast<int64_t>(nb[g]) * a.c_src + kb * 32 + kq * 8);
        } else {
          bf = Frag{};
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[g][mb] = Mfma<T>::run(af[mb], bf, acc[g][mb]);
      }
    }
  }

  OT* dst = static_cast<OT*>(a.dst);
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (tbase + g >= a.n_tiles) continue;
    const int32_t row = a.tile_rows[(tbase + g) * kTile + col];
    if (row < 0) continue;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (mb0 + mb >= a.mbt) continue;
      OT* out = dst + static_cast<int64_t>(row) * a.c_dst + (mb0 + mb) * 16 + kq * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) out[e] = from_f32<OT>(acc[g][mb][e]);
    }
  }
}

// ---------------------------------------------------------------- direct (FMA)
struct DirectK {
  const uint64_t* tile_mask;
  const int32_t* tile_rows;
  const int32_t* pool;
  int64_t n_tiles;
  int kvol;
  const void* src;
  int c_src;
  const void* w;
  int w_cin, w_cout;
  bool transpose, mirror;
  void* dst;
  int c_dst;
};

// 256 threads = 16 tiles x 16 rows; each thread owns 8 destination channels
// (grid.y walks the 8-channel chunks).
template <typename T, typename OT>
__global__ __launch_bounds__(256) void k_direct(DirectK a) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 16 + (threadIdx.x >> 4);
  const int r = threadIdx.x & 15;
  if (t >= a.n_tiles) return;
  const int c0 = blockIdx.y * 8;
  const uint64_t tm = a.tile_mask[t];
  const T* src = static_cast<const T*>(a.src);
  const T* w = static_cast<const T*>(a.w);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int k = 0;
  for (uint64_t mm = tm; mm; mm &= mm - 1, ++k) {
    const int o = __builtin_ctzll(mm);
    const int32_t nb = a.pool[(t * a.kvol + k) * kTile + r];
    if (nb < 0) continue;
    const int os = a.mirror ? a.kvol - 1 - o : o;
    const T* wo = w + static_cast<int64_t>(os) * a.w_cin * a.w_cout;
    const T* xs = src + static_cast<int64_t>(nb) * a.c_src;
    for (int ci = 0; ci < a.c_src; ++ci) {
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
  const int32_t row = a.tile_rows[t * kTile + r];
  if (row < 0) return;
  OT* out = static_cast<OT*>(a.dst) + static_cast<int64_t>(row) * a.c_dst;
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (c0 + e < a.c_dst) out[c0 + e] = from_f32<OT>(acc[e]);
}

// ---------------------------------------------------------------- gather-scatter
// One launch per offset o: thread = (pair, 8-channel chunk).  acc (fp32
// [n_dest][c_dst]) += src[src_row] . W[o] at dst_row.
template <typename T>
__global__ __launch_bounds__(256) void k_gs_offset(const int64_t* __restrict__ pair_start, int o,
                                                   const int32_t* __restrict__ src_rows,
                                                   const int32_t* __restrict__ dst_rows, const T* __restrict__ src,
                                                   int c_src, const T* __restrict__ w, int w_cin, int w_cout,
                                                   bool transpose, float* __restrict__ acc, int c_dst) {
  const int nchunk = (c_dst + 7) / 8;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t p = pair_start[o] + i / nchunk;
  if (p >= pair_start[o + 1]) return;
  const int c0 = static_cast<int>(i % nchunk) * 8;
  const T* xs = src + static_cast<int64_t>(src_rows[p]) * c_src;
  const T* wo = w + static_cast<int64_t>(o) * w_cin * w_cout;
  float sum[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int ci = 0; ci < c_src; ++ci) {
    const float xv = to_f32(xs[ci]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = c0 + e;
      if (c < c_dst) {
        const T wv = transpose ? wo[static_cast<int64_t>(c) * w_cout + ci] : wo[static_cast<int64_t>(ci) * w_cout + c];
        sum[e] = fmaf(xv, to_f32(wv), sum[e]);
      }
    }
  }
  float* out = acc + static_cast<int64_t>(dst_rows[p]) * c_dst;
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

// ---------------------------------------------------------------- dispatch helpers
template <typename T, typename OT, int MB, int WM>
hipError_t igemm_launch_mb(const IgemmK& k, hipStream_t s) {
  constexpr int G = 2;
  dim3 grid(static_cast<unsigned>(ceil_div<int64_t>(k.n_tiles, 4 * G)), static_cast<unsigned>(ceil_div(k.mbt, MB)));
  k_igemm<T, OT, MB, G, WM><<<grid, 256, 0, s>>>(k);
  return hipGetLastError();
}

template <typename T, typename OT, int WM>
hipError_t igemm_launch_w(const IgemmK& k, hipStream_t s) {
  if (k.mbt >= 8) return igemm_launch_mb<T, OT, 8, WM>(k, s);
  if (k.mbt >= 4) return igemm_launch_mb<T, OT, 4, WM>(k, s);
  if (k.mbt >= 2) return igemm_launch_mb<T, OT, 2, WM>(k, s);
  return igemm_launch_mb<T, OT, 1, WM>(k, s);
}

template <typename T, typename OT>
hipError_t igemm_launch(const IgemmK& k, int wm, hipStream_t s) {
  if (wm == kWPacked) return igemm_launch_w<T, OT, kWPacked>(k, s);
  if (wm == kWContig) return igemm_launch_w<T, OT, kWContig>(k, s);
  return igemm_launch_w<T, OT, kWStrided>(k, s);
}

template <typename T>
hipError_t pack_launch(const ConvArgs& a, void* wpack, hipStream_t s) {
  const int64_t total = static_cast<int64_t>(a.kvol) * (a.c_dst / 16) * (a.c_src / 32) * 512;
  k_pack_w<T><<<static_cast<unsigned>(ceil_div<int64_t>(total, 256)), 256, 0, s>>>(
      static_cast<const T*>(a.w), a.w_cin, a.w_cout, a.kvol, a.c_src, a.c_dst, a.transpose, a.mirror,
      static_cast<T*>(wpack));
  return hipGetLastError();
}

template <typename T, typename OT>
hipError_t direct_launch(const DirectK& k, hipStream_t s) {
  dim3 grid(static_cast<unsigned>(ceil_div<int64_t>(k.n_tiles, 16)), static_cast<unsigned>(ceil_div(k.c_dst, 8)));
  k_direct<T, OT><<<grid, 256, 0, s>>>(k);
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

bool igemm_supported(int c_src, int c_dst, ts_dtype in_dtype) {
  return in_dtype != TS_F32 && c_src % 32 == 0 && c_dst % 16 == 0 && c_src > 0 && c_dst > 0;
}

// Packing the forward weights into fragment order is optional: the direct
// (strided) loads avoid a second kernel launch per call.
static bool igemm_pack_forward() {
  static const bool pack = [] {
    const char* e = getenv("TS_IGEMM_PACK");
    return e && e[0] == '1';
  }();
  return pack;
}

size_t igemm_workspace_bytes(int kvol, int c_src, int c_dst) {
  return align_up(static_cast<size_t>(kvol) * c_src * c_dst * 2, 256);
}

hipError_t launch_igemm(const ConvArgs& a, void* ws, hipStream_t s) {
  const ts_rel& rel = *a.rel;
  if (rel.n_tiles == 0) return hipSuccess;
  int wm = a.transpose ? kWContig : kWStrided;
  if (wm == kWStrided && igemm_pack_forward() && ws) {
    hipError_t e = a.in_dtype == TS_F16 ? pack_launch<_Float16>(a, ws, s) : pack_launch<__bf16>(a, ws, s);
    if (e != hipSuccess) return e;
    wm = kWPacked;
  }
  IgemmK k;
  k.tile_mask = rel.tile_mask;
  k.tile_rows = rel.tile_rows;
  k.pool = rel.pool;
  k.n_tiles = rel.n_tiles;
  k.kvol = a.kvol;
  k.src = a.src;
  k.c_src = a.c_src;
  k.wpack = ws;
  k.w = a.w;
  k.w_cout = a.w_cout;
  k.mirror = a.mirror ? 1 : 0;
  k.dst = a.dst;
  k.c_dst = a.c_dst;
  k.mbt = a.c_dst / 16;
  k.kbt = a.c_src / 32;
  if (a.in_dtype == TS_F16) {
    switch (a.out_dtype) {
      case TS_F32: return igemm_launch<_Float16, float>(k, wm, s);
      case TS_F16: return igemm_launch<_Float16, _Float16>(k, wm, s);
      default: return igemm_launch<_Float16, __bf16>(k, wm, s);
    }
  }
  switch (a.out_dtype) {
    case TS_F32: return igemm_launch<__bf16, float>(k, wm, s);
    case TS_F16: return igemm_launch<__bf16, _Float16>(k, wm, s);
    default: return igemm_launch<__bf16, __bf16>(k, wm, s);
  }
}

hipError_t launch_direct(const ConvArgs& a, hipStream_t s) {
  const ts_rel& rel = *a.rel;
  if (rel.n_tiles == 0) return hipSuccess;
  DirectK k;
  k.tile_mask = rel.tile_mask;
  k.tile_rows = rel.tile_rows;
  k.pool = rel.pool;
  k.n_tiles = rel.n_tiles;
  k.kvol = a.kvol;
  k.src = a.src;
  k.c_src = a.c_src;
  k.w = a.w;
  k.w_cin = a.w_cin;
  k.w_cout = a.w_cout;
  k.transpose = a.transpose;
  k.mirror = a.mirror;
  k.dst = a.dst;
  k.c_dst = a.c_dst;
  switch (a.in_dtype) {
    case TS_F32: return direct_dispatch_out<float>(k, a.out_dtype, s);
    case TS_F16: return direct_dispatch_out<_Float16>(k, a.out_dtype, s);
    default: return direct_dispatch_out<__bf16>(k, a.out_dtype, s);
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
  for (int o = 0; o < a.kvol; ++o) {
    k_gs_offset<T><<<grid, 256, 0, s>>>(map->pair_start, o, src_rows, dst_rows, static_cast<const T*>(a.src), a.c_src,
                                        static_cast<const T*>(a.w), a.w_cin, a.w_cout, a.transpose, acc, a.c_dst);
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
