// Implicit-GEMM contraction on MFMA (fp16 / bf16 in, fp32 accumulate).
//
// Computes, over a tiled relation, D[row][n] = sum_o sum_k A_o[n][k] X[src(row,o)][k]
// where A_o is the weight slice of offset o:
//   forward:  A_o[n][k] = W[o][k][n]      (W = [kvol][c_src][c_dst])
//   dgrad:    A_o[n][k] = W[o'][n][k]     (W = [kvol][c_dst][c_src]; o' = kvol-1-o
//                                          for a submanifold map, else o)
// The TorchSparse++ abstract credits this dataflow (computation overlapped
// with memory access) for its speed; the relation is the kernel map of the
// torch-lattice page "Migrating from TorchSparse".
//
// First a small kernel packs the weights into MFMA fragment order (16-byte
// chunks, fragment (o, mb, kb) = 64 consecutive chunks), so every later copy
// of a slice is a straight coalesced 16-byte copy.
//
// Work split.  A block of 4 waves owns 4*G tiles of 16 destination rows (each
// wave G tiles, the output channels of one block column).  The block walks
// the union of its tiles' offset masks in ascending order.  Per offset:
//   * the packed weight slice is copied into LDS once per block;
//   * each wave gathers, for each of its tiles that has the offset, the 16
//     source rows straight into B fragments (16 bytes per lane);
//   * v_mfma_f32_16x16x32 with D = A . X^T, so a lane ends holding 4
//     consecutive output channels of one row.
// Latency: the neighbour rows of a tile's 16 rows (the source row of each
// slot at each offset) are loaded once, up front, into registers and picked
// per offset with a lane shuffle, so no load address waits on another load
// inside the loop.  Gathers and weight loads run two offsets ahead (three register sets
// of gathers, two LDS weight buffers, one barrier per offset); each step first
// stores the weights loaded one step earlier into the free LDS buffer, then
// issues the next weight loads before its gathers, so that the in-order load
// counter never forces a gather to land early.  Every output
// row is written once, no atomics.  Blocks are numbered so that each XCD walks
// a contiguous range of tiles (its L2 keeps the gathered rows).
#include <stdlib.h>

#include "common.h"
#include "launch.h"

namespace ts {

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));  // one 16-byte chunk

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

// Neighbours held per tile and lane: lane (col, q) keeps offsets o = q*kNbRegs
// + j, j < kNbRegs, of the row in slot col, so kernels of up to 4 * kNbRegs
// offsets are supported.
constexpr int kNbRegs = 7;
constexpr int kMaxIgemmKvol = 4 * kNbRegs;

struct IgK {
  const uint64_t* tile_mask;
  const int32_t* tile_rows;
  const int32_t* nbr;  // [rows][kvol]
  int64_t n_tiles;
  int kvol;
  const void* src;
  int c_src;
  const u32x4* wp;  // packed fragments [kvol][mbt][c_src/32][64]
  int mbt;          // fragments of 16 output channels in the packed weights
  void* dst;
  int c_dst;
  int out_dtype;
  int64_t nblk;  // logical blocks
  int64_t nb8;   // ceil(nblk / 8)
  int xcd_map;   // number blocks so that each XCD walks a contiguous range
};

// Packed chunk i = ((o * mbt + mb) * kbn + kb) * 64 + lane holds A_o[n][k..k+7]
// with n = mb*16 + lane%16, k = kb*32 + (lane/16)*8; zero for n >= c_dst.
template <typename T>
__global__ __launch_bounds__(256) void k_wpack(const T* __restrict__ w, int kvol, int c_src, int c_dst, int mbt,
                                               int trans, int mirror, u32x4* __restrict__ out) {
  const int kbn = c_src / 32;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= static_cast<int64_t>(kvol) * mbt * kbn * 64) return;
  const int lane = static_cast<int>(i & 63);
  int64_t r = i >> 6;
  const int kb = static_cast<int>(r % kbn);
  r /= kbn;
  const int mb = static_cast<int>(r % mbt);
  const int o = static_cast<int>(r / mbt);
  const int n = mb * 16 + (lane & 15);
  const int k0 = kb * 32 + (lane >> 4) * 8;
  const int64_t slice = static_cast<int64_t>(c_src) * c_dst;
  u32x4 v = {0u, 0u, 0u, 0u};
  if (n < c_dst) {
    if (trans) {
      const int os = mirror ? kvol - 1 - o : o;
      v = *reinterpret_cast<const u32x4*>(w + os * slice + static_cast<int64_t>(n) * c_src + k0);
    } else {
      unsigned short e[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) e[j] = __builtin_bit_cast(unsigned short, w[o * slice + static_cast<int64_t>(k0 + j) * c_dst + n]);
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = static_cast<unsigned>(e[2 * j]) | (static_cast<unsigned>(e[2 * j + 1]) << 16);
    }
  }
  out[i] = v;
}

__device__ __forceinline__ int next_bit(uint64_t u, int o) {
  if (o < 0 || o >= 63) return -1;
  const uint64_t rest = u & ~((2ull << o) - 1);
  return rest ? __builtin_ctzll(rest) : -1;
}

template <typename T, int MB, int KB, int G>
__global__ __launch_bounds__(256) void k_igemm(IgK a) {
  typedef typename Mfma<T>::frag Frag;
  constexpr int FR = MB * KB;                      // fragments per offset and block column
  constexpr int CHUNKS = FR * 64;                  // 16-byte chunks per weight slice
  constexpr int CH = (CHUNKS + 255) / 256;         // per thread
  __shared__ u32x4 wl[2][CHUNKS];
  __shared__ uint64_t wunion[4];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15;
  const int kq = lane >> 4;
  const int64_t hb = blockIdx.x;
  const int64_t lb = a.xcd_map ? (hb & 7) * a.nb8 + (hb >> 3) : hb;  // XCD-contiguous numbering
  if (lb >= a.nblk) return;                        // whole block, before any barrier
  const int mb0 = blockIdx.y * MB;
  const int64_t t0 = (lb * 4 + wave) * G;
  const int kvol = a.kvol;

  // masks, destination rows and their neighbours (first loads of the kernel)
  uint64_t m[G];
  int32_t pr[G][kNbRegs];
  uint64_t u = 0;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const bool live = t0 + g < a.n_tiles;
    const int64_t tile = live ? t0 + g : 0;
    m[g] = live ? a.tile_mask[tile] : 0ull;
    u |= m[g];
    const int32_t drow = a.tile_rows[tile * kTile + col];
    const int32_t* nrow = a.nbr + static_cast<int64_t>(drow >= 0 ? drow : 0) * kvol;
#pragma unroll
    for (int j = 0; j < kNbRegs; ++j) {
      const int o = kq * kNbRegs + j;
      const int32_t v = nrow[o < kvol ? o : 0];
      pr[g][j] = drow >= 0 ? v : -1;
    }
  }
  if (lane == 0) wunion[wave] = u;
  __syncthreads();
  const uint64_t U = wunion[0] | wunion[1] | wunion[2] | wunion[3];

  f32x4 acc[G][MB];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[g][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const T* src = static_cast<const T*>(a.src);
  const int c_src = a.c_src, c_dst = a.c_dst;

  // Source row of slot `col` of tile g at offset o: register o % kNbRegs of
  // lane col + 16 * (o / kNbRegs).
  auto pool_row = [&](int g, int o) -> int32_t {
    const int q = o / kNbRegs, j = o - q * kNbRegs;
    int32_t v = pr[g][0];
#pragma unroll
    for (int jj = 1; jj < kNbRegs; ++jj) v = (j == jj) ? pr[g][jj] : v;
    return __shfl(v, col + 16 * q, 64);
  };
  // Gathers of offset o, branch-free (row 0 when there is nothing to fetch);
  // ok[g] marks a present row, and consumers zero the others.
  auto gather = [&](int o, Frag (&x)[G][KB], bool (&ok)[G]) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int32_t nb = pool_row(g, o);
      ok[g] = ((m[g] >> o) & 1) && nb >= 0;
      const T* row = src + static_cast<int64_t>(ok[g] ? nb : 0) * c_src + kq * 8;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) x[g][kb] = __builtin_bit_cast(Frag, *reinterpret_cast<const u32x4*>(row + kb * 32));
    }
  };
  // This thread's chunks of the packed slice of offset o.  Chunks of
  // fragments past the packed column count read the slice start: they land in
  // fragment rows of output channels that are never written out.
  auto wload = [&](int o, u32x4 (&r)[CH]) {
    const int64_t base = (static_cast<int64_t>(o) * a.mbt + mb0) * KB * 64;
    const int64_t lim = (static_cast<int64_t>(o) * a.mbt + a.mbt) * KB * 64;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int i = threadIdx.x + c * 256;
      const int64_t idx = base + (i < CHUNKS ? i : 0);
      r[c] = a.wp[idx < lim ? idx : base];
    }
  };
  auto wstore = [&](const u32x4 (&r)[CH], u32x4* buf) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int i = threadIdx.x + c * 256;
      if ((c + 1) * 256 <= CHUNKS || i < CHUNKS) buf[i] = r[c];
    }
  };

  if (U) {
    // Offsets u_0 < u_1 < ... of U.  Entering step i: LDS buffer i%2 holds
    // W(u_i); the weight registers hold W(u_{i+1}); gather set i%3 holds
    // X(u_i) (issued at step i-2) and set (i+1)%3 holds X(u_{i+1}).  Past the
    // last offset the prefetches repeat a valid offset (harmless loads).
    int o0 = __builtin_ctzll(U);
    int o1 = next_bit(U, o0);
    int o2 = o1 >= 0 ? next_bit(U, o1) : -1;
    Frag x0[G][KB], x1[G][KB], x2[G][KB];
    bool k0[G], k1[G], k2[G];
    u32x4 wr[CH];
    wload(o0, wr);
    gather(o0, x0, k0);
    gather(o1 >= 0 ? o1 : o0, x1, k1);
    wstore(wr, wl[0]);
    wload(o1 >= 0 ? o1 : o0, wr);
    __syncthreads();

    auto step = [&](Frag (&xc)[G][KB], bool (&kc)[G], Frag (&xf)[G][KB], bool (&kf)[G], u32x4 (&w)[CH],
                    int b) -> bool {
      const int okeep = o2 >= 0 ? o2 : (o1 >= 0 ? o1 : o0);
      wstore(w, wl[b ^ 1]);                       // W(u_{i+1}), loaded one step ago
      wload(okeep, w);                            // W(u_{i+2}), before the gathers
      gather(okeep, xf, kf);                      // X(u_{i+2})
      const u32x4* lw = wl[b];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        Frag af[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) af[mb] = __builtin_bit_cast(Frag, lw[(mb * KB + kb) * 64 + lane]);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          if (!((m[g] >> o0) & 1)) continue;  // wave-uniform
          const Frag bx = kc[g] ? xc[g][kb] : Frag{};
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) acc[g][mb] = Mfma<T>::run(af[mb], bx, acc[g][mb]);
        }
      }
      if (o1 < 0) return false;
      __syncthreads();
      o0 = o1;
      o1 = o2;
      o2 = o2 >= 0 ? next_bit(U, o2) : -1;
      return true;
    };
    while (step(x0, k0, x2, k2, wr, 0) && step(x1, k1, x0, k0, wr, 1) && step(x2, k2, x1, k1, wr, 0) &&
           step(x0, k0, x2, k2, wr, 1) && step(x1, k1, x0, k0, wr, 0) && step(x2, k2, x1, k1, wr, 1)) {
    }
  }

  // write each destination row once
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (t0 + g >= a.n_tiles) continue;
    const int32_t row = a.tile_rows[(t0 + g) * kTile + col];
    if (row < 0) continue;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int n = (mb0 + mb) * 16 + kq * 4;
      if (n >= c_dst) continue;
      const int64_t off = static_cast<int64_t>(row) * c_dst + n;
      const f32x4 v = acc[g][mb];
      if (a.out_dtype == TS_F32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(a.dst) + off) = v;
      } else if (a.out_dtype == TS_F16) {
        typedef _Float16 h4 __attribute__((ext_vector_type(4)));
        h4 h = {static_cast<_Float16>(v[0]), static_cast<_Float16>(v[1]), static_cast<_Float16>(v[2]),
                static_cast<_Float16>(v[3])};
        *reinterpret_cast<h4*>(static_cast<_Float16*>(a.dst) + off) = h;
      } else {
        typedef __bf16 b4 __attribute__((ext_vector_type(4)));
        b4 h = {static_cast<__bf16>(v[0]), static_cast<__bf16>(v[1]), static_cast<__bf16>(v[2]),
                static_cast<__bf16>(v[3])};
        *reinterpret_cast<b4*>(static_cast<__bf16*>(a.dst) + off) = h;
      }
    }
  }
}

// Tiles per wave.  Default 1: more blocks in flight and a smaller offset
// union per block beat sharing a weight slice across more tiles; the
// environment variable TS_IGEMM_G (1, 2 or 4) overrides it for tuning.
static int tiles_per_wave(int mb) {
  static const int forced = [] {
    const char* e = getenv("TS_IGEMM_G");
    return e ? atoi(e) : 0;
  }();
  (void)mb;
  if (forced == 1 || forced == 2 || forced == 4) return forced;
  return 1;
}

// Workgroups are dealt to the 8 XCDs round-robin; numbering blocks so that
// XCD x gets a contiguous range keeps each XCD's gathers in its own L2.
// TS_IGEMM_XCD=0 switches the renumbering off (tuning).
static int xcd_map_on() {
  static const int on = [] {
    const char* e = getenv("TS_IGEMM_XCD");
    return e && e[0] == '0' ? 0 : 1;
  }();
  return on;
}

template <typename T, int MB, int KB, int G>
hipError_t launch_g(IgK k, hipStream_t s) {
  k.nblk = ceil_div<int64_t>(k.n_tiles, 4 * G);
  k.nb8 = ceil_div<int64_t>(k.nblk, 8);
  k.xcd_map = xcd_map_on();
  dim3 grid(static_cast<unsigned>(k.xcd_map ? k.nb8 * 8 : k.nblk), static_cast<unsigned>(ceil_div(k.c_dst / 16, MB)));
  k_igemm<T, MB, KB, G><<<grid, 256, 0, s>>>(k);
  return hipGetLastError();
}

template <typename T, int MB, int KB>
hipError_t launch_mb_kb(const IgK& k, hipStream_t s) {
  switch (tiles_per_wave(MB)) {
    case 1: return launch_g<T, MB, KB, 1>(k, s);
    case 2: return launch_g<T, MB, KB, 2>(k, s);
    default: return launch_g<T, MB, KB, 4>(k, s);
  }
}

template <typename T, int MB>
hipError_t launch_mb(const IgK& k, hipStream_t s) {
  switch (k.c_src / 32) {
    case 1: return launch_mb_kb<T, MB, 1>(k, s);
    case 2: return launch_mb_kb<T, MB, 2>(k, s);
    case 3: return launch_mb_kb<T, MB, 3>(k, s);
    default: return launch_mb_kb<T, MB, 4>(k, s);
  }
}

// Output channels per block column: up to 128 (8 fragments) by default;
// TS_IGEMM_MB (1, 2, 4 or 8 fragments of 16 channels) lowers it for tuning.
static int max_mb() {
  static const int forced = [] {
    const char* e = getenv("TS_IGEMM_MB");
    const int v = e ? atoi(e) : 0;
    return (v == 1 || v == 2 || v == 4 || v == 8) ? v : 8;
  }();
  return forced;
}

template <typename T>
hipError_t launch_t(const IgK& k, hipStream_t s) {
  int mbt = k.c_dst / 16;
  if (mbt > max_mb()) mbt = max_mb();
  if (mbt > 4) return launch_mb<T, 8>(k, s);
  if (mbt > 2) return launch_mb<T, 4>(k, s);
  if (mbt > 1) return launch_mb<T, 2>(k, s);
  return launch_mb<T, 1>(k, s);
}

}  // namespace

bool igemm_supported(int kvol, int c_src, int c_dst, ts_dtype in_dtype) {
  return in_dtype != TS_F32 && kvol >= 1 && kvol <= kMaxIgemmKvol && c_src % 32 == 0 && c_dst % 16 == 0 &&
         c_src > 0 && c_src <= 128 && c_dst > 0;
}

size_t igemm_workspace_bytes(int kvol, int c_src, int c_dst) {
  return static_cast<size_t>(kvol) * ceil_div(c_dst, 16) * (c_src / 32) * 64 * 16;
}

hipError_t launch_igemm(const ConvArgs& a, void* ws, hipStream_t s) {
  const ts_rel& rel = *a.rel;
  if (rel.n_tiles == 0) return hipSuccess;
  IgK k;
  k.tile_mask = rel.tile_mask;
  k.tile_rows = rel.tile_rows;
  k.nbr = rel.nbr;
  k.n_tiles = rel.n_tiles;
  k.kvol = a.kvol;
  k.src = a.src;
  k.c_src = a.c_src;
  k.wp = static_cast<const u32x4*>(ws);
  k.mbt = ceil_div(a.c_dst, 16);
  k.dst = a.dst;
  k.c_dst = a.c_dst;
  k.out_dtype = a.out_dtype;
  k.nblk = 0;
  k.nb8 = 0;
  const int64_t chunks = static_cast<int64_t>(a.kvol) * k.mbt * (a.c_src / 32) * 64;
  const unsigned pg = static_cast<unsigned>(ceil_div<int64_t>(chunks, 256));
  if (a.in_dtype == TS_F16) {
    k_wpack<_Float16><<<pg, 256, 0, s>>>(static_cast<const _Float16*>(a.w), a.kvol, a.c_src, a.c_dst, k.mbt,
                                         a.transpose ? 1 : 0, a.mirror ? 1 : 0, static_cast<u32x4*>(ws));
    return launch_t<_Float16>(k, s);
  }
  k_wpack<__bf16><<<pg, 256, 0, s>>>(static_cast<const __bf16*>(a.w), a.kvol, a.c_src, a.c_dst, k.mbt,
                                     a.transpose ? 1 : 0, a.mirror ? 1 : 0, static_cast<u32x4*>(ws));
  return launch_t<__bf16>(k, s);
}

}  // namespace ts
