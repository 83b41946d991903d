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
// Work split.  A block of 4 waves owns 4*G tiles of 16 destination rows (each
// wave G tiles, all output channels of one 128-channel column).  The block
// walks the union of its tiles' offset masks in ascending order; per offset:
//   * the weight slice is copied from global memory into LDS once per block,
//     already in MFMA fragment order (the forward transposes on the way);
//   * each wave gathers, for each of its tiles that has the offset, the 16
//     source rows straight into B fragments (16 bytes per lane);
//   * v_mfma_f32_16x16x32 with D = A . X^T, so a lane ends holding 4
//     consecutive output channels of one row.
// Software pipeline: while offset i is multiplied, the gathers and weight
// slice of offset i+1 and the pool indices and weight loads of offset i+2 are
// in flight; the LDS weight buffer is double-buffered, one barrier per offset.  Every output
// row is written once, no atomics.  Blocks are numbered so that each XCD
// walks a contiguous range of tiles (its L2 keeps the gathered rows).
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

struct IgK {
  const uint64_t* tile_mask;
  const int32_t* tile_rows;
  const int32_t* pool;
  int64_t n_tiles;
  int kvol;
  const void* src;
  int c_src;
  const void* w;
  int trans;   // dgrad layout
  int mirror;  // dgrad of a submanifold map
  void* dst;
  int c_dst;
  int out_dtype;
  int64_t nblk;  // logical blocks
  int64_t nb8;   // ceil(nblk / 8)
  int xcd_map;   // number blocks so that each XCD walks a contiguous range
};

__device__ __forceinline__ int next_bit(uint64_t u, int o) {
  if (o < 0 || o >= 63) return -1;
  const uint64_t rest = u & ~((2ull << o) - 1);
  return rest ? __builtin_ctzll(rest) : -1;
}

template <typename T, int MB, int KB, int G>
__global__ __launch_bounds__(256) void k_igemm(IgK a) {
  typedef typename Mfma<T>::frag Frag;
  constexpr int FR = MB * KB;                      // fragments per offset
  constexpr int CHUNKS = FR * 64;                  // 16-byte chunks per weight slice
  constexpr int CH = (CHUNKS + 255) / 256;         // per thread
  __shared__ uint4 wl[2][FR * 64];
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

  uint64_t m[G];
  uint64_t u = 0;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = (t0 + g < a.n_tiles) ? a.tile_mask[t0 + g] : 0ull;
    u |= m[g];
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
  const T* w = static_cast<const T*>(a.w);
  const int c_src = a.c_src, c_dst = a.c_dst;
  const int64_t slice = static_cast<int64_t>(c_src) * c_dst;

  // ---- helpers.  No load is issued under a branch: every load reads a valid
  // address (row or tile 0 when there is nothing to fetch), and masking is
  // applied only where the value is consumed, so the compiler can count
  // outstanding loads exactly and the prefetches really overlap the multiplies.
  auto pool_idx = [&](int o, int32_t* nb) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const bool has = (m[g] >> o) & 1;
      const int k = __popcll(m[g] & ((1ull << o) - 1));
      const int64_t tile = has ? t0 + g : 0;
      nb[g] = a.pool[(tile * a.kvol + (has ? k : 0)) * kTile + col];  // meaningful only when `has`
    }
  };
  // gathers of offset o; ok[g] = row present (consumers zero the others)
  auto gather = [&](int o, const int32_t* nb, Frag (*x)[KB], bool* ok) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      ok[g] = ((m[g] >> o) & 1) && nb[g] >= 0;
      const T* row = src + static_cast<int64_t>(ok[g] ? nb[g] : 0) * c_src + kq * 8;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) x[g][kb] = __builtin_bit_cast(Frag, *reinterpret_cast<const uint4*>(row + kb * 32));
    }
  };
  // global -> registers: this thread's chunks of the weight slice of offset o.
  // Chunks past c_dst read a clamped address: they land in fragment rows of
  // output channels that are never written out.
  auto wload = [&](int o, uint4* r) {
    const int os = (a.trans && a.mirror) ? a.kvol - 1 - o : o;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int i0 = threadIdx.x + c * 256;
      const int i = i0 < CHUNKS ? i0 : 0;
      int64_t off;
      if (a.trans) {
        // A[n][k] = W[o'][n][k]; chunk = (n, 8 consecutive k)
        const int n = mb0 * 16 + i / (KB * 4);
        const int k = (i % (KB * 4)) * 8;
        off = os * slice + static_cast<int64_t>(n < c_dst ? n : 0) * c_src + k;
      } else {
        // A[n][k] = W[o][k][n]; chunk = (k, 8 consecutive n)
        const int k = i / (MB * 2);
        const int n = mb0 * 16 + (i % (MB * 2)) * 8;
        off = os * slice + static_cast<int64_t>(k) * c_dst + (n < c_dst ? n : 0);
      }
      r[c] = *reinterpret_cast<const uint4*>(w + off);
    }
  };
  // registers -> LDS in fragment order: slot (mb, kb, lane) holds A[n][k..k+7]
  // with n = mb*16 + lane%16, k = kb*32 + (lane/16)*8
  auto wstore = [&](const uint4* r, uint4* buf) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int i = threadIdx.x + c * 256;
      if (i >= CHUNKS) continue;
      if (a.trans) {
        const int nl = i / (KB * 4);
        const int k = (i % (KB * 4)) * 8;
        const int slot = ((nl >> 4) * KB + (k >> 5)) * 64 + (nl & 15) + 16 * ((k & 31) >> 3);
        buf[slot] = r[c];
      } else {
        const int k = i / (MB * 2);
        const int nl = (i % (MB * 2)) * 8;
        const T* v = reinterpret_cast<const T*>(&r[c]);
        T* b = reinterpret_cast<T*>(buf);
        const int base = ((nl >> 4) * KB + (k >> 5)) * 64 + 16 * ((k & 31) >> 3);
#pragma unroll
        for (int e = 0; e < 8; ++e) b[(base + ((nl + e) & 15)) * 8 + (k & 7)] = v[e];
      }
    }
  };

  if (U) {
    // Pipeline over the union of offsets, unrolled by two with ping-pong
    // register sets (A/B) so nothing is copied between iterations.  Entering
    // a step for offset oc: LDS buffer `buf` holds W(oc); xcur = gathers of
    // oc (issued one step earlier); nbnxt = pool indices of o1; wnxt = W(o1)
    // loads (issued one step earlier).  Each load thus has a whole step of
    // multiplies and barrier to land.  Past the last offset the prefetches
    // repeat a valid offset (harmless loads, no branches).
    int oc = __builtin_ctzll(U);
    int o1 = next_bit(U, oc);
    int o2 = o1 >= 0 ? next_bit(U, o1) : -1;
    Frag xA[G][KB], xB[G][KB];
    bool okA[G], okB[G];
    int32_t nbA[G], nbB[G];
    uint4 wA[CH], wB[CH];
    wload(oc, wA);
    pool_idx(oc, nbA);
    gather(oc, nbA, xA, okA);
    pool_idx(o1 >= 0 ? o1 : oc, nbB);
    wstore(wA, wl[0]);
    wload(o1 >= 0 ? o1 : oc, wB);
    __syncthreads();
    int buf = 0;
    auto step = [&](Frag (&xcur)[G][KB], bool (&okcur)[G], Frag (&xnxt)[G][KB], bool (&oknxt)[G],
                    int32_t (&nbcur)[G], int32_t (&nbnxt)[G], uint4 (&wcur)[CH], uint4 (&wnxt)[CH]) -> bool {
      const int okeep = o1 >= 0 ? o1 : oc;
      gather(okeep, nbnxt, xnxt, oknxt);          // X(o1)
      pool_idx(o2 >= 0 ? o2 : okeep, nbcur);      // pool(o2)
      const uint4* lw = wl[buf];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        Frag af[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) af[mb] = __builtin_bit_cast(Frag, lw[(mb * KB + kb) * 64 + lane]);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          if (!((m[g] >> oc) & 1)) continue;  // wave-uniform
          const Frag bx = okcur[g] ? xcur[g][kb] : Frag{};
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) acc[g][mb] = Mfma<T>::run(af[mb], bx, acc[g][mb]);
        }
      }
      if (o1 < 0) return false;
      wstore(wnxt, wl[buf ^ 1]);                  // W(o1), loaded one step ago
      wload(o2 >= 0 ? o2 : okeep, wcur);          // W(o2)
      __syncthreads();
      buf ^= 1;
      oc = o1;
      o1 = o2;
      o2 = o2 >= 0 ? next_bit(U, o2) : -1;
      return true;
    };
    while (step(xA, okA, xB, okB, nbA, nbB, wA, wB) && step(xB, okB, xA, okA, nbB, nbA, wB, wA)) {
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

// Tiles per wave.  Default: 4 for up to 64 output channels, 2 above; the
// environment variable TS_IGEMM_G (1, 2 or 4) overrides it for tuning.
static int tiles_per_wave(int mb) {
  static const int forced = [] {
    const char* e = getenv("TS_IGEMM_G");
    return e ? atoi(e) : 0;
  }();
  if (forced == 1 || forced == 2 || forced == 4) return forced;
  return mb <= 4 ? 4 : 2;
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

bool igemm_supported(int c_src, int c_dst, ts_dtype in_dtype) {
  return in_dtype != TS_F32 && c_src % 32 == 0 && c_dst % 16 == 0 && c_src > 0 && c_src <= 128 && c_dst > 0;
}

size_t igemm_workspace_bytes(int, int, int) { return 0; }

hipError_t launch_igemm(const ConvArgs& a, void*, hipStream_t s) {
  const ts_rel& rel = *a.rel;
  if (rel.n_tiles == 0) return hipSuccess;
  IgK k;
  k.tile_mask = rel.tile_mask;
  k.tile_rows = rel.tile_rows;
  k.pool = rel.pool;
  k.n_tiles = rel.n_tiles;
  k.kvol = a.kvol;
  k.src = a.src;
  k.c_src = a.c_src;
  k.w = a.w;
  k.trans = a.transpose ? 1 : 0;
  k.mirror = a.mirror ? 1 : 0;
  k.dst = a.dst;
  k.c_dst = a.c_dst;
  k.out_dtype = a.out_dtype;
  k.nblk = 0;
  k.nb8 = 0;
  return a.in_dtype == TS_F16 ? launch_t<_Float16>(k, s) : launch_t<__bf16>(k, s);
}

}  // namespace ts
