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
// Weights reach LDS in one of two layouts.  Forward-layout weights on
// 16-byte-aligned storage are copied as stored, row by row with a chunk
// swizzle, and fragments are built with gfx950's transposing LDS reads (no
// extra launch).  Otherwise (dgrad, 128-channel columns of the barrier-
// stepped kernel, unaligned or pre-packed weights) a small kernel first packs
// them into MFMA fragment order (16-byte chunks, fragment (o, mb, kb) = 64
// consecutive chunks), so every copy of a slice is a straight coalesced
// 16-byte copy.
//
// Work split.  A block of NW wavefronts owns NW*G tiles of 16 destination
// rows (each wavefront G tiles, the output channels of one block column) and
// walks the union of its tiles' offset masks in ascending order.  Per offset:
//   * the packed weight slice is copied into one of two LDS buffers with
//     direct global-to-LDS loads (no register staging);
//   * each wavefront gathers, for each of its tiles that has the offset, the
//     16 source rows straight into B fragments (16 bytes per lane);
//   * v_mfma_f32_16x16x32 with D = A . X^T, so a lane ends holding 4
//     consecutive output channels of one row; with G = 2 each A fragment read
//     from LDS feeds two MFMAs.
// Latency: the neighbour rows of a tile's 16 rows (the source row of each
// slot at each offset) are loaded once, up front, into registers and picked
// per offset with a lane shuffle, so no load address waits on another load
// inside the loop.  Gathers run two offsets ahead in three register sets.
// Each step waits on the vector-memory counter only for its own copy of the
// slice and meets the other wavefronts at a barrier without a memory fence,
// so gathers for later offsets stay in flight across it.  Gathers are buffer
// loads: an absent row reads out of range and returns zeros without a
// memory access.  Every output row is written once, no atomics.  Blocks are
// numbered so that each XCD walks a contiguous range of tiles (its L2 keeps
// the gathered rows).
#include <stdint.h>

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
  uint32_t src_bytes;  // < 2^31: a buffer offset of 2^31 is out of range
  int64_t n_src;       // rows of src and of dst (bounds-check build)
  int64_t n_dest;
  int c_src;
  const u32x4* wp;  // packed fragments [kvol][mbt][c_src/32][64]
  int mbt;          // fragments of 16 output channels in the packed weights
  void* dst;
  int c_dst;
  int out_dtype;
  int64_t nblk;  // logical blocks
  int64_t nb8;   // ceil(nblk / 8)
  int xcd_map;   // number blocks so that each XCD walks a contiguous range
  int in_order;  // tiles keep rows in index order (launch choice only)
  int ncol;      // weight-resident kernel: block columns
  const void* w;  // the layer's weights as stored (wmode 1)
  int wmode;      // weight source: 0 packed fragments (wp), 1 forward rows of w
  int mirror;     // wmode 1: offset o reads W[kvol-1-o]
};

// Packed chunk i = ((o * mbt + mb) * kbn + kb) * 64 + lane holds A_o[n][k..k+7]
// with n = mb*16 + lane%16, k = kb*32 + (lane/16)*8; zero for n >= c_dst.
template <typename T>
__global__ __launch_bounds__(256) void k_wpack(const T* __restrict__ w, int kvol, int c_src, int c_dst, int mbt,
                                               int trans, int mirror, int vec, u32x4* __restrict__ out) {
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
    const int os = mirror ? kvol - 1 - o : o;
    if (trans && vec) {  // 16-byte aligned weights: the 8 values are one aligned chunk
      v = *reinterpret_cast<const u32x4*>(w + os * slice + static_cast<int64_t>(n) * c_src + k0);
    } else if (trans) {
      unsigned short e[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) e[j] = __builtin_bit_cast(unsigned short, w[os * slice + static_cast<int64_t>(n) * c_src + k0 + j]);
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = static_cast<unsigned>(e[2 * j]) | (static_cast<unsigned>(e[2 * j + 1]) << 16);
    } else {
      unsigned short e[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) e[j] = __builtin_bit_cast(unsigned short, w[os * slice + static_cast<int64_t>(k0 + j) * c_dst + n]);
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = static_cast<unsigned>(e[2 * j]) | (static_cast<unsigned>(e[2 * j + 1]) << 16);
    }
  }
  out[i] = v;
}

// Stores 4 consecutive output channels (fp32 accumulators) in the output type.
__device__ __forceinline__ void store4(void* dst, int out_dtype, int64_t off, f32x4 v) {
  if (out_dtype == TS_F32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(dst) + off) = v;
  } else if (out_dtype == TS_F16) {
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    h4 h = {static_cast<_Float16>(v[0]), static_cast<_Float16>(v[1]), static_cast<_Float16>(v[2]),
            static_cast<_Float16>(v[3])};
    *reinterpret_cast<h4*>(static_cast<_Float16*>(dst) + off) = h;
  } else {
    typedef __bf16 b4 __attribute__((ext_vector_type(4)));
    b4 h = {static_cast<__bf16>(v[0]), static_cast<__bf16>(v[1]), static_cast<__bf16>(v[2]),
            static_cast<__bf16>(v[3])};
    *reinterpret_cast<b4*>(static_cast<__bf16*>(dst) + off) = h;
  }
}

__device__ __forceinline__ int next_bit(uint64_t u, int o) {
  if (o < 0 || o >= 63) return -1;
  const uint64_t rest = u & ~((2ull << o) - 1);
  return rest ? __builtin_ctzll(rest) : -1;
}

// Compile-time step index, so that register sets picked by step stay static.
template <int I>
struct Ic {
  static constexpr int v = I;
};
template <int I, int N>
struct Seq {
  template <typename F>
  __device__ __forceinline__ static bool go(F& f) {
    return f(Ic<I>{}) && Seq<I + 1, N>::go(f);
  }
};
template <int N>
struct Seq<N, N> {
  template <typename F>
  __device__ __forceinline__ static bool go(F&) {
    return true;
  }
};

// Waits until at most n vector-memory operations of this wave are
// outstanding (loads retire in issue order); the other counters are left
// unconstrained.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | 0x70 | 0xF00 | ((N >> 4) << 14));
}
// 16 bytes per lane from global memory straight into LDS: lane l writes
// dst + l (dst is wave-uniform).  Completion is counted by the vector-memory
// counter.  Kept out of the kernel templates: clang emits no host launch
// stub for a kernel template whose body names this builtin.
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
__device__ __forceinline__ void lds_copy16(const u32x4* src, lds_u32x4* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}
// All of this wave's LDS reads have returned.
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// Workgroup barrier with no memory fence: the waits it needs are explicit at
// each use, so that loads in flight (gathers for later offsets) stay in
// flight across it.  The empty asm statements keep the compiler from moving
// memory operations across the barrier.
__device__ __forceinline__ void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Chunk swizzle of the row-by-row layout (WM 1): chunk cc of row ci sits at
// cc ^ (2 * wswz<MB>(ci)) within its row (pairs of chunks, i.e. 16 output
// channels, move together).  Chosen so that the 64 lanes of one transposing
// read (16 rows, 2 chunks each) fall on every 16-byte bank group of a
// 256-byte period exactly twice for MB = 2, 4 and 8; unswizzled rows of 128
// or 256 bytes would put 8 or 16 of them on the same banks.
template <int MB>
__device__ __forceinline__ int wswz(int ci) {
  return MB >= 8 ? ((ci & 7) + 2 * ((ci >> 3) & 3)) & 7 : ((ci >> 3) & 3) & (MB - 1);
}

// Source of the 16-byte weight chunk r * 64 + lane of offset o for the block
// column whose first fragment row is mb0:
//   WM 0: the packed fragments (fragment r of the column);
//   WM 1: W[o] as the forward stores it, [c_src][c_dst]: the column's slice
//         kept row by row (row ci = 2*MB chunks of 8 output channels, in the
//         swizzled order of wswz), for the transposing fragment reads.
// Output channels past c_dst read channel 0: they feed accumulators that are
// never stored.
template <typename T, int MB, int KB, int WM>
__device__ __forceinline__ const u32x4* wchunk(const IgK& a, int o, int mb0, int r, int lane) {
  if constexpr (WM == 0) {
    const int live = (a.mbt - mb0) * KB;  // fragments of this column inside the packing
    const int64_t base = (static_cast<int64_t>(o) * a.mbt + mb0) * KB;
    return a.wp + (base + (r < live ? r : 0)) * 64 + lane;
  } else {
    const int os = a.mirror ? a.kvol - 1 - o : o;
    const T* w = static_cast<const T*>(a.w);
    const int c = r * 64 + lane;  // the LDS chunk this lane fills
    const int ci = c / (2 * MB), cc = (c - ci * (2 * MB)) ^ (2 * wswz<MB>(ci));
    int co = mb0 * 16 + cc * 8;
    if (co >= a.c_dst) co = 0;
    return reinterpret_cast<const u32x4*>(w + (static_cast<int64_t>(os) * a.c_src + ci) * a.c_dst + co);
  }
}

// Transposing LDS reads (gfx950).  In each group of 16 lanes, lane q + 4m
// (q, m < 4) names 4 consecutive 16-bit values and lane 4q + r receives value
// r of the 4-value runs named by lanes q, q+4, q+8, q+12.  With W[o] held row
// by row ([c_src][MB*16] 16-bit values) and lane (g, q + 4m) of group g naming
// row 8g + m (+4 for the second read) at column 16*mb + 4q, lane (g, j) gets
// rows 8g..8g+7 of column 16*mb + j: the A fragment of output channel j and
// contracted channels 8g..8g+7.  `p0` and `p4` are that lane's byte
// addresses in LDS for the first and the second four rows.  Kept out of the
// kernel templates, like the global-to-LDS copy.
typedef __attribute__((__vector_size__(4 * sizeof(__fp16)))) __fp16 h4tr;
typedef __attribute__((address_space(3))) h4tr lds_h4tr;
__device__ __forceinline__ u32x4 lds_tr_frag(const char* p0, const char* p4) {
  const h4tr lo = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_h4tr*)p0);
  const h4tr hi = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_h4tr*)p4);
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 l = __builtin_bit_cast(u32x2, lo), h = __builtin_bit_cast(u32x2, hi);
  return u32x4{l[0], l[1], h[0], h[1]};
}

template <typename T, int MB, int KB, int G, int D, int NW, int WM>
__global__ __launch_bounds__(NW * 64) void k_igemm(IgK a) {
  constexpr bool TR = WM == 1;  // transposing fragment reads of the row-by-row layout
  typedef typename Mfma<T>::frag Frag;
  constexpr int FR = MB * KB;                      // fragments per offset and block column
  constexpr int CHUNKS = FR * 64;                  // 16-byte chunks per weight slice
  constexpr int FW = (FR + NW - 1) / NW;           // fragments copied per wave (at most)
  constexpr int GL = G * KB;                       // gather loads per wave and offset
  __shared__ u32x4 wl[2][CHUNKS];
  __shared__ uint64_t wunion[NW];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15;
  const int kq = lane >> 4;
  const int64_t hb = blockIdx.x;
  const int64_t lb = a.xcd_map ? (hb & 7) * a.nb8 + (hb >> 3) : hb;  // XCD-contiguous numbering
  if (lb >= a.nblk) return;                        // whole block, before any barrier
  const int mb0 = blockIdx.y * MB;
  const int64_t t0 = (lb * NW + wave) * G;
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
    const int32_t drow = dbg_opt(a.tile_rows[tile * kTile + col], a.n_dest, TS_DEBUG_DST_ROW);
    const int32_t* nrow = a.nbr + static_cast<int64_t>(drow >= 0 ? drow : 0) * kvol;
#pragma unroll
    for (int j = 0; j < kNbRegs; ++j) {
      const int o = kq * kNbRegs + j;
      const int32_t v = dbg_opt(nrow[o < kvol ? o : 0], a.n_src, TS_DEBUG_SRC_ROW);
      pr[g][j] = drow >= 0 ? v : -1;
    }
  }
  if (lane == 0) wunion[wave] = u;
  __syncthreads();
  uint64_t U = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) U |= wunion[w];
  uint64_t mine = 0;
#pragma unroll
  for (int g = 0; g < G; ++g) mine |= m[g];

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
  // Gathers of offset o as buffer loads over the source matrix: a row that is
  // absent (or a tile without the offset) gets an out-of-range offset, which
  // returns zeros without a memory access, so no select is needed at use and
  // no cache access is spent on it.  Exactly GL loads, always issued.
  const __amdgpu_buffer_rsrc_t xr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(src), 0, static_cast<int>(a.src_bytes), 0x00020000);
  auto gather = [&](int o, Frag (&x)[G][KB]) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int32_t nb = pool_row(g, o);
      const bool ok = ((m[g] >> o) & 1) && nb >= 0;
      const uint32_t off = ok ? static_cast<uint32_t>(nb * c_src + kq * 8) * 2u : 0x80000000u;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        x[g][kb] = __builtin_bit_cast(Frag, __builtin_amdgcn_raw_buffer_load_b128(xr, static_cast<int>(off + kb * 64), 0, 0));
    }
  };
  // Copy of the packed slice of offset o into LDS buffer `buf` by direct
  // global-to-LDS loads: wave w moves fragments w, w+NW, ... (1 KB each, lane
  // l to chunk l) into buffer bb.  Fragments past the packed column count copy the slice
  // start: they feed rows of output channels that are never written out.
  // Wave-uniform; FW loads when the wave has FW fragments, fewer otherwise.
  auto wcopy = [&](int o, int bb) {
#pragma unroll
    for (int j = 0; j < FW; ++j) {
      const int f = wave + NW * j;
      if (FR % NW != 0 && f >= FR) break;
      lds_copy16(wchunk<T, MB, KB, WM>(a, o, mb0, f, lane), (lds_u32x4*)&wl[bb][f * 64]);
    }
  };
  // transposing reads: this lane's byte offsets within a slice, for the
  // first and the second four rows (row 8*kq + m (+4), column pair q >> 1,
  // half q & 1), and the swizzle of those rows as a byte mask
  const int trq = lane & 3, trm = (lane >> 2) & 3;
  const int tr_b0 = (8 * kq + trm) * (MB * 32) + (trq >> 1) * 16 + (trq & 1) * 8;
  const int tr_b4 = tr_b0 + 4 * MB * 32;
  const int tr_x0 = 32 * wswz<MB>(8 * kq + trm), tr_x4 = 32 * wswz<MB>(8 * kq + 4 + trm);

  if (U) {
    // Offsets u_0 < u_1 < ... of U.  Weights: two LDS buffers, W(u_j) in
    // buffer j % 2.  Gathers: R = D + 1 register sets, X(u_j) in set j % R,
    // issued D steps ahead.  Step i:
    //   wait for this wave's copy of W(u_i) (only the GL gathers issued after
    //   it may stay in flight) and for its LDS reads of step i-1; barrier;
    //   multiply X(u_i) by W(u_i); copy W(u_{i+1}) into buffer (i+1) % 2
    //   (read at step i-1: every wave is past it); gather X(u_{i+D}).
    // The copy goes after the fragment reads because the compiler makes any
    // LDS read wait for every copy into LDS still in flight.  Issue order is
    // the same in the prologue, so the wait count is the same constant at
    // every step.  Past the last offset the gathers repeat a valid offset
    // (harmless loads); no copy is issued past it.
    constexpr int R = D + 1;
    Frag xs[R][G][KB];
    int oc = __builtin_ctzll(U);  // u_i
    const int last = 63 - __builtin_clzll(U);
    int onx = oc;                 // u_{i+D-1} before a step's gather, then u_{i+D}
#pragma unroll
    for (int j = 0; j + 1 < D; ++j) {
      gather(onx, xs[j]);
      onx = onx < last ? next_bit(U, onx) : onx;
    }
    wcopy(oc, 0);
    gather(onx, xs[D - 1]);
    auto step = [&](auto ic) -> bool {
      constexpr int i = decltype(ic)::v;
      constexpr int cur = i % R, fill = (i + D) % R, b = i % 2;
      wait_vm<GL>();
      wait_lds();
      bare_barrier();
      if ((mine >> oc) & 1) {  // wave-uniform: no fragment reads for a wave without the offset
        const u32x4* lw = wl[b];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          Frag af[MB];
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            if constexpr (TR) {
              const char* sl = reinterpret_cast<const char*>(lw) + kb * 32 * MB * 32;
              af[mb] = __builtin_bit_cast(Frag, lds_tr_frag(sl + tr_b0 + ((mb * 32) ^ tr_x0),
                                                            sl + tr_b4 + ((mb * 32) ^ tr_x4)));
            } else {
              af[mb] = __builtin_bit_cast(Frag, lw[(mb * KB + kb) * 64 + lane]);
            }
          }
#pragma unroll
          for (int g = 0; g < G; ++g) {
            if (!((m[g] >> oc) & 1)) continue;  // wave-uniform
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) acc[g][mb] = Mfma<T>::run(af[mb], xs[cur][g][kb], acc[g][mb]);
          }
        }
      }
      if (oc == last) return false;
      oc = next_bit(U, oc);
      asm volatile("" ::: "memory");
      wcopy(oc, b ^ 1);                           // W(u_{i+1})
      onx = onx < last ? next_bit(U, onx) : onx;  // u_{i+D}
      gather(onx, xs[fill]);
      return true;
    };
    while (Seq<0, 2 * R>::go(step)) {
    }
    wait_vm<0>();  // no copy into LDS may still be in flight when the block ends
  }

  // write each destination row once
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (t0 + g >= a.n_tiles) continue;
    const int32_t row = dbg_opt(a.tile_rows[(t0 + g) * kTile + col], a.n_dest, TS_DEBUG_DST_ROW);
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

// Weight-resident variant, for layers whose weights (one block column of
// output channels, every offset) fit in LDS: kvol * MB * KB fragments of
// 1 KB, at most kResFrags.  The grid is one block per compute unit.  Each
// block copies its column's weights into LDS once and then holds them; its
// wavefronts walk tile groups independently, each over the union of its own
// G tiles' masks only, with no barrier and no weight copy inside the loop,
// so a step costs its fragment reads and MFMAs and waits only for the
// gathers issued D steps earlier.
//   * Block b serves XCD b % 8 (workgroups are dealt to XCDs round-robin) and
//     column (b / 8) % ncol; XCD x walks the x-th eighth of the tile groups,
//     each of its blocks a contiguous share, and the block's waves take the
//     groups of that share from an LDS counter as they finish the last one.
//     A single global counter per XCD was measured 2.6x slower: its atomics
//     serialise.
//   * The next group's masks, rows and neighbour rows load while the current
//     group runs, so only a group's first gathers are exposed.
//   * Every step issues its gathers, past the last offset out of range (no
//     memory access), so all paths carry the same loads and the compiler's
//     wait before a step covers that step's gathers only.
constexpr int kResFrags = 144;

template <typename T, int MB, int KB, int G, int D, int NW, int WM>
__global__ __launch_bounds__(NW * 64) void k_igemm_res(IgK a) {
  constexpr bool TR = WM == 1;
  typedef typename Mfma<T>::frag Frag;
  constexpr int FR = MB * KB;   // fragments per offset and block column
  constexpr int GL = G * KB;    // gather loads per wave and offset
  __shared__ u32x4 wl[kResFrags * 64];
  __shared__ unsigned next_group;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15;
  const int kq = lane >> 4;
  const int xcd = blockIdx.x & 7;
  const int bi = blockIdx.x >> 3;
  const int column = bi % a.ncol;
  const int bj = bi / a.ncol;
  const int mb0 = column * MB;
  const int kvol = a.kvol;
  // transposing reads: this lane's byte offsets within a slice (see k_igemm)
  const int trq = lane & 3, trm = (lane >> 2) & 3;
  const int tr_b0 = (8 * kq + trm) * (MB * 32) + (trq >> 1) * 16 + (trq & 1) * 8;
  const int tr_b4 = tr_b0 + 4 * MB * 32;
  const int tr_x0 = 32 * wswz<MB>(8 * kq + trm), tr_x4 = 32 * wswz<MB>(8 * kq + 4 + trm);

  // the column's weights, every offset: fragment f = o * FR + mb * KB + kb
  {
    for (int f = wave; f < kvol * FR; f += NW) {
      const int o = f / FR, r = f - o * FR;
      lds_copy16(wchunk<T, MB, KB, WM>(a, o, mb0, r, lane), (lds_u32x4*)&wl[f * 64]);
    }
    if (threadIdx.x == 0) next_group = 0u;
    wait_vm<0>();
    __syncthreads();
  }

  const T* src = static_cast<const T*>(a.src);
  const int c_src = a.c_src, c_dst = a.c_dst;
  const __amdgpu_buffer_rsrc_t xr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(src), 0, static_cast<int>(a.src_bytes), 0x00020000);
  // XCD x walks the x-th eighth of the tile groups; each of its blocks of
  // this column a contiguous share of that.
  const int64_t ng = a.nblk;  // tile groups
  const int64_t xlo = ng * xcd / 8, xn = ng * (xcd + 1) / 8 - xlo;
  const int64_t lo = xlo + xn * bj / a.nb8, hi = xlo + xn * (bj + 1) / a.nb8;

  // Tile metadata (masks, destination rows, then neighbour rows) of the
  // wave's next group is loaded while the current group runs: the masks and
  // rows after the current group's first gathers, the neighbour rows after
  // its first D steps, so only the first gathers of a group wait.
  uint64_t m[G];
  int32_t drow[G], pr[G][kNbRegs];
  auto load_meta = [&](int64_t g0, uint64_t (&mm)[G], int32_t (&dr)[G]) {
#pragma unroll
    for (int g = 0; g < G; ++g) {  // a tile past the end reads tile 0 and is masked off
      const bool live = g0 >= 0 && g0 + g < a.n_tiles;
      const int64_t tile = live ? g0 + g : 0;
      const uint64_t v = a.tile_mask[tile];
      mm[g] = live ? v : 0ull;
      const int32_t r = dbg_opt(a.tile_rows[tile * kTile + col], a.n_dest, TS_DEBUG_DST_ROW);
      dr[g] = live ? r : -1;
    }
  };
  auto load_nbr = [&](const int32_t (&dr)[G], int32_t (&p)[G][kNbRegs]) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int32_t* nrow = a.nbr + static_cast<int64_t>(dr[g] >= 0 ? dr[g] : 0) * kvol;
#pragma unroll
      for (int j = 0; j < kNbRegs; ++j) {
        const int o = kq * kNbRegs + j;
        const int32_t v = dbg_opt(nrow[o < kvol ? o : 0], a.n_src, TS_DEBUG_SRC_ROW);
        p[g][j] = dr[g] >= 0 ? v : -1;
      }
    }
  };
  // Groups of the block's share are dealt by an LDS ticket: a wave takes the
  // next group when it starts one, so waves that drew short groups take more.
  auto ticket = [&]() -> unsigned {  // issued by lane 0; the value is read later
    unsigned v = 0u;
    if (lane == 0) v = atomicAdd(&next_group, 1u);
    return v;
  };
  int64_t gi = lo + static_cast<int64_t>(__builtin_amdgcn_readfirstlane(ticket()));
  load_meta(gi < hi ? gi * G : -1, m, drow);
  load_nbr(drow, pr);

  while (gi < hi) {
    const unsigned tk = ticket();
    int64_t gn = hi, gnext = -1;
    uint64_t mine = 0;
#pragma unroll
    for (int g = 0; g < G; ++g) mine |= m[g];
    uint64_t nm[G];
    int32_t ndrow[G], npr[G][kNbRegs];
    bool nbr_issued = false;

    f32x4 acc[G][MB];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[g][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto pool_row = [&](int g, int o) -> int32_t {
      const int q = o / kNbRegs, j = o - q * kNbRegs;
      int32_t v = pr[g][0];
#pragma unroll
      for (int jj = 1; jj < kNbRegs; ++jj) v = (j == jj) ? pr[g][jj] : v;
      return __shfl(v, col + 16 * q, 64);
    };
    // live = false (past the wave's last offset): out of range, no memory access
    auto gather = [&](int o, bool live, Frag (&x)[G][KB]) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int32_t nb = pool_row(g, o);
        const bool ok = live && ((m[g] >> o) & 1) && nb >= 0;
        const uint32_t off = ok ? static_cast<uint32_t>(nb * c_src + kq * 8) * 2u : 0x80000000u;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          x[g][kb] = __builtin_bit_cast(Frag, __builtin_amdgcn_raw_buffer_load_b128(xr, static_cast<int>(off + kb * 64), 0, 0));
      }
    };

    if (mine) {
      // Offsets u_0 < u_1 < ... < u_{n-1} of this wave's union; X(u_j) in
      // register set j % R, gathered D steps ahead.  The walk runs a whole
      // number of R-step rounds: steps past u_{n-1} do no math and gather
      // out of range, so every path issues the same loads and no step has
      // to wait for more than its own gathers.
      constexpr int R = D + 1;
      Frag xs[R][G][KB];
      const int nst = __builtin_popcountll(mine);
      int oc = __builtin_ctzll(mine);
      int onx = oc;
      int ng = 0;  // gathers issued
#pragma unroll
      for (int j = 0; j < D; ++j) {
        gather(onx, ng < nst, xs[j]);
        ++ng;
        onx = next_bit(mine, onx);
      }
      gn = lo + static_cast<int64_t>(__builtin_amdgcn_readfirstlane(tk));
      gnext = gn < hi ? gn * G : -1;
      load_meta(gnext, nm, ndrow);
      for (int st = 0; st < nst; st += R) {
#pragma unroll
        for (int i = 0; i < R; ++i) {
          const int cur = i, fill = (i + D) % R;
          if (st + i < nst) {  // wave-uniform
            const u32x4* lw = wl + oc * FR * 64;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
              Frag af[MB];
#pragma unroll
              for (int mb = 0; mb < MB; ++mb) {
                if constexpr (TR) {
                  const char* sl = reinterpret_cast<const char*>(lw) + kb * 32 * MB * 32;
                  af[mb] = __builtin_bit_cast(Frag, lds_tr_frag(sl + tr_b0 + ((mb * 32) ^ tr_x0),
                                                                sl + tr_b4 + ((mb * 32) ^ tr_x4)));
                } else {
                  af[mb] = __builtin_bit_cast(Frag, lw[(mb * KB + kb) * 64 + lane]);
                }
              }
#pragma unroll
              for (int g = 0; g < G; ++g) {
                if (!((m[g] >> oc) & 1)) continue;  // wave-uniform
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) acc[g][mb] = Mfma<T>::run(af[mb], xs[cur][g][kb], acc[g][mb]);
              }
            }
            oc = next_bit(mine, oc);
          }
          gather(onx < 0 ? 0 : onx, ng < nst, xs[fill]);  // X(u_{st+i+D})
          ++ng;
          onx = next_bit(mine, onx);
          if (st + i == D - 1) {  // wave-uniform
            load_nbr(ndrow, npr);
            nbr_issued = true;
          }
        }
      }
    } else {
      gn = lo + static_cast<int64_t>(__builtin_amdgcn_readfirstlane(tk));
      gnext = gn < hi ? gn * G : -1;
      load_meta(gnext, nm, ndrow);
    }
    if (!nbr_issued) load_nbr(ndrow, npr);

#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int32_t row = drow[g];  // -1 past the end or for an empty slot
      if (row < 0) continue;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int n = (mb0 + mb) * 16 + kq * 4;
        if (n >= c_dst) continue;
        store4(a.dst, a.out_dtype, static_cast<int64_t>(row) * c_dst + n, acc[g][mb]);
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m[g] = nm[g];
      drow[g] = ndrow[g];
#pragma unroll
      for (int j = 0; j < kNbRegs; ++j) pr[g][j] = npr[g][j];
    }
    gi = gn;
  }
  (void)GL;
}

// Tiles per wave.  Two when a weight slice is at least 32 fragments (e.g.
// 128x128): each fragment read from LDS then feeds two MFMAs, which halves
// the LDS reads per row and doubles the math per barrier.  Two as well when
// tiles keep rows in index order: a block's offset union then covers nearly
// every offset whatever its size.  Otherwise one, which keeps the union of a
// mask-grouped block small.
static int tiles_per_wave(int fr, int in_order) { return (fr >= 32 || in_order) ? 2 : 1; }

// Workgroups are dealt to the 8 XCDs round-robin; blocks are numbered so
// that XCD x gets a contiguous range, which keeps each XCD's gathers in its
// own L2.

// Waves per block: 4, or 8 when tiles keep rows in index order (every block
// then walks nearly all offsets whatever its size, so a larger block only
// shares each weight copy among more rows).
static int waves_per_block(int in_order) { return in_order ? 8 : 4; }

template <typename T, int MB, int KB, int G, int NW>
hipError_t launch_gw(IgK k, hipStream_t s) {
  k.nblk = ceil_div<int64_t>(k.n_tiles, NW * G);
  k.nb8 = ceil_div<int64_t>(k.nblk, 8);
  k.xcd_map = 1;
  dim3 grid(static_cast<unsigned>(k.xcd_map ? k.nb8 * 8 : k.nblk), static_cast<unsigned>(ceil_div(k.c_dst / 16, MB)));
  if (k.wmode == 1)
    k_igemm<T, MB, KB, G, 2, NW, 1><<<grid, NW * 64, 0, s>>>(k);
  else
    k_igemm<T, MB, KB, G, 2, NW, 0><<<grid, NW * 64, 0, s>>>(k);
  return hipGetLastError();
}

template <typename T, int MB, int KB, int G>
hipError_t launch_g(IgK k, hipStream_t s) {
  if (waves_per_block(k.in_order) == 8) return launch_gw<T, MB, KB, G, 8>(k, s);
  return launch_gw<T, MB, KB, G, 4>(k, s);
}

template <typename T, int MB, int KB>
hipError_t launch_mb_kb(const IgK& k, hipStream_t s) {
  switch (tiles_per_wave(MB * KB, k.in_order)) {
    case 2: return launch_g<T, MB, KB, 2>(k, s);
    default: return launch_g<T, MB, KB, 1>(k, s);
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

// Weight-resident launch.  Gathers in flight per wave: D offsets of G * KB
// 16-byte loads.  Waves per block from the register need of acc, the gather
// ring and the fragments (one block per compute unit: the weights take most
// of the LDS).
template <typename T, int MB, int KB>
hipError_t launch_res_mk(IgK k, int ncu, hipStream_t s) {
  constexpr int G = 2;
  constexpr int D = KB >= 4 ? 2 : (KB == 1 ? 4 : 3);
  constexpr int NW = MB * KB <= 2 ? 16 : (MB * KB <= 8 && MB < 8 ? 12 : 8);
  k.nblk = ceil_div<int64_t>(k.n_tiles, G);
  int64_t per = ncu / (8 * k.ncol);
  if (per < 1) per = 1;
  const int64_t need = ceil_div<int64_t>(ceil_div<int64_t>(k.nblk, 8), NW);  // blocks that have a group
  k.nb8 = per < need ? per : need;
  dim3 grid(static_cast<unsigned>(8 * k.ncol * k.nb8));
  if (k.wmode == 1)
    k_igemm_res<T, MB, KB, G, D, NW, 1><<<grid, NW * 64, 0, s>>>(k);
  else
    k_igemm_res<T, MB, KB, G, D, NW, 0><<<grid, NW * 64, 0, s>>>(k);
  return hipGetLastError();
}

template <typename T, int MB>
hipError_t launch_res_m(const IgK& k, int ncu, hipStream_t s) {
  switch (k.c_src / 32) {
    case 1: return launch_res_mk<T, MB, 1>(k, ncu, s);
    case 2: return launch_res_mk<T, MB, 2>(k, ncu, s);
    case 3: return launch_res_mk<T, MB, 3>(k, ncu, s);
    default: return launch_res_mk<T, MB, 4>(k, ncu, s);
  }
}

// Fragments of 16 output channels per block for the weight-resident kernel
// (all output channels in one block column), or 0 when those weights do not
// fit in LDS.  Split into two columns (e.g. 27 offsets of 64 x 64), each
// column would gather every source row and read the neighbour table again:
// measured slower than the barrier-stepped kernel on the ring scan (50 vs
// 42 us) and on its generated support (404 vs 340 us), so such layers stay on
// that kernel.
static int res_mb(int kvol, int c_src, int c_dst) {
  const int mbt = ceil_div(c_dst, 16), kb = c_src / 32;
  int mb = 1;
  while (mb < mbt) mb *= 2;
  return (mb <= 8 && kvol * mb * kb <= kResFrags) ? mb : 0;
}

static int cu_count() {
  static int n[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (n[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    n[dev] = v;
  }
  return n[dev];
}

template <typename T>
hipError_t launch_res(IgK k, int mb, hipStream_t s) {
  k.ncol = ceil_div(k.mbt, mb);
  const int ncu = cu_count();
  switch (mb) {
    case 1: return launch_res_m<T, 1>(k, ncu, s);
    case 2: return launch_res_m<T, 2>(k, ncu, s);
    case 4: return launch_res_m<T, 4>(k, ncu, s);
    default: return launch_res_m<T, 8>(k, ncu, s);
  }
}

template <typename T>
hipError_t launch_t(const IgK& k, hipStream_t s) {
  const int mbt = k.c_dst / 16;
  if (mbt > 4) return launch_mb<T, 8>(k, s);
  if (mbt > 2) return launch_mb<T, 4>(k, s);
  if (mbt > 1) return launch_mb<T, 2>(k, s);
  return launch_mb<T, 1>(k, s);
}

}  // namespace

bool igemm_supported(int kvol, int64_t n_src, int c_src, int c_dst, ts_dtype in_dtype) {
  const int64_t bytes = n_src * c_src * 2;
  return in_dtype != TS_F32 && kvol >= 1 && kvol <= kMaxIgemmKvol && c_src % 32 == 0 && c_dst % 16 == 0 &&
         c_src > 0 && c_src <= 128 && c_dst > 0 && bytes < (int64_t{1} << 31);
}

size_t igemm_workspace_bytes(int kvol, int c_src, int c_dst) {
  return static_cast<size_t>(kvol) * ceil_div(c_dst, 16) * (c_src / 32) * 64 * 16;
}

hipError_t launch_wpack(const ConvArgs& a, void* ws, hipStream_t s) {
  const int mbt = ceil_div(a.c_dst, 16);
  const int64_t chunks = static_cast<int64_t>(a.kvol) * mbt * (a.c_src / 32) * 64;
  const unsigned pg = static_cast<unsigned>(ceil_div<int64_t>(chunks, 256));
  const int vec = (reinterpret_cast<uintptr_t>(a.w) & 15) == 0 ? 1 : 0;
  if (a.in_dtype == TS_F16)
    k_wpack<_Float16><<<pg, 256, 0, s>>>(static_cast<const _Float16*>(a.w), a.kvol, a.c_src, a.c_dst, mbt,
                                         a.transpose ? 1 : 0, a.mirror ? 1 : 0, vec, static_cast<u32x4*>(ws));
  else
    k_wpack<__bf16><<<pg, 256, 0, s>>>(static_cast<const __bf16*>(a.w), a.kvol, a.c_src, a.c_dst, mbt,
                                       a.transpose ? 1 : 0, a.mirror ? 1 : 0, vec, static_cast<u32x4*>(ws));
  return hipGetLastError();
}

hipError_t launch_igemm(const ConvArgs& a, void* ws, hipStream_t s) {
  const ts_rel& rel = *a.rel;
  // The kernels copy forward-layout weights straight from w (16-byte aligned)
  // into a row-by-row LDS layout read with transposing loads, so no pack
  // launch precedes them.  Measured faster for the weight-resident kernel
  // and for block columns of up to 64 output channels; a 128-channel column
  // of the barrier-stepped kernel reads its fragments faster packed (train
  // forward 138.6 vs 141 us), as does dgrad, whose chunks would come from
  // 16 rows apiece.  Weights packed ahead use the packed layout.
  const int rmb = res_mb(a.kvol, a.c_src, a.c_dst);
  const bool direct = !a.prepacked && !a.transpose &&
                      (reinterpret_cast<uintptr_t>(a.w) & 15) == 0 && (rmb != 0 || ceil_div(a.c_dst, 16) <= 4);
  if (!a.prepacked && !direct) {
    const hipError_t e = launch_wpack(a, ws, s);
    if (e != hipSuccess) return e;
  }
  if (rel.n_tiles == 0) return hipSuccess;
  IgK k;
  k.tile_mask = rel.tile_mask;
  k.tile_rows = rel.tile_rows;
  k.nbr = rel.nbr;
  k.n_tiles = rel.n_tiles;
  k.kvol = a.kvol;
  k.src = a.src;
  k.src_bytes = static_cast<uint32_t>(a.n_src * a.c_src * 2);
  k.n_src = a.n_src;
  k.n_dest = rel.n_dest_cap;
  k.c_src = a.c_src;
  k.wp = static_cast<const u32x4*>(ws);
  k.mbt = ceil_div(a.c_dst, 16);
  k.dst = a.dst;
  k.c_dst = a.c_dst;
  k.out_dtype = a.out_dtype;
  k.nblk = 0;
  k.nb8 = 0;
  k.in_order = a.rows_in_order ? 1 : 0;
  k.ncol = 1;
  k.w = a.w;
  k.wmode = direct ? 1 : 0;
  k.mirror = a.mirror ? 1 : 0;
  if (a.in_dtype == TS_F16) return rmb ? launch_res<_Float16>(k, rmb, s) : launch_t<_Float16>(k, s);
  return rmb ? launch_res<__bf16>(k, rmb, s) : launch_t<__bf16>(k, s);
}

}  // namespace ts

TS_DEBUG_TU(igemm)
