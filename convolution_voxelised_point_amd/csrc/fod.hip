// Fetch-on-demand contraction (the third dataflow the torch-lattice page
// "Migrating from TorchSparse" names in section "Backend and configuration
// differences"; the TorchSparse++ abstract credits dataflows that overlap
// computation with memory access).  It walks a relation stored as per-tile
// pair groups: the destination rows are cut into tiles of TS_GTILE rows, and
// inside a tile the pairs of each offset are listed in destination order and
// padded to whole groups of 16, so group g of a tile occupies entries
// [16g, 16g + 16) of the tile's lists.  Every group is one 16-pair MFMA
// product with a single offset's weights: only the source rows that exist are
// fetched, straight from the source matrix into MFMA operands (no gather
// buffer), and the products are added into the destination rows of an fp32
// accumulator tile held in LDS, which is written out once per tile.  There
// are no atomics: within a group the destination rows are distinct, and one
// wave owns each accumulator tile and adds its groups in a fixed order, so
// results are bitwise repeatable.
//
// Work split.  A block owns one column of CB = 16 * MW output channels and
// keeps that column's weights for every offset resident in LDS (loaded once
// per block; the only barrier of the kernel follows that load).  Its waves
// take tiles of the block's share from an LDS ticket; a wave's accumulator is
// R x CB fp32 in its own LDS region.  Blocks are numbered so that each XCD
// walks a contiguous eighth of the tiles for every column (the columns of a
// tile then fetch the same source rows from the same L2).
//
// Weights reach LDS as stored: the forward layout W[o][c_src][c_dst] row by
// row (fragments built with gfx950's transposing LDS reads), the dgrad
// layout W[o][c_dst][c_src] row by row (fragments are plain 16-byte reads);
// a mirrored map stores W[kvol-1-o] in slot o.
//
// Pipeline per wave (constant load pattern per group, so the compiler's
// wait before a use covers only that use's loads): the source rows and
// slots of group g + DM, the source-row fetches of group g + DB, then the
// MFMAs of group g and the read-add-write of its accumulator rows.
#include "common.h"
#include "launch.h"

namespace ts {

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct FMfma;
template <>
struct FMfma<_Float16> {
  typedef f16x8 frag;
  static __device__ __forceinline__ f32x4 run(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};
template <>
struct FMfma<__bf16> {
  typedef bf16x8 frag;
  static __device__ __forceinline__ f32x4 run(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

constexpr int kR = TS_GTILE;                     // destination rows per tile
constexpr int kLdsChunks = (156 * 1024) / 16;    // 16-byte chunks of LDS per block
constexpr int kRingM = 16;                       // register sets of (source row, slot), group mod 16
constexpr int kRingB = 8;                        // register sets of fetched rows, group mod 8
constexpr int kDM = 15;                          // groups the slot loads run ahead
constexpr int kDB = 7;                           // groups the row fetches run ahead

struct FodK {
  const int32_t* gcount;  // [n_gtiles][kvol]
  const int32_t* gsrc;    // [n_gtiles][kvol * kR]
  const uint8_t* gslot;   // [n_gtiles][kvol * kR]
  int64_t n_gtiles;
  const int64_t* n_dest;  // device destination-row count (NULL: n_dest_cap)
  int64_t n_dest_cap;
  int kvol;
  const void* src;
  uint32_t src_bytes;     // < 2^31: an offset of 2^31 reads out of range
  int c_src;
  const void* w;
  int w_vec;              // w is 16-byte aligned
  int mirror;             // slot o holds W[kvol - 1 - o]
  void* dst;
  int c_dst;
  int out_dtype;
  int ncol;               // output-channel columns
  int nsub;               // blocks per (XCD, column)
  int acc_base;           // first LDS chunk of the accumulators
};

// Swizzle of 16-byte chunk c in row r of a table whose rows hold nch chunks:
// c is XORed with bits of r below sw, the largest power of two (<= 16) that
// divides nch, so it stays inside its aligned run of sw chunks.  For nch a
// power of two, 16 consecutive rows read at one column land on 16 different
// 16-byte bank groups.
__device__ __forceinline__ int chunk_swz(int r, int c, int nch) {
  int sw = nch & -nch;
  if (sw > 16) sw = 16;
  const int per = nch >= 16 ? 1 : 16 / nch;
  return c ^ ((r / per) & (sw - 1));
}

// Forward layout, row-by-row: chunk cc (8 output channels) of row ci sits at
// cc ^ (2 * wswz(ci)) within its row; with MW column blocks of 16 channels
// per row, the 64 lanes of one transposing read fall on every 16-byte bank
// group of a 256-byte period at most twice.
template <int MW>
__device__ __forceinline__ int wswz(int ci) {
  return MW >= 8 ? ((ci & 7) + 2 * ((ci >> 3) & 3)) & 7 : ((ci >> 3) & 3) & (MW - 1);
}

// Transposing LDS reads (gfx950): in each 16-lane group, lane q + 4m names 4
// consecutive 16-bit values and lane 4q + r receives value r of the runs
// named by lanes q, q+4, q+8, q+12.  Rows of W[o] ([c_src][CB] 16-bit values)
// give lane (g, j) rows 8g..8g+7 of column j: the A fragment of output
// channel j over contracted channels 8g..8g+7.
typedef __attribute__((__vector_size__(4 * sizeof(__fp16)))) __fp16 h4tr;
typedef __attribute__((address_space(3))) h4tr lds_h4tr;
__device__ __forceinline__ u32x4 lds_tr_frag(const char* p0, const char* p4) {
  const h4tr lo = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_h4tr*)p0);
  const h4tr hi = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_h4tr*)p4);
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 l = __builtin_bit_cast(u32x2, lo), h = __builtin_bit_cast(u32x2, hi);
  return u32x4{l[0], l[1], h[0], h[1]};
}

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

template <int I>
struct Fi {
  static constexpr int v = I;
};

// Waves per block at most: 12 (three per SIMD, up to 168 registers per
// lane), or 8 for 96 and 128 contracted channels or 32-channel columns,
// whose operand rings need more.
constexpr int fod_max_waves(int kb, int mw) { return (kb >= 3 || mw >= 2) ? 8 : 12; }

template <typename T, int KB, int MW, int WM>
__global__ __launch_bounds__(64 * fod_max_waves(KB, MW)) void k_fod(FodK a) {
  typedef typename FMfma<T>::frag Frag;
  constexpr int CB = 16 * MW;         // output channels of the block column
  constexpr int NCH = CB / 4;         // 16-byte fp32 chunks per accumulator row
  constexpr int C_SRC = 32 * KB;      // contracted channels
  constexpr int WROW = WM == 0 ? CB * 2 : C_SRC * 2;  // bytes per stored weight row in LDS
  constexpr int WROWS = WM == 0 ? C_SRC : CB;         // weight rows per offset
  constexpr int WSLICE = WROW * WROWS;                // bytes per offset
  __shared__ u32x4 lds[kLdsChunks];
  __shared__ unsigned ticket;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwave = blockDim.x >> 6;
  const int col = lane & 15, kq = lane >> 4;
  const int xcd = blockIdx.x & 7;
  const int bk = blockIdx.x >> 3;
  const int column = bk % a.ncol;
  const int sub = bk / a.ncol;
  const int n0 = column * CB;
  const int kvol = a.kvol;
  char* const ldsb = reinterpret_cast<char*>(lds);

  // the column's weights for every offset, as stored, into LDS: each thread
  // issues up to 8 chunk loads before it stores any (one memory round trip
  // per 8 chunks); chunks outside the weights (channels past c_dst) load
  // element 0 and store zeros
  {
    const T* w = static_cast<const T*>(a.w);
    const int per_slice = WSLICE / 16;
    const int total = kvol * per_slice;
    auto chunk_of = [&](int i, int64_t* g, int* lpos) {
      const int o = i / per_slice, r = i - o * per_slice;
      const int os = a.mirror ? kvol - 1 - o : o;
      int lp;
      if (WM == 0) {
        const int ci = r / (CB / 8), part = r - ci * (CB / 8);
        const int co = n0 + 8 * part;
        *g = co < a.c_dst ? (static_cast<int64_t>(os) * C_SRC + ci) * a.c_dst + co : -1;
        lp = ci * WROW + 16 * (part ^ (2 * wswz<MW>(ci)));
      } else {
        const int nl = r / (C_SRC / 8), part = r - nl * (C_SRC / 8);
        const int n = n0 + nl;
        *g = n < a.c_dst ? (static_cast<int64_t>(os) * a.c_dst + n) * C_SRC + 8 * part : -1;
        lp = nl * WROW + 16 * chunk_swz(nl, part, C_SRC / 8 < 16 ? C_SRC / 8 : 16);
      }
      *lpos = o * WSLICE + lp;
    };
    for (int i0 = threadIdx.x; i0 < total; i0 += 8 * blockDim.x) {
      u32x4 v[8];
      int lpos[8];
      bool take[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * static_cast<int>(blockDim.x);
        int64_t g = -1;
        lpos[u] = 0;
        if (i < total) chunk_of(i, &g, &lpos[u]);
        take[u] = i < total;
        const int64_t gs = g >= 0 ? g : 0;
        if (a.w_vec) {
          v[u] = *reinterpret_cast<const u32x4*>(w + gs);
        } else {
          unsigned short e[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) e[j] = __builtin_bit_cast(unsigned short, w[gs + j]);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            v[u][j] = static_cast<unsigned>(e[2 * j]) | (static_cast<unsigned>(e[2 * j + 1]) << 16);
        }
        if (g < 0) v[u] = u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (take[u]) *reinterpret_cast<u32x4*>(ldsb + lpos[u]) = v[u];
    }
    if (threadIdx.x == 0) ticket = 0u;
    __syncthreads();
  }

  // this block's share of the tiles: XCD x walks the x-th eighth, its
  // blocks of this column a contiguous part each
  const int64_t nt = a.n_gtiles;
  const int64_t xlo = nt * xcd / 8, xn = nt * (xcd + 1) / 8 - xlo;
  const int64_t lo = xlo + xn * sub / a.nsub, hi = xlo + xn * (sub + 1) / a.nsub;
  const int64_t n_dest = a.n_dest ? (*a.n_dest < a.n_dest_cap ? *a.n_dest : a.n_dest_cap) : a.n_dest_cap;
  char* const accb = ldsb + static_cast<int64_t>(a.acc_base + wave * (kR * NCH)) * 16;
  const T* src = static_cast<const T*>(a.src);
  const __amdgpu_buffer_rsrc_t xr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(src), 0, static_cast<int>(a.src_bytes), 0x00020000);
  const int c_src = a.c_src;
  (void)nwave;

  // transposing-read addresses of this lane inside a forward-layout slice
  const int trq = lane & 3, trm = (lane >> 2) & 3;
  const int tr_b0 = (8 * kq + trm) * WROW + (trq >> 1) * 16 + (trq & 1) * 8;
  const int tr_b4 = tr_b0 + 4 * WROW;
  const int tr_x0 = 32 * wswz<MW>(8 * kq + trm), tr_x4 = 32 * wswz<MW>(8 * kq + 4 + trm);

  for (;;) {
    unsigned tk = 0u;
    if (lane == 0) tk = atomicAdd(&ticket, 1u);
    const int64_t t = lo + static_cast<int64_t>(__builtin_amdgcn_readfirstlane(tk));
    if (t >= hi) break;

    // zero the accumulator tile
#pragma unroll
    for (int i = 0; i < kR * NCH / 64; ++i)
      *reinterpret_cast<f32x4*>(accb + (i * 64 + lane) * 16) = f32x4{0.f, 0.f, 0.f, 0.f};

    // groups of the tile: lane o < kvol holds its offset's pair count, the
    // offset's first group (exclusive prefix of the group counts) and the
    // end of its groups
    const int cnt = lane < kvol ? a.gcount[t * kvol + lane] : 0;
    const int ng = (cnt + 15) >> 4;
    int incl = ng;
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) {
      const int y = __shfl_up(incl, sh, 64);
      incl += lane >= sh ? y : 0;
    }
    const int gfirst = incl - ng;
    const int G = __builtin_amdgcn_readlane(incl, 63);
    const int64_t ebase = t * static_cast<int64_t>(kvol) * kR;
    // offset of group g (wave-uniform g < G): the offsets whose groups all
    // come before g, counted
    auto offset_of = [&](int g) -> int {
      return __builtin_popcountll(__ballot(lane < kvol && incl <= g));
    };
    // valid lanes of group g: pairs left in its offset past 16 per earlier group
    auto live_of = [&](int g, int o) -> int {
      const int c = __builtin_amdgcn_readlane(cnt, o), f = __builtin_amdgcn_readlane(gfirst, o);
      return c - 16 * (g - f);
    };

    // Register rings indexed by group mod 8 (compile-time positions):
    // source row and slot of each lane (loaded DM groups ahead), the fetched
    // source rows (DB groups ahead), and the group's offset and live lane
    // count (decoded when its rows are fetched).
    int32_t msrc[kRingM];
    int32_t mslot[kRingM];
    Frag xs[kRingB][KB];
    int ro[kRingB], rl[kRingB];
    Frag af[MW][KB];
    int o_cur = -1;

    auto step = [&](int v, auto pc) {
      constexpr int p = decltype(pc)::v;
      // slots and source rows of group v + DM
      {
        const int g = v + kDM;
        const bool ok = g >= 0 && g < G;
        const int64_t e = ebase + (ok ? 16 * g : 0) + col;
        msrc[(p + kDM) % kRingM] = a.gsrc[e];
        mslot[(p + kDM) % kRingM] = a.gslot[e];
      }
      // source rows of group v + DB, fetched into MFMA operands (absent rows
      // read out of range: zeros, no memory access)
      {
        const int g = v + kDB;
        int o = 0, live = 0;
        if (g >= 0 && g < G) {  // wave-uniform
          o = offset_of(g);
          live = live_of(g, o);
        }
        ro[(p + kDB) % kRingB] = o;
        rl[(p + kDB) % kRingB] = live;
        const int32_t s = msrc[(p + kDB) % kRingM];
        const uint32_t off = col < live ? static_cast<uint32_t>(s * c_src + kq * 8) * 2u : 0x80000000u;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          xs[(p + kDB) % kRingB][kb] =
              __builtin_bit_cast(Frag, __builtin_amdgcn_raw_buffer_load_b128(xr, static_cast<int>(off + kb * 64), 0, 0));
      }
      if (v < 0 || v >= G) return;  // wave-uniform
      const int o = ro[p % kRingB];
      const bool live = col < rl[p % kRingB];
      const int slot = mslot[p % kRingM];
      // the accumulator rows of this group, read before the operands are
      // needed: they enter the MFMAs as the C operand
      f32x4 acc[MW];
      char* arow = accb + slot * (NCH * 16);
#pragma unroll
      for (int mb = 0; mb < MW; ++mb)
        acc[mb] = live ? *reinterpret_cast<const f32x4*>(arow + chunk_swz(slot, 4 * mb + kq, NCH) * 16)
                       : f32x4{0.f, 0.f, 0.f, 0.f};
      if (o != o_cur) {  // wave-uniform: this offset's fragments from the resident weights
        o_cur = o;
        const char* sl = ldsb + o * WSLICE;
#pragma unroll
        for (int mb = 0; mb < MW; ++mb)
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            if constexpr (WM == 0) {
              const char* s2 = sl + kb * 32 * WROW;
              af[mb][kb] = __builtin_bit_cast(Frag, lds_tr_frag(s2 + tr_b0 + ((mb * 32) ^ tr_x0),
                                                                s2 + tr_b4 + ((mb * 32) ^ tr_x4)));
            } else {
              const int nl = 16 * mb + col;
              const int c = chunk_swz(nl, 4 * kb + kq, C_SRC / 8 < 16 ? C_SRC / 8 : 16);
              af[mb][kb] = __builtin_bit_cast(Frag, *reinterpret_cast<const u32x4*>(sl + nl * WROW + 16 * c));
            }
          }
      }
#pragma unroll
      for (int mb = 0; mb < MW; ++mb) {
        f32x4 d = acc[mb];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) d = FMfma<T>::run(af[mb][kb], xs[p % kRingB][kb], d);
        if (live) *reinterpret_cast<f32x4*>(arow + chunk_swz(slot, 4 * mb + kq, NCH) * 16) = d;
      }
    };

    // virtual groups v = -16 .. G-1 in rounds of 16 (the ring positions are
    // compile-time), the first round only issuing loads; a tile without
    // pairs only writes zeros
    if (G > 0) {
      for (int v0 = -16; v0 < G; v0 += 16) {
        step(v0 + 0, Fi<0>{});
        step(v0 + 1, Fi<1>{});
        step(v0 + 2, Fi<2>{});
        step(v0 + 3, Fi<3>{});
        step(v0 + 4, Fi<4>{});
        step(v0 + 5, Fi<5>{});
        step(v0 + 6, Fi<6>{});
        step(v0 + 7, Fi<7>{});
        step(v0 + 8, Fi<8>{});
        step(v0 + 9, Fi<9>{});
        step(v0 + 10, Fi<10>{});
        step(v0 + 11, Fi<11>{});
        step(v0 + 12, Fi<12>{});
        step(v0 + 13, Fi<13>{});
        step(v0 + 14, Fi<14>{});
        step(v0 + 15, Fi<15>{});
      }
    }

    // write the tile's rows once (rows at or past the device count are not
    // written); lane l takes accumulator chunks l, l + 64, ...
    for (int it = 0; it < kR * NCH / 64; ++it) {
      const int i = it * 64 + lane;
      const int r = i / NCH, c = i - r * NCH;
      const int64_t row = t * kR + r;
      const int n = n0 + 4 * c;
      if (row < n_dest && n < a.c_dst) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(accb + (r * NCH + chunk_swz(r, c, NCH)) * 16);
        store4(a.dst, a.out_dtype, row * a.c_dst + n, v);
      }
    }
  }
}

int fod_cu_count() {
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

// LDS bytes of the resident weights of one column of 16 * mw channels.
size_t fod_weight_bytes(int kvol, int c_src, int mw) { return static_cast<size_t>(kvol) * c_src * 16 * mw * 2; }

// Column width (MFMA blocks of 16 channels per column) and waves per block:
// the widest column whose weights leave room for at least eight waves'
// accumulators, else the narrowest that leaves room for two; 0 when even
// that does not fit.
void fod_shape(int kvol, int c_src, int c_dst, int* mw_out, int* nw_out) {
  *mw_out = 0;
  *nw_out = 0;
  const size_t lds = static_cast<size_t>(kLdsChunks) * 16;
  for (int mw = 2; mw >= 1; mw >>= 1) {
    if (mw == 2 && c_dst < 32) continue;
    const int max_nw = fod_max_waves(c_src / 32, mw);
    const size_t wb = fod_weight_bytes(kvol, c_src, mw);
    if (wb >= lds) continue;
    const size_t accw = static_cast<size_t>(kR) * 16 * mw * 4;
    int nw = static_cast<int>((lds - wb) / accw);
    if (nw > max_nw) nw = max_nw;
    if (nw >= 6 || (mw == 1 && nw >= 2)) {
      *mw_out = mw;
      *nw_out = nw;
      return;
    }
  }
}

template <typename T, int KB, int MW>
hipError_t launch_kb_mw(FodK k, int wm, int nw, hipStream_t s) {
  const int ncu = fod_cu_count();
  k.ncol = ceil_div(k.c_dst, 16 * MW);
  int nsub = ncu / (8 * k.ncol);
  if (nsub < 1) nsub = 1;
  const int64_t per_xcd = ceil_div<int64_t>(k.n_gtiles, 8);
  if (nsub > per_xcd) nsub = static_cast<int>(per_xcd > 0 ? per_xcd : 1);
  k.nsub = nsub;
  k.acc_base = static_cast<int>(fod_weight_bytes(k.kvol, k.c_src, MW) / 16);
  const dim3 grid(static_cast<unsigned>(8 * k.ncol * nsub));
  if (wm == 0)
    k_fod<T, KB, MW, 0><<<grid, nw * 64, 0, s>>>(k);
  else
    k_fod<T, KB, MW, 1><<<grid, nw * 64, 0, s>>>(k);
  return hipGetLastError();
}

template <typename T, int KB>
hipError_t launch_kb(const FodK& k, int mw, int wm, int nw, hipStream_t s) {
  if (mw == 2) return launch_kb_mw<T, KB, 2>(k, wm, nw, s);
  return launch_kb_mw<T, KB, 1>(k, wm, nw, s);
}

template <typename T>
hipError_t launch_t(const FodK& k, int mw, int wm, int nw, hipStream_t s) {
  switch (k.c_src / 32) {
    case 1: return launch_kb<T, 1>(k, mw, wm, nw, s);
    case 2: return launch_kb<T, 2>(k, mw, wm, nw, s);
    case 3: return launch_kb<T, 3>(k, mw, wm, nw, s);
    default: return launch_kb<T, 4>(k, mw, wm, nw, s);
  }
}

}  // namespace

bool fod_supported(int kvol, int64_t n_src, int c_src, int c_dst, ts_dtype in_dtype) {
  if (in_dtype == TS_F32 || kvol < 1 || c_src % 32 != 0 || c_src < 32 || c_src > 128 || c_dst % 16 != 0 ||
      c_dst < 16)
    return false;
  if (n_src * c_src * 2 >= (int64_t{1} << 31)) return false;
  int mw, nw;
  fod_shape(kvol, c_src, c_dst, &mw, &nw);
  return mw > 0;
}

hipError_t launch_fod(const ConvArgs& a, hipStream_t s) {
  const ts_rel& rel = *a.rel;
  if (rel.n_gtiles == 0) return hipSuccess;
  int mw, nw;
  fod_shape(a.kvol, a.c_src, a.c_dst, &mw, &nw);
  if (mw == 0) return hipErrorInvalidValue;
  FodK k;
  k.gcount = rel.gcount;
  k.gsrc = rel.gsrc;
  k.gslot = rel.gslot;
  k.n_gtiles = rel.n_gtiles;
  k.n_dest = rel.n_dest;
  k.n_dest_cap = rel.n_dest_cap;
  k.kvol = a.kvol;
  k.src = a.src;
  k.src_bytes = static_cast<uint32_t>(a.n_src * a.c_src * 2);
  k.c_src = a.c_src;
  k.w = a.w;
  k.w_vec = (reinterpret_cast<uintptr_t>(a.w) & 15) == 0 ? 1 : 0;
  k.mirror = a.mirror ? 1 : 0;
  k.dst = a.dst;
  k.c_dst = a.c_dst;
  k.out_dtype = a.out_dtype;
  k.ncol = 1;
  k.nsub = 1;
  k.acc_base = 0;
  const int wm = a.transpose ? 1 : 0;
  if (a.in_dtype == TS_F16) return launch_t<_Float16>(k, mw, wm, nw, s);
  return launch_t<__bf16>(k, mw, wm, nw, s);
}

}  // namespace ts
