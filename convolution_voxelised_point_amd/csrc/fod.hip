// Fetch-on-demand contraction (the third dataflow the torch-lattice page
// "Migrating from TorchSparse" names in section "Backend and configuration
// differences"; the TorchSparse++ abstract credits dataflows that overlap
// computation with memory access).  It walks a relation stored as per-tile
// pair groups: the destination rows are cut into tiles of TS_GTILE rows, and
// inside a tile the pairs of each offset are listed in destination order and
// padded to whole groups of 16 (pads name no source row and the sink slot
// TS_GTILE), so group g of a tile occupies entries [16g, 16g + 16).  Every
// group is one 16-pair MFMA product with a single offset's weights: only the
// source rows that exist are fetched, straight from the source matrix into
// MFMA operands (no gather buffer), and the products are added into the
// destination rows of an fp32 accumulator tile held in LDS, which is written
// out once.  There are no atomics: within a group the destination rows are
// distinct, and one wave owns each accumulator tile and adds its groups in
// a fixed offset order, so results are bitwise repeatable.
//
// Work split.  A block covers one column of output channels -- 32 for
// layers of up to 64 outputs, else 64 -- for NT tiles, with one compute
// wave per 32 channels of a tile (a 64-channel column is split into halves:
// smaller accumulators, more waves to overlap each other's waits), and one
// loader wave.  The block steps through the
// offsets in lockstep: barrier k means that step k's weights sit in LDS (a
// ring of three slices, loaded by the loader wave two steps ahead with
// direct global-to-LDS copies) and that every compute wave is done with the
// steps before k.  A
// compute wave passes the barriers of the steps its tile lacks without
// work, and its gathers run ahead of the barriers (they do not depend on the
// weights).  Blocks are numbered so that each XCD walks a contiguous range
// of block indexes (a tile's columns fetch the same source rows from the
// same L2); block b holds tiles b, b + nblk, ... (nblk blocks per column).
//
// Weights reach LDS as stored: the forward layout W[o][c_src][c_dst] row by
// row (fragments built with gfx950's transposing LDS reads), the dgrad
// layout W[o][c_dst][c_src] row by row (fragments are plain 16-byte reads);
// a mirrored map takes W[kvol-1-o] for offset o.
//
// Pipeline per compute wave (constant load pattern per group, so the
// compiler's wait before a use covers only that use's loads): the source-row
// fetches of group g + DB, the source rows and slots of group g + DM, then
// the MFMAs of group g and the read-add-write of its accumulator rows.  The
// loads are in flight for DB and DM groups: a gather from HBM takes
// microseconds under load, so the depth, not the instruction count, sets the
// time per group.
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

constexpr int kR = TS_GTILE;          // destination rows per tile (row kR of an accumulator: pad sink)
constexpr int kSlots = 3;             // weight slots in LDS: steps k, k + 1, k + 2
constexpr int kLdsBytes = 160 * 1024; // LDS of one block
// Pipeline depths (groups in flight per wave): the fetched source rows of
// RB groups (4 when three waves share a SIMD's registers, else 8), the
// entries of RM = 2 RB groups; a round is RM groups.
constexpr int fod_rb(int waves) { return waves > 8 ? 4 : 8; }

// Bytes of one offset's weight slice (c_src = 32 KB channels by 16 MW
// output channels, 16-bit) and of one wave's accumulator (kR + 1 rows of
// 16 MH fp32, MH the MFMA blocks of 16 output channels a wave owns).
constexpr int fod_slice_bytes(int kb, int mw) { return 1024 * kb * mw; }
constexpr int fod_acc_bytes(int mh) { return (kR + 1) * 64 * mh; }
// Compute waves per block at most: 8 (with the loader, three waves on one
// SIMD) for up to 64 contracted channels, else 6 (two per SIMD: their
// fetched rows need the registers).
constexpr int fod_max_nw(int kb) { return kb <= 2 ? 8 : 6; }
// Tiles per block: as many tiles' accumulators (MW / MH waves each) as fit
// beside the weight ring (slots of `ops` slices), within that wave count.
constexpr int fod_tiles(int kb, int mw, int mh, int ops) {
  return (kLdsBytes - kSlots * ops * fod_slice_bytes(kb, mw)) / (fod_acc_bytes(mh) * (mw / mh)) * (mw / mh) >
                 fod_max_nw(kb)
             ? fod_max_nw(kb) / (mw / mh)
             : (kLdsBytes - kSlots * ops * fod_slice_bytes(kb, mw)) / (fod_acc_bytes(mh) * (mw / mh));
}
// Offsets per lockstep step: two when slots of two slices still leave room
// for as many tiles as slots of one, else one.
constexpr int fod_ops(int kb, int mw, int mh) { return fod_tiles(kb, mw, mh, 2) >= fod_tiles(kb, mw, mh, 1) ? 2 : 1; }
#define FOD_OPS_OVERRIDE(x) (x)

struct FodK {
  const int32_t* gcount;  // [n_gtiles][kvol]
  const int32_t* gsrc;    // [n_gtiles][kvol * kR]
  const uint8_t* gslot;   // [n_gtiles][kvol * kR]
  int64_t n_gtiles;
  const int64_t* n_dest;  // device destination-row count (NULL: n_dest_cap)
  int64_t n_dest_cap;
  int kvol;
  const void* src;
  uint32_t src_bytes;     // < 2^31: an offset of 2^31 or more reads out of range
  int64_t n_src;          // source rows (bounds-check build)
  int c_src;
  const void* w;
  int w_vec;              // w is 16-byte aligned
  int mirror;             // step o takes W[kvol - 1 - o]
  void* dst;
  int c_dst;
  int out_dtype;
  int ncol;               // output-channel columns
  int64_t nblk;           // blocks of NT tiles
  int64_t nb8;            // ceil(nblk / 8)
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

// 16 bytes per lane from global memory straight into LDS: lane l writes
// dst + 16 l (dst is wave-uniform).  Completion is counted by the
// vector-memory counter.  Not a template: clang emits no host launch stub for
// a kernel template whose body names this builtin directly.
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
__device__ __forceinline__ void lds_copy16(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds(static_cast<const u32x4*>(src), (lds_u32x4*)dst, 16, 0, 0);
}
// Waits until at most N vector-memory operations of this wave are
// outstanding (they retire in issue order); other counters unconstrained.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | 0x70 | 0xF00 | ((N >> 4) << 14));
}
// All of this wave's LDS operations have completed.
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// Workgroup barrier with no memory fence: each wave states the waits it
// needs before it, so gathers in flight stay in flight across it.  The empty
// asm statements keep the compiler from moving memory operations across.
__device__ __forceinline__ void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
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

// A wave-uniform address, stated as such (kept in scalar registers: a
// buffer descriptor built from a vector register is used lane group by lane
// group).
__device__ __forceinline__ void* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
}

template <int I>
struct Fi {
  static constexpr int v = I;
};
// f(Fi<0>{}), ..., f(Fi<N-1>{}) in order, unrolled at compile time.
template <int N, int I = 0>
struct Unroll {
  template <class F>
  static __device__ __forceinline__ void run(F&& f) {
    f(Fi<I>{});
    Unroll<N, I + 1>::run(f);
  }
};
template <int N>
struct Unroll<N, N> {
  template <class F>
  static __device__ __forceinline__ void run(F&&) {}
};

template <typename T, int KB, int MW, int MH, int WM, int OPS>
__global__ __launch_bounds__(64 * (fod_tiles(KB, MW, MH, OPS) * (MW / MH) + 1)) void k_fod(FodK a) {
  typedef typename FMfma<T>::frag Frag;
  constexpr int WPT = MW / MH;        // compute waves per tile (one per MH blocks of 16 channels)
  constexpr int NT = fod_tiles(KB, MW, MH, OPS);  // tiles per block
  constexpr int NW = NT * WPT;        // compute waves per block
  constexpr int CB = 16 * MW;         // output channels of the block column
  constexpr int NCH = 4 * MH;         // 16-byte fp32 chunks per accumulator row
  constexpr int C_SRC = 32 * KB;      // contracted channels
  constexpr int WROW = WM == 0 ? CB * 2 : C_SRC * 2;  // bytes per stored weight row in LDS
  constexpr int SLICE = fod_slice_bytes(KB, MW);      // bytes per offset
  constexpr int COPIES = SLICE / 1024;                // 16-byte copies per lane and offset
  constexpr int SLOT = OPS * SLICE;                   // bytes per step
  constexpr int ACC = fod_acc_bytes(MH);
  static_assert(kSlots * SLOT + NW * ACC <= kLdsBytes, "LDS budget");
  __shared__ __attribute__((aligned(1024))) char lds[kSlots * SLOT + NW * ACC];

  constexpr int RB = fod_rb(NW + 1);  // fetched-row register sets
  constexpr int DB = RB - 1;          // groups the row fetches run ahead
  constexpr int RM = 2 * RB;          // slot register sets, and groups per round
  constexpr int DM = RM - 1;          // groups the entry loads run ahead
  // source-row entries live DM - DB = RB groups (loaded DM, used DB groups
  // ahead); every ring's length divides the round so positions repeat
  constexpr int RS = RM;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, kq = lane >> 4;
  const int hb = blockIdx.x;
  const int k8 = hb >> 3;
  const int column = k8 % a.ncol;
  const int64_t tb = static_cast<int64_t>(hb & 7) * a.nb8 + k8 / a.ncol;
  if (tb >= a.nblk) return;  // the whole block, before any barrier
  const int n0 = column * CB;
  const int kvol = a.kvol;
  // The block takes the offsets in order, OPS of them per lockstep step
  // (offset k: step k / OPS, slice k % OPS of its slot).  Every block starts
  // at offset 0: starting each block at its own offset, so that blocks
  // running at once copy different slices, measured slower on the ring scan.
  const int nsteps = (kvol + OPS - 1) / OPS;

  if (wave == NW) {
    // Loader: step s's weights into slot s % 3, two steps ahead of the
    // compute waves, with direct global-to-LDS copies (element by element
    // through registers when the weights are not 16-byte aligned).  Chunk p
    // of a slot (16 bytes): forward layout row ci = p / (CB/8) at swizzled
    // column, dgrad layout row nl = p / (C_SRC/8) likewise; chunks of output
    // channels past c_dst copy a valid chunk of the slice (they feed
    // accumulator channels that are never written out).  A last step with
    // fewer than OPS offsets copies its first slice again into the unused
    // ones, so every step issues the same number of copies.
    const T* w = static_cast<const T*>(a.w);
    auto chunk_src = [&](int os, int p) -> int64_t {
      if constexpr (WM == 0) {
        const int ci = p / (CB / 8), sc = p - ci * (CB / 8);
        const int part = sc ^ (2 * wswz<MW>(ci));
        const int co = n0 + 8 * part;
        return (static_cast<int64_t>(os) * C_SRC + ci) * a.c_dst + (co < a.c_dst ? co : 0);
      } else {
        const int nl = p / (C_SRC / 8), sc = p - nl * (C_SRC / 8);
        const int part = chunk_swz(nl, sc, C_SRC / 8 < 16 ? C_SRC / 8 : 16);
        const int n = n0 + nl;
        return (static_cast<int64_t>(os) * a.c_dst + (n < a.c_dst ? n : 0)) * C_SRC + 8 * part;
      }
    };
    auto copy_slice = [&](int o, char* slot) __attribute__((always_inline)) {
      const int os = a.mirror ? kvol - 1 - o : o;
      if (a.w_vec) {
#pragma unroll
        for (int j = 0; j < COPIES; ++j) lds_copy16(w + chunk_src(os, 64 * j + lane), slot + 1024 * j);
      } else {
        for (int j = 0; j < COPIES; ++j) {
          const T* g = w + chunk_src(os, 64 * j + lane);
          u32x4 v;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            v[q] = static_cast<unsigned>(__builtin_bit_cast(unsigned short, g[2 * q])) |
                   (static_cast<unsigned>(__builtin_bit_cast(unsigned short, g[2 * q + 1])) << 16);
          *reinterpret_cast<u32x4*>(slot + 1024 * j + 16 * lane) = v;
        }
      }
    };
    auto copy = [&](int st) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < OPS; ++j) {
        const int k = st * OPS + j;
        copy_slice(k < kvol ? k : st * OPS, lds + (st % kSlots) * SLOT + j * SLICE);
      }
    };
    copy(0);
    if (nsteps > 1) copy(1);
    for (int st = 0; st < nsteps; ++st) {
      // step st's weights have landed (only step st + 1's copies may still
      // be in flight)
      if (a.w_vec) {
        if (st + 1 < nsteps)
          wait_vm<OPS * COPIES>();
        else
          wait_vm<0>();
      } else {
        wait_lds();
      }
      bare_barrier();
      if (st + 2 < nsteps) copy(st + 2);  // into the slot of step st - 1: every wave is past it
    }
    return;
  }

  // compute wave: tile t, output channels n0 + 16 MH h .. + 16 MH.  The
  // block's tiles are tb, tb + nblk, tb + 2 nblk, ...: tiles from distant
  // parts of the scene share a block, so that blocks whose lockstep steps
  // wait on their densest tile carry similar loads (on the ring scan in row
  // order, 26 against 28.5 us with NT consecutive tiles per block).
  const int h = wave % WPT;
  const int64_t t = tb + static_cast<int64_t>(wave / WPT) * a.nblk;
  const bool has_tile = t < a.n_gtiles;
  const int nw0 = n0 + 16 * MH * h;
  const int acc_off = kSlots * SLOT + wave * ACC;  // this wave's accumulator (row-size aligned)
  char* const accb = lds + acc_off;
#pragma unroll
  for (int i = 0; i < kR * NCH / 64; ++i)
    *reinterpret_cast<f32x4*>(accb + (i * 64 + lane) * 16) = f32x4{0.f, 0.f, 0.f, 0.f};

  const int64_t ebase = t * static_cast<int64_t>(kvol) * kR;
  const T* src = static_cast<const T*>(a.src);
  const __amdgpu_buffer_rsrc_t xr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(src), 0, static_cast<int>(a.src_bytes), 0x00020000);

  // Register rings indexed by group (compile-time positions): source row and
  // slot of each lane (loaded DM groups ahead), the fetched source rows (DB
  // groups ahead).  A slot is loaded as the aligned word that holds it (a
  // group's entries start at a multiple of 16, so lane col's byte is byte
  // col % 4 of its word) and taken out at its use: a ring of byte loads
  // would be widened where the rounds loop back, which waits for them all.
  // Entry loads go through buffer descriptors over the tile's entries, the
  // group's position in the scalar offset (a wave without a tile gets empty
  // descriptors: its loads read zeros and touch no memory).  Source-row
  // fetches are not masked: pads (-1) read out of range (zeros, no access),
  // and groups past the tile's last fetch rows that are never used.
  int32_t msrc[RS];
  uint32_t mslot[RM];
  Frag xs[RB][KB];
  Frag af[MH][KB];
  const int slot_shift = 8 * (col & 3);
  const __amdgpu_buffer_rsrc_t er_src =
      __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(a.gsrc + ebase), 0, has_tile ? kvol * kR * 4 : 0, 0x00020000);
  const __amdgpu_buffer_rsrc_t er_slot =
      __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(a.gslot + ebase), 0, has_tile ? kvol * kR : 0, 0x00020000);
  // the entries of groups 0 .. DM-1 (the first round's) go out before the
  // group counts are read: they need no count (entries past the tile's
  // groups feed no MFMA)
  Unroll<DM>::run([&](auto ic) {
    constexpr int i = decltype(ic)::v;
    msrc[i % RS] = __builtin_bit_cast(int32_t, __builtin_amdgcn_raw_buffer_load_b32(er_src, 4 * col, 64 * i, 0));
    mslot[i % RM] = __builtin_amdgcn_raw_buffer_load_b32(er_slot, col & ~3, 16 * i, 0);
  });
  // groups of the tile in offset order: lane k < kvol holds the group count
  // of offset k and the end of its groups (inclusive prefix)
  const int cnt = has_tile && lane < kvol ? dbg_req(a.gcount[t * kvol + lane], kR + 1, TS_DEBUG_DST_ROW) : 0;
  const int ng = (cnt + 15) >> 4;
  int incl = ng;
#pragma unroll
  for (int sh = 1; sh < 64; sh <<= 1) {
    const int y = __shfl_up(incl, sh, 64);
    incl += lane >= sh ? y : 0;
  }
  const int G = __builtin_amdgcn_readlane(incl, 63);
  const uint64_t present = __ballot(lane < kvol && ng > 0);

  // transposing-read addresses of this lane inside a forward-layout slice
  const int trq = lane & 3, trm = (lane >> 2) & 3;
  const int tr_b0 = (8 * kq + trm) * WROW + (trq >> 1) * 16 + (trq & 1) * 8;
  const int tr_b4 = tr_b0 + 4 * WROW;
  const int tr_x0 = 32 * wswz<MW>(8 * kq + trm), tr_x4 = 32 * wswz<MW>(8 * kq + 4 + trm);

  int k_cur = -1;  // offset whose fragments are held
  int s_cur = -1;  // barriers 0..s_cur passed
  int e_cur = 0;   // end of offset k_cur's groups

  // accumulator chunk swizzle: chunk c of row r sits at c ^ sw(r) (the
  // chunk_swz layout), so the MH chunks of a lane's row are the address of
  // chunk kq ^ sw(r) with bit 6 and up XORed by 64 mb (rows are 64 MH bytes,
  // row-size aligned)
  constexpr int SW_PER = NCH >= 16 ? 1 : 16 / NCH;
  constexpr int SW_MASK = (NCH >= 16 ? 16 : NCH) - 1;

  // one group position p of a round: the fetch of group v0 + p + DB's
  // source rows, then the entry loads of group v0 + p + DM (groups past the
  // tile's last read stored group 0; the first round's entries are loaded
  // before the counts), then, outside the first round, the
  // MFMAs of group v0 + p.  The fetch reads its source-row entry before the
  // entry load of the same step reuses that register.
  auto step = [&](int v0, auto pc, auto firstc) {
    constexpr int p = decltype(pc)::v;
    constexpr bool FIRST = decltype(firstc)::v;
    if constexpr (!FIRST || p + DB >= RM) {
      int32_t ms = msrc[(p + DB) % RS];
      // (the bounds-check build checks the entries of the tile's groups:
      // the first round's may lie past them)
      if constexpr (kDebugChecks) ms = v0 + p + DB < G ? dbg_opt(ms, a.n_src, TS_DEBUG_SRC_ROW) : ms;
      const uint32_t off = static_cast<uint32_t>(ms) * (C_SRC * 2) + kq * 16;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        xs[(p + DB) % RB][kb] =
            __builtin_bit_cast(Frag, __builtin_amdgcn_raw_buffer_load_b128(xr, static_cast<int>(off + kb * 64), 0, 0));
    }
    if constexpr (!FIRST) {  // (the first round's entries are loaded above)
      const int g = v0 + p + DM;
      const int sg = g < G ? g : 0;
      msrc[(p + DM) % RS] = __builtin_bit_cast(int32_t, __builtin_amdgcn_raw_buffer_load_b32(er_src, 4 * col, 64 * sg, 0));
      mslot[(p + DM) % RM] = __builtin_amdgcn_raw_buffer_load_b32(er_slot, col & ~3, 16 * sg, 0);
    }
    if constexpr (FIRST) return;
    const int v = v0 + p;
    if (v >= G) return;  // wave-uniform
    if (v >= e_cur) {  // wave-uniform: the first group of the next offset the tile has
      const int k_new = __builtin_ctzll(present & (~0ull << (k_cur + 1)));
      e_cur = __builtin_amdgcn_readlane(incl, k_new);
      const int s_new = k_new / OPS;
      for (int st = s_cur + 1; st <= s_new; ++st) bare_barrier();
      s_cur = s_new;
      k_cur = k_new;
      const char* sl = lds + (s_new % kSlots) * SLOT + (k_new - s_new * OPS) * SLICE;
#pragma unroll
      for (int mb = 0; mb < MH; ++mb)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const int mg = MH * h + mb;  // block of the slice
          if constexpr (WM == 0) {
            const char* s2 = sl + kb * 32 * WROW;
            af[mb][kb] = __builtin_bit_cast(Frag, lds_tr_frag(s2 + tr_b0 + ((mg * 32) ^ tr_x0),
                                                              s2 + tr_b4 + ((mg * 32) ^ tr_x4)));
          } else {
            const int nl = 16 * mg + col;
            const int c = chunk_swz(nl, 4 * kb + kq, C_SRC / 8 < 16 ? C_SRC / 8 : 16);
            af[mb][kb] = __builtin_bit_cast(Frag, *reinterpret_cast<const u32x4*>(sl + nl * WROW + 16 * c));
          }
        }
    }
    // the group's accumulator rows (the pad sink included) enter the MFMAs
    // as the C operand and are written back
    uint32_t slot = (mslot[p % RM] >> slot_shift) & 0xffu;
    if constexpr (kDebugChecks) slot = static_cast<uint32_t>(dbg_req(static_cast<int32_t>(slot), kR + 1, TS_DEBUG_DST_ROW));
    const uint32_t abase = static_cast<uint32_t>(acc_off) + slot * (NCH * 16) +
                           16u * (static_cast<uint32_t>(kq) ^ ((slot / SW_PER) & SW_MASK));
    f32x4 acc[MH];
#pragma unroll
    for (int mb = 0; mb < MH; ++mb) acc[mb] = *reinterpret_cast<const f32x4*>(lds + (abase ^ (64u * mb)));
#pragma unroll
    for (int mb = 0; mb < MH; ++mb) {
      f32x4 d = acc[mb];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) d = FMfma<T>::run(af[mb][kb], xs[p % RB][kb], d);
      *reinterpret_cast<f32x4*>(lds + (abase ^ (64u * mb))) = d;
    }
  };
  auto round = [&](int v0, auto firstc) { Unroll<RM>::run([&](auto pc) { step(v0, pc, firstc); }); };

  // groups in rounds of RM (the ring positions are compile-time): a first
  // round of loads only (entries of groups 0..DM-1, rows of groups
  // 0..DB-1), then rounds that each compute RM groups
  if (G > 0) {
    round(-RM, Fi<1>{});
    for (int v0 = 0; v0 < G; v0 += RM) round(v0, Fi<0>{});
  }
  // the barriers of the steps past the tile's last one
  for (int st = s_cur + 1; st < nsteps; ++st) bare_barrier();
  if (!has_tile) return;

  // write the tile's rows once (rows at or past the device count are not
  // written); lane l takes accumulator chunks l, l + 64, ..., read eight at
  // a time before they are stored
  const int64_t n_dest = a.n_dest ? (*a.n_dest < a.n_dest_cap ? *a.n_dest : a.n_dest_cap) : a.n_dest_cap;
  const int64_t left = n_dest - t * kR;
  const int rows = static_cast<int>(left < kR ? (left > 0 ? left : 0) : kR);
  constexpr int ITS = kR * NCH / 64;
  constexpr int UN = ITS < 8 ? ITS : 8;
  for (int it0 = 0; it0 < ITS; it0 += UN) {
    f32x4 v[UN];
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int i = (it0 + u) * 64 + lane;
      const int r = i / NCH, c = i - r * NCH;
      v[u] = *reinterpret_cast<const f32x4*>(accb + (r * NCH + chunk_swz(r, c, NCH)) * 16);
    }
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int i = (it0 + u) * 64 + lane;
      const int r = i / NCH, c = i - r * NCH;
      const int n = nw0 + 4 * c;
      if (r < rows && n < a.c_dst) store4(a.dst, a.out_dtype, (t * kR + r) * a.c_dst + n, v[u]);
    }
  }
}

// Column width in MFMA blocks of 16 output channels.  Layers of up to 64
// output channels take columns of 32: a block then holds eight tiles (one
// wave each) instead of four (two waves each), and the two columns fetch
// every source row once each; on the ring scan (64 -> 64) that measured
// 25.0 against 26.0 us.  Wider layers keep columns of 64.
int fod_mw(int c_dst) { return c_dst > 64 ? 4 : (c_dst > 16 ? 2 : 1); }

template <typename T, int KB, int MW>
hipError_t launch_kb_mw(FodK k, int wm, hipStream_t s) {
  constexpr int MH = MW >= 2 ? 2 : 1;  // two compute waves per tile for 64-channel columns
  constexpr int OPS = FOD_OPS_OVERRIDE(fod_ops(KB, MW, MH));
  constexpr int NT = fod_tiles(KB, MW, MH, OPS);
  constexpr int NW = NT * (MW / MH);
  static_assert(NT >= 1, "a tile fits");
  k.ncol = ceil_div(k.c_dst, 16 * MW);
  k.nblk = ceil_div<int64_t>(k.n_gtiles, NT);
  k.nb8 = ceil_div<int64_t>(k.nblk, 8);
  const int64_t blocks = 8 * k.nb8 * k.ncol;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(blocks));
  if (wm == 0)
    k_fod<T, KB, MW, MH, 0, OPS><<<grid, (NW + 1) * 64, 0, s>>>(k);
  else
    k_fod<T, KB, MW, MH, 1, OPS><<<grid, (NW + 1) * 64, 0, s>>>(k);
  return hipGetLastError();
}

template <typename T, int KB>
hipError_t launch_kb(const FodK& k, int wm, hipStream_t s) {
  switch (fod_mw(k.c_dst)) {
    case 4: return launch_kb_mw<T, KB, 4>(k, wm, s);
    case 2: return launch_kb_mw<T, KB, 2>(k, wm, s);
    default: return launch_kb_mw<T, KB, 1>(k, wm, s);
  }
}

template <typename T>
hipError_t launch_t(const FodK& k, int wm, hipStream_t s) {
  switch (k.c_src / 32) {
    case 1: return launch_kb<T, 1>(k, wm, s);
    case 2: return launch_kb<T, 2>(k, wm, s);
    case 3: return launch_kb<T, 3>(k, wm, s);
    default: return launch_kb<T, 4>(k, wm, s);
  }
}

}  // namespace

bool fod_supported(int kvol, int64_t n_src, int c_src, int c_dst, ts_dtype in_dtype) {
  if (in_dtype == TS_F32 || kvol < 1 || kvol > TS_MAX_KVOL || c_src % 32 != 0 || c_src < 32 || c_src > 128 ||
      c_dst % 16 != 0 || c_dst < 16)
    return false;
  return n_src * c_src * 2 < (int64_t{1} << 31);
}

hipError_t launch_fod(const ConvArgs& a, hipStream_t s) {
  const ts_rel& rel = *a.rel;
  if (rel.n_gtiles == 0) return hipSuccess;
  if (!fod_supported(a.kvol, a.n_src, a.c_src, a.c_dst, a.in_dtype)) return hipErrorInvalidValue;
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
  k.n_src = a.n_src;
  k.c_src = a.c_src;
  k.w = a.w;
  k.w_vec = (reinterpret_cast<uintptr_t>(a.w) & 15) == 0 ? 1 : 0;
  k.mirror = a.mirror ? 1 : 0;
  k.dst = a.dst;
  k.c_dst = a.c_dst;
  k.out_dtype = a.out_dtype;
  k.ncol = 1;
  k.nblk = 0;
  k.nb8 = 0;
  const int wm = a.transpose ? 1 : 0;
  if (a.in_dtype == TS_F16) return launch_t<_Float16>(k, wm, s);
  return launch_t<__bf16>(k, wm, s);
}

}  // namespace ts

TS_DEBUG_TU(fod)
