// Kernel-map construction (the "kernel-map construction" that the
// torch-lattice page "Migrating from TorchSparse" names in section "Sparse
// tensor expectations"): for each destination row and kernel offset, the
// source row at the displaced coordinate (a row-major [rows][kvol] table),
// plus per-row and per-tile offset masks so that the contraction skips empty
// offsets.
//
// Three relations share the code, differing only in how the probed
// coordinate is formed from the destination coordinate c and offset delta:
//   submanifold  (dest = outputs = inputs):  c + delta       in the input table
//   downsampling (dest = strided outputs):   s*c + delta     in the input table
//   transposed   (dest = inputs):            (c - delta)/s   in the output table,
//                                            only when s divides c - delta
//
// Probing: a lane owns one destination row; the coordinate table is a grid
// of voxel blocks, so all offsets of a row resolve through at most 2^D block
// lookups (issued together) and then one cell load per offset.
//
// Tiles: rows are either kept in index order (spatially local) or, by
// default, sorted by offset mask inside windows of 4096 rows so that the 16
// rows of a tile share most offsets and the contraction pads less.  The sort
// is stable (ties keep row order), so the map is deterministic.
#include "common.h"
#include "launch.h"

namespace ts {

namespace {

constexpr int kSortItems = 4;  // rows per sorting thread

struct RelK {
  const int32_t* dc;
  int64_t n_dest_cap;
  const int64_t* n_dest;
  int ndim, stride, kvol, centre;
  int stride_shift;  // log2(stride) when stride is a power of two, else -1
  Offsets offs;
  Table src;
  Table own;
  int64_t n_tiles;
  uint64_t* tile_mask;
  int32_t* tile_rows;
  int32_t* nbr;
  uint64_t* row_mask;
  int64_t n_gtiles;  // pair-group tiles (0: no groups)
  int32_t* gcount;
  int32_t* gsrc;
  uint8_t* gslot;
};

__device__ __forceinline__ int64_t dest_count(const int64_t* n_dest, int64_t cap) {
  if (!n_dest) return cap;
  const int64_t n = *n_dest;
  return n < cap ? n : cap;
}

// Compile-time kernel geometry: offsets as packed key displacements.  A key
// is [batch:16][axis0+2^15:16][axis1+2^15:16][axis2+2^15:16] (2-D keys keep
// the last field at 2^15), so displacing a coordinate by delta adds
// delta0*2^32 + delta1*2^16 + delta2 to its key as long as no field leaves
// [0, 65535] -- which each probe checks per axis.
template <int ND, int K>
struct Geo {
  static constexpr int KV = ND == 3 ? K * K * K : K * K;
  static constexpr int R = (K - 1) / 2;
  int8_t d[KV][3];
  int64_t packed[KV];
  constexpr Geo() : d{}, packed{} {
    for (int o = 0; o < KV; ++o) {
      int rem = o;
      for (int ax = ND - 1; ax >= 0; --ax) {
        d[o][ax] = static_cast<int8_t>(rem % K - R);
        rem /= K;
      }
      packed[o] = d[o][0] * (int64_t{1} << 32) + d[o][1] * (int64_t{1} << 16) + (ND == 3 ? d[o][2] : 0);
    }
  }
};

// Biased fields (value + 2^15) of a coordinate, as int64; false when the
// batch or a field is out of range.
template <int ND>
__device__ __forceinline__ bool fields_of(int64_t b, const int64_t* v, int64_t* f) {
  if (b < 0 || b > 65534) return false;
  bool ok = true;
#pragma unroll
  for (int ax = 0; ax < 3; ++ax) {
    f[ax] = ax < ND ? v[ax] + 32768 : 32768;
    ok = ok && f[ax] >= 0 && f[ax] <= 65535;
  }
  return ok;
}

__device__ __forceinline__ uint64_t key_of_fields(int64_t b, const int64_t* f) {
  return (static_cast<uint64_t>(b) << 48) | (static_cast<uint64_t>(f[0]) << 32) | (static_cast<uint64_t>(f[1]) << 16) |
         static_cast<uint64_t>(f[2]);
}

// Key probed at offset o from the base fields f (already scaled by the
// stride for the downsampling relation); false when a field leaves range.
template <int ND, int K>
__device__ __forceinline__ bool offset_key(const Geo<ND, K>& g, uint64_t base, const int64_t* f, int o,
                                           uint64_t* key) {
  bool ok = true;
#pragma unroll
  for (int ax = 0; ax < ND; ++ax) {
    const int64_t v = f[ax] + g.d[o][ax];
    ok = ok && v >= 0 && v <= 65535;
  }
  *key = base + static_cast<uint64_t>(g.packed[o]);
  return ok;
}

// All offsets of one row against the two-level table.  The displaced
// coordinates of a kernel of size K span at most two blocks per axis, i.e. at
// most 2^ND "corner" blocks:
//   phase 1: the slots of the needed corner blocks, looked up together in
//            rounds (every round issues the loads of all unresolved corners);
//   phase 2: one cell load per offset, all issued before any is used.
// No load sits under a branch (invalid ones read cell 0 and are masked), so
// a row costs two memory round trips plus rare collision rounds.  Whether an
// offset's coordinate lies in the upper block, in range, and its cell bits
// depend on each axis's displacement alone, so they are worked out per axis
// and displacement (K values) and combined per offset: the corner slot of an
// offset is picked by a tree of selects (x, then y, then z) shared between
// offsets, rather than compared against all 2^ND corners.  `valid` false
// probes nothing.
template <int ND, int K>
__device__ __forceinline__ void probe_fields(const Table& t, uint64_t base, const int64_t* f, bool valid,
                                             int32_t (&nb)[Geo<ND, K>::KV]) {
  constexpr int KV = Geo<ND, K>::KV;
  constexpr int LB = ND == 3 ? 2 : 3;  // log2 of the block side
  constexpr int NC = 1 << ND;
  constexpr int DMIN = -Geo<ND, K>::R, DMAX = K - 1 - Geo<ND, K>::R;
  const uint64_t b = base >> 48;
  int64_t lo[3] = {0, 0, 0}, hi[3] = {0, 0, 0};
  bool live = valid;
#pragma unroll
  for (int ax = 0; ax < ND; ++ax) {
    const int64_t vmin = f[ax] + DMIN, vmax = f[ax] + DMAX;
    live = live && vmax >= 0 && vmin <= 65535;
    lo[ax] = (vmin < 0 ? 0 : vmin) >> LB;
    hi[ax] = (vmax > 65535 ? 65535 : vmax) >> LB;
  }
  // per axis and displacement DMIN + i: upper block, in range, cell bits
  bool up[3][K], inr[3][K];
  uint32_t cb[3][K];
  uint32_t seen[3] = {1u, 1u, 1u};  // block bits that occur on each axis (bit 0: lower, bit 1: upper)
#pragma unroll
  for (int ax = 0; ax < ND; ++ax) {
    seen[ax] = 0;
#pragma unroll
    for (int i = 0; i < K; ++i) {
      const int64_t v = f[ax] + DMIN + i;
      up[ax][i] = (v >> LB) != lo[ax];
      inr[ax][i] = v >= 0 && v <= 65535;
      cb[ax][i] = static_cast<uint32_t>(v) & ((1u << LB) - 1);
      seen[ax] |= up[ax][i] ? 2u : 1u;
    }
  }
  // the corners needed: every combination of the block bits that occur
  uint32_t need = 0;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    bool use = live;
#pragma unroll
    for (int ax = 0; ax < ND; ++ax) use = use && ((seen[ax] >> ((c >> ax) & 1)) & 1);
    need |= use ? 1u << c : 0u;
  }
  // phase 1: corner block slots
  uint64_t bk[NC];
  uint32_t slot[NC];
  int32_t found[NC];
  uint32_t pend = need;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const uint64_t b0 = (c & 1) ? hi[0] : lo[0];
    const uint64_t b1 = (c & 2) ? hi[1] : lo[1];
    const uint64_t b2 = ND == 3 ? static_cast<uint64_t>((c & 4) ? hi[2] : lo[2]) : static_cast<uint64_t>(f[2]);
    bk[c] = (b << 48) | (b0 << 32) | (b1 << 16) | b2;
    slot[c] = static_cast<uint32_t>(first_slot(t, bk[c]));
    found[c] = -1;
  }
  // each round reads kProbeRead consecutive slots (16 bytes) at every pending
  // corner's probe position -- half of an aligned group, which keeps the
  // registers of 8 corners in flight low -- and resolves the first slot that
  // holds the key or is empty
  constexpr int kProbeRead = 2;
  for (uint64_t round = 0; round <= t.mask && __ballot(pend != 0); ++round) {
    uint4 g[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) g[c] = *reinterpret_cast<const uint4*>(t.keys + (((pend >> c) & 1) ? slot[c] : 0));
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (!((pend >> c) & 1)) continue;
      const uint64_t k2[2] = {~((static_cast<uint64_t>(g[c].y) << 32) | g[c].x),
                              ~((static_cast<uint64_t>(g[c].w) << 32) | g[c].z)};
      int hit = -1;
      bool stop = false;
#pragma unroll
      for (int j = kProbeRead - 1; j >= 0; --j) {  // first position that holds the key or is empty
        if (k2[j] == bk[c]) { hit = j; stop = true; }
        else if (k2[j] == kEmptyKey) { hit = -1; stop = true; }
      }
      if (stop) {
        if (hit >= 0) found[c] = static_cast<int32_t>(slot[c] + hit);
        pend &= ~(1u << c);
      } else {
        slot[c] = static_cast<uint32_t>((slot[c] + kProbeRead) & t.mask);
      }
    }
  }
  // phase 2: the corner slot of each offset by selects along x, then y, then
  // z; then its cell
  int32_t r[KV];
  bool ok[KV];
  if constexpr (ND == 3) {
    int32_t sx[K][4];  // by x displacement: the slots of the four (y, z) corners
#pragma unroll
    for (int i0 = 0; i0 < K; ++i0)
#pragma unroll
      for (int yz = 0; yz < 4; ++yz) sx[i0][yz] = up[0][i0] ? found[1 | (yz << 1)] : found[yz << 1];
#pragma unroll
    for (int i0 = 0; i0 < K; ++i0)
#pragma unroll
      for (int i1 = 0; i1 < K; ++i1) {
        const int32_t z0 = up[1][i1] ? sx[i0][1] : sx[i0][0];
        const int32_t z1 = up[1][i1] ? sx[i0][3] : sx[i0][2];
        const bool in01 = live && inr[0][i0] && inr[1][i1];
        const uint32_t c01 = (cb[0][i0] << 4) | (cb[1][i1] << 2);
#pragma unroll
        for (int i2 = 0; i2 < K; ++i2) {
          const int o = (i0 * K + i1) * K + i2;
          const int32_t sl = up[2][i2] ? z1 : z0;
          ok[o] = in01 && inr[2][i2] && sl >= 0;
          const uint32_t ci = ok[o] ? static_cast<uint32_t>(sl) * kCells + (c01 | cb[2][i2]) : 0u;  // < 2^31
          r[o] = t.cells[ci];
        }
      }
  } else {
#pragma unroll
    for (int i0 = 0; i0 < K; ++i0) {
      const int32_t y0 = up[0][i0] ? found[1] : found[0];
      const int32_t y1 = up[0][i0] ? found[3] : found[2];
#pragma unroll
      for (int i1 = 0; i1 < K; ++i1) {
        const int o = i0 * K + i1;
        const int32_t sl = up[1][i1] ? y1 : y0;
        ok[o] = live && inr[0][i0] && inr[1][i1] && sl >= 0;
        const uint32_t ci = ok[o] ? static_cast<uint32_t>(sl) * kCells + ((cb[0][i0] << 3) | cb[1][i1]) : 0u;
        r[o] = t.cells[ci];
      }
    }
  }
#pragma unroll
  for (int o = 0; o < KV; ++o) nb[o] = ok[o] ? cell_row(static_cast<uint32_t>(r[o])) : -1;
}

// Base fields of destination `row` for the submanifold (c) and downsampling
// (s*c) relations; false when the row takes no part.
template <int MODE, int ND>
__device__ __forceinline__ bool dest_fields(const RelK& a, int64_t row, uint64_t* base, int64_t* f) {
  const int32_t* c = a.dc + row * (ND + 1);
  int64_t v[3] = {0, 0, 0};
#pragma unroll
  for (int ax = 0; ax < ND; ++ax) v[ax] = c[1 + ax];
  int64_t f0[3];
  if (!fields_of<ND>(c[0], v, f0)) return false;  // the row's own coordinate must be valid
  if (MODE == kModeDown) {
#pragma unroll
    for (int ax = 0; ax < ND; ++ax) v[ax] *= a.stride;
  }
  // scaled fields may leave range; offset_key checks every probe
#pragma unroll
  for (int ax = 0; ax < 3; ++ax) f[ax] = ax < ND ? v[ax] + 32768 : 32768;
  *base = (static_cast<uint64_t>(c[0]) << 48) + (static_cast<uint64_t>(f[0]) << 32) +
          (static_cast<uint64_t>(f[1]) << 16) + static_cast<uint64_t>(f[2]);
  return true;
}

// Destination coordinate of `row`; false when the row takes no part.
template <int MODE>
__device__ __forceinline__ bool dest_load(const RelK& a, int64_t row, int64_t* b, int64_t* s) {
  const int32_t* c = a.dc + row * (a.ndim + 1);
  *b = c[0];
  s[0] = s[1] = s[2] = 0;
  for (int d = 0; d < a.ndim; ++d) s[d] = c[1 + d];
  uint64_t key;
  if (!make_key(a.ndim, *b, s, &key)) return false;
  if (MODE == kModeUp) return table_find(a.own, key) == static_cast<int32_t>(row);
  return true;
}

// Key probed for offset o; false when no source row can exist there.
template <int MODE>
__device__ __forceinline__ bool probe_key(const RelK& a, const int8_t* offs, int64_t b, const int64_t* s, int o,
                                          uint64_t* key) {
  int64_t p[3] = {0, 0, 0};
  for (int d = 0; d < a.ndim; ++d) {
    const int64_t dd = offs[o * 3 + d];
    if (MODE == kModeSubm) {
      p[d] = s[d] + dd;
    } else if (MODE == kModeDown) {
      p[d] = static_cast<int64_t>(a.stride) * s[d] + dd;
    } else {
      // the transposed relation: (p - delta) / s where exact; coordinates
      // fit in 32 bits, and a power-of-two stride needs no division
      const int32_t t = static_cast<int32_t>(s[d] - dd);
      if (a.stride_shift >= 0) {
        if (t & ((1 << a.stride_shift) - 1)) return false;
        p[d] = t >> a.stride_shift;  // exact: arithmetic shift of a multiple
      } else {
        if (t % a.stride != 0) return false;
        p[d] = t / a.stride;
      }
    }
  }
  return make_key(a.ndim, b, p, key);
}

template <int MODE>
__device__ __forceinline__ int32_t probe(const RelK& a, const int8_t* offs, int64_t b, const int64_t* s, int o) {
  uint64_t key;
  if (!probe_key<MODE>(a, offs, b, s, o, &key)) return -1;
  return table_find(a.src, key);
}

__device__ __forceinline__ uint64_t group16_or(uint64_t v) {
  uint32_t lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(v >> 32);
#pragma unroll
  for (int sh = 8; sh >= 1; sh >>= 1) {
    lo |= __shfl_xor(lo, sh, 64);
    hi |= __shfl_xor(hi, sh, 64);
  }
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ void load_offsets(const RelK& a, int8_t* offs) {
  const int8_t* src_offs = &a.offs.d[0][0];
  for (int i = threadIdx.x; i < a.kvol * 3; i += blockDim.x) offs[i] = src_offs[i];
  __syncthreads();
}

// A wave-uniform address, stated as such (a buffer descriptor built from a
// vector register would be used lane group by lane group).
template <typename P>
__device__ __forceinline__ P* wave_uniform(P* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<P*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Group tiles of a 256-row workgroup: TS_GTILE rows are kWpt wavefronts,
// and a workgroup covers kTpb tiles.
constexpr int kWpt = TS_GTILE / 64;
constexpr int kTpb = 256 / TS_GTILE;
static_assert(TS_GTILE % 64 == 0 && 256 % TS_GTILE == 0, "group tiles of whole wavefronts within a workgroup");

// Pair groups of the kTpb group tiles of a workgroup of 256 destination
// rows, one lane per row (thread i = slot i % TS_GTILE of tile
// kTpb * blockIdx.x + i / TS_GTILE).  `nb(o)` is the lane's source row at
// offset o, read only where bit o of `mask` is set.  Per offset, each
// wavefront counts its rows by a ballot; the first wavefront of each tile
// turns the counts into the offsets' padded runs (an exclusive scan over
// offsets of whole groups of 16) and the tile's counts; every lane then
// writes its pairs at its run's start plus its rank among the tile's rows
// with that offset, so each run lists destination rows in order.  Every
// thread must call this (barriers).
template <int KVMAX, typename NB>
__device__ __forceinline__ void emit_groups(const RelK& a, int kvol, uint64_t mask, NB nb) {
  __shared__ int gw[4][KVMAX];         // pairs per wavefront and offset
  __shared__ int gstart[kTpb][KVMAX];  // first entry of each offset's run, per tile
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // unrolled for the compile-time kernel sizes (at most 27 offsets); the
  // runtime-size instance (up to TS_MAX_KVOL) keeps its loops
  constexpr int kUnroll = KVMAX <= 32 ? KVMAX : 1;
#pragma unroll kUnroll
  for (int o = 0; o < KVMAX; ++o) {
    if (o >= kvol) break;
    const uint64_t b = __ballot((mask >> o) & 1);
    if (lane == 0) gw[wave][o] = __popcll(b);
  }
  __syncthreads();
  const int h = wave / kWpt, wt = wave % kWpt;  // tile of the workgroup, wavefront of the tile
  const int64_t gt = static_cast<int64_t>(blockIdx.x) * kTpb + h;
  if (wt == 0) {  // wave-uniform: the first wavefront of each tile
    int c = 0;
#pragma unroll
    for (int i = 0; i < kWpt; ++i) c += lane < kvol ? gw[wave + i][lane] : 0;
    const int n16 = (c + 15) & ~15;
    int incl = n16;
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) {
      const int y = __shfl_up(incl, sh, 64);
      incl += lane >= sh ? y : 0;
    }
    if (lane < kvol) {
      gstart[h][lane] = incl - n16;
      if (gt < a.n_gtiles) a.gcount[gt * kvol + lane] = c;
    }
  }
  __syncthreads();
  if (gt >= a.n_gtiles) return;
  const int64_t ebase = gt * kvol * TS_GTILE;
  const uint8_t slot = static_cast<uint8_t>(threadIdx.x % TS_GTILE);
  // lane o < kvol holds where this wavefront's rows with offset o start in
  // the tile's entries: the run start plus the tile's rows with o in earlier
  // wavefronts (read per offset with a readlane)
  int run_at = 0;
  if (lane < kvol) {
    int before = 0;
#pragma unroll
    for (int i = 0; i < kWpt - 1; ++i) before += i < wt ? gw[wave - wt + i][lane] : 0;
    run_at = gstart[h][lane] + before;
  }
  // the tile's entries through buffer descriptors (32-bit offsets; the base
  // is wave-uniform, stated as such)
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(wave_uniform(a.gsrc + ebase), 0, kvol * TS_GTILE * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t rq =
      __builtin_amdgcn_make_buffer_rsrc(wave_uniform(a.gslot + ebase), 0, kvol * TS_GTILE, 0x00020000);
#pragma unroll kUnroll
  for (int o = 0; o < KVMAX; ++o) {
    if (o >= kvol) break;
    const bool has = (mask >> o) & 1;
    const uint64_t b = __ballot(has);
    if (!has) continue;
    const int pos = __builtin_amdgcn_readlane(run_at, o) +
                    static_cast<int>(__builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(b >> 32),
                                                                __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(b), 0u)));
    __builtin_amdgcn_raw_buffer_store_b32(nb(o), rs, 4 * pos, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b8(slot, rq, pos, 0, 0);
  }
  // the pad entries that complete each offset's last group: no source row
  // and the sink slot TS_GTILE
  for (int idx = threadIdx.x % TS_GTILE; idx < kvol * 16; idx += TS_GTILE) {
    const int o = idx >> 4, k = idx & 15;
    int c = 0;
#pragma unroll
    for (int i = 0; i < kWpt; ++i) c += gw[kWpt * h + i][o];
    const int rem = c & 15;
    if (rem != 0 && k >= rem) {
      const int64_t e = ebase + gstart[h][o] + (c - rem) + k;
      a.gsrc[e] = -1;
      a.gslot[e] = static_cast<uint8_t>(TS_GTILE);
    }
  }
}

// Pass 1: one lane per destination row in index order.  Writes the row's
// mask and, with TB, its neighbours (and with `natural` the tiles: rows
// stay in index order); with GR the pair groups.
template <int MODE, int ND, int K, bool TB, bool GR>
__global__ __launch_bounds__(256) void k_rel_probe(RelK a, int natural, int64_t* n_out_fill) {
  constexpr int KV = Geo<ND, K>::KV;
  // The workgroup's 256 rows own one contiguous span of the neighbour table:
  // lanes stage their rows in LDS, and the span is then written with
  // coalesced 16-byte stores (a lane's own row is KV scattered words).
  __shared__ __attribute__((aligned(16))) int32_t staged[256 * KV];
  const int64_t t = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) / kTile;
  const int r = threadIdx.x & (kTile - 1);
  if (n_out_fill && blockIdx.x == 0 && threadIdx.x == 0) *n_out_fill = a.n_dest_cap;
  const bool live = t < a.n_tiles;  // every lane stays for the barrier below
  const int64_t n_dest = dest_count(a.n_dest, a.n_dest_cap);
  const int64_t row = t * kTile + r;
  uint64_t base = 0;
  int64_t f[3] = {0, 0, 0};
  const bool valid = live && row < n_dest && dest_fields<MODE, ND>(a, row, &base, f);
  int32_t nb[KV];
  probe_fields<ND, K>(a.src, base, f, valid, nb);
  uint64_t mask = 0;
#pragma unroll
  for (int o = 0; o < KV; ++o)
    if (nb[o] >= 0) mask |= 1ull << o;
  // a submanifold output takes part only when it owns its coordinate
  if (MODE == kModeSubm && nb[(KV - 1) / 2] != static_cast<int32_t>(row)) mask = 0;
  if (live && row < a.n_dest_cap) a.row_mask[row] = mask;
  if constexpr (GR) emit_groups<KV>(a, KV, mask, [&](int o) {
      int32_t v = nb[0];
#pragma unroll
      for (int j = 1; j < KV; ++j) v = o == j ? nb[j] : v;
      return v;
    });
  if constexpr (!TB) return;
#pragma unroll
  for (int o = 0; o < KV; ++o) staged[threadIdx.x * KV + o] = ((mask >> o) & 1) ? nb[o] : -1;
  if (natural) {
    const uint64_t tmask = group16_or(mask);
    if (live && r == 0) a.tile_mask[t] = tmask;
    if (live) a.tile_rows[t * kTile + r] = row < n_dest ? static_cast<int32_t>(row) : -1;
  }
  __syncthreads();
  // rows at or past the device count are never read through the table
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * 256;
  const int64_t rows = n_dest - row0 < 256 ? n_dest - row0 : 256;
  if (rows <= 0) return;
  const int words = static_cast<int>(rows) * KV;  // span start row0 * KV * 4 bytes is 16-byte aligned
  int32_t* dst = a.nbr + row0 * KV;
  const uint4* s4 = reinterpret_cast<const uint4*>(staged);
  uint4* d4 = reinterpret_cast<uint4*>(dst);
  for (int i = threadIdx.x; i < words / 4; i += 256) d4[i] = s4[i];
  const int tail = words & 3;
  if (threadIdx.x < tail) dst[words - tail + threadIdx.x] = staged[words - tail + threadIdx.x];
}

// Runtime-kvol versions, for kernel sizes and modes without a compile-time
// instance: a lane per row probes every offset into its LDS row, and the
// workgroup's 256 rows are then written as one coalesced span.
template <int MODE>
__global__ __launch_bounds__(256) void k_rel_probe_any(RelK a, int natural) {
  extern __shared__ int32_t nbr_lds[];  // [256][kvol]
  __shared__ int8_t offs[TS_MAX_KVOL * 3];
  load_offsets(a, offs);
  const int64_t t = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) / kTile;
  const int r = threadIdx.x & (kTile - 1);
  const bool live = t < a.n_tiles;  // every lane stays for the barrier below
  const int64_t n_dest = dest_count(a.n_dest, a.n_dest_cap);
  const int64_t row = t * kTile + r;
  int64_t b = 0, s[3] = {0, 0, 0};
  const bool valid = live && row < n_dest && dest_load<MODE>(a, row, &b, s);
  int32_t* my = nbr_lds + threadIdx.x * a.kvol;
  uint64_t mask = 0;
  for (int o = 0; o < a.kvol; ++o) {
    const int32_t n = valid ? probe<MODE>(a, offs, b, s, o) : -1;
    my[o] = n;
    if (n >= 0) mask |= 1ull << o;
  }
  // a submanifold output takes part only when it owns its coordinate
  if (MODE == kModeSubm && valid && my[a.centre] != static_cast<int32_t>(row)) {
    mask = 0;
    for (int o = 0; o < a.kvol; ++o) my[o] = -1;
  }
  if (live && row < a.n_dest_cap) a.row_mask[row] = mask;
  const uint64_t tmask = group16_or(mask);  // a 16-lane group is live or not as a whole
  if (natural && live) {
    if (r == 0) a.tile_mask[t] = tmask;
    a.tile_rows[t * kTile + r] = row < n_dest ? static_cast<int32_t>(row) : -1;
  }
  __syncthreads();
  // rows at or past the device count are never read through the table
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * 256;
  const int64_t rows = n_dest - row0 < 256 ? n_dest - row0 : 256;
  if (rows <= 0) return;
  const int words = static_cast<int>(rows) * a.kvol;
  int32_t* dst = a.nbr + row0 * a.kvol;
  for (int k = threadIdx.x; k < words; k += 256) dst[k] = nbr_lds[k];
}

// Pair groups of a relation that has its neighbour table (relations the
// runtime-kvol probe builds): one lane per destination row, 256 rows (kTpb
// group tiles) per workgroup.
__global__ __launch_bounds__(256) void k_groups_from_table(RelK a) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t n_dest = dest_count(a.n_dest, a.n_dest_cap);
  const uint64_t mask = row < n_dest ? a.row_mask[row] : 0ull;
  const int32_t* nr = a.nbr + (row < n_dest ? row : 0) * a.kvol;
  emit_groups<TS_MAX_KVOL>(a, a.kvol, mask, [&](int o) { return nr[o]; });
}

// Pass 2: stable sort of each window's rows by offset mask: an LSD radix
// sort with 4-bit digits in LDS.  1024 threads; thread t holds window
// elements t, t+1024, t+2048, t+3072 (element order = row order).  Per pass:
//   * inside a wave, a row's rank among the rows of its item and digit comes
//     from four ballots (one per digit bit) and a lane-mask popcount;
//   * the (digit, item, wave) counts, laid out digit-major, are
//     exclusive-scanned once across the block, which yields every row's
//     destination directly;
// ties keep their order, so the map is deterministic.
constexpr int kDigits = 16;

// Lanes whose digit equals d, from the four per-bit ballots.
__device__ __forceinline__ uint64_t digit_lanes(const uint64_t (&bal)[4], uint32_t d) {
  uint64_t m = ~0ull;
#pragma unroll
  for (int b = 0; b < 4; ++b) m &= ((d >> b) & 1) ? bal[b] : ~bal[b];
  return m;
}

template <int kSortThreads>
__global__ __launch_bounds__(kSortThreads) void k_rel_sort(const uint64_t* __restrict__ row_mask, int64_t n_dest_cap,
                                                           const int64_t* n_dest_p, int nbits, int64_t n_slots,
                                                           int32_t* __restrict__ tile_rows,
                                                           uint64_t* __restrict__ tile_mask) {
  constexpr int kItems = kSortItems;
  constexpr int kSortWindow = kSortThreads * kItems;
  constexpr int kSortWaves = kSortThreads / 64;
  __shared__ uint2 buf[kSortWindow];
  // [digit][item][wave] -> exclusive start, one pad word after every 64: the
  // per-digit writes and reads stride by kItems * kSortWaves words, which
  // unpadded would put a wavefront's lanes on one LDS bank
  constexpr int kHist = kDigits * kItems * kSortWaves;
  __shared__ int hist[kHist + kHist / 64];
  auto hx = [](int l) { return l + (l >> 6); };
  __shared__ int wsum[kSortWaves];
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kSortWindow;
  const int64_t n_dest = dest_count(n_dest_p, n_dest_cap);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t lt = (1ull << lane) - 1;
  uint32_t key[kItems];
  int32_t row[kItems];
#pragma unroll
  for (int i = 0; i < kItems; ++i) {
    const int64_t r = base + i * kSortThreads + threadIdx.x;
    const bool ok = r < n_dest;
    const uint64_t m = ok ? row_mask[r] : 0;
    key[i] = ok ? static_cast<uint32_t>(m ^ (m >> 32)) : 0xffffffffu;
    row[i] = ok ? static_cast<int32_t>(r) : -1;
  }
  for (int sh = 0; sh < nbits; sh += 4) {
    int rank[kItems];
    uint32_t d[kItems];
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      d[i] = (key[i] >> sh) & (kDigits - 1);
      uint64_t bal[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) bal[b] = __ballot((d[i] >> b) & 1);
      rank[i] = __popcll(digit_lanes(bal, d[i]) & lt);
      if (lane < kDigits) hist[hx((lane * kItems + i) * kSortWaves + wave)] = __popcll(digit_lanes(bal, lane));
    }
    __syncthreads();
    // block-wide exclusive scan of the 1024 counts (one per thread)
    const int v = hist[hx(threadIdx.x)];
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      x += lane >= o ? y : 0;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int before = 0;
#pragma unroll
    for (int w = 0; w < kSortWaves; ++w) before += w < wave ? wsum[w] : 0;
    hist[hx(threadIdx.x)] = before + x - v;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      const int dest = hist[hx((d[i] * kItems + i) * kSortWaves + wave)] + rank[i];
      buf[dest] = make_uint2(key[i], static_cast<uint32_t>(row[i]));
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      const uint2 e = buf[i * kSortThreads + threadIdx.x];
      key[i] = e.x;
      row[i] = static_cast<int32_t>(e.y);
    }
    __syncthreads();  // reads of buf and hist done before the next pass writes them
  }
  // a tile = 16 consecutive slots = 16 consecutive lanes of one item
#pragma unroll
  for (int i = 0; i < kItems; ++i) {
    const int64_t slot = base + i * kSortThreads + threadIdx.x;
    if (slot < n_slots) tile_rows[slot] = row[i];
    const uint64_t tm = group16_or(row[i] >= 0 ? row_mask[row[i]] : 0ull);
    if ((lane & 15) == 0 && slot < n_slots) tile_mask[slot / kTile] = tm;
  }
}

// Per-offset pair lists, destination rows in index order.  Blocks of 256
// destination rows count their pairs per offset; an exclusive scan over the
// (offset, block) counts gives each block its write positions.
__global__ __launch_bounds__(256) void k_pairs_count(const uint64_t* __restrict__ row_mask, int64_t n_dest_cap,
                                                     const int64_t* n_dest_p, int kvol, int64_t nblk,
                                                     int32_t* __restrict__ cnt) {
  __shared__ int wave_cnt[4][TS_MAX_KVOL];
  const int64_t n_dest = dest_count(n_dest_p, n_dest_cap);
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const uint64_t mask = row < n_dest ? row_mask[row] : 0;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int o = 0; o < kvol; ++o) {
    const uint64_t bal = __ballot((mask >> o) & 1);
    if (lane == 0) wave_cnt[wave][o] = __popcll(bal);
  }
  __syncthreads();
  if (threadIdx.x < kvol) {
    const int o = threadIdx.x;
    cnt[o * nblk + blockIdx.x] = wave_cnt[0][o] + wave_cnt[1][o] + wave_cnt[2][o] + wave_cnt[3][o];
  }
}

// Writes the pairs of a block of 256 destination rows.  The write position
// of each (wavefront, offset) -- the block's scanned base plus the counts of
// the wavefronts before it -- is computed once into LDS.  Block 0 also
// writes pair_start.
__global__ __launch_bounds__(256) void k_pairs_fill(RelK a, int64_t nblk, const int32_t* __restrict__ base,
                                                    const int64_t* total, int64_t pair_cap,
                                                    int64_t* __restrict__ pair_start, int32_t* __restrict__ pair_in,
                                                    int32_t* __restrict__ pair_out) {
  __shared__ int wave_pos[4][TS_MAX_KVOL];
  const int64_t n_dest = dest_count(a.n_dest, a.n_dest_cap);
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const uint64_t mask = row < n_dest ? a.row_mask[row] : 0;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint64_t below = (1ull << lane) - 1;
  if (blockIdx.x == 0 && threadIdx.x <= a.kvol) {  // clamped: lists never run past their capacity
    const int64_t v = threadIdx.x < a.kvol ? base[threadIdx.x * nblk] : *total;
    pair_start[threadIdx.x] = v < pair_cap ? v : pair_cap;
  }
  for (int o = 0; o < a.kvol; ++o) {
    const uint64_t bal = __ballot((mask >> o) & 1);
    if (lane == 0) wave_pos[wave][o] = __popcll(bal);
  }
  __syncthreads();
  if (threadIdx.x < a.kvol) {  // counts -> exclusive positions, per offset
    const int o = threadIdx.x;
    int p = base[o * nblk + blockIdx.x];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int c = wave_pos[w][o];
      wave_pos[w][o] = p;
      p += c;
    }
  }
  __syncthreads();
  for (int o = 0; o < a.kvol; ++o) {
    const bool has = (mask >> o) & 1;
    const uint64_t bal = __ballot(has);  // every lane takes part
    if (!has) continue;
    const int pos = wave_pos[wave][o] + __popcll(bal & below);
    if (pos >= pair_cap) continue;
    pair_out[pos] = static_cast<int32_t>(row);
    pair_in[pos] = a.nbr[row * a.kvol + o];
  }
}

// k_pairs_fill for a relation without its neighbour table: the source row
// of a (row, offset) pair is read from the pair groups -- entry
// (offset's run start) + (the row's rank among its tile's rows with the
// offset), the rank from the same ballots that place the pair.
__global__ __launch_bounds__(256) void k_pairs_fill_groups(RelK a, int64_t nblk, const int32_t* __restrict__ base,
                                                           const int64_t* total, int64_t pair_cap,
                                                           int64_t* __restrict__ pair_start,
                                                           int32_t* __restrict__ pair_in,
                                                           int32_t* __restrict__ pair_out) {
  __shared__ int wave_pos[4][TS_MAX_KVOL];
  __shared__ int wave_cnt[4][TS_MAX_KVOL];
  __shared__ int run0[kTpb][TS_MAX_KVOL];
  const int64_t n_dest = dest_count(a.n_dest, a.n_dest_cap);
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const uint64_t mask = row < n_dest ? a.row_mask[row] : 0;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint64_t below = (1ull << lane) - 1;
  const int h = wave / kWpt, wt = wave % kWpt;  // tile of the workgroup, wavefront of the tile
  const int64_t gt = static_cast<int64_t>(blockIdx.x) * kTpb + h;
  if (blockIdx.x == 0 && threadIdx.x <= a.kvol) {  // clamped: lists never run past their capacity
    const int64_t v = threadIdx.x < a.kvol ? base[threadIdx.x * nblk] : *total;
    pair_start[threadIdx.x] = v < pair_cap ? v : pair_cap;
  }
  for (int o = 0; o < a.kvol; ++o) {
    const uint64_t bal = __ballot((mask >> o) & 1);
    if (lane == 0) wave_cnt[wave][o] = __popcll(bal);
  }
  if (wt == 0) {  // the tile's run starts, from its group counts
    const int c = lane < a.kvol && gt < a.n_gtiles ? a.gcount[gt * a.kvol + lane] : 0;
    const int n16 = (c + 15) & ~15;
    int incl = n16;
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) {
      const int y = __shfl_up(incl, sh, 64);
      incl += lane >= sh ? y : 0;
    }
    if (lane < a.kvol) run0[h][lane] = incl - n16;
  }
  __syncthreads();
  if (threadIdx.x < a.kvol) {  // counts -> exclusive positions, per offset
    const int o = threadIdx.x;
    int p = base[o * nblk + blockIdx.x];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      wave_pos[w][o] = p;
      p += wave_cnt[w][o];
    }
  }
  __syncthreads();
  const int64_t ebase = gt * a.kvol * TS_GTILE;
  for (int o = 0; o < a.kvol; ++o) {
    const bool has = (mask >> o) & 1;
    const uint64_t bal = __ballot(has);  // every lane takes part
    if (!has) continue;
    const int rank = __popcll(bal & below);
    const int pos = wave_pos[wave][o] + rank;
    if (pos >= pair_cap) continue;
    int before = 0;  // the tile's rows with the offset in earlier wavefronts
#pragma unroll
    for (int i = 0; i < kWpt - 1; ++i) before += i < wt ? wave_cnt[wave - wt + i][o] : 0;
    const int in_tile = run0[h][o] + before + rank;
    pair_out[pos] = static_cast<int32_t>(row);
    pair_in[pos] = a.gsrc[ebase + in_tile];
  }
}

RelK make_relk(const RelBuild& bld, const ts_rel& rel) {
  RelK a;
  a.dc = bld.dest_coords;
  a.n_dest_cap = bld.n_dest_cap;
  a.n_dest = bld.n_dest;
  a.ndim = bld.ndim;
  a.stride = bld.stride;
  a.stride_shift = -1;
  for (int k = 0; k < 17; ++k)
    if (bld.stride == (1 << k)) a.stride_shift = k;
  a.kvol = bld.kvol;
  a.centre = (bld.kvol - 1) / 2;
  a.offs = make_offsets(bld.ndim, bld.ksize);
  a.src = table_view(bld.src_table, bld.src_cap, bld.ndim);
  a.own = bld.own_table ? table_view(bld.own_table, bld.own_cap, bld.ndim) : a.src;
  a.n_tiles = rel.n_tiles;
  a.tile_mask = rel.tile_mask;
  a.tile_rows = rel.tile_rows;
  a.nbr = rel.nbr;
  a.row_mask = rel.row_mask;
  a.n_gtiles = rel.n_gtiles;
  a.gcount = rel.gcount;
  a.gsrc = rel.gsrc;
  a.gslot = rel.gslot;
  return a;
}

// Rows sorted together: kSortItems * kSortThreads (one window per
// workgroup).
constexpr int kSortThreads = 1024;

void launch_sort(const RelK& a, hipStream_t s) {
  const int64_t slots = a.n_tiles * kTile;
  const int nbits = a.kvol < 32 ? a.kvol : 32;
  const unsigned grid =
      static_cast<unsigned>(ceil_div<int64_t>(slots, static_cast<int64_t>(kSortThreads) * kSortItems));
  k_rel_sort<kSortThreads><<<grid, kSortThreads, 0, s>>>(a.row_mask, a.n_dest_cap, a.n_dest, nbits, slots,
                                                         a.tile_rows, a.tile_mask);
}

// With a neighbour table (TB) the tiles are written in index order or
// sorted; the pair groups come from the probe itself (GR).
template <int MODE, int ND, int K>
void launch_rel_geo(const RelK& a, bool natural, unsigned grid, int64_t* n_out_fill, hipStream_t s) {
  const bool tb = a.nbr != nullptr, gr = a.n_gtiles > 0;
  const int nat = natural ? 1 : 0;
  if (tb && gr)
    k_rel_probe<MODE, ND, K, true, true><<<grid, 256, 0, s>>>(a, nat, n_out_fill);
  else if (tb)
    k_rel_probe<MODE, ND, K, true, false><<<grid, 256, 0, s>>>(a, nat, n_out_fill);
  else
    k_rel_probe<MODE, ND, K, false, true><<<grid, 256, 0, s>>>(a, nat, n_out_fill);
  if (tb && !natural) launch_sort(a, s);
}

template <int MODE>
void launch_rel_any(const RelK& a, bool natural, unsigned grid, int64_t* n_out_fill, hipStream_t s) {
  const size_t lds = static_cast<size_t>(256) * a.kvol * sizeof(int32_t);
  if (n_out_fill) (void)fill_i64(n_out_fill, 1, a.n_dest_cap, s);
  k_rel_probe_any<MODE><<<grid, 256, lds, s>>>(a, natural ? 1 : 0);
  if (!natural) launch_sort(a, s);
  if (a.n_gtiles > 0) k_groups_from_table<<<grid, 256, 0, s>>>(a);
}

template <int ND, int K>
constexpr bool geo_instanced() {
  return (ND == 3 && (K == 1 || K == 2 || K == 3)) || (ND == 2 && (K == 2 || K == 3 || K == 5));
}

template <int MODE>
void launch_rel_mode(const RelK& a, int ksize, bool natural, unsigned grid, int64_t* n_out_fill, hipStream_t s) {
  if (a.ndim == 3 && ksize == 3) return launch_rel_geo<MODE, 3, 3>(a, natural, grid, n_out_fill, s);
  if (a.ndim == 3 && ksize == 2) return launch_rel_geo<MODE, 3, 2>(a, natural, grid, n_out_fill, s);
  if (a.ndim == 3 && ksize == 1) return launch_rel_geo<MODE, 3, 1>(a, natural, grid, n_out_fill, s);
  if (a.ndim == 2 && ksize == 3) return launch_rel_geo<MODE, 2, 3>(a, natural, grid, n_out_fill, s);
  if (a.ndim == 2 && ksize == 2) return launch_rel_geo<MODE, 2, 2>(a, natural, grid, n_out_fill, s);
  if (a.ndim == 2 && ksize == 5) return launch_rel_geo<MODE, 2, 5>(a, natural, grid, n_out_fill, s);
  return launch_rel_any<MODE>(a, natural, grid, n_out_fill, s);
}

}  // namespace

size_t rel_scratch_bytes(int64_t, int) { return 0; }

bool rel_probe_emits_groups(int mode, int ndim, int ksize) {
  if (mode != kModeSubm && mode != kModeDown) return false;
  return (ndim == 3 && ksize >= 1 && ksize <= 3) || (ndim == 2 && (ksize == 2 || ksize == 3 || ksize == 5));
}

hipError_t launch_rel_build(const RelBuild& bld, const ts_rel& rel, bool natural, int64_t* n_out_fill,
                            hipStream_t s) {
  if (rel.n_tiles == 0) return n_out_fill ? fill_i64(n_out_fill, 1, bld.n_dest_cap, s) : hipSuccess;
  RelK a = make_relk(bld, rel);
  const unsigned grid = static_cast<unsigned>(ceil_div<int64_t>(rel.n_tiles * kTile, 256));
  switch (bld.mode) {
    case kModeSubm: launch_rel_mode<kModeSubm>(a, bld.ksize, natural, grid, n_out_fill, s); break;
    case kModeDown: launch_rel_mode<kModeDown>(a, bld.ksize, natural, grid, n_out_fill, s); break;
    default: launch_rel_any<kModeUp>(a, natural, grid, n_out_fill, s); break;
  }
  return hipGetLastError();
}

size_t pairs_scratch_bytes(int64_t n_dest_cap, int kvol) {
  const int64_t nblk = ceil_div<int64_t>(n_dest_cap, 256);
  const int64_t n = nblk * kvol;
  return align_up(static_cast<size_t>(n > 0 ? n : 1) * 4, 256) + scan_tmp_bytes(n);
}

hipError_t launch_pairs_build(const RelBuild& bld, const ts_rel& rel, int64_t pair_cap, int64_t* pair_start,
                              int32_t* pair_in, int32_t* pair_out, void* scratch, hipStream_t s) {
  const int64_t nblk = ceil_div<int64_t>(bld.n_dest_cap, 256);
  if (nblk == 0) return fill_i64(pair_start, bld.kvol + 1, 0, s);
  const int64_t n = nblk * bld.kvol;
  int32_t* cnt = static_cast<int32_t*>(scratch);
  void* tmp = static_cast<char*>(scratch) + align_up(static_cast<size_t>(n) * 4, 256);
  k_pairs_count<<<static_cast<unsigned>(nblk), 256, 0, s>>>(rel.row_mask, bld.n_dest_cap, bld.n_dest, bld.kvol,
                                                              nblk, cnt);
  hipError_t e = scan_exclusive_i32(cnt, cnt, n, pair_start + bld.kvol, tmp, s);
  if (e != hipSuccess) return e;
  RelK a = make_relk(bld, rel);
  if (rel.nbr)
    k_pairs_fill<<<static_cast<unsigned>(nblk), 256, 0, s>>>(a, nblk, cnt, pair_start + bld.kvol, pair_cap,
                                                               pair_start, pair_in, pair_out);
  else
    k_pairs_fill_groups<<<static_cast<unsigned>(nblk), 256, 0, s>>>(a, nblk, cnt, pair_start + bld.kvol, pair_cap,
                                                                      pair_start, pair_in, pair_out);
  return hipGetLastError();
}

}  // namespace ts
