// Weight gradient: dW[o] = sum over the pairs (i, j) of offset o of
// x[i]^T dy[j]  -- one (Cin x M_o) . (M_o x Cout) product per offset, needed
// for the mixed-precision training the TorchSparse++ abstract reports.
//
// The pairs of each offset are cut into chunks of kChunk pairs.  A block
// reduces one chunk for one (Cin, Cout) tile into a private fp32 partial;
// k_wgrad_reduce then sums the partials of each offset in chunk order, so
// the result does not depend on scheduling (no atomics).
//
// fp16/bf16 with channel counts that are multiples of 16 use MFMA.  A block
// owns a TW x TW tile of dW[o] (2 x 2 waves) and walks its chunk in steps of
// 64 pairs.  Per step, each staging thread gathers 8 rows x 8 channels
// (16-byte loads of x[pair_in] or dy[pair_out]), transposes the 8 x 8 block
// in registers and writes 8 channel rows of 8 consecutive pairs to LDS, so
// every MFMA fragment (8 consecutive pairs of one channel) is one 16-byte
// LDS read.  Pair indices are loaded three steps ahead and rows two steps
// ahead (register rings), the LDS slab is double-buffered, one barrier per
// step.
#include "common.h"
#include "launch.h"

namespace ts {

namespace {

constexpr int kChunk = 2048;   // pairs per partial
constexpr int kWStep = 64;     // pairs per step
constexpr int kWStride = kWStep;  // halves per LDS channel row (128 bytes)

// LDS address (in halves) of the 16-byte chunk pc (8 pairs) of channel row
// ch.  The chunk index is XOR-swizzled with bits of ch so that the 16 lanes
// of a fragment read (16 consecutive channels, one chunk) hit 16 different
// 16-byte bank groups, and the transposed stores (16 channels 8 apart) at
// most two lanes per group.
__device__ __forceinline__ int slab_at(int ch, int pc) { return ch * kWStride + ((pc ^ ((ch >> 1) ^ (ch >> 3))) & 7) * 8; }

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

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

template <int I>
struct WIc {
  static constexpr int v = I;
};

template <typename T, int TW>
__global__ __launch_bounds__(256, 2) void k_wgrad_mfma(const int32_t* __restrict__ chunk_base,
                                                    const int64_t* __restrict__ pair_start, int kvol,
                                                    const int32_t* __restrict__ pair_in,
                                                    const int32_t* __restrict__ pair_out, const T* __restrict__ x,
                                                    int cin, const T* __restrict__ dy, int cout,
                                                    float* __restrict__ partial, int64_t n_x, int64_t n_dy) {
  typedef typename WMfma<T>::frag Frag;
  constexpr int HT = TW / 2;   // channels per wave in each dim
  constexpr int NT = HT / 16;  // 16 x 16 MFMA tiles per wave in each dim
  constexpr int CG = TW / 8;   // 8-channel groups per operand
  __shared__ __attribute__((aligned(16))) T slab[2][2][TW * kWStride];  // [buffer][x | dy][channel][pair]
  const int c = blockIdx.x;
  int o;
  int64_t p0, p1;
  if (!chunk_range(chunk_base, pair_start, kvol, c, &o, &p0, &p1)) return;
  const int ci0 = blockIdx.y * TW, co0 = blockIdx.z * TW;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // staging role: operand, 8-pair group, 8-channel group
  const int op = threadIdx.x >> 7;
  const int tt = threadIdx.x & 127;
  const bool stager = tt < 8 * CG;
  const int pg = tt / CG, cg = tt % CG;
  const T* src = op ? dy : x;
  const int C = op ? cout : cin;
  const int ch = (op ? co0 : ci0) + cg * 8;
  const bool cok = stager && ch < C;
  const int32_t* rows = op ? pair_out : pair_in;
  const int nsteps = static_cast<int>((p1 - p0 + kWStep - 1) / kWStep);

  f32x4 acc[NT][NT];
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Pair r of this thread's group at step st exists when it lies inside the
  // chunk (validity never depends on a loaded value, so no load is ever
  // placed under a branch).
  auto valid = [&](int st, int r) -> bool {
    return cok && p0 + static_cast<int64_t>(st) * kWStep + pg * 8 + r < p1;
  };
  // row indices of step st (clamped address; meaningful where valid)
  auto load_idx = [&](int st, int32_t (&id)[8]) {
    const int64_t q = p0 + static_cast<int64_t>(st) * kWStep + pg * 8;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int64_t p = q + r;
      id[r] = rows[p < p1 ? p : p1 - 1];
    }
  };
  // rows of step st; absent pairs read row 0 and are zeroed when staged
  auto load_rows = [&](int st, const int32_t (&id)[8], u32x4 (&v)[8]) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int32_t row = valid(st, r) ? dbg_req(id[r], op ? n_dy : n_x, op ? TS_DEBUG_DST_ROW : TS_DEBUG_SRC_ROW) : 0;
      v[r] = *reinterpret_cast<const u32x4*>(src + static_cast<int64_t>(row) * C + (cok ? ch : 0));
    }
  };
  // 8 x 8 transpose of 16-bit values: out row e = channel ch+e over the 8 pairs
  auto stage = [&](int st, u32x4 (&in)[8], T* buf) {
    if (!stager) return;
#pragma unroll
    for (int r = 0; r < 8; ++r) in[r] = valid(st, r) ? in[r] : u32x4{0u, 0u, 0u, 0u};  // in place
    T* base = buf + (op ? TW * kWStride : 0);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      u32x4 outv;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t a = in[2 * m][e >> 1], b = in[2 * m + 1][e >> 1];
        outv[m] = (e & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
      }
      *reinterpret_cast<u32x4*>(base + slab_at(cg * 8 + e, pg)) = outv;
    }
  };
  auto mma = [&](const T* buf) {
    const T* xa = buf;
    const T* yb = buf + TW * kWStride;
#pragma unroll
    for (int kb = 0; kb < kWStep / 32; ++kb) {
      Frag af[NT], bf[NT];
#pragma unroll
      for (int i = 0; i < NT; ++i)
        af[i] = __builtin_bit_cast(
            Frag, *reinterpret_cast<const u32x4*>(xa + slab_at(wm * HT + i * 16 + (lane & 15), kb * 4 + (lane >> 4))));
#pragma unroll
      for (int j = 0; j < NT; ++j)
        bf[j] = __builtin_bit_cast(
            Frag, *reinterpret_cast<const u32x4*>(yb + slab_at(wn * HT + j * 16 + (lane & 15), kb * 4 + (lane >> 4))));
#pragma unroll
      for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = WMfma<T>::run(af[i], bf[j], acc[i][j]);
    }
  };

  // prologue: indices of steps 0..2, rows of steps 0..1, slab of step 0.
  // Index sets alternate: the set of step s+3 is loaded at step s into the
  // one whose rows (step s+1) were issued at step s-1.
  int32_t id[2][8];
  u32x4 rv[2][8];
  load_idx(0, id[0]);
  load_idx(1, id[1]);
  load_rows(0, id[0], rv[0]);
  load_rows(1, id[1], rv[1]);
  load_idx(2, id[0]);
  stage(0, rv[0], &slab[0][0][0]);
  __syncthreads();
  int s = 0;
  // step s: indices of s+3, rows of s+2, multiplies of s, staging of s+1
  auto step = [&](auto ic) -> bool {
    constexpr int i = decltype(ic)::v;
    load_idx(s + 3, id[(i + 3) & 1]);
    load_rows(s + 2, id[(i + 2) & 1], rv[i & 1]);
    mma(&slab[i & 1][0][0]);
    if (++s >= nsteps) return false;
    stage(s, rv[(i + 1) & 1], &slab[(i + 1) & 1][0][0]);
    __syncthreads();
    return true;
  };
  while (step(WIc<0>{}) && step(WIc<1>{}) && step(WIc<2>{}) && step(WIc<3>{})) {
  }

  // D[m][n]: lane holds n = lane%16, m = 4*(lane/16) + e
  float* part = partial + static_cast<int64_t>(c) * cin * cout;
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int co = co0 + wn * HT + j * 16 + (lane & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ci = ci0 + wm * HT + i * 16 + (lane >> 4) * 4 + e;
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
                                                   float* __restrict__ partial, int64_t n_x, int64_t n_dy) {
  const int c = blockIdx.x;
  int o;
  int64_t p0, p1;
  if (!chunk_range(chunk_base, pair_start, kvol, c, &o, &p0, &p1)) return;
  const int64_t e = static_cast<int64_t>(blockIdx.y) * 256 + threadIdx.x;
  if (e >= static_cast<int64_t>(cin) * cout) return;
  const int ci = static_cast<int>(e / cout), co = static_cast<int>(e % cout);
  float acc = 0.f;
  for (int64_t p = p0; p < p1; ++p)
    acc = fmaf(static_cast<float>(x[static_cast<int64_t>(dbg_req(pair_in[p], n_x, TS_DEBUG_SRC_ROW)) * cin + ci]),
               static_cast<float>(dy[static_cast<int64_t>(dbg_req(pair_out[p], n_dy, TS_DEBUG_DST_ROW)) * cout + co]),
               acc);
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
  const int c0 = chunk_base[o], c1 = chunk_base[o + 1];
  float s = 0.f;
  int c = c0;
  for (; c + 8 <= c1; c += 8) {  // loads issued together, summed in chunk order
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = partial[static_cast<int64_t>(c + u) * elems + e];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; c < c1; ++c) s += partial[static_cast<int64_t>(c) * elems + e];
  dw[i] = s;
}

int64_t max_chunks(const ts_kmap* map) { return map->pair_cap / kChunk + map->kvol + 1; }

dim3 grid_chunks(unsigned nch, int cin, int cout, int tw) {
  return dim3(nch, static_cast<unsigned>(ceil_div(cin, tw)), static_cast<unsigned>(ceil_div(cout, tw)));
}

template <int TW>
void launch_wgrad_mfma(dim3 grid, ts_dtype dt, const ts_kmap* map, const void* x, int cin, const void* dy, int cout,
                       const int32_t* chunk_base, float* partial, hipStream_t s) {
  if (dt == TS_F16)
    k_wgrad_mfma<_Float16, TW><<<grid, 256, 0, s>>>(chunk_base, map->pair_start, map->kvol, map->pair_in,
                                                     map->pair_out, static_cast<const _Float16*>(x), cin,
                                                     static_cast<const _Float16*>(dy), cout, partial, map->n_in,
                                                     map->n_out_cap);
  else
    k_wgrad_mfma<__bf16, TW><<<grid, 256, 0, s>>>(chunk_base, map->pair_start, map->kvol, map->pair_in,
                                                   map->pair_out, static_cast<const __bf16*>(x), cin,
                                                   static_cast<const __bf16*>(dy), cout, partial, map->n_in,
                                                   map->n_out_cap);
}

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
  // The MFMA kernel stages rows with 16-byte loads: rows of 16-channel
  // multiples are 16-byte aligned when the matrices are; otherwise the FMA
  // kernel, which reads element by element, takes the layer.
  const bool aligned = (reinterpret_cast<uintptr_t>(x) & 15) == 0 && (reinterpret_cast<uintptr_t>(dy) & 15) == 0;
  const bool mfma = dt != TS_F32 && cin % 16 == 0 && cout % 16 == 0 && aligned;
  if (mfma) {
    if (cin >= 128 && cout >= 128)
      launch_wgrad_mfma<128>(grid_chunks(nch, cin, cout, 128), dt, map, x, cin, dy, cout, chunk_base, partial, s);
    else
      launch_wgrad_mfma<64>(grid_chunks(nch, cin, cout, 64), dt, map, x, cin, dy, cout, chunk_base, partial, s);
  } else {
    dim3 grid(nch, static_cast<unsigned>(ceil_div<int64_t>(elems, 256)));
    switch (dt) {
      case TS_F32:
        k_wgrad_fma<float><<<grid, 256, 0, s>>>(chunk_base, map->pair_start, map->kvol, map->pair_in, map->pair_out,
                                                 static_cast<const float*>(x), cin, static_cast<const float*>(dy), cout,
                                                 partial, map->n_in, map->n_out_cap);
        break;
      case TS_F16:
        k_wgrad_fma<_Float16><<<grid, 256, 0, s>>>(chunk_base, map->pair_start, map->kvol, map->pair_in,
                                                    map->pair_out, static_cast<const _Float16*>(x), cin,
                                                    static_cast<const _Float16*>(dy), cout, partial, map->n_in,
                                                   map->n_out_cap);
        break;
      default:
        k_wgrad_fma<__bf16><<<grid, 256, 0, s>>>(chunk_base, map->pair_start, map->kvol, map->pair_in, map->pair_out,
                                                  static_cast<const __bf16*>(x), cin, static_cast<const __bf16*>(dy),
                                                  cout, partial, map->n_in, map->n_out_cap);
        break;
    }
  }
  const int64_t total = elems * map->kvol;
  k_wgrad_reduce<<<static_cast<unsigned>(ceil_div<int64_t>(total, 256)), 256, 0, s>>>(chunk_base, map->kvol, partial,
                                                                                     elems, dw);
  return hipGetLastError();
}

}  // namespace ts

TS_DEBUG_TU(wgrad)
