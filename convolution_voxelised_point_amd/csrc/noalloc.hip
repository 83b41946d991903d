// The allocation-free variant of dgrad: the same kernels as
// ts_conv_bwd_dgrad, with the implicit GEMM's packed weights in a static
// device array of the library instead of a caller workspace.  Meant for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation).
//
// Each GPU the library runs on holds its own copy of `scratch` until the
// process ends.  Host code never names the array in a kernel argument or a
// copy (the name is a host-side stand-in, not a device address): the device
// address is looked up once per device, with that device current, and kept.
#include <mutex>

#include "common.h"
#include "launch.h"

namespace {

constexpr size_t kScratchBytes = size_t{4} << 20;  // TS_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == TS_NOALLOC_SCRATCH_BYTES, "header and library disagree on the scratch size");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_addr[kMaxDevices] = {};

// Device address of this device's `scratch`, or NULL when the lookup fails.
void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> g(g_lock);
  if (!g_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_addr[dev] = p;
  }
  return g_addr[dev];
}

}  // namespace

extern "C" ts_status ts_conv_bwd_dgrad_noalloc(const ts_kmap* map, const void* dy, int cout, const void* w, int cin,
                                               void* dx, ts_dtype in_dtype, ts_dtype out_dtype, hipStream_t stream) {
  if (!map) return TS_ERR_INVALID_ARG;
  // The gather-scatter dataflow's fp32 accumulator grows with the rows, so
  // only the implicit GEMM (packed weights, bounded by the kernel volume and
  // channel counts) and the direct kernel (no scratch) run here.
  const size_t need = ts_conv_workspace_bytes(map, cin, cout, TS_OP_DGRAD, in_dtype, TS_DATAFLOW_IMPLICIT_GEMM);
  if (need > kScratchBytes) return TS_ERR_UNSUPPORTED;
  void* ws = nullptr;
  if (need > 0) {
    ws = scratch_address();
    if (!ws) return TS_ERR_HIP;
  }
  return ts_conv_bwd_dgrad(map, dy, cout, w, cin, dx, in_dtype, out_dtype, TS_DATAFLOW_IMPLICIT_GEMM, ws, need,
                           stream);
}
