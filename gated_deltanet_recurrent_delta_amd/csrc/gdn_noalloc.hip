// gdn_prefill_noalloc: gdn_prefill with its workspace in a static device
// array instead of caller memory, for callers that cannot allocate (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  The kernels are gdn_prefill's; only where their scratch
// lives differs.
//
// `scratch` is a file-scope device array.  Its name in host code is a host
// stand-in, not a device address, so host code never passes it to a kernel
// or a copy: on the first call on each device, with that device current,
// hipGetSymbolAddress gives that device's own copy of the array, and every
// later call on the device uses that pointer.  The array lives as long as
// the process; every call on one device shares it, so calls that overlap on
// one device (on different streams, or from different host threads without
// ordering) race on it.  Nothing in it has to start at zero: the prepare
// phase writes every byte the scan then reads.
#include <mutex>

#include "gdn.h"
#include "gdn_launch.hpp"

namespace {

static __device__ __attribute__((aligned(256))) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_ptr[kMaxDevices] = {};

// This device's copy of `scratch`, looked up once per device.
int scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GDN_EHIP;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return GDN_EHIP;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return GDN_OK;
}

}  // namespace

extern "C" int gdn_prefill_noalloc(const void* q, const void* k, const void* v,
                                   const float* alpha, const float* beta,
                                   const float* S0, void* o, float* ST, int B,
                                   int T, int H, int dk, int dv, int in_dtype,
                                   int out_dtype, void* stream) {
  // argument and size checks first, before any HIP call
  int st = gdn::prefill_args(q, k, v, alpha, beta, S0, o, ST, B, T, H, dk, dv,
                             in_dtype, out_dtype);
  if (st != GDN_OK) return st;
  void* ws = nullptr;
  if (T > 0) {
    if (gdn_prefill_workspace_bytes(B, T, H, dk, dv) > GDN_NOALLOC_SCRATCH_BYTES)
      return GDN_EWORKSPACE;
    st = scratch_ptr(&ws);
    if (st != GDN_OK) return st;
  }
  return gdn_prefill(q, k, v, alpha, beta, S0, o, ST, B, T, H, dk, dv, in_dtype,
                     out_dtype, ws, T > 0 ? GDN_NOALLOC_SCRATCH_BYTES : 0, stream);
}
