// noalloc.hip -- ulys_attn_fwd_noalloc: the forward attention for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).
//
// It is ulys_attn_fwd_ws with the workspace taken from a fixed device array of
// kScratchBytes that this file defines: the split path's partial states or the
// unit counter live there instead of in caller memory.  The array is resolved
// to a device address once per device (hipGetSymbolAddress, with that device
// current) and the address is kept; the kernels receive it as the workspace
// argument, exactly as they receive a caller's workspace.  Every call on one
// device shares that device's array, so calls that overlap in time on one
// device (different streams, or different host threads) race on it; calls
// ordered on one stream do not.  The kernels clear the counter with a kernel
// of their own on every call and write every partial state before reading it,
// so no contents carry over from an earlier call.  Nothing here allocates.
#include <mutex>

#include "internal.h"
#include "ulysses.h"

namespace {

constexpr int kMaxDevices = 64;
constexpr int64_t kScratchBytes = ULYS_NOALLOC_SCRATCH_BYTES;

// The scratch array.  In host code `scratch` names a host-side stand-in, not
// device memory: only the address hipGetSymbolAddress returns is used.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, looked up on the first call on
// that device; nullptr (and *err set) when the runtime fails.
void* scratch_on_current_device(int* err) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *err = ULYS_ERR_HIP;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      *err = ULYS_ERR_HIP;
      return nullptr;
    }
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" int ulys_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o,
                                     float* lse, int64_t s, int64_t b, int64_t h, int64_t h_kv,
                                     int64_t d_h, int32_t P, int32_t causal, int32_t dtype,
                                     void* stream) {
  // the argument checks of ulys_attn_fwd run first, on every path
  if (!q || !k || !v || !o) return ULYS_ERR_NULL;
  const int64_t need =
      ulys_attn_fwd_workspace_size(s, b, h, h_kv, d_h, P, causal, dtype);
  if (need < 0) return (int)need;
  if (need > kScratchBytes) return ULYS_ERR_DIM;  // beyond the fixed scratch
  void* ws = nullptr;
  if (need > 0) {
    int err = ULYS_OK;
    ws = scratch_on_current_device(&err);
    if (!ws) return err;
  }
  return ulys_attn_fwd_ws(q, k, v, o, lse, s, b, h, h_kv, d_h, P, causal, dtype, ws, need,
                          stream);
}
