// fa_bwd_noalloc: the backward with its workspace in a fixed device array of this library, for
// callers that cannot allocate (declared in include/fa.h).
//
// The backward's only scratch memory is the two fp32 row vectors D_i = rowsum(dO * O) and
// LSE_i * log2(e) (8 bytes per query row). Here they live in `scratch`, a file-scope device
// array of kScratchBytes that every GPU the library runs on holds until the process ends. In
// host code the array's name is only a host-side stand-in, so its device address is looked up
// once per device with hipGetSymbolAddress (with that device current) and kept; kernels get
// that address, never the name. Nothing in the array has to start at zero: the first kernel of
// every call writes each row it later reads. Calls that overlap on one GPU share the array and
// race.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/fa.h"
#include "fa_launch.h"

constexpr size_t kScratchBytes = size_t(16) << 20;   // 16 MiB: B * H * T up to 2^21 rows

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

std::mutex g_mu;
void* g_addr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up on the first call there.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FA_ERR_HIP;
    g_addr[dev] = p;
  }
  *out = g_addr[dev];
  return FA_OK;
}

}  // namespace

extern "C" {

size_t fa_bwd_noalloc_max_bytes(void) { return kScratchBytes; }

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv, int B, int H, int T, int D,
                   float scale, int causal, int dtype, void* stream) {
  // every argument is validated before the runtime is touched
  if (int rc = fa::check_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, T, D, scale, causal, dtype))
    return rc;
  if (fa_bwd_workspace_bytes(B, H, T, D) > kScratchBytes) return FA_ERR_SCRATCH;
  void* ws = nullptr;
  if (int rc = scratch_address(&ws)) return rc;
  return fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, ws, kScratchBytes, B, H, T, D, scale, causal,
                dtype, stream);
}

}  // extern "C"
