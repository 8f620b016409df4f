// bitnet_quantize_static: bitnet_quantize with its scratch in a file-scope
// device array instead of a caller-provided workspace, for callers that
// cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid allocation).
//
// The only scratch of bitnet_quantize is the weight absmean's fixed set of
// fp64 partial sums and, for the one-pass launch, one record per workgroup
// (its partial and a publication word tagged per launch;
// bitnet_ternarize_workspace_bytes(): 6144 bytes, the same for every N, K). `scratch` holds kStaticScratchBytes; each device
// the library runs on holds its own copy until the process ends. In host
// code `scratch` names a host-side stand-in, so its device address is looked
// up once per device with hipGetSymbolAddress (with that device current, on
// the first call there) and that address is what the kernels get. Every
// partial is written before it is read in each call, and a publication
// word left by an earlier call never matches a later call's, so nothing
// needs clearing. Calls that overlap on one device share the array and race.

#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/bitnet.h"
#include "internal.h"

namespace {

constexpr size_t kStaticScratchBytes = 8192;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device (looked up on the
// first call on that device), or NULL if the runtime cannot give it.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" {

bitnet_status bitnet_quantize_static(const void* W, bitnet_dtype w_dtype, int64_t N, int64_t K, const uint16_t* x,
                                     int64_t M, uint8_t* w_packed, float* gamma, int8_t* x_q, float* s_x,
                                     void* stream) {
  // the scratch this call needs, against the array's fixed size
  if (N >= 1 && K >= 1 && bitnet_ternarize_workspace_bytes(N, K) > kStaticScratchBytes) return BITNET_ERR_WORKSPACE;
  void* ws = scratch_on_current_device();
  if (ws == nullptr) return BITNET_ERR_HIP;
  return bitnet_quantize(W, w_dtype, N, K, x, M, w_packed, gamma, x_q, s_x, ws, kStaticScratchBytes, stream);
}

}  // extern "C"
