// Allocation-free variant of socket_decode_step for callers that cannot call
// hipMalloc (code under HIP graph capture, tight serving loops, harnesses
// that forbid allocation).  Its scratch memory -- the table images, selection
// histograms, counters, bitmaps, candidates, internal scores and attention
// partials that socket_decode_step keeps in the caller's workspace -- is one
// file-scope device array instead.
//
// Every GPU the library runs on holds its own copy of the array (allocated
// when this code object is loaded on that device, kept until the process
// ends).  In host code the array's name is only a host-side stand-in, so its
// device address is looked up once per device with hipGetSymbolAddress and
// only that address is ever handed to kernels.
#include <mutex>

#include "../../include/socket_lsh.h"
#include "common.h"

namespace {

__device__ __align__(256) unsigned char scratch[SOCKET_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call there, with that device current).
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SOCKET_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return SOCKET_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SOCKET_EHIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return SOCKET_OK;
}

}  // namespace

extern "C" int socket_decode_step_noalloc(const void* q, const void* K, const void* V, int dtype,
                                          int B, int Hq, int Hkv, int d, const void* W, int L,
                                          int P, float tau, uint8_t* ids, float* vnorm,
                                          const int32_t* lens, int64_t n_cap, const int32_t* ks,
                                          int k_max, int sink, int window, float scale,
                                          int32_t* idx, float* scores, float* out,
                                          void* stream) {
  const size_t need = socket_decode_step_workspace(B, Hq, Hkv, n_cap, L, P, k_max);
  if (need > (size_t)SOCKET_NOALLOC_SCRATCH_BYTES) return SOCKET_ENOSPC;
  void* ws = nullptr;
  const int rc = scratch_address(&ws);
  if (rc != SOCKET_OK) return rc;
  // Invalid or unsupported sizes (need == 0) are reported by socket_decode_step
  // with the status a call with a large enough workspace would get; nothing is
  // enqueued then.
  return socket_decode_step(q, K, V, dtype, B, Hq, Hkv, d, W, L, P, tau, ids, vnorm, lens, n_cap,
                            ks, k_max, sink, window, scale, idx, scores, out, ws,
                            (size_t)SOCKET_NOALLOC_SCRATCH_BYTES, stream);
}
