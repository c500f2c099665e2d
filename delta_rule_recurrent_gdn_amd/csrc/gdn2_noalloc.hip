// gdn2_noalloc.hip -- gdn2_fwd_chunked_noalloc: the two-stage chunked forward
// with its workspace in a device array that the library owns, for callers that
// cannot allocate device memory (code under graph capture, tight serving loops).
//
// The array is a file-scope __device__ variable: every GPU the library runs on
// holds its own copy, at its own address, until the process ends. Host code
// never uses the variable's name as an address (on the host that name is only a
// stand-in); the device address comes from hipGetSymbolAddress, taken once per
// device with that device current, and every kernel gets that pointer.

#include <stdint.h>

#include <mutex>

#include "gdn2.h"
#include "gdn2_internal.h"

namespace {

static_assert(GDN2_NOALLOC_SCRATCH_BYTES % 256 == 0, "whole 256-byte blocks");
__device__ __align__(256) char scratch[GDN2_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, null until first use there

// The current device's copy of the array.
int device_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GDN2_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return GDN2_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GDN2_OK;
}

}  // namespace

extern "C" int gdn2_fwd_chunked_noalloc(const void* q, const void* k, const void* v, const float* log_alpha,
                                        const void* b, const void* w, const float* S0, float* o, float* S_final,
                                        float* chunk_states, int B, int T, int H, int Dk, int Dv, int chunk, int dt,
                                        void* stream) {
  // sizes first (host arithmetic only): an invalid size returns 0 here and is reported below by the
  // regular entry point; a valid one beyond the array is refused before any device call
  const size_t need = gdn2_workspace_bytes(GDN2_OP_FWD, B, T, H, Dk, Dv, chunk, dt);
  if (need > (size_t)GDN2_NOALLOC_SCRATCH_BYTES) return GDN2_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    const int st = device_scratch(&ws);
    if (st != GDN2_OK) return st;
  }
  return gdn2_fwd_chunked(q, k, v, log_alpha, b, w, S0, o, S_final, chunk_states, ws,
                          need > 0 ? (size_t)GDN2_NOALLOC_SCRATCH_BYTES : 0, B, T, H, Dk, Dv, chunk, dt, stream);
}
