// Decode entry point that allocates nothing and takes no workspace: the
// scratch memory the decode kernels need (the absorbed queries, the per-split
// partial outputs and their softmax statistics) lives in a file-scope device
// array of fixed size, one copy per GPU, held until the process ends.
//
// Host code never passes the array's name to a kernel or a copy: in host code
// the name is a host-side stand-in, not a device address. The device address
// of each GPU's copy is looked up once per device (hipGetSymbolAddress, with
// that device current) on the first call on that device and kept.
#include <mutex>
#include <stdio.h>
#include <stdlib.h>

#include "launch.h"
#include "mla.h"

namespace {

static __device__ __align__(256) char scratch[MLA_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void* g_ptr[MAX_DEVICES];  // device address of `scratch` on each device, once looked up

// Device address of this device's scratch array (the current device), or
// nullptr if it cannot be found.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" {

size_t mla_noalloc_scratch_bytes(void) { return (size_t)MLA_NOALLOC_SCRATCH_BYTES; }

mla_status mla_decode_noalloc(const mla_dims* d, int32_t batch, int32_t q_len, const void* q_nope,
                              const void* q_pe, const void* w_uk, const void* w_uv, const mla_cache* cache,
                              void* out, void* stream) {
  size_t need = 0;
  const int32_t max_context = cache ? cache->max_context : 0;
  mla_status st = mla_decode_multi_workspace_size(d, batch, q_len, max_context, &need);
  if (st != MLA_OK) return st;
  if (need > (size_t)MLA_NOALLOC_SCRATCH_BYTES) {
    if (getenv("MLA_TRACE"))
      fprintf(stderr, "[mla] decode_noalloc: needs %zu bytes of scratch, the fixed array holds %zu\n", need,
              (size_t)MLA_NOALLOC_SCRATCH_BYTES);
    return MLA_ERR_WORKSPACE;
  }
  void* ws = nullptr;
  if (need > 0 && batch > 0) {
    ws = device_scratch();
    if (!ws) return MLA_ERR_HIP;
  }
  // the same checks, plan and kernels as mla_decode_multi, on the fixed array
  return mla_decode_multi(d, batch, q_len, q_nope, q_pe, w_uk, w_uv, cache, out, ws, need, stream);
}

}  // extern "C"
