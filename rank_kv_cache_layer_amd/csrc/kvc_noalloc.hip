// The per-hop correction without a caller workspace, for callers that cannot allocate device
// memory (code under stream capture, tight serving loops, harnesses that forbid allocation).
// Its scratch is a file-scope device array of KVC_NOALLOC_SCRATCH_BYTES, one copy per GPU, held
// until the process ends; every call on a GPU reuses that GPU's copy.
#include <mutex>

#include "kvc_internal.h"

namespace {

// the scratch buffer itself; host code never passes this name to a kernel: on the host it is a
// stand-in, not a device address (see scratch_of)
static __device__ __align__(256) char scratch[KVC_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];    // device address of `scratch` on each device, taken once per device

// The device address of this device's copy of `scratch` (looked up on the first call on the
// device, with that device current).
hipError_t scratch_of(int dev, void** out) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" kvc_status kvc_correct_hop_noalloc(const void* k_src, const void* v_src, void* k_out, void* v_out,
                                              kvc_dtype dtype, kvc_shape shape, int64_t p_src, int64_t p_tgt,
                                              const kvc_rope* rope, const kvc_pool* pool, const kvc_params* params,
                                              kvc_match_out* out, void* stream) {
  // a request that does not fit launches nothing; an invalid one (size query 0) gets its own error
  // from kvc_correct_hop's validation, before any launch
  const size_t need = kvc_workspace_size(KVC_CALL_CORRECT, shape, pool, params);
  if (need > (size_t)KVC_NOALLOC_SCRATCH_BYTES)
    return kvc::report(KVC_E_WORKSPACE, "no-alloc hop: needs %zu bytes of scratch, the maximum is %zu (%d MiB)",
                       need, (size_t)KVC_NOALLOC_SCRATCH_BYTES, KVC_NOALLOC_SCRATCH_BYTES >> 20);
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return kvc::report(KVC_E_HIP, "no-alloc hop: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return kvc::report(KVC_E_PARAM, "no-alloc hop: device %d out of range", dev);
  void* ws = nullptr;
  if ((e = scratch_of(dev, &ws)) != hipSuccess)
    return kvc::report(KVC_E_HIP, "no-alloc hop: scratch address: %s", hipGetErrorString(e));
  return kvc_correct_hop(k_src, v_src, k_out, v_out, dtype, shape, p_src, p_tgt, rope, pool, params, out, ws,
                         (size_t)KVC_NOALLOC_SCRATCH_BYTES, stream);
}
