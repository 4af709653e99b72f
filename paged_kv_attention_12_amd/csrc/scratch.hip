// Allocation-free decode step: pkv_paged_decode_store with its split
// workspace taken from a static device array instead of a caller buffer, for
// callers that cannot allocate device memory at all (code under graph
// capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The array lives in this file's code object, one copy per device, for the
// life of the process.  Its device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept; host code never
// passes the array's own name to a kernel (on the host it is only a stand-in
// for the symbol).  Every call on a device shares that device's copy, so calls
// that overlap on one device (two streams, two threads) race; the split
// kernel writes every partial it later merges, so nothing needs clearing
// between calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/pkv.h"
#include "launch.hpp"

namespace {

static __device__ __align__(256) char scratch[PKV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on first
// use per device, with that device current).
pkv_status scratch_of_current_device(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (pkv_status)pkv::note_hip_error(e);
  if (dev < 0 || dev >= kMaxDevices) return PKV_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return (pkv_status)pkv::note_hip_error(e != hipSuccess ? e : hipErrorInvalidSymbol);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status pkv_paged_decode_store_noalloc(const pkv_pool *pool, int32_t layer_id,
                                          const pkv_step *step, const void *q, const void *k_new,
                                          const void *v_new, int32_t n_heads, float sm_scale,
                                          int32_t num_splits, void *out, void *stream) {
  if (!pool || !step) return PKV_ERR_NULL;
  if (step->batch < 0 || n_heads <= 0 || num_splits <= 0) return PKV_ERR_SHAPE;
  if (step->batch == 0) return PKV_OK;
  const size_t need =
      pkv_decode_workspace_bytes(step->batch, n_heads,
                                 pool->v_head_dim > 0 ? pool->v_head_dim : pool->head_dim,
                                 num_splits);
  if (need == 0) return PKV_ERR_SHAPE;
  if (need > (size_t)PKV_NOALLOC_SCRATCH_BYTES) return PKV_ERR_SCRATCH_LIMIT;
  void *ws = nullptr;
  const pkv_status st = scratch_of_current_device(&ws);
  if (st != PKV_OK) return st;
  return pkv_paged_decode_store(pool, layer_id, step, q, k_new, v_new, n_heads, sm_scale,
                                num_splits, ws, (size_t)PKV_NOALLOC_SCRATCH_BYTES, out, stream);
}

}  // extern "C"
