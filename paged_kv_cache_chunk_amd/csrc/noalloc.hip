// pkv_attn_bwd_noalloc: the attention backward of pkv_attn_bwd with its
// scratch (D = rowsum(dO * O), the base-2 log-sum-exp and, in top-K mode, the
// dK/dV work list) in a fixed device array of the library instead of memory
// that the pool grows with hipMalloc, for callers that cannot allocate.
//
// The array lives in the code object; each GPU the library runs on holds its
// own copy at its own address, kept until the process ends.  Host code never
// passes the array's name to a kernel (on the host it is only a stand-in for
// the symbol): the device address is looked up with hipGetSymbolAddress on
// the first call on each device and kept per device.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pkv_pool.h"

namespace pkv {
namespace {

constexpr int64_t kScratchBytes = 16ll << 20;  // per GPU
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of `scratch` on the current device.
pkv_status scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return pool_hip_fail(e, "pkv_attn_bwd_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return pool_fail(PKV_EUNSUPPORTED, "pkv_attn_bwd_noalloc: device index beyond 63");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return pool_hip_fail(e, "pkv_attn_bwd_noalloc: hipGetSymbolAddress");
    if (!ptr) return pool_fail(PKV_EHIP, "pkv_attn_bwd_noalloc: no device address for the scratch");
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return PKV_OK;
}

}  // namespace
}  // namespace pkv

extern "C" pkv_status pkv_attn_bwd_noalloc(pkv_pool* pool, int32_t layer, int64_t q_pos0,
                                           int64_t n_q, int32_t n_q_heads, float scale,
                                           const void* q, const void* o, const void* dout,
                                           const float* lse, const pkv_sel* sel, float* dq,
                                           hipStream_t stream) {
  void* buf = nullptr;
  const pkv_status st = pkv::scratch_address(&buf);
  if (st != PKV_OK) return st;
  return pkv::attn_bwd_impl(pool, layer, q_pos0, n_q, n_q_heads, scale, q, o, dout, lse, sel, dq,
                            stream, buf, pkv::kScratchBytes, "pkv_attn_bwd_noalloc");
}

