// Routing without any device allocation: the route workspace lives in a static
// device array of fixed size instead of caller memory.  For callers that cannot
// allocate (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).
#include <hip/hip_runtime.h>

#include <mutex>

#include "abs.h"
#include "internal.h"
#include "route_internal.h"

// The workspace of abs_route_noalloc.  Each GPU the library runs on holds its
// own copy until the process ends.  In host code this name is only a stand-in
// for the symbol: the device address of each GPU's copy comes from
// hipGetSymbolAddress and is the only form passed to kernels.
static __device__ __align__(256) unsigned char scratch[ABS_ROUTE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device

// Device address of the current device's copy of `scratch`; looked up once per
// device, with that device current.
hipError_t scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

using namespace abs_impl;

extern "C" abs_status abs_route_noalloc(const abs_plan* plan, const void* q, const void* k,
                                        float p, int32_t k_floor, float slack,
                                        const abs_mask* mask, void* stream) {
  if (!plan || plan->num_blocks <= 0 || plan->rows <= 0 || plan->block_tokens <= 0 ||
      (plan->s.dtype != ABS_F32 && plan->s.dtype != ABS_BF16) || plan->heads_per_phase < 1)
    return ABS_EINVAL;
  if (!q || !k || !mask || !mask->row_ptr || !mask->col_idx || !mask->head_nnz)
    return ABS_EINVAL;
  if (!(p > 0.0f && p <= 1.0f)) return ABS_EINVAL;
  if (k_floor < 1) return ABS_EINVAL;
  if (!(slack >= 0.0f && slack < 1.0f)) return ABS_EINVAL;
  const Geo g = make_geo(plan);
  const RouteWs L = route_ws_layout(g, slack > 0.0f);
  if (L.total > (size_t)ABS_ROUTE_NOALLOC_SCRATCH_BYTES) return ABS_ETOOBIG;
  // the stream's device must be the current one: that is the copy looked up
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ABS_EHIP;
  if (stream) {
    int sdev = -1;
    if (hipStreamGetDevice((hipStream_t)stream, &sdev) != hipSuccess) return ABS_EHIP;
    if (sdev != dev) return ABS_EINVAL;
  }
  void* ws = nullptr;
  if (scratch_address(dev, &ws) != hipSuccess) return ABS_EHIP;
  const int kf = k_floor > g.nb ? g.nb : k_floor;
  const hipError_t e = launch_route(g, plan->s.dtype, q, k, p, kf, slack, mask, (char*)ws, L,
                                    (hipStream_t)stream);
  return e == hipSuccess ? ABS_OK : ABS_EHIP;
}
