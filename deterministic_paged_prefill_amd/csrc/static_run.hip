// dpp_run_static: dpp_run over a scratch array the library owns, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc). Same checks, same kernels, same bits as dpp_run.
//
// The scratch holds what dpp_run's workspace holds: the plan's work list at its head, then
// the split partials of the largest pass. A file-scope device array gives every device the
// library runs on its own copy, held until the process ends. Its device address is resolved
// once per device with hipGetSymbolAddress while that device is current; host code only ever
// passes that address (the array's own name is a host-side stand-in, not a device pointer).
//
// Nothing in the scratch needs to start at zero: the upload writes the whole work list
// (zero chunk and reserved words included), and the merge reads only the partial slots that
// the same run's prefill launch wrote. Every call on one device shares that device's array, so
// calls that overlap on one GPU (two streams, two threads) race.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "plan.h"

static __device__ __align__(256) unsigned char scratch[DPP_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];   // the array's device address on each device, once resolved
uint32_t g_owner[kMaxDevices];  // plan id of the work list last uploaded into that scratch

dpp_status hip_fail(hipError_t e, const char* what) {
  return dpp::fail(DPP_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

}  // namespace

extern "C" dpp_status dpp_run_static(const dpp_plan* plan, const void* q, int64_t q_rows, const void* k_pool,
                                     const void* v_pool, int64_t num_pages, const int32_t* kv_indices,
                                     int64_t num_kv_indices, void* o, float* lse, uint32_t flags,
                                     void* stream_ptr) {
  dpp_status st = dpp::check_run_args(plan, "dpp_run_static", q, q_rows, k_pool, v_pool, num_pages, kv_indices,
                                      num_kv_indices, o, lse, flags);
  if (st != DPP_OK) return st;
  if (plan->workspace_bytes > (size_t)DPP_STATIC_SCRATCH_BYTES)
    return dpp::fail(DPP_ERR_WORKSPACE, "dpp_run_static: the plan needs " + std::to_string(plan->workspace_bytes) +
                                            " B of workspace, above the static scratch's " +
                                            std::to_string((size_t)DPP_STATIC_SCRATCH_BYTES) +
                                            " B; plan with workspace_cap_bytes <= DPP_STATIC_SCRATCH_BYTES");
  if (plan->num_items == 0) return DPP_OK;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return dpp::fail(DPP_ERR_UNSUPPORTED, "dpp_run_static: device index above 63");
  hipStream_t stream = (hipStream_t)stream_ptr;
  void* ws = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
      g_scratch[dev] = p;
    }
    ws = g_scratch[dev];
    if (flags & DPP_RUN_REUSE_UPLOAD) {
      if (g_owner[dev] != plan->plan_id)
        return dpp::fail(DPP_ERR_INVALID, "dpp_run_static: DPP_RUN_REUSE_UPLOAD, but the scratch of this device "
                                          "holds another plan's work list (or none)");
    } else {
      // the plan's pinned copy if an earlier dpp_run made one, else its pageable host copy
      // (which the runtime stages); no allocation either way
      const size_t hbytes = plan->header.size() * sizeof(int32_t);
      const void* src;
      {
        std::lock_guard<std::mutex> plock(plan->pinned_mu);
        src = plan->pinned ? plan->pinned : (const void*)plan->header.data();
      }
      e = hipMemcpyAsync(ws, src, hbytes, hipMemcpyHostToDevice, stream);
      if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(work list -> scratch)");
      g_owner[dev] = plan->plan_id;
    }
  }
  return dpp::launch_passes(plan, q, k_pool, v_pool, num_pages, kv_indices, o, lse, ws, stream_ptr);
}
