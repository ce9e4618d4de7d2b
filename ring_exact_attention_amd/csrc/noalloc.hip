// attn_bwd_noalloc: the dense backward with its scratch in a static device array, for
// callers that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid allocation).
//
// The backward's scratch -- D and the log-sum-exp per (batch, q head, row), and the fp32
// dk/dv partials when a GQA group's heads are split over several workgroups -- lives in
// `scratch`, a file-scope array of kScratchBytes that each GPU holds from the moment the
// library's code object is loaded until the process ends.  In host code `scratch` only
// names the symbol; its device address is looked up once per device with
// hipGetSymbolAddress (each GPU has its own copy at its own address) and only that
// address is handed to the kernels.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "attn.h"
#include "launch.h"

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;   // ATTN_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == ATTN_NOALLOC_SCRATCH_BYTES, "attn.h states the scratch size");
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of this GPU's `scratch` (looked up on the first call on each device,
// with that device current).  NULL and a message on failure.
void* scratch_ptr(int* status) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *status = rea::report_error(ATTN_ERR_HIP, e != hipSuccess ? hipGetErrorString(e)
                                                               : "device index out of range");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      char msg[160];
      snprintf(msg, sizeof msg, "hipGetSymbolAddress of the scratch array failed: %s",
               e != hipSuccess ? hipGetErrorString(e) : "null address");
      *status = rea::report_error(ATTN_ERR_HIP, msg);
      return nullptr;
    }
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" int attn_bwd_noalloc(const attn_params* params, const void* q, const void* k, const void* v,
                                const void* o, const void* dout, const float* m, const float* l, void* dq,
                                void* dk, void* dv, void* stream) {
  if (params && params->sel_idx)
    return rea::report_error(ATTN_ERR_UNSUPPORTED, "attn_bwd_noalloc: dense mode only (sel_idx must be NULL)");
  const size_t need = attn_bwd_workspace_bytes(params);
  if (need == 0) {
    // invalid params: attn_bwd reports why, before it touches the workspace or the device
    return attn_bwd(params, q, k, v, o, dout, m, l, dq, dk, dv, nullptr, 0, stream);
  }
  if (need > kScratchBytes) {
    char msg[200];
    snprintf(msg, sizeof msg,
             "attn_bwd_noalloc: these params need %zu bytes of scratch, above the static %zu bytes; "
             "use attn_bwd with a workspace",
             need, kScratchBytes);
    return rea::report_error(ATTN_ERR_WORKSPACE, msg);
  }
  int st = ATTN_OK;
  void* ws = scratch_ptr(&st);
  if (!ws) return st;
  return attn_bwd(params, q, k, v, o, dout, m, l, dq, dk, dv, ws, kScratchBytes, stream);
}
