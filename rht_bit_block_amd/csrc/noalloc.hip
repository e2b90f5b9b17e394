// Level statistics of a row-wise quantization without any device allocation:
// the variant of ufp4_quant_diag for callers that cannot allocate (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The workgroups' partial sums, which ufp4_quant_diag keeps in the caller's
// workspace, live here in `scratch`, a file-scope device array of
// kDiagWorkspaceBytes (8 KiB) that each GPU the library runs on holds until
// the process ends.  Its device address is resolved once per device with
// hipGetSymbolAddress (that device current) and only that address is handed
// to the kernels.  Every call on a GPU shares the array: each call clears it
// with a kernel before use, and calls that overlap on one GPU race.
//
// [UFP4] = "Rethinking Shrinkage Bias in FP4 Pretraining of LLMs ... the UFP4
// Recipe" (hyper.ai summary, Method: the bin-asymmetry equation and bucket
// utilisation these statistics measure).
#include <atomic>
#include <mutex>

#include "ufp4_internal.h"

namespace {

// The scratch the no-allocation entry point uses, at most this size: the
// workgroups fold into kDiagSlots partial sets whatever the input's size.
static __device__ __align__(256) unsigned long long scratch[ufp4::kDiagWorkspaceBytes / 8];
static_assert(sizeof(scratch) == ufp4::kDiagWorkspaceBytes, "scratch holds the partial sets");

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];   // device address of scratch per device
std::mutex g_resolve;

// Device address of `scratch` on the current device, resolved on the first
// call made on that device.
int scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return UFP4_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return UFP4_ERR_UNSUPPORTED;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_resolve);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return UFP4_ERR_HIP;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return UFP4_OK;
}

}  // namespace

extern "C" int ufp4_quant_diag_noalloc(const void* x, int64_t rows, int64_t cols, int64_t ld,
                                       const ufp4_quant_cfg* cfg, uint64_t* stats,
                                       void* stream) {
  ufp4::QuantLaunch q;
  int st = ufp4::diag_prepare(x, rows, cols, ld, cfg, stats, q);
  if (st) return st;
  void* partials = nullptr;
  st = scratch_on_current_device(&partials);
  if (st) return st;
  const hipError_t e =
      ufp4::launch_quant_diag(q, reinterpret_cast<unsigned long long*>(stats),
                              reinterpret_cast<unsigned long long*>(partials),
                              (hipStream_t)stream);
  return e == hipSuccess ? UFP4_OK : UFP4_ERR_HIP;
}
