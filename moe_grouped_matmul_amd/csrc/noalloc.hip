// Static split-K scratch for the allocation-free dense GEMM entry point
// (dg_fp8_gemm_nt_noalloc): callers that cannot allocate (code under graph
// capture, tight serving loops, harnesses that forbid allocation) pass only
// their inputs and outputs, and the K-split partials and completion counters
// live in this file-scope device array instead of a caller workspace.
//
// The array exists once per GPU the library runs on (every device that loads
// the code object holds its own copy, until the process ends).  Host code
// never passes the array's name to a kernel (on the host it is only a
// stand-in symbol): the first call on a device resolves the device address
// with hipGetSymbolAddress, with that device current, and keeps it per
// device.  The counter area at the start of the array (see dg_internal.hpp)
// must be zero before a K-split launch uses it; device globals start zeroed,
// the first call on a device clears the area once more with a fill kernel
// on the caller's stream (a memset node would not be safe in a captured
// graph), and every launch leaves its counters at zero again.  Calls that
// overlap on one GPU share the array and race.

#include <atomic>
#include <mutex>

#include "dg_internal.hpp"

namespace dg {
namespace {

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];
std::mutex g_scratch_mu;

__global__ void __launch_bounds__(256) clear_words(uint32_t* p, int n) {
  for (int i = (int)threadIdx.x; i < n; i += (int)blockDim.x) p[i] = 0u;
}

}  // namespace

hipError_t scratch_for_current_device(void** out, hipStream_t stream) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(clear_words, dim3(1), dim3(256), 0, stream, static_cast<uint32_t*>(p),
                         (int)(kWsCounterBytes / 4));
      e = hipGetLastError();
      if (e != hipSuccess) return e;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace dg
