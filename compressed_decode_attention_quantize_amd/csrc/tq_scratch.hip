// tq_scratch.hip -- the decode workspace that tq_decode_attention_noalloc
// uses in place of a caller's: one file-scope device array (each GPU the
// library runs on holds its own copy until the process ends), found once per
// device with hipGetSymbolAddress.  In host code the array's name is only a
// stand-in; kernels receive the device address looked up here.

#include <mutex>

#include "tq_internal.h"

namespace tq {
namespace {

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};

__global__ __launch_bounds__(256) void clear_words_kernel(uint32_t* p, int n_words) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n_words) p[i] = 0u;
}

}  // namespace

hipError_t scratch_workspace(void** out, hipStream_t stream) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    // the completion counters must start at zero (every decode leaves the
    // ones it used at zero again); cleared by a kernel, not a memset, so that
    // a first call under graph capture records a kernel node
    const int n_words = static_cast<int>(kScratchCounterBytes / 4);
    hipLaunchKernelGGL(clear_words_kernel, dim3((n_words + 255) / 256), dim3(256), 0, stream,
                       static_cast<uint32_t*>(p), n_words);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace tq
