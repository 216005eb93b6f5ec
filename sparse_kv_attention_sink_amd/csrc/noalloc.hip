// The tree verify for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid it): the
// same kernels as spec_attn_verify_tree, with the workspace taken from a
// file-scope device array instead of a caller buffer.
#include <stdio.h>

#include <mutex>

#include "spec_internal.h"

// The static workspace: header (error word), counter region, split
// partials.  Each GPU the library runs on holds its own copy, from the first
// use until the process ends.  In host code `scratch` names a host-side
// stand-in, never the device memory: kernels get the address that
// hipGetSymbolAddress returns for the current device.
static constexpr size_t kStaticScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device

__global__ __launch_bounds__(256) void clear_words_kernel(uint32_t* p, size_t words) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < words; i += (size_t)gridDim.x * 256) p[i] = 0;
}

}  // namespace

#pragma GCC visibility push(default)
extern "C" spec_status spec_attn_verify_tree_noalloc(
    const spec_dims* dims, const void* q, int32_t n_nodes, const spec_kv* cache,
    const int32_t* cache_len, const uint8_t* pad_or_null, int64_t pad_stride_b,
    const spec_kv* tree, const int32_t* parents, int64_t parents_stride_b, void* out,
    float* lse_or_null, int32_t* pos_ids_or_null, void* stream) {
  using namespace spec;
  size_t need = 0;
  spec_status st = verify_impl(dims, q, n_nodes, cache, cache_len, pad_or_null, pad_stride_b, tree,
                               parents, parents_stride_b, out, lse_or_null, pos_ids_or_null,
                               nullptr, 0, stream, &need);
  if (st != SPEC_OK || need == 0) return st;   // invalid, or nothing to launch (batch 0)
  if (need > kStaticScratchBytes) {
    char msg[160];
    snprintf(msg, sizeof msg, "this shape needs %zu bytes of scratch; the static array holds %zu",
             need, kStaticScratchBytes);
    return set_error(SPEC_E_UNSUPPORTED, msg);
  }
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(SPEC_E_HIP, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return set_error(SPEC_E_UNSUPPORTED, "device index beyond 63");
  void* ptr = nullptr;
  bool first = false;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch_ptr[dev] == nullptr) {
      // once per device, with that device current: the device address of
      // this GPU's copy of the array
      e = hipGetSymbolAddress(&g_scratch_ptr[dev], HIP_SYMBOL(scratch));
      if (e != hipSuccess || g_scratch_ptr[dev] == nullptr) {
        g_scratch_ptr[dev] = nullptr;
        return set_error(SPEC_E_HIP, e != hipSuccess ? hipGetErrorString(e) : "no device address");
      }
      first = true;
    }
    ptr = g_scratch_ptr[dev];
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (first) {
    // Counters must start at zero.  The array is zero-initialised when its
    // code object loads, and every call leaves the counters it used at zero;
    // clearing the header and counter region once more on first use costs one
    // small launch.  (A fill kernel, not a memset node: this may run under
    // graph capture.)
    hipLaunchKernelGGL(clear_words_kernel, dim3(64), dim3(256), 0, s, static_cast<uint32_t*>(ptr),
                       kScratchOff / 4);
    if ((e = hipGetLastError()) != hipSuccess) return set_error(SPEC_E_HIP, hipGetErrorString(e));
  }
  return verify_impl(dims, q, n_nodes, cache, cache_len, pad_or_null, pad_stride_b, tree, parents,
                     parents_stride_b, out, lse_or_null, pos_ids_or_null, ptr, kStaticScratchBytes,
                     stream, nullptr);
}
#pragma GCC visibility pop
