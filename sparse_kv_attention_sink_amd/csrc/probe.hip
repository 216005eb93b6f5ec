// Measurement kernels (libspecprobe): the HBM read rate a streaming kernel
// reaches on this GPU through each of the two load paths the attention
// kernels use, and the cost of a launch that does no work.  They compute
// nothing of the method; the benchmark reports the attention kernels'
// rates against them.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dev_common.h"
#include "spec_probe.h"

namespace spec {
namespace {

constexpr int kBlock = 4096;          // bytes one workgroup reads per load round
constexpr int kStage = 16384;         // bytes per LDS stage (ring path)

// Workgroup w reads blocks w, w + W, ...: IF blocks per round, every load
// of a round issued before any is used.  Each block is one 16-byte
// non-temporal buffer load per thread, from a descriptor based at the
// block (so the 32-bit offsets never overflow, whatever the buffer size).
template <int IF>
__global__ __launch_bounds__(256) void probe_read_kernel(const char* src, int64_t n_blocks, uint32_t* sink) {
  const int64_t W = gridDim.x;
  const uint32_t off = threadIdx.x * 16u;
  uint32_t x = 0;
  for (int64_t b0 = blockIdx.x; b0 < n_blocks; b0 += W * IF) {
    i32x4 v[IF];
#pragma unroll
    for (int i = 0; i < IF; ++i) {
      const int64_t bi = b0 + (int64_t)i * W;
      const int64_t bb = bi < n_blocks ? bi : b0;   // past the end: re-read this round's first block
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(src + bb * kBlock), 0, kBlock, kRsrcWord3);
      v[i] = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2 /* non-temporal */);
    }
#pragma unroll
    for (int i = 0; i < IF; ++i) x ^= (uint32_t)(v[i].x ^ v[i].y ^ v[i].z ^ v[i].w);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x ^= (uint32_t)__shfl_xor((int)x, m, 64);
  __shared__ uint32_t red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

// Wait until at most n (0 <= n <= MAXN) stages of copies are in flight,
// 4 copy instructions per stage and wavefront.
template <int MAXN>
__device__ __forceinline__ void wait_stages(int n) {
  if constexpr (MAXN <= 0) {
    wait_vm<0>();
  } else {
    if (n >= MAXN) wait_vm<MAXN * 4>();
    else wait_stages<MAXN - 1>(n);
  }
}

// Workgroup w streams the 16 KiB stages w, w + W, ... into a ring of NS LDS
// stages with global_load_lds_dwordx4 (each wavefront copies 4 KiB of every
// stage), NS - 1 stages in flight, and XORs one word of each landed stage.
template <int NS>
__global__ __launch_bounds__(256) void probe_read_lds_kernel(const char* src, int64_t n_stages, uint32_t* sink) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[NS * kStage];
  const int64_t W = gridDim.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t mine = blockIdx.x < n_stages ? (n_stages - 1 - blockIdx.x) / W + 1 : 0;
  const uint32_t base = lds_addr(ring);
  auto issue = [&](int64_t j, int slot) __attribute__((always_inline)) {
    const char* g = src + (blockIdx.x + j * W) * kStage + wave * 4096;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      copy16_to_lds(g + u * 1024 + lane * 16,
                    __builtin_amdgcn_readfirstlane(base + slot * kStage + wave * 4096 + u * 1024));
  };
  uint32_t x = 0;
  for (int j = 0; j < NS - 1; ++j)
    if (j < mine) issue(j, j);
  for (int64_t j = 0; j < mine; ++j) {
    const int64_t newer = mine - 1 - j;   // stages issued after stage j, at most NS - 2
    wait_stages<NS - 2>((int)(newer < NS - 2 ? newer : NS - 2));
    barrier_only();                        // every wave's copies of stage j landed; stage j-1 is consumed
    if (j + NS - 1 < mine) issue(j + NS - 1, (int)((j + NS - 1) % NS));
    x ^= *SPEC_LDS(const uint32_t, (uintptr_t)(base + (uint32_t)(j % NS) * kStage + threadIdx.x * 64));
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x ^= (uint32_t)__shfl_xor((int)x, m, 64);
  __shared__ uint32_t red[4];
  if (lane == 0) red[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

__global__ __launch_bounds__(256) void probe_empty_kernel(uint32_t* sink) {
  if (threadIdx.x == 0) sink[blockIdx.x] = blockIdx.x;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace
}  // namespace spec

using namespace spec;

#pragma GCC visibility push(default)
extern "C" {

int32_t spec_probe_read(const void* src, size_t bytes, int32_t workgroups, int32_t in_flight,
                        uint32_t* sink, void* stream) {
  if (src == nullptr || sink == nullptr || !aligned16(src) || bytes == 0 || bytes % kBlock ||
      workgroups < 1 || workgroups > (1 << 20))
    return -1;
  const int64_t n = (int64_t)(bytes / kBlock);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const char* s = static_cast<const char*>(src);
  switch (in_flight) {
    case 4: hipLaunchKernelGGL(probe_read_kernel<4>, dim3(workgroups), dim3(256), 0, st, s, n, sink); break;
    case 8: hipLaunchKernelGGL(probe_read_kernel<8>, dim3(workgroups), dim3(256), 0, st, s, n, sink); break;
    case 16: hipLaunchKernelGGL(probe_read_kernel<16>, dim3(workgroups), dim3(256), 0, st, s, n, sink); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int32_t spec_probe_read_lds(const void* src, size_t bytes, int32_t workgroups, int32_t stages,
                            uint32_t* sink, void* stream) {
  if (src == nullptr || sink == nullptr || !aligned16(src) || bytes == 0 || bytes % kStage ||
      workgroups < 1 || workgroups > (1 << 20))
    return -1;
  const int64_t n = (int64_t)(bytes / kStage);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const char* s = static_cast<const char*>(src);
  switch (stages) {
    case 2: hipLaunchKernelGGL(probe_read_lds_kernel<2>, dim3(workgroups), dim3(256), 0, st, s, n, sink); break;
    case 4: hipLaunchKernelGGL(probe_read_lds_kernel<4>, dim3(workgroups), dim3(256), 0, st, s, n, sink); break;
    case 6: hipLaunchKernelGGL(probe_read_lds_kernel<6>, dim3(workgroups), dim3(256), 0, st, s, n, sink); break;
    case 8: hipLaunchKernelGGL(probe_read_lds_kernel<8>, dim3(workgroups), dim3(256), 0, st, s, n, sink); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int32_t spec_probe_empty(int32_t workgroups, uint32_t* sink, void* stream) {
  if (sink == nullptr || workgroups < 1 || workgroups > (1 << 20)) return -1;
  hipLaunchKernelGGL(probe_empty_kernel, dim3(workgroups), dim3(256), 0, static_cast<hipStream_t>(stream), sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
#pragma GCC visibility pop
