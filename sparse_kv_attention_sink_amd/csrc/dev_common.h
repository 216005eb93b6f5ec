// Device helpers shared by the gfx950 kernels: bf16 conversion, cross-lane
// reductions, LDS transpose reads, direct global-to-LDS copies and explicit
// memory-counter waits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "spec_internal.h"

namespace spec {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

#define SPEC_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

// 16-byte streaming load (non-temporal hint: the data is read once).
__device__ __forceinline__ float4 load_stream_f4(const void* p) {
  const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

// fp32 -> bf16 bits, round to nearest even (gfx950 converts in hardware,
// v_cvt_pk_bf16_f32); NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float shfl_xor(float x, int m) { return __shfl_xor(x, m, 64); }

__device__ __forceinline__ void raise_error(uint32_t* err, uint32_t bit) {
  atomicOr(err, bit);
}

// LDS byte address of a __shared__ object (the value M0 takes for a copy).
template <typename T>
__device__ __forceinline__ uint32_t lds_addr(T* p) {
  return (uint32_t)(uintptr_t)SPEC_LDS(T, p);
}

// Direct 16-byte-per-lane copy global -> LDS (global_load_lds_dwordx4).
// Lane i's 16 bytes land at LDS address m0 + 16 * i; m0 must be wave-uniform.
// Issued through inline assembly so that the compiler does not insert a
// full memory-counter wait before every LDS read: the kernels that use it
// count their copies themselves and wait with wait_vm<N>().
__device__ __forceinline__ void copy16_to_lds(const void* gaddr, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gaddr), "s"(m0)
               : "memory", "m0");
}

// The same copy from a wave-uniform base (SGPR pair) plus a 32-bit per-lane
// byte offset: no 64-bit address arithmetic per lane.  The base and m0 go
// through readfirstlane so that they are scalar whatever the compiler can
// prove about their uniformity (an "s" operand it believes divergent would
// otherwise be handed over in VGPRs).
__device__ __forceinline__ void copy16_to_lds_s(const void* sbase, uint32_t voff, uint32_t m0) {
  // (readfirstlane returns a signed int: both halves are taken back as
  // unsigned 32-bit values before they are joined, so the low half is never
  // sign-extended into the high one)
  const uint64_t b = reinterpret_cast<uint64_t>(sbase);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint64_t bs = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(reinterpret_cast<const void*>(bs)), "s"(__builtin_amdgcn_readfirstlane(m0))
               : "memory", "m0");
}

// Wait until at most N vector-memory operations of this wave are in flight
// (gfx9 s_waitcnt encoding; expcnt and lgkmcnt left unconstrained).
// Inline assembly with a memory clobber, so that no LDS read is moved above it.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Workgroup barrier without the memory fence __syncthreads() implies (which
// would also wait for every copy still in flight).
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" : : : "memory"); }

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// with M[i][e] the e-th 16-bit value at lane i's address, lane l receives
// M[4j + l/4][l%4] as its j-th value (j = 0..3).
__device__ __forceinline__ s16x4 lds_read_tr16(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(SPEC_LDS(s16x4, (uintptr_t)addr));
}

// ---------------------------------------------------------------- split merge
// Partial results cross workgroups through the workspace.  They are written
// and read with device-coherent (sc1) buffer accesses: an sc1 store goes
// through the XCD's L2 to the device coherence point, and an sc1 load fetches
// from it, so no L2 write-back or invalidate (what a device-scope fence
// costs on a multi-XCD part) is needed; a wait for the stores to complete
// before the arrival atomic orders them.

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
constexpr int kSc1 = 16;                     // cache-policy bit SC1 of buffer accesses
constexpr int32_t kRsrcWord3 = 0x00020000;   // raw 32-bit buffer (gfx9 descriptor word 3)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcWord3);
}
__device__ __forceinline__ void store_sc1_f4(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, off, 0, kSc1);
}
__device__ __forceinline__ void store_sc1_f1(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int32_t, v), r, off, 0, kSc1);
}
__device__ __forceinline__ f32x4 load_sc1_f4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kSc1));
}
__device__ __forceinline__ float load_sc1_f1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kSc1));
}

// Arrival at the end of a split: returns true (in every thread of the
// workgroup) iff this workgroup is the last of `splits` to arrive on
// `counter`; that workgroup resets the counter to zero and may then read,
// with sc1 loads, what the others wrote with sc1 stores before arriving.
__device__ __forceinline__ bool arrive_last(uint32_t* counter, int splits) {
  __shared__ int s_last;
  wait_vm<0>();      // this thread's sc1 stores have reached the coherence point
  __syncthreads();   // ... and every other thread's
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = prev + 1 == (uint32_t)splits;
    if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = last ? 1 : 0;
  }
  __syncthreads();
  return s_last != 0;
}

}  // namespace spec
