// Device helpers shared by the gfx950 kernels: bf16 conversion, cross-lane
// reductions, partial-result stores.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "spec_internal.h"

namespace spec {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load (non-temporal hint: the data is read once).
__device__ __forceinline__ uint4 load_stream(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 load_stream_f4(const void* p) {
  const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

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

// Data-parallel-primitive moves within 16-lane rows (gfx9 DPP controls).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppRor4 = 0x124;      // row_ror:4
constexpr int kDppRor8 = 0x128;      // row_ror:8
constexpr int kDppHalfMirror = 0x141;

// Sum over groups of LANES consecutive lanes (8 or 16); every lane of the
// group receives the group's sum.
template <int LANES>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (LANES == 16) {
    x += dpp<kDppRor8>(x);
    x += dpp<kDppRor4>(x);
  } else {
    static_assert(LANES == 8, "group of 8 or 16 lanes");
    x += dpp<kDppHalfMirror>(x);
  }
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  return x;
}

__device__ __forceinline__ float shfl_xor(float x, int m) { return __shfl_xor(x, m, 64); }

__device__ __forceinline__ void raise_error(uint32_t* err, uint32_t bit) {
  atomicOr(err, bit);
}

// Store one row's result: the final output (splits == 1) or an fp32 partial.
// `vals` holds NV consecutive head-dim values starting at d0.
template <int NV>
__device__ __forceinline__ void store_row_values(const AttnArgs& a, int dtype, int pair, int z,
                                                 int s, int i, int d0, const float* vals) {
  const int r = z * a.rb + i;
  if (a.splits > 1) {
    size_t base = ((((size_t)pair * a.n_rb + z) * a.splits + s) * a.rb + i) * a.D + d0;
    float* dst = a.o_part + base;
#pragma unroll
    for (int e = 0; e < NV; e += 4)
      *reinterpret_cast<float4*>(dst + e) = make_float4(vals[e], vals[e + 1], vals[e + 2], vals[e + 3]);
    return;
  }
  const int b = pair / a.Hkv, g = pair % a.Hkv;
  const int t = r / a.G, hh = r % a.G;
  size_t o = (((size_t)b * a.T + t) * a.Hq + g * a.G + hh) * a.D + d0;
  if (dtype == SPEC_BF16) {
    uint16_t* dst = reinterpret_cast<uint16_t*>(a.out) + o;
#pragma unroll
    for (int e = 0; e < NV; e += 4) {
      uint2 w = make_uint2(pack_bf16x2(vals[e], vals[e + 1]), pack_bf16x2(vals[e + 2], vals[e + 3]));
      *reinterpret_cast<uint2*>(dst + e) = w;
    }
  } else {
    float* dst = reinterpret_cast<float*>(a.out) + o;
#pragma unroll
    for (int e = 0; e < NV; e += 4)
      *reinterpret_cast<float4*>(dst + e) = make_float4(vals[e], vals[e + 1], vals[e + 2], vals[e + 3]);
  }
}

// Store one row's log2-domain sum-exp (partial) or natural-log lse (final).
__device__ __forceinline__ void store_row_lse(const AttnArgs& a, int pair, int z, int s, int i,
                                              float lse2) {
  const int r = z * a.rb + i;
  if (a.splits > 1) {
    a.lse_part[(((size_t)pair * a.n_rb + z) * a.splits + s) * a.rb + i] = lse2;
    return;
  }
  if (a.lse == nullptr) return;
  const int b = pair / a.Hkv, g = pair % a.Hkv;
  const int t = r / a.G, hh = r % a.G;
  a.lse[((size_t)b * a.T + t) * a.Hq + g * a.G + hh] = lse2 * kLn2;
}

}  // namespace spec
