// Split-K combine and the plain fp32 attention kernel (all modes).
//
// The combine merges the per-split partials of a query row: with split s
// holding o_s (normalised by its own softmax sum) and its log2 sum-exp x_s,
// the row's result is sum_s 2^(x_s - M) o_s / sum_s 2^(x_s - M) with
// M = max_s x_s, and lse = (M + log2 sum_s 2^(x_s - M)) * ln 2.  This is the
// exact softmax over the union of the splits' keys.
//
// The fp32 kernels are the plain path for fp32 inputs (one wavefront per query
// row and split; lanes take one key each for q.k, then the head dimension for
// P.V).  It serves the draft view (window or budget list) and the tree verify
// with the same definitions as the bf16 kernels.
#include "dev_common.h"

namespace spec {

// One block per (pair, row): 256 threads; thread (d, g) sums the splits
// s = g, g + 256/D, ... for head-dim element d; empty splits hold o = 0 and
// x = -inf, so their weight 2^(x - M) is exactly 0 and no branch is needed.
__global__ __launch_bounds__(256) void combine_kernel(AttnArgs a, int dtype) {
  const int row = blockIdx.x % a.R;
  const int pair = blockIdx.x / a.R;
  const int z = row / a.rb, i = row % a.rb;
  const int tid = threadIdx.x;
  const int S = a.splits, D = a.D;
  const size_t base = (((size_t)pair * a.n_rb + z) * S) * a.rb + i;
  __shared__ float s_max[4];
  __shared__ float s_o[256], s_w[256];

  float M = -INFINITY;
  bool nan = false;
  for (int s = tid; s < S; s += 256) {
    const float x = a.lse_part[base + (size_t)s * a.rb];
    nan |= isnan(x);
    M = fmaxf(M, x);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) M = fmaxf(M, __shfl_xor(M, m, 64));
  if ((tid & 63) == 0) s_max[tid >> 6] = M;
  nan = __syncthreads_or(nan);
  M = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));

  const int groups = 256 / D;
  const int d = tid % D, grp = tid / D;
  float o = 0.f, w = 0.f;
  if (!nan && M != -INFINITY) {
#pragma unroll 4
    for (int s = grp; s < S; s += groups) {
      const size_t ps = base + (size_t)s * a.rb;
      const float ws = __builtin_amdgcn_exp2f(a.lse_part[ps] - M);
      w += ws;
      o += ws * a.o_part[ps * D + d];
    }
  }
  s_o[tid] = o;
  s_w[tid] = w;
  __syncthreads();
  if (grp != 0) return;
  for (int g2 = 1; g2 < groups; ++g2) {
    o += s_o[g2 * D + d];
    w += s_w[g2 * D + d];
  }
  float lse2;
  if (nan) {
    o = NAN;
    lse2 = NAN;
  } else if (M == -INFINITY) {
    o = 0.f;
    lse2 = -INFINITY;
  } else {
    o /= w;
    lse2 = M + log2f(w);
  }
  const int b = pair / a.Hkv, g = pair % a.Hkv;
  const int t = row / a.G, hh = row % a.G;
  const size_t oi = (((size_t)b * a.T + t) * a.Hq + g * a.G + hh);
  if (dtype == SPEC_BF16)
    reinterpret_cast<uint16_t*>(a.out)[oi * D + d] = (uint16_t)f32_to_bf16(o);
  else
    reinterpret_cast<float*>(a.out)[oi * D + d] = o;
  if (d == 0 && a.lse != nullptr) a.lse[oi] = lse2 * kLn2;
}

hipError_t launch_combine(const AttnArgs& a, int dtype, hipStream_t st) {
  const int64_t blocks = (int64_t)a.B * a.Hkv * a.R;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a, dtype);
  return hipGetLastError();
}

// ------------------------------------------------------------------ fp32

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

template <int MODE>
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs a) {
  const int lane = threadIdx.x;
  int w = blockIdx.x;
  const int s = w % a.splits;
  w /= a.splits;
  const int r = w % a.n_rb;          // rb == 1: one row per wavefront
  const int pair = w / a.n_rb;
  const int b = pair / a.Hkv, g = pair % a.Hkv;
  const int t = r / a.G, hh = r % a.G;
  const int D = a.D;

  int L = a.cache_len[b];
  bool bad;
  if (MODE == kVerify) bad = a.bad[b] != 0;
  else bad = L < a.T || (a.kv_ring == 0 && L > a.capacity);   // a ring keeps the logical length
  if (bad) L = 0;

  __shared__ float qs[128];
  const float* qrow = reinterpret_cast<const float*>(a.q) + (((size_t)b * a.T + t) * a.Hq + g * a.G + hh) * D;
  for (int d = lane; d < D; d += 64) qs[d] = qrow[d];
  __syncthreads();

  const float* kc = reinterpret_cast<const float*>(a.k) + b * a.kb + g * a.kh;
  const float* vc = reinterpret_cast<const float*>(a.v) + b * a.kb + g * a.kh;
  const int e = L - a.T + t + 1;     // draft: first position the query cannot see

  int n_keys = 0, s_len = 0, w_start = 0;
  uint64_t anc = 0;
  if (!bad) {
    if (MODE == kDraftWindow) {
      s_len = min(a.n_sink, L);
      w_start = min(max(max(a.n_sink, L - a.T + 1 - a.window), 0), L);
      n_keys = s_len + (L - w_start);
    } else if (MODE == kDraftGather) {
      n_keys = a.budget;
    } else {
      n_keys = L + a.T;
      anc = a.anc[(size_t)b * a.T + t];
    }
  }
  // Splits are planned over the cache capacity; in verify mode the last split
  // also takes the N tree keys that follow the cache positions.
  const int p0 = s * a.chunk;
  const int p1 = (MODE == kVerify && s == a.splits - 1) ? n_keys : min(n_keys, p0 + a.chunk);

  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  bool idx_bad = false;
  for (int c = p0; c < p1; c += 64) {
    const int pos = c + lane;
    bool vis = pos < p1;
    const float* krow = kc;
    const float* vrow = vc;
    if (vis) {
      if (MODE == kDraftWindow) {
        const int j = pos < s_len ? pos : w_start + (pos - s_len);
        vis = j < e && (j < a.n_sink || j >= e - a.window);
        const int jr = (a.kv_ring == 0 || j < a.n_sink) ? j : a.n_sink + (j - a.n_sink) % a.kv_ring;
        krow = kc + (int64_t)jr * a.kt;
        vrow = vc + (int64_t)jr * a.kt;
      } else if (MODE == kDraftGather) {
        const int j = a.idx[b * a.idx_sb + g * a.idx_sh + pos];
        if (j == -1) {          // padding entry: selects nothing
          vis = false;
        } else if (j < 0 || j >= L) {
          idx_bad = true;
          vis = false;
        } else {
          vis = j < e;
          krow = kc + (int64_t)j * a.kt;
          vrow = vc + (int64_t)j * a.kt;
        }
      } else if (pos < L) {
        vis = a.pad == nullptr || a.pad[b * a.pad_sb + pos] == 0;
        krow = kc + (int64_t)pos * a.kt;
        vrow = vc + (int64_t)pos * a.kt;
      } else {
        const int node = pos - L;
        vis = (anc >> node) & 1ull;
        krow = reinterpret_cast<const float*>(a.tk) + b * a.tkb + g * a.tkh + (int64_t)node * a.tkt;
        vrow = reinterpret_cast<const float*>(a.tv) + b * a.tkb + g * a.tkh + (int64_t)node * a.tkt;
      }
    }
    float sc = -INFINITY;
    if (vis) {
      float acc = 0.f;
      for (int d = 0; d < D; d += 4) {
        const float4 kv = *reinterpret_cast<const float4*>(krow + d);
        acc += kv.x * qs[d] + kv.y * qs[d + 1] + kv.z * qs[d + 2] + kv.w * qs[d + 3];
      }
      sc = acc * a.scale_log2;
    }
    const float mn = fmaxf(m, wave_max(sc));
    if (mn == -INFINITY) continue;
    const float alpha = exp2f(m - mn);
    const float p = exp2f(sc - mn);
    l = l * alpha + wave_sum(p);
    o0 *= alpha;
    o1 *= alpha;
    const uint64_t vaddr = reinterpret_cast<uint64_t>(vrow);
    for (int j = 0; j < 64; ++j) {
      const float pj = __shfl(p, j, 64);
      if (pj == 0.f) continue;
      const uint32_t lo = __shfl((uint32_t)vaddr, j, 64);
      const uint32_t hi = __shfl((uint32_t)(vaddr >> 32), j, 64);
      const float* vj = reinterpret_cast<const float*>(((uint64_t)hi << 32) | lo);
      o0 += pj * vj[lane < D ? lane : 0];
      if (D > 64) o1 += pj * vj[lane + 64];
    }
    m = mn;
  }

  const bool poison = bad || __any(idx_bad);
  if (lane == 0) {
    if (MODE != kVerify && bad) raise_error(a.err, SPEC_DEV_CACHE_LEN);
    if (!bad && poison) raise_error(a.err, SPEC_DEV_INDEX);
  }
  float inv, lse2;
  if (poison) {
    inv = NAN;
    lse2 = NAN;
  } else if (l > 0.f) {
    inv = 1.f / l;
    lse2 = m + log2f(l);
  } else {
    inv = 0.f;
    lse2 = -INFINITY;
  }
  o0 = poison ? NAN : o0 * inv;
  o1 = poison ? NAN : o1 * inv;
  if (a.splits > 1) {
    const size_t ps = (((size_t)pair * a.n_rb + r) * a.splits + s);
    if (lane < D) a.o_part[ps * D + lane] = o0;
    if (D > 64) a.o_part[ps * D + lane + 64] = o1;
    if (lane == 0) a.lse_part[ps] = lse2;
  } else {
    const size_t oi = (((size_t)b * a.T + t) * a.Hq + g * a.G + hh);
    float* out = reinterpret_cast<float*>(a.out) + oi * D;
    if (lane < D) out[lane] = o0;
    if (D > 64) out[lane + 64] = o1;
    if (lane == 0 && a.lse != nullptr) a.lse[oi] = lse2 * kLn2;
  }
}

// ------------------------------------------------------------------ fp32 verify prep
// One block per sequence: validates cache_len and parents, builds each
// node's ancestor-or-self bitmask, and writes the remapped positions
// (non-padding slots before cache_len, plus the node's depth).
__global__ __launch_bounds__(256) void verify_prep_kernel(
    int N, int capacity, const int32_t* __restrict__ cache_len, const uint8_t* __restrict__ pad,
    int64_t pad_sb, const int32_t* __restrict__ parents, int64_t par_sb, int32_t* pos_ids,
    uint64_t* anc_ws, int32_t* bad_ws, uint32_t* err) {
  const int b = blockIdx.x, tid = threadIdx.x;
  __shared__ int par_s[kMaxNodes];
  __shared__ int cnt_s[4];
  const int L = cache_len[b];
  const bool bad_len = L < 0 || L > capacity;
  bool bad_par = false;
  if (tid < N) {
    const int p = parents[b * par_sb + tid];
    par_s[tid] = p;
    bad_par = !(p >= -1 && p < tid);
  }
  const bool any_bad_par = __syncthreads_or(bad_par);

  int cnt = 0;
  if (pad != nullptr && pos_ids != nullptr && !bad_len) {
    const uint8_t* row = pad + b * pad_sb;
    for (int j = tid * 4; j < L; j += 256 * 4) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(row + j);
      const int nb = min(4, L - j);
#pragma unroll
      for (int e = 0; e < 4; ++e) cnt += (e < nb) && ((w >> (8 * e)) & 0xffu);
    }
  }
#pragma unroll
  for (int msk = 32; msk >= 1; msk >>= 1) cnt += __shfl_xor(cnt, msk, 64);
  if ((tid & 63) == 0) cnt_s[tid >> 6] = cnt;
  __syncthreads();

  const int n_pad = cnt_s[0] + cnt_s[1] + cnt_s[2] + cnt_s[3];
  const bool bad = bad_len || any_bad_par;
  if (tid == 0) {
    if (bad_len) raise_error(err, SPEC_DEV_CACHE_LEN);
    if (any_bad_par) raise_error(err, SPEC_DEV_PARENT);
    bad_ws[b] = bad ? 1 : 0;
  }
  if (tid < N) {
    // walk to the root: parents precede children, so this ends
    uint64_t anc = 0;
    int depth = -1;
    if (!bad) {
      for (int j = tid; j >= 0; j = par_s[j]) {
        anc |= 1ull << j;
        ++depth;
      }
    }
    anc_ws[(size_t)b * N + tid] = anc;
    if (pos_ids != nullptr) pos_ids[(size_t)b * N + tid] = bad ? -1 : (L - n_pad) + depth;
  }
}

hipError_t launch_verify_prep(const AttnArgs& a, const int32_t* parents, int64_t parents_sb,
                              int32_t* pos_ids, uint64_t* anc_ws, int32_t* bad_ws,
                              hipStream_t st) {
  hipLaunchKernelGGL(verify_prep_kernel, dim3(a.B), dim3(256), 0, st, a.T, a.capacity,
                     a.cache_len, a.pad, a.pad_sb, parents, parents_sb, pos_ids, anc_ws,
                     bad_ws, a.err);
  return hipGetLastError();
}

hipError_t launch_attn_f32(const AttnArgs& a, int mode, hipStream_t st) {
  const int64_t waves = (int64_t)a.B * a.Hkv * a.n_rb * a.splits;
  dim3 grid((unsigned)waves), block(64);
  if (mode == kDraftWindow) hipLaunchKernelGGL(attn_f32_kernel<kDraftWindow>, grid, block, 0, st, a);
  else if (mode == kDraftGather) hipLaunchKernelGGL(attn_f32_kernel<kDraftGather>, grid, block, 0, st, a);
  else hipLaunchKernelGGL(attn_f32_kernel<kVerify>, grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace spec
