// Verify-phase tree attention, bf16 MFMA path (gfx950).
//
// Method: "SpecMemo: Speculative Decoding is in Your Pocket" (Pith review),
// "What carries the argument" and Figure 9: N speculated tree nodes are
// verified in one pass under a tree attention mask; batched verification
// pads accepted tokens to a uniform shape, remaps position IDs so padding is
// ignored and gives cached padding slots -inf.  Each node attends to every
// valid cache slot plus its ancestors and itself.
//
// Kernel shape: (tree nodes x GQA group) query rows against the keys of one
// KV head form a dense contraction, so both products run on bf16 MFMA
// (v_mfma_f32_16x16x32_bf16, fp32 accumulation):
//   S^T[key][row] = K[key][:] . Q[row][:]    (A = K from LDS, B = Q^T in VGPRs)
//   O^T[d][row]  += V^T[d][key] . P^T[key][row]
// Computing the transposed products leaves each lane owning one query row
// (lane % 16) in both the score and the output accumulators, so the online
// softmax state (max, sum, rescale) is lane-local and P goes from the score
// accumulator straight into the next MFMA operand without an LDS round trip.
// One wavefront per (sequence, KV head, row block, split) streams 32-key
// tiles: 16-byte coalesced global loads into registers, then K into a padded
// LDS tile and V transposed into a swizzled LDS tile (the V operand needs 8
// keys per lane at a fixed head-dim column); the next tile's loads are in
// flight while the current one is multiplied.
#include "dev_common.h"

namespace spec {

// ------------------------------------------------------------------ prep
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

// ------------------------------------------------------------------ tile staging

__device__ __forceinline__ uint32_t u4get(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Issue the global loads of one 32-key tile (K rows natural, V rows in groups
// of 4 keys x 8 head-dim elements per lane).  Addresses are a wave-uniform
// tile base plus per-lane 32-bit byte offsets; keys at or past `limit` (only
// in a split's last, partial tile) re-read the last valid row, and their
// scores are masked.
template <int D>
__device__ __forceinline__ void load_tile(uint4 (&kreg)[(32 * D / 8) / 64], uint4 (&vreg)[D / 8 / 8 * 4],
                                          const uint16_t* kp, const uint16_t* vp, int64_t st,
                                          int base, int limit, int lane) {
  constexpr int LPR = D / 8, RPI = 64 / LPR, NIK = 32 / RPI, NU = LPR / 8;
  const int row_in = lane / LPR, ch = lane % LPR;
  const uint32_t stb = (uint32_t)st * 2u;                 // row stride in bytes
  const char* kb = reinterpret_cast<const char*>(kp + (int64_t)base * st);
  const char* vb = reinterpret_cast<const char*>(vp + (int64_t)base * st);
  const uint32_t col = (uint32_t)ch * 16u;
  if (base + 32 <= limit) {
#pragma unroll
    for (int j = 0; j < NIK; ++j)
      kreg[j] = load_stream(kb + ((uint32_t)(j * RPI + row_in) * stb + col));
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int kg = lane / LPR + (64 / LPR) * u;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        vreg[u * 4 + r4] = load_stream(vb + ((uint32_t)(kg * 4 + r4) * stb + col));
    }
  } else {
    const int last = limit - 1 - base;
#pragma unroll
    for (int j = 0; j < NIK; ++j)
      kreg[j] = load_stream(kb + ((uint32_t)min(j * RPI + row_in, last) * stb + col));
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int kg = lane / LPR + (64 / LPR) * u;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        vreg[u * 4 + r4] = load_stream(vb + ((uint32_t)min(kg * 4 + r4, last) * stb + col));
    }
  }
}

// K rows go to a padded LDS tile; V goes transposed (head-dim major, 4-key
// groups swizzled by head-dim block) so that the P.V operand of a lane (8
// keys at one head-dim column) is two 8-byte LDS reads.
template <int D>
__device__ __forceinline__ void store_tile(uint8_t* k_lds, uint8_t* v_lds,
                                           const uint4 (&kreg)[(32 * D / 8) / 64],
                                           const uint4 (&vreg)[D / 8 / 8 * 4], int lane) {
  constexpr int LPR = D / 8, RPI = 64 / LPR, NIK = 32 / RPI, NU = LPR / 8;
  constexpr int KP = 2 * D + 16, VP = 72;
  const int row_in = lane / LPR, ch = lane % LPR;
#pragma unroll
  for (int j = 0; j < NIK; ++j)
    *reinterpret_cast<uint4*>(k_lds + (j * RPI + row_in) * KP + ch * 16) = kreg[j];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int kg = lane / LPR + (64 / LPR) * u;
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      // head-dim pair (2*e2, 2*e2+1) of keys kg*4 .. kg*4+3
      const uint32_t a0 = u4get(vreg[u * 4 + 0], e2), a1 = u4get(vreg[u * 4 + 1], e2);
      const uint32_t a2 = u4get(vreg[u * 4 + 2], e2), a3 = u4get(vreg[u * 4 + 3], e2);
      const uint2 lo = make_uint2(__builtin_amdgcn_perm(a1, a0, 0x05040100u),
                                  __builtin_amdgcn_perm(a3, a2, 0x05040100u));
      const uint2 hi = make_uint2(__builtin_amdgcn_perm(a1, a0, 0x07060302u),
                                  __builtin_amdgcn_perm(a3, a2, 0x07060302u));
      const int d0 = ch * 8 + 2 * e2, d1 = d0 + 1;
      *reinterpret_cast<uint2*>(v_lds + d0 * VP + ((kg ^ ((d0 >> 4) & 7)) * 8)) = lo;
      *reinterpret_cast<uint2*>(v_lds + d1 * VP + ((kg ^ ((d1 >> 4) & 7)) * 8)) = hi;
    }
  }
}

// ------------------------------------------------------------------ MFMA kernel

template <int D, int RT>
__global__ __launch_bounds__(64) void verify_mfma_kernel(AttnArgs a) {
  constexpr int ND = D / 32;            // 32-wide head-dim chunks (q.k MFMA steps)
  constexpr int NDT = D / 16;           // 16-wide head-dim tiles of the output
  constexpr int KP = 2 * D + 16;        // K tile row pitch (bytes), padded
  constexpr int VP = 72;                // V^T tile row pitch (bytes): 32 keys + 8
  constexpr int LPR = D / 8;            // lanes per key row in a 16-byte load
  constexpr int RPI = 64 / LPR;         // key rows per load instruction
  constexpr int NIK = 32 / RPI;         // K load instructions per tile
  constexpr int NU = LPR / 8;           // V units (4 keys x 8 dims) per lane
  (void)KP;
  __shared__ __attribute__((aligned(16))) uint8_t k_lds[32 * KP];
  __shared__ __attribute__((aligned(16))) uint8_t v_lds[D * VP];

  const int lane = threadIdx.x;
  const int l16 = lane & 15, q4 = lane >> 4;

  int w = blockIdx.x;
  const int s = w % a.splits;
  w /= a.splits;
  const int z = w % a.n_rb;
  const int pair = w / a.n_rb;
  const int b = pair / a.Hkv, g = pair % a.Hkv;
  const bool bad = a.bad[b] != 0;
  const int L = bad ? 0 : a.cache_len[b];
  const int N = a.T;

  // Query fragments (B operand of S^T) and ancestor masks, one row per lane.
  bf16x8 qf[RT][ND];
  uint64_t anc[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = z * a.rb + rt * 16 + l16;
    anc[rt] = 0;
#pragma unroll
    for (int c = 0; c < ND; ++c) qf[rt][c] = bf16x8{};
    if (row < a.R) {
      const int node = row / a.G, hh = row % a.G;
      anc[rt] = bad ? 0ull : a.anc[(size_t)b * N + node];
      const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) +
                           (((size_t)b * N + node) * a.Hq + g * a.G + hh) * D + q4 * 8;
#pragma unroll
      for (int c = 0; c < ND; ++c)
        qf[rt][c] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + c * 32));
    }
  }

  f32x4 acc[RT][NDT];
  float m[RT], lsum[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m[rt] = -INFINITY;
    lsum[rt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int c0 = s * a.chunk;
  const int c1 = min(L, c0 + a.chunk);
  const int n_cache_tiles = (!bad && c1 > c0) ? (c1 - c0 + 31) / 32 : 0;
  const int n_tree_tiles = (!bad && s == a.splits - 1) ? (N + 31) / 32 : 0;
  const int n_tiles = n_cache_tiles + n_tree_tiles;

  const uint16_t* kc = reinterpret_cast<const uint16_t*>(a.k) + b * a.kb + g * a.kh;
  const uint16_t* vc = reinterpret_cast<const uint16_t*>(a.v) + b * a.kb + g * a.kh;
  const uint16_t* tkp = reinterpret_cast<const uint16_t*>(a.tk) + b * a.tkb + g * a.tkh;
  const uint16_t* tvp = reinterpret_cast<const uint16_t*>(a.tv) + b * a.tkb + g * a.tkh;
  const uint8_t* padrow = a.pad ? a.pad + b * a.pad_sb : nullptr;

  uint4 kreg[NIK], vreg[NU * 4];

  if (n_tiles > 0) {
    const bool tree0 = n_cache_tiles == 0;
    load_tile<D>(kreg, vreg, tree0 ? tkp : kc, tree0 ? tvp : vc, tree0 ? a.tkt : a.kt,
                 tree0 ? 0 : c0, tree0 ? N : c1, lane);
  }

  for (int tile = 0; tile < n_tiles; ++tile) {
    const bool tree = tile >= n_cache_tiles;
    const int base = tree ? (tile - n_cache_tiles) * 32 : c0 + tile * 32;
    const int limit = tree ? N : c1;

    __syncthreads();   // previous tile's LDS reads are done
    store_tile<D>(k_lds, v_lds, kreg, vreg, lane);
    __syncthreads();
    if (tile + 1 < n_tiles) {
      const bool ntree = tile + 1 >= n_cache_tiles;
      const int nbase = ntree ? (tile + 1 - n_cache_tiles) * 32 : c0 + (tile + 1) * 32;
      load_tile<D>(kreg, vreg, ntree ? tkp : kc, ntree ? tvp : vc, ntree ? a.tkt : a.kt, nbase,
                   ntree ? N : c1, lane);
    }

    // Visibility of this lane's 8 keys: base + h*16 + q4*4 + i.
    uint32_t padw[2] = {0u, 0u};
    if (!tree && padrow != nullptr) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k0 = base + h * 16 + q4 * 4;
        if (k0 < limit) padw[h] = *reinterpret_cast<const uint32_t*>(padrow + k0);
      }
    }

#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      f32x4 sc[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x4 c = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int cc = 0; cc < ND; ++cc) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(k_lds + (h * 16 + l16) * KP + cc * 64 + q4 * 16);
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[rt][cc], c, 0, 0, 0);
        }
        sc[h] = c;
      }
      float t[8];
      float mloc = -INFINITY;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = base + h * 16 + q4 * 4 + i;
          bool vis = key < limit;
          if (tree) vis = vis && ((anc[rt] >> key) & 1ull);
          else vis = vis && (((padw[h] >> (8 * i)) & 0xffu) == 0u);
          const float x = vis ? sc[h][i] * a.scale_log2 : -INFINITY;
          t[h * 4 + i] = x;
          mloc = fmaxf(mloc, x);
        }
      }
      mloc = fmaxf(mloc, shfl_xor(mloc, 16));
      mloc = fmaxf(mloc, shfl_xor(mloc, 32));
      const float mn = fmaxf(m[rt], mloc);
      float p[8];
      if (mn == -INFINITY) {
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = 0.f;
      } else {
        const float alpha = __builtin_amdgcn_exp2f(m[rt] - mn);
        float ps = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = __builtin_amdgcn_exp2f(t[e] - mn);
          ps += p[e];
        }
        lsum[rt] = lsum[rt] * alpha + ps;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) acc[rt][dt] *= alpha;
        m[rt] = mn;
      }
      const uint4 pw = make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                                  pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7]));
      const bf16x8 pf = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int d = dt * 16 + l16;
        const uint8_t* vrow = v_lds + d * VP;
        const uint2 lo = *reinterpret_cast<const uint2*>(vrow + ((q4 ^ (dt & 7)) * 8));
        const uint2 hi = *reinterpret_cast<const uint2*>(vrow + (((4 + q4) ^ (dt & 7)) * 8));
        const bf16x8 vf = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
        acc[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, acc[rt][dt], 0, 0, 0);
      }
    }
  }

#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float lr = lsum[rt];
    lr += shfl_xor(lr, 16);
    lr += shfl_xor(lr, 32);
    const int i = rt * 16 + l16;
    if (z * a.rb + i >= a.R) continue;
    float lse2;
    float scale;
    if (bad) {
      scale = NAN;
      lse2 = NAN;
    } else if (lr > 0.f) {
      scale = 1.f / lr;
      lse2 = m[rt] + log2f(lr);
    } else {
      scale = 0.f;
      lse2 = -INFINITY;
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      float vals[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) vals[e] = bad ? NAN : acc[rt][dt][e] * scale;
      store_row_values<4>(a, SPEC_BF16, pair, z, s, i, dt * 16 + q4 * 4, vals);
    }
    if (q4 == 0) store_row_lse(a, pair, z, s, i, lse2);
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

hipError_t launch_verify_bf16(const AttnArgs& a, hipStream_t st) {
  const int64_t waves = (int64_t)a.B * a.Hkv * a.n_rb * a.splits;
  dim3 grid((unsigned)waves), block(64);
  if (a.D == 128) {
    if (a.rb == 16) hipLaunchKernelGGL((verify_mfma_kernel<128, 1>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((verify_mfma_kernel<128, 2>), grid, block, 0, st, a);
  } else {
    if (a.rb == 16) hipLaunchKernelGGL((verify_mfma_kernel<64, 1>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((verify_mfma_kernel<64, 2>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace spec
