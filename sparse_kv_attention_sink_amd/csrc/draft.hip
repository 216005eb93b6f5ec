// Draft-phase attention over a sparse view of the KV cache, bf16 path (gfx950).
//
// Method: "Windowed-MTP: Removing the Full-Context Draft-KV Tax at
// Million-Token Context" (Pith review), "What carries the argument": the draft
// reads only the first n_sink tokens plus the last W tokens of the cache;
// "BudgetDraft: Acceptance-Aware Multi-View Training for Sparse-KV Speculative
// Decoding" (Pith review), abstract: the drafter reads a sparse KV view under
// a fixed budget of positions.
//
// Kernel shape (one wavefront per (sequence, KV head, row block, split)):
// the draft is a handful of query rows (Tq * G, 4 to 16) against a few
// hundred to a few thousand keys, far below the MFMA ridge, so it runs on the
// vector ALUs.  Each key row (D bf16 = 16 lanes x 16 B) is loaded with fully
// coalesced 16-byte loads; a lane holds 8 head-dim elements of one key, forms
// partial q.k with packed bf16 dot products (v_dot2_f32_bf16) and a 16-lane
// DPP reduction completes the score.  Each group of lanes that shares a key
// slot keeps its own online-softmax state (m, l, o), merged across the
// wavefront once at the end, so the main loop has no cross-row shuffles.
#include "dev_common.h"

namespace spec {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_acc(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

// The union of the sink range and the window ranges of all Tq chained
// queries, as a contiguous "view position" sequence: positions [0, s_len) are
// the sink slots 0..s_len-1, positions [s_len, n) are slots w_start.. .
struct WindowView {
  int s_len, w_start, n;
};

__device__ __forceinline__ WindowView window_view(int L, int T, int n_sink, int W) {
  const int e_last = L, e_first = L - T + 1;
  const int s_len = min(n_sink, e_last);
  int w_start = max(max(n_sink, e_first - W), 0);
  w_start = min(w_start, e_last);
  return {s_len, w_start, s_len + (e_last - w_start)};
}

template <int D, int RB, bool GATHER>
__global__ __launch_bounds__(64) void draft_bf16_kernel(AttnArgs a) {
  constexpr int LPK = D / 8;          // lanes per key row
  constexpr int KPI = 64 / LPK;       // key rows per load instruction
  constexpr int NI = RB <= 8 ? 8 : 4; // load instructions per chunk
  constexpr int CH = KPI * NI;        // keys per chunk
  const int lane = threadIdx.x;
  const int dc = lane % LPK, ks = lane / LPK;

  int w = blockIdx.x;
  const int s = w % a.splits;
  w /= a.splits;
  const int z = w % a.n_rb;
  const int pair = w / a.n_rb;
  const int b = pair / a.Hkv, g = pair % a.Hkv;
  const int L = a.cache_len[b];
  const bool bad_len = L < a.T || L > a.capacity;

  // Query rows of this block: r = t*G + hh.
  uint4 qv[RB];
  int erow[RB];
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    const int r = z * RB + i;
    erow[i] = 0;
    qv[i] = make_uint4(0, 0, 0, 0);
    if (r < a.R) {
      const int t = r / a.G, hh = r % a.G;
      erow[i] = L - a.T + t + 1;
      const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) +
                           (((size_t)b * a.T + t) * a.Hq + g * a.G + hh) * D + dc * 8;
      qv[i] = *reinterpret_cast<const uint4*>(qp);
    }
  }

  float m[RB], l[RB], o[RB][8];
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[i][e] = 0.f;
  }

  bool idx_bad = false;
  if (!bad_len) {
    WindowView wv{0, 0, 0};
    int n_view;
    if constexpr (GATHER) {
      n_view = a.budget;
    } else {
      wv = window_view(L, a.T, a.n_sink, a.window);
      n_view = wv.n;
    }
    const int p0 = s * a.chunk;
    const int p1 = min(n_view, p0 + a.chunk);
    const uint16_t* kbase = reinterpret_cast<const uint16_t*>(a.k) + b * a.kb + g * a.kh + dc * 8;
    const uint16_t* vbase = reinterpret_cast<const uint16_t*>(a.v) + b * a.kb + g * a.kh + dc * 8;
    const int32_t* ibase = GATHER ? a.idx + b * a.idx_sb + g * a.idx_sh : nullptr;

    for (int p = p0; p < p1; p += CH) {
      uint4 kr[NI], vr[NI];
      int slot[NI];
      bool valid[NI];
#pragma unroll
      for (int n = 0; n < NI; ++n) {
        const int pos = p + n * KPI + ks;
        valid[n] = pos < p1;
        int j;
        if constexpr (GATHER) {
          j = valid[n] ? ibase[pos] : 0;
          if (valid[n] && (j < 0 || j >= L)) {
            idx_bad = true;
            valid[n] = false;
          }
        } else {
          j = pos < wv.s_len ? pos : wv.w_start + (pos - wv.s_len);
        }
        if (!valid[n]) j = 0;
        slot[n] = j;
        kr[n] = *reinterpret_cast<const uint4*>(kbase + (int64_t)j * a.kt);
        vr[n] = *reinterpret_cast<const uint4*>(vbase + (int64_t)j * a.kt);
      }
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        float sc[NI];
        float cm = -INFINITY;
#pragma unroll
        for (int n = 0; n < NI; ++n) {
          float acc = 0.f;
          acc = dot2_acc(kr[n].x, qv[i].x, acc);
          acc = dot2_acc(kr[n].y, qv[i].y, acc);
          acc = dot2_acc(kr[n].z, qv[i].z, acc);
          acc = dot2_acc(kr[n].w, qv[i].w, acc);
          acc = group_sum<LPK>(acc) * a.scale_log2;
          const int j = slot[n], e = erow[i];
          bool vis = valid[n] && j < e;
          if constexpr (!GATHER) vis = vis && (j < a.n_sink || j >= e - a.window);
          sc[n] = vis ? acc : -INFINITY;
          cm = fmaxf(cm, sc[n]);
        }
        const float mn = fmaxf(m[i], cm);
        if (mn == -INFINITY) continue;
        const float alpha = exp2f(m[i] - mn);
        l[i] *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[i][e] *= alpha;
#pragma unroll
        for (int n = 0; n < NI; ++n) {
          const float pr = exp2f(sc[n] - mn);
          l[i] += pr;
          o[i][0] += pr * bf16lo(vr[n].x);
          o[i][1] += pr * bf16hi(vr[n].x);
          o[i][2] += pr * bf16lo(vr[n].y);
          o[i][3] += pr * bf16hi(vr[n].y);
          o[i][4] += pr * bf16lo(vr[n].z);
          o[i][5] += pr * bf16hi(vr[n].z);
          o[i][6] += pr * bf16lo(vr[n].w);
          o[i][7] += pr * bf16hi(vr[n].w);
        }
        m[i] = mn;
      }
    }
  }

  const bool poison = bad_len || __any(idx_bad);
  if (lane == 0) {
    if (bad_len) raise_error(a.err, SPEC_DEV_CACHE_LEN);
    if (!bad_len && poison) raise_error(a.err, SPEC_DEV_INDEX);
  }

  // Merge the KPI key-slot groups, then store.
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    float M = m[i];
#pragma unroll
    for (int msk = LPK; msk < 64; msk <<= 1) M = fmaxf(M, shfl_xor(M, msk));
    const float sc = (m[i] == -INFINITY) ? 0.f : exp2f(m[i] - M);
    float li = l[i] * sc;
    float oi[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) oi[e] = o[i][e] * sc;
#pragma unroll
    for (int msk = LPK; msk < 64; msk <<= 1) {
      li += shfl_xor(li, msk);
#pragma unroll
      for (int e = 0; e < 8; ++e) oi[e] += shfl_xor(oi[e], msk);
    }
    const int r = z * RB + i;
    if (r >= a.R || ks != 0) continue;
    float lse2;
    if (poison) {
#pragma unroll
      for (int e = 0; e < 8; ++e) oi[e] = NAN;
      lse2 = NAN;
    } else if (li > 0.f) {
      const float inv = 1.f / li;
#pragma unroll
      for (int e = 0; e < 8; ++e) oi[e] *= inv;
      lse2 = M + log2f(li);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) oi[e] = 0.f;
      lse2 = -INFINITY;
    }
    store_row_values<8>(a, SPEC_BF16, pair, z, s, i, dc * 8, oi);
    if (dc == 0) store_row_lse(a, pair, z, s, i, lse2);
  }
}

template <int D, bool GATHER>
static hipError_t launch_draft_rb(const AttnArgs& a, hipStream_t st) {
  const int64_t waves = (int64_t)a.B * a.Hkv * a.n_rb * a.splits;
  dim3 grid((unsigned)waves), block(64);
  switch (a.rb) {
    case 4: hipLaunchKernelGGL((draft_bf16_kernel<D, 4, GATHER>), grid, block, 0, st, a); break;
    case 8: hipLaunchKernelGGL((draft_bf16_kernel<D, 8, GATHER>), grid, block, 0, st, a); break;
    case 12: hipLaunchKernelGGL((draft_bf16_kernel<D, 12, GATHER>), grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL((draft_bf16_kernel<D, 16, GATHER>), grid, block, 0, st, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_draft_bf16(const AttnArgs& a, hipStream_t st) {
  const bool gather = a.idx != nullptr;
  if (a.D == 128) return gather ? launch_draft_rb<128, true>(a, st) : launch_draft_rb<128, false>(a, st);
  return gather ? launch_draft_rb<64, true>(a, st) : launch_draft_rb<64, false>(a, st);
}

}  // namespace spec
