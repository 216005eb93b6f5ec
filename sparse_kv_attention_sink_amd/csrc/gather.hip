// Partial KV cache gather (gfx950).
//
// Method: "SpecPV: Improving Self-Speculative Decoding for Long-Context
// Generation via Partial Verification", section 3.2 "Partial Verification":
// verification attends to a partial cache of a sink, retrieved blocks, a
// local window and a buffer, kept contiguous in token order and handled as
// one KV segment; section 3.3: a full verification refreshes it.
//
// The partial cache is built from one budget list per sequence: slot j of
// every KV head receives the K and V rows of the listed position; a -1 entry
// (or a bad one, which raises SPEC_DEV_INDEX) gives a padding slot with zero
// K/V.  One workgroup copies kGatherSlots slots of one sequence for every
// KV head: each thread moves 16-byte chunks, consecutive threads consecutive
// chunks of a row, so reads and writes are coalesced per row.  HBM-bound:
// budget x Hkv x 2 x D x esz bytes read and as many written.
#include "dev_common.h"

namespace spec {

namespace {

constexpr int kGatherSlots = 8;
constexpr int kGatherUnroll = 8;   // chunks a thread loads before it stores them

__global__ __launch_bounds__(256) void kv_gather_kernel(GatherArgs a) {
  const int b = blockIdx.y, tid = threadIdx.x;
  const int j0 = blockIdx.x * kGatherSlots;
  __shared__ int pos_s[kGatherSlots];
  const int L0 = a.cache_len[b];
  const bool bad_len = L0 < 0 || L0 > a.capacity;      // a bad length lists nothing
  const int L = bad_len ? 0 : L0;
  if (bad_len && blockIdx.x == 0 && tid == 0) raise_error(a.err, SPEC_DEV_CACHE_LEN);
  if (tid < kGatherSlots) {
    const int j = j0 + tid;
    int p = -1;
    if (j < a.budget) {
      p = a.idx[(int64_t)b * a.idx_sb + j];
      const bool ok = p >= 0 && p < L;
      if (!ok && p != -1 && !bad_len) raise_error(a.err, SPEC_DEV_INDEX);
      if (!ok) p = -1;
      a.partial_pad[(int64_t)b * a.pad_sb + j] = ok ? 0 : 1;
    }
    pos_s[tid] = p;
  }
  if (blockIdx.x == 0 && tid == 0) a.partial_len[b] = a.budget;
  __syncthreads();
  const int CH = a.row_chunks;
  const int per_slot = a.n_kv_heads * CH;              // chunks of one slot (K or V)
  const int n = min(kGatherSlots, a.budget - j0) * per_slot;
  // every thread loads its chunks of a round first, then stores them
  for (int w0 = 0; w0 < 2 * n; w0 += 256 * kGatherUnroll) {
    u32x4 val[kGatherUnroll];
    char* dst[kGatherUnroll];
#pragma unroll
    for (int u = 0; u < kGatherUnroll; ++u) {
      const int w = w0 + u * 256 + tid;
      val[u] = u32x4{0, 0, 0, 0};
      dst[u] = nullptr;
      if (w < 2 * n) {
        const int which = w >= n;                      // 0: K, 1: V
        const int r = which ? w - n : w;
        const int jj = r / per_slot, h = (r / CH) % a.n_kv_heads, ch = r % CH;
        const int p = pos_s[jj];
        if (p >= 0)
          val[u] = *reinterpret_cast<const u32x4*>((which ? a.v : a.k) + (int64_t)b * a.c_sb +
                                                   (int64_t)h * a.c_sh + (int64_t)p * a.c_st +
                                                   ch * 16);
        dst[u] = (which ? a.pv : a.pk) + (int64_t)b * a.p_sb + (int64_t)h * a.p_sh +
                 (int64_t)(j0 + jj) * a.p_st + ch * 16;
      }
    }
#pragma unroll
    for (int u = 0; u < kGatherUnroll; ++u)
      if (dst[u] != nullptr) *reinterpret_cast<u32x4*>(dst[u]) = val[u];
  }
}

}  // namespace

hipError_t launch_kv_gather(const GatherArgs& a, hipStream_t st) {
  const unsigned gx = (unsigned)((a.budget + kGatherSlots - 1) / kGatherSlots);
  hipLaunchKernelGGL(kv_gather_kernel, dim3(gx, (unsigned)a.batch), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace spec
