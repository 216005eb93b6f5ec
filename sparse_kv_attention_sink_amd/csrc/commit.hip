// KV commit of the accepted path (gfx950).
//
// Method: "SpecMemo: Speculative Decoding is in Your Pocket" (Pith review),
// "What carries the argument" and Figure 9: batched verification keeps each
// sequence's accepted tokens and pads the batch to one uniform shape, the pad
// slots being scored -inf afterwards; "SpecPV: Improving Self-Speculative
// Decoding for Long-Context Generation via Partial Verification", section
// 3.3: candidates that were not accepted leave the cache once verification is
// done.
//
// One workgroup per sequence.  Every workgroup first derives the batch's
// append count P = 1 + max accepted length (over sequences whose acceptance
// result is valid), so no second launch or cross-workgroup wait is needed.
// The copy is column-parallel: a thread owns one 16-byte column (K or V,
// KV head, head-dim chunk) and moves the accepted rows into it in path
// order, up to 8 rows loaded before any is stored.  The tree rows may alias
// the cache slots at or after cache_len: node n of a path sits at depth
// <= n, so path[j] >= j, and a store to slot cache_len + j never hits a row
// that a later group still has to read.
#include "dev_common.h"

namespace spec {

namespace {

constexpr int kCommitGroup = 8;   // rows loaded before they are stored

// Accept length of sequence bb if its acceptance result is valid, else -1;
// the path entries are loaded in groups (independent loads in flight
// together) and, when `keep` is set, staged in `path_out`.
__device__ __forceinline__ int commit_tau(const CommitArgs& a, int bb, bool keep, int* path_out) {
  const int tau = a.accept_len[bb];
  bool ok = tau >= 0 && tau <= a.max_depth && tau <= a.n_nodes;
  const int cnt = ok ? tau : 0;
  const int32_t* p = a.accept_path + (int64_t)bb * a.max_depth;
  for (int j0 = 0; j0 < cnt; j0 += kCommitGroup) {
    int n[kCommitGroup];
#pragma unroll
    for (int i = 0; i < kCommitGroup; ++i) n[i] = j0 + i < cnt ? p[j0 + i] : 0;
#pragma unroll
    for (int i = 0; i < kCommitGroup; ++i) {
      ok = ok && n[i] >= 0 && n[i] < a.n_nodes;
      if (keep && j0 + i < cnt) path_out[j0 + i] = n[i];
    }
  }
  return ok ? tau : -1;
}

__global__ __launch_bounds__(256) void kv_commit_kernel(CommitArgs a) {
  const int b = blockIdx.x, tid = threadIdx.x;
  __shared__ int s_max[4];
  __shared__ int s_tau;
  __shared__ int s_path[kMaxNodes];
  const int L = a.cache_len[b];   // in flight while P is found

  // P over the whole batch (each workgroup computes the same value); the
  // thread that checks this workgroup's own sequence stages its path
  int m = 0;
  for (int bb = tid; bb < a.batch; bb += 256) {
    const int t = commit_tau(a, bb, bb == b, s_path);
    m = max(m, t);
    if (bb == b) s_tau = t;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = max(m, __shfl_xor(m, o, 64));
  if ((tid & 63) == 0) s_max[tid >> 6] = m;
  __syncthreads();
  const int P = 1 + max(max(s_max[0], s_max[1]), max(s_max[2], s_max[3]));
  const int tau = s_tau;
  const bool fits = L >= 0 && L <= a.capacity - P;
  if (tid == 0) {
    if (tau < 0) raise_error(a.err, SPEC_DEV_COMMIT);
    if (!fits) raise_error(a.err, SPEC_DEV_CACHE_LEN);
    if (b == 0 && a.n_appended != nullptr) *a.n_appended = P;
  }
  if (!fits) return;

  const int per_head = a.row_chunks;
  const int cols = 2 * a.n_kv_heads * per_head;
  for (int c = tid; c < cols; c += 256) {
    const int which = c / (a.n_kv_heads * per_head);
    const int h = (c / per_head) % a.n_kv_heads, ch = c % per_head;
    char* dst = (which ? a.v : a.k) + (int64_t)b * a.c_sb + (int64_t)h * a.c_sh + ch * 16;
    const char* src = (which ? a.tv : a.tk) + (int64_t)b * a.t_sb + (int64_t)h * a.t_sh + ch * 16;
    for (int j0 = 0; j0 < tau; j0 += kCommitGroup) {
      uint4 r[kCommitGroup];
#pragma unroll
      for (int i = 0; i < kCommitGroup; ++i)
        if (j0 + i < tau) r[i] = *reinterpret_cast<const uint4*>(src + (int64_t)s_path[j0 + i] * a.t_st);
#pragma unroll
      for (int i = 0; i < kCommitGroup; ++i)
        if (j0 + i < tau) *reinterpret_cast<uint4*>(dst + (int64_t)(L + j0 + i) * a.c_st) = r[i];
    }
  }
  // accepted slots and the bonus slot are valid, the rest of the P are pads
  for (int j = tid; j < P; j += 256) a.pad[(int64_t)b * a.pad_sb + L + j] = j <= tau ? 0 : 1;
  __syncthreads();   // every thread has read cache_len[b]
  if (tid == 0) a.cache_len[b] = L + P;
}

}  // namespace

hipError_t launch_kv_commit(const CommitArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(kv_commit_kernel, dim3((unsigned)a.batch), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace spec
