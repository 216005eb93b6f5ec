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

// ------------------------------------------------------------ compaction
//
// Dropping the pad slots that batched commits leave behind (SpecMemo review,
// Figure 9; SpecPV section 3.3): the valid slots below cache_len keep their
// order and move to the front, cache_len becomes their count and the pad
// bytes below the old cache_len are cleared.
//
// kv_compact_scan_kernel (capacities above kCompactScanSlots only):
// kCompactSlices workgroups per sequence, each scanning one slice of the pad
// bytes below cache_len with 16-byte loads for the slice's first pad slot
// and pad count.  A shorter pad row is scanned by the move kernel itself,
// which saves a launch.
// kv_compact_move_kernel: one workgroup per (sequence, KV head), in place.
// It finds the sequence's first pad slot f and pad count (from the slices'
// summaries, or by its own scan); slots below f stay where they are.  From f
// on, chunks of 256 slots are handled in increasing order: a block prefix
// sum of the chunk's pad bytes gives each valid slot j its destination
// d(j) = j - (pads before j) <= j.  The rows of a chunk move in passes of
// 64 to 256 rows (kCompactItems 16-byte pieces per thread), each loading all
// its rows before storing any.  A store
// lands at d(j) <= j, below every row a later pass or chunk reads, and on a
// row of its own pass only after that pass's loads have completed; distinct
// valid slots have distinct destinations.  So no row is overwritten before
// it has been read.
// kv_compact_finish_kernel: one workgroup per sequence, after the moves:
// cache_len and the pad bytes.

constexpr int kCompactChunk = 256;   // slots per prefix-sum chunk (one per thread)
constexpr int kCompactItems = 8;     // 16-byte pieces each thread moves per pass

__device__ __forceinline__ int nonzero_bytes(uint32_t w) {
  return __popc(((w & 0x7f7f7f7fu) + 0x7f7f7f7fu | w) & 0x80808080u);
}
__device__ __forceinline__ int first_nonzero_byte(uint32_t w) {   // 4 if none
  const uint32_t m = ((w & 0x7f7f7f7fu) + 0x7f7f7f7fu | w) & 0x80808080u;
  return m ? (__ffs(m) - 1) >> 3 : 4;
}

// First pad slot (INT_MAX if none) and pad count of pad bytes [lo, hi) of
// `prow`, reduced over the workgroup; every thread gets the result.
__device__ void scan_pads(const uint8_t* prow, int lo, int hi, int& first_out, int& cnt_out) {
  __shared__ int s_first[4], s_cnt[4];
  const int tid = threadIdx.x;
  int first = INT_MAX, cnt = 0;
  const int n = max(hi - lo, 0);
  const uint8_t* p = prow + lo;
  const int head = min(n, (int)((16 - (reinterpret_cast<uintptr_t>(p) & 15)) & 15));
  if (tid < head && p[tid]) {
    first = lo + tid;
    cnt = 1;
  }
  const int nvec = (n - head) / 16;
  const uint4* pv = reinterpret_cast<const uint4*>(p + head);
  for (int i0 = 0; i0 < nvec; i0 += 256 * 8) {
    uint4 w[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * 256 + tid;
      w[u] = i < nvec ? pv[i] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int base = lo + head + 16 * (i0 + u * 256 + tid);
      const uint32_t q[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        cnt += nonzero_bytes(q[e]);
        const int f = first_nonzero_byte(q[e]);
        if (f < 4) first = min(first, base + 4 * e + f);
      }
    }
  }
  for (int j = head + 16 * nvec + tid; j < n; j += 256)
    if (p[j]) {
      first = min(first, lo + j);
      ++cnt;
    }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    first = min(first, __shfl_xor(first, m, 64));
    cnt += __shfl_xor(cnt, m, 64);
  }
  if ((tid & 63) == 0) {
    s_first[tid >> 6] = first;
    s_cnt[tid >> 6] = cnt;
  }
  __syncthreads();
  first_out = min(min(s_first[0], s_first[1]), min(s_first[2], s_first[3]));
  cnt_out = s_cnt[0] + s_cnt[1] + s_cnt[2] + s_cnt[3];
}

// The sequence's first pad slot (INT_MAX if none) and pad count from its
// slices' summaries; every thread gets the result.
__device__ void combine_slices(const int32_t* sum_b, int& first_out, int& cnt_out) {
  __shared__ int s_first, s_cnt;
  const int tid = threadIdx.x;
  if (tid < 64) {
    int first = tid < kCompactSlices ? sum_b[2 * tid] : INT_MAX;
    int cnt = tid < kCompactSlices ? sum_b[2 * tid + 1] : 0;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      first = min(first, __shfl_xor(first, m, 64));
      cnt += __shfl_xor(cnt, m, 64);
    }
    if (tid == 0) {
      s_first = first;
      s_cnt = cnt;
    }
  }
  __syncthreads();
  first_out = s_first;
  cnt_out = s_cnt;
}

__global__ __launch_bounds__(256) void kv_compact_scan_kernel(CompactArgs a) {
  const int b = blockIdx.x / kCompactSlices, sl = blockIdx.x % kCompactSlices;
  const int L = a.cache_len[b];
  if (L < 0 || L > a.capacity) return;   // (the move kernel reports it)
  const int per = (L + kCompactSlices - 1) / kCompactSlices;
  const int lo = min(L, sl * per), hi = min(L, lo + per);
  int first, cnt;
  scan_pads(a.pad + (int64_t)b * a.pad_sb, lo, hi, first, cnt);
  if (threadIdx.x == 0) {
    a.summary[(b * kCompactSlices + sl) * 2] = first;
    a.summary[(b * kCompactSlices + sl) * 2 + 1] = cnt;
  }
}

__global__ __launch_bounds__(256) void kv_compact_move_kernel(CompactArgs a) {
  const int b = blockIdx.x / a.n_kv_heads, h = blockIdx.x % a.n_kv_heads;
  const int tid = threadIdx.x;
  __shared__ int dest_s[kCompactChunk];
  __shared__ int scan_s[kCompactChunk];
  const int L = a.cache_len[b];
  if (L < 0 || L > a.capacity) {
    if (h == 0 && tid == 0) raise_error(a.err, SPEC_DEV_CACHE_LEN);
    return;
  }
  const uint8_t* prow = a.pad + (int64_t)b * a.pad_sb;
  int32_t* const sum_b = a.summary + (int64_t)b * kCompactSlices * 2;
  int first, cnt;
  if (a.sliced) {
    combine_slices(sum_b, first, cnt);
  } else {
    scan_pads(prow, 0, L, first, cnt);
    // the finish kernel reads slice summaries: the whole row as slice 0
    if (h == 0 && tid < kCompactSlices) {
      sum_b[2 * tid] = tid == 0 ? first : INT_MAX;
      sum_b[2 * tid + 1] = tid == 0 ? cnt : 0;
    }
  }
  if (first == INT_MAX) return;   // no pad: nothing moves

  // ---- moves, chunk by chunk from the first pad
  const int rc = a.row_chunks;
  const int rows_per_pass = 256 * kCompactItems / rc;   // rc divides 256 * kCompactItems
  char* const base_k = a.k + (int64_t)b * a.c_sb + (int64_t)h * a.c_sh;
  char* const base_v = a.v + (int64_t)b * a.c_sb + (int64_t)h * a.c_sh;
  int before = 0;   // pads in [first, c0)
  for (int c0 = first; c0 < L; c0 += kCompactChunk) {
    const int j = c0 + tid;
    const int flag = j < L ? (prow[j] != 0) : 1;
    // inclusive block scan of the flags (Hillis-Steele in LDS)
    scan_s[tid] = flag;
    __syncthreads();
    for (int o = 1; o < kCompactChunk; o <<= 1) {
      const int add = tid >= o ? scan_s[tid - o] : 0;
      __syncthreads();
      scan_s[tid] += add;
      __syncthreads();
    }
    const int excl = scan_s[tid] - flag;
    dest_s[tid] = flag ? -1 : j - (before + excl);
    const int total = scan_s[kCompactChunk - 1];
    __syncthreads();
    before += total;
    for (int tsr = 0; tsr < 2; ++tsr) {
      char* const base = tsr ? base_v : base_k;
      for (int r0 = 0; r0 < kCompactChunk; r0 += rows_per_pass) {
        uint4 val[kCompactItems];
        int dst[kCompactItems];
#pragma unroll
        for (int u = 0; u < kCompactItems; ++u) {
          const int it = u * 256 + tid;
          const int r = r0 + it / rc, ch = it % rc;
          const int d = r < kCompactChunk ? dest_s[r] : -1;
          dst[u] = d == c0 + r ? -1 : d;   // destination slot of a row that moves, else -1
          if (dst[u] >= 0)
            val[u] = *reinterpret_cast<const uint4*>(base + (int64_t)(c0 + r) * a.c_st + ch * 16);
        }
        wait_vm<0>();
        __syncthreads();   // every load of this pass has returned
#pragma unroll
        for (int u = 0; u < kCompactItems; ++u) {
          if (dst[u] < 0) continue;
          const int ch = (u * 256 + tid) % rc;
          *reinterpret_cast<uint4*>(base + (int64_t)dst[u] * a.c_st + ch * 16) = val[u];
        }
      }
    }
    __syncthreads();   // dest_s and scan_s are rewritten by the next chunk
  }
}

__global__ __launch_bounds__(256) void kv_compact_finish_kernel(CompactArgs a) {
  const int b = blockIdx.x, tid = threadIdx.x;
  const int L = a.cache_len[b];
  if (L < 0 || L > a.capacity) return;
  int first, cnt;
  combine_slices(a.summary + (int64_t)b * kCompactSlices * 2, first, cnt);
  uint8_t* prow = a.pad + (int64_t)b * a.pad_sb;
  for (int j = first == INT_MAX ? L : first + tid; j < L; j += 256) prow[j] = 0;
  __syncthreads();   // every thread has read cache_len[b]
  if (tid == 0) a.cache_len[b] = L - cnt;
}

}  // namespace

hipError_t launch_kv_commit(const CommitArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(kv_commit_kernel, dim3((unsigned)a.batch), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_kv_compact(const CompactArgs& a, hipStream_t st) {
  if (a.sliced) {
    hipLaunchKernelGGL(kv_compact_scan_kernel, dim3((unsigned)(a.batch * kCompactSlices)), dim3(256), 0, st, a);
    hipError_t e0 = hipGetLastError();
    if (e0 != hipSuccess) return e0;
  }
  hipLaunchKernelGGL(kv_compact_move_kernel, dim3((unsigned)(a.batch * a.n_kv_heads)), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kv_compact_finish_kernel, dim3((unsigned)a.batch), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace spec
