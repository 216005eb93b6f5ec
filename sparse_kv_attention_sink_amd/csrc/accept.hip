// Greedy tree acceptance (gfx950).
//
// Method: "BudgetDraft: Acceptance-Aware Multi-View Training for Sparse-KV
// Speculative Decoding" (Pith review), Figure 2: the full-cache verifier
// produces greedy targets; "Windowed-MTP: Removing the Full-Context Draft-KV
// Tax at Million-Token Context" (Pith review), losslessness: the target
// decides every accepted token; "SpecPV: Improving Self-Speculative Decoding
// for Long-Context Generation via Partial Verification", section 4.1
// "Metrics": the accept length may be 0.
//
// One kernel.  Each block scans a contiguous slice of one logits row with
// 16-byte loads and reduces (value, index) pairs under the rule "larger value
// wins, NaN beats every number, ties go to the smaller index"; the slice's
// winner lands in the workspace.  The block that finishes a row's slices last
// (arrival counter per row) merges them into the row's argmax, and the block
// that finishes a sequence's rows last (arrival counter per sequence) walks
// the tree in node order (parents precede children).  Two levels keep the
// arrivals on one counter few (a sequence of 4 rows in 31 slices each had
// 124 on one address); where the counter region cannot hold a counter per
// row, the per-sequence counter takes every slice's arrival and the walk
// merges the slices.
#include "dev_common.h"

namespace spec {

struct ArgBest {
  float v;
  int i;
};

// true iff (v1, i1) should win over (v2, i2)
__device__ __forceinline__ bool arg_better(float v1, int i1, float v2, int i2) {
  const bool n1 = isnan(v1), n2 = isnan(v2);
  if (n1 || n2) return n1 && (!n2 || i1 < i2);
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

__device__ __forceinline__ void arg_consider(float& bv, int& bi, float v, int i) {
  if (arg_better(v, i, bv, bi)) {
    bv = v;
    bi = i;
  }
}

// Within one thread indices only increase, so a strict ">" keeps the first
// maximum and a NaN, once held, is never replaced; the first element is
// always taken (a row of -inf still has an argmax).  The full rule (with
// index tie-breaks) is only needed when merging across threads.
__device__ __forceinline__ void scan_one(float& bv, int& bi, float v, int i) {
  const bool take = v > bv || (isnan(v) && !isnan(bv)) || bi == INT_MAX;
  bv = take ? v : bv;
  bi = take ? i : bi;
}

// Argmax of one logits slice (all 256 threads); returns the winner in thread 0.
__device__ ArgBest slice_argmax(const float* __restrict__ x, int64_t v0, int64_t v1) {
  const int tid = threadIdx.x;
  float bv = -INFINITY;
  int bi = INT_MAX;
  // unaligned head, 16-byte body (8 loads in flight per thread), tail
  int64_t a0 = v0;
  const int64_t mis = (reinterpret_cast<uintptr_t>(x + v0) >> 2) & 3;
  if (mis) a0 = min(v1, v0 + (4 - mis));
  for (int64_t v = v0 + tid; v < a0; v += 256) arg_consider(bv, bi, x[v], (int)v);
  const int64_t nvec = (v1 - a0) / 4;
  const float4* xv = reinterpret_cast<const float4*>(x + a0);
  // thread-local results are merged with arg_consider, so each thread may scan
  // its own index sequence in increasing order
  float tv = -INFINITY;
  int ti = INT_MAX;
  int64_t k = tid;
  constexpr int U = 8;
  for (; k + (U - 1) * 256 < nvec; k += U * 256) {
    float4 f[U];
#pragma unroll
    for (int u = 0; u < U; ++u) f[u] = load_stream_f4(xv + k + u * 256);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int base = (int)(a0 + 4 * (k + u * 256));
      scan_one(tv, ti, f[u].x, base);
      scan_one(tv, ti, f[u].y, base + 1);
      scan_one(tv, ti, f[u].z, base + 2);
      scan_one(tv, ti, f[u].w, base + 3);
    }
  }
  for (; k < nvec; k += 256) {
    const float4 f = xv[k];
    const int base = (int)(a0 + 4 * k);
    scan_one(tv, ti, f.x, base);
    scan_one(tv, ti, f.y, base + 1);
    scan_one(tv, ti, f.z, base + 2);
    scan_one(tv, ti, f.w, base + 3);
  }
  if (ti != INT_MAX) arg_consider(bv, bi, tv, ti);
  for (int64_t v = a0 + 4 * nvec + tid; v < v1; v += 256) arg_consider(bv, bi, x[v], (int)v);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float ov = __shfl_xor(bv, m, 64);
    const int oi = __shfl_xor(bi, m, 64);
    arg_consider(bv, bi, ov, oi);
  }
  __shared__ float sv[4];
  __shared__ int si[4];
  if ((tid & 63) == 0) {
    sv[tid >> 6] = bv;
    si[tid >> 6] = bi;
  }
  __syncthreads();
  if (tid == 0)
    for (int w = 1; w < 4; ++w) arg_consider(bv, bi, sv[w], si[w]);
  return ArgBest{bv, bi};
}

// Acceptance of sequence b from the per-slice winners: greedy target of every
// row, accepted(i) = every node on i's root path carries its parent's target
// (ancestor masks by walking parents), result = deepest accepted node, ties
// to the smallest index.  Runs in one block; nodes live in the first wave.
__device__ void accept_walk(int b, int N, int vsplits, __amdgpu_buffer_rsrc_t prs,
                            const int32_t* __restrict__ tokens, const int32_t* __restrict__ parents,
                            int64_t par_sb, int max_depth, int32_t* accept_len,
                            int32_t* accept_path, int32_t* bonus, uint32_t* err) {
  const int tid = threadIdx.x;
  __shared__ int am[kMaxNodes + 1];
  __shared__ int par_s[kMaxNodes];
  __shared__ int on_path[kMaxNodes];
  if (tid <= N) {
    const uint32_t p0 = (uint32_t)(((int64_t)b * (N + 1) + tid) * vsplits * sizeof(ArgBest));
    float bv = load_sc1_f1(prs, p0);
    int bi = __float_as_int(load_sc1_f1(prs, p0 + 4));
    for (int s = 1; s < vsplits; ++s)
      arg_consider(bv, bi, load_sc1_f1(prs, p0 + s * 8), __float_as_int(load_sc1_f1(prs, p0 + s * 8 + 4)));
    am[tid] = bi;
  }
  bool bad = false;
  int pr = -1, tok = 0;
  if (tid < N) {
    pr = parents[b * par_sb + tid];
    tok = tokens[(int64_t)b * N + tid];
    par_s[tid] = pr;
    bad = !(pr >= -1 && pr < tid);
  }
  const bool any_bad = __syncthreads_or(bad);
  int32_t* path = accept_path + (int64_t)b * max_depth;
  if (any_bad) {
    if (tid == 0) {
      raise_error(err, SPEC_DEV_PARENT);
      accept_len[b] = -1;
      bonus[b] = -1;
    }
    for (int k = tid; k < max_depth; k += 256) path[k] = -1;
    return;
  }
  int best = -1, len = 0;
  uint64_t anc = 0;
  int depth = -1;
  if (tid < 64) {   // N <= 64: every node is a lane of the first wavefront
    const bool match = tid < N && tok == am[pr + 1];
    const uint64_t match_mask = __ballot(match);
    if (tid < N)
      for (int j = tid; j >= 0; j = par_s[j]) {
        anc |= 1ull << j;
        ++depth;
      }
    const bool acc = tid < N && (anc & ~match_mask) == 0;
    int key = acc ? (depth << 8) | (255 - tid) : -1;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) key = max(key, __shfl_xor(key, m, 64));
    best = key < 0 ? -1 : 255 - (key & 255);
    len = key < 0 ? 0 : (key >> 8) + 1;
    const uint64_t best_anc = best < 0 ? 0ull : __shfl(anc, best, 64);
    if (tid < N && ((best_anc >> tid) & 1ull)) on_path[depth] = tid;
  }
  __syncthreads();
  if (tid < 64) {
    for (int k = tid; k < max_depth; k += 64) path[k] = k < len ? on_path[k] : -1;
    if (tid == 0) {
      if (len > max_depth) raise_error(err, SPEC_DEV_DEPTH);
      accept_len[b] = len;
      bonus[b] = am[best + 1];
    }
  }
}

// part: [rows][vsplits] slice winners, then [rows] row winners (two
// levels); counters: [B] per sequence, then [rows] per row (two levels).
__global__ __launch_bounds__(256) void accept_kernel(
    const float* __restrict__ logits, int64_t V, int N, int vsplits, int64_t vchunk, int two_level,
    ArgBest* __restrict__ part, uint32_t* counters, const int32_t* __restrict__ tokens,
    const int32_t* __restrict__ parents, int64_t par_sb, int max_depth, int32_t* accept_len,
    int32_t* accept_path, int32_t* bonus, uint32_t* err) {
  const int row = blockIdx.x / vsplits, sp = blockIdx.x % vsplits;
  const int rows = (int)(gridDim.x / vsplits), B = rows / (N + 1);
  const int b = row / (N + 1);
  const int64_t v0 = (int64_t)sp * vchunk;
  const int64_t v1 = min(V, v0 + vchunk);
  const ArgBest best = slice_argmax(logits + (int64_t)row * V, v0, v1);
  const __amdgpu_buffer_rsrc_t prs = coherent_rsrc(part, (uint32_t)(gridDim.x * sizeof(ArgBest)));
  const __amdgpu_buffer_rsrc_t rrs = coherent_rsrc(part + gridDim.x, (uint32_t)(rows * sizeof(ArgBest)));
  auto store_best = [&](__amdgpu_buffer_rsrc_t rs, int i, float v, int idx) __attribute__((always_inline)) {
    store_sc1_f1(rs, (uint32_t)(i * sizeof(ArgBest)), v);
    store_sc1_f1(rs, (uint32_t)(i * sizeof(ArgBest) + 4), __int_as_float(idx));
  };
  if (!two_level) {
    if (threadIdx.x == 0) store_best(prs, blockIdx.x, best.v, best.i);
    if (!arrive_last(counters + b, (N + 1) * vsplits)) return;
    accept_walk(b, N, vsplits, prs, tokens, parents, par_sb, max_depth, accept_len, accept_path,
                bonus, err);
    return;
  }
  if (vsplits == 1) {
    if (threadIdx.x == 0) store_best(rrs, row, best.v, best.i);
  } else {
    if (threadIdx.x == 0) store_best(prs, blockIdx.x, best.v, best.i);
    if (!arrive_last(counters + B + row, vsplits)) return;
    if (threadIdx.x < 64) {   // the row's slices (at most 64), one per lane
      float bv = -INFINITY;
      int bi = INT_MAX;
      if ((int)threadIdx.x < vsplits) {
        const uint32_t o = (uint32_t)((row * vsplits + threadIdx.x) * sizeof(ArgBest));
        bv = load_sc1_f1(prs, o);
        bi = __float_as_int(load_sc1_f1(prs, o + 4));
      }
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        const float ov = __shfl_xor(bv, m, 64);
        const int oi = __shfl_xor(bi, m, 64);
        arg_consider(bv, bi, ov, oi);
      }
      if (threadIdx.x == 0) store_best(rrs, row, bv, bi);
    }
  }
  if (!arrive_last(counters + b, N + 1)) return;
  accept_walk(b, N, 1, rrs, tokens, parents, par_sb, max_depth, accept_len, accept_path, bonus,
              err);
}

size_t accept_part_offset(int) { return kScratchOff; }

hipError_t launch_accept(int B, int N, int V, const float* logits, const int32_t* tokens,
                         const int32_t* parents, int64_t parents_sb, int max_depth,
                         int32_t* accept_len, int32_t* accept_path, int32_t* bonus, void* ws,
                         int vsplits, int two_level, hipStream_t st, uint32_t* err) {
  uint8_t* w = reinterpret_cast<uint8_t*>(ws);
  uint32_t* counters = reinterpret_cast<uint32_t*>(w + kHeaderBytes);
  ArgBest* part = reinterpret_cast<ArgBest*>(w + accept_part_offset(B));
  const int64_t vchunk = cdiv(V, vsplits);
  const int64_t rows = (int64_t)B * (N + 1);
  hipLaunchKernelGGL(accept_kernel, dim3((unsigned)(rows * vsplits)), dim3(256), 0, st, logits,
                     (int64_t)V, N, vsplits, vchunk, two_level, part, counters, tokens, parents,
                     parents_sb, max_depth, accept_len, accept_path, bonus, err);
  return hipGetLastError();
}

}  // namespace spec
