// Budget selection by block-mean scoring (gfx950).
//
// Method: "SpecPV: Improving Self-Speculative Decoding for Long-Context
// Generation via Partial Verification", section 3.2 "Partial Verification"
// (the partial cache is chosen block by block, as KV cache managers keep the
// cache in blocks, and is kept together with a sink and a local window) and
// section 4.1 (mean reduction for the retrieval); "BudgetDraft:
// Acceptance-Aware Multi-View Training for Sparse-KV Speculative Decoding"
// (Pith review), abstract: the drafter reads a sparse KV view under a fixed
// budget.
//
// block_means_kernel: the mean key of every cache block over its valid
// (below cache_len, not padding) positions, fp32.  One wavefront per block,
// rows read as coalesced 16-byte chunks; it streams the K cache once.
//
// score_blocks_kernel: every block that meets the middle between sink and
// window is scored with (mean query of the KV head) . (mean key), fp32,
// several workgroups per (sequence, KV head), into the workspace.
//
// select_blocks_kernel: one workgroup per (sequence, KV head).  The n_select
// best scores are found exactly by a radix select on order-preserving 32-bit keys
// (ties to the smaller block index through a prefix count); the list of sink,
// chosen blocks and window positions, without pads, is written in increasing
// order and padded with -1.
#include "dev_common.h"

namespace spec {

namespace {

constexpr int kMeanBlocksPerWG = 4;   // one block per wavefront
constexpr int kScoreSteps = 8;
constexpr int kWindowSegs = 64;      // pieces the window is listed in
constexpr int kScoreBlocksPerWG = 16 * kScoreSteps;   // 4 wavefronts x 4 blocks x steps

__global__ __launch_bounds__(256) void block_means_kernel(MeansArgs a) {
  const int b = blockIdx.z, g = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int L0 = a.cache_len[b];
  const bool bad = L0 < 0 || L0 > a.capacity;
  if (bad && threadIdx.x == 0 && blockIdx.x == 0 && g == 0) raise_error(a.err, SPEC_DEV_CACHE_LEN);
  const int L = bad ? 0 : L0;
  const int CH = a.row_chunks;              // 16-byte chunks per key row
  const int RPI = 64 / CH;                  // rows per wavefront step
  const int r_in = lane / CH, ch = lane % CH;
  const char* kb = a.k + (int64_t)b * a.k_sb + (int64_t)g * a.k_sh + ch * 16;
  const uint8_t* pr = a.pad == nullptr ? nullptr : a.pad + (int64_t)b * a.pad_sb;
  float* mb = a.means + ((int64_t)b * a.n_kv_heads + g) * a.max_blocks * a.head_dim;
  const int c_end = a.first_block + a.n_blocks;
  for (int i = wave; i < kMeanBlocksPerWG; i += 4) {
    const int c = a.first_block + blockIdx.x * kMeanBlocksPerWG + i;
    if (c >= c_end) break;
    const int r0 = c * a.block, r1 = min(r0 + a.block, L);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int cnt = 0;
    for (int rb = r0; rb < r1; rb += 4 * RPI) {
      u32x4 v[4];
      bool ok[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int row = rb + u * RPI + r_in;
        ok[u] = row < r1 && (pr == nullptr || pr[row] == 0);
        v[u] = ok[u] ? *reinterpret_cast<const u32x4*>(kb + (int64_t)row * a.k_st) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (!ok[u]) continue;
        ++cnt;
        if (a.bf16) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[2 * e] += __uint_as_float(v[u][e] << 16);
            acc[2 * e + 1] += __uint_as_float(v[u][e] & 0xffff0000u);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] += __uint_as_float(v[u][e]);
        }
      }
    }
    // the RPI row groups of the same chunk are lanes CH apart
    for (int o = CH; o < 64; o <<= 1) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], o, 64);
      cnt += __shfl_xor(cnt, o, 64);
    }
    if (r_in == 0) {
      const int epc = a.bf16 ? 8 : 4;
      float* dst = mb + (int64_t)c * a.head_dim + ch * epc;
      const float inv = cnt > 0 ? 1.f / (float)cnt : 0.f;
      for (int e = 0; e < epc; ++e) dst[e] = cnt > 0 ? acc[e] * inv : NAN;
    }
  }
}

// Order-preserving key of a score (larger score, larger key); 0 means "no
// score" (NaN: a block without a valid position).
__device__ __forceinline__ uint32_t score_key(float s) {
  if (isnan(s)) return 0u;
  const uint32_t u = __float_as_uint(s);
  const uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return max(k, 1u);
}

// Block-wide exclusive prefix sum of one int per thread (256 threads).
__device__ __forceinline__ int block_exclusive_sum(int x, int* red4, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) red4[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    before += w < wave ? red4[w] : 0;
    all += red4[w];
  }
  __syncthreads();
  *total = all;
  return before + incl - x;
}

// Candidate blocks of a sequence: those meeting [n_sink, L - window).
__device__ __forceinline__ void candidate_range(const SelectArgs& a, int L, int* c_lo, int* nc) {
  const int mid_lo = a.n_sink, mid_hi = L - a.window;
  *c_lo = 0;
  *nc = 0;
  if (mid_hi > mid_lo) {
    *c_lo = mid_lo / a.block;
    *nc = min((mid_hi - 1) / a.block + 1, a.max_blocks) - *c_lo;
  }
}

// Scores of kScoreBlocksPerWG consecutive blocks of one (sequence, KV head):
// (mean query) . (mean key) in fp32, NaN for blocks that are not candidates
// or have no mean.  16 lanes per block, 4 blocks per wavefront step, all of a
// wavefront's steps in flight together.
__global__ __launch_bounds__(256) void score_blocks_kernel(SelectArgs a) {
  const int b = blockIdx.z, g = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  __shared__ float qbar_s[128];
  const int L = a.cache_len[b];
  const bool bad = L < 0 || L > a.capacity;
  const int D = a.head_dim, G = a.G, rows = a.T * G;
  if (tid < D) {
    float s = 0.f;
    for (int r = 0; r < rows; ++r) {
      const int t = r / G, hh = r % G;
      const int64_t o = (((int64_t)b * a.T + t) * a.Hq + g * G + hh) * D + tid;
      s += a.bf16 ? __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(a.q)[o] << 16)
                  : reinterpret_cast<const float*>(a.q)[o];
    }
    qbar_s[tid] = s / (float)rows;
  }
  __syncthreads();
  int c_lo, nc;
  candidate_range(a, bad ? 0 : L, &c_lo, &nc);
  const int c_hi = c_lo + (bad ? 0 : nc);
  const float* mb = a.means + ((int64_t)b * a.n_kv_heads + g) * a.max_blocks * D;
  float* so = a.sc_ws + ((int64_t)b * a.n_kv_heads + g) * a.max_blocks;
  const int per = D / 16, sub = lane & 15;
  float qv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) qv[e] = e < per ? qbar_s[sub * per + e] : 0.f;
  const int c0 = blockIdx.x * kScoreBlocksPerWG + wave * 4 + (lane >> 4);
  f32x4 m[kScoreSteps][2];
#pragma unroll
  for (int u = 0; u < kScoreSteps; ++u) {
    const int c = min(c0 + u * 16, a.max_blocks - 1);
    const f32x4* src = reinterpret_cast<const f32x4*>(mb + (int64_t)c * D + sub * per);
    const bool live = c >= c_lo && c < c_hi;
    m[u][0] = live ? src[0] : f32x4{0.f, 0.f, 0.f, 0.f};
    m[u][1] = live && per == 8 ? src[1] : f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int u = 0; u < kScoreSteps; ++u) {
    const int c = c0 + u * 16;
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) s += m[u][e >> 2][e & 3] * qv[e];
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
    if (sub == 0 && c < a.max_blocks) so[c] = (c >= c_lo && c < c_hi) ? s : NAN;
  }
}

__global__ __launch_bounds__(256) void select_blocks_kernel(SelectArgs a) {
  const int b = blockIdx.y, g = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  __shared__ uint32_t key_s[kMaxSelectBlocks];
  __shared__ int hist_s[256];
  __shared__ int red4[4];
  __shared__ int s_digit, s_above;
  __shared__ int sel_s[kMaxSelect];
  __shared__ int segcnt_s[kMaxSelect + 1 + kWindowSegs];

  // one list per (sequence, KV head), or per sequence when shared (g = 0)
  const int n_lists = a.shared ? 1 : a.n_kv_heads;
  int32_t* out = a.idx + ((int64_t)b * n_lists + g) * a.budget;
  float* sc_out = a.scores == nullptr ? nullptr
                                      : a.scores + ((int64_t)b * n_lists + g) * a.max_blocks;
  const int L0 = a.cache_len[b];
  if (L0 < 0 || L0 > a.capacity) {
    if (tid == 0 && g == 0) raise_error(a.err, SPEC_DEV_CACHE_LEN);
    for (int i = tid; i < a.budget; i += 256) out[i] = -1;
    if (sc_out != nullptr)
      for (int i = tid; i < a.max_blocks; i += 256) sc_out[i] = NAN;
    return;
  }
  const int L = L0;

  // candidate blocks and their scores (score_blocks_kernel)
  const int mid_lo = a.n_sink, mid_hi = L - a.window;
  int c_lo, nc;
  candidate_range(a, L, &c_lo, &nc);
  const float* sw = a.sc_ws + ((int64_t)b * a.n_kv_heads + g) * a.max_blocks;
  const int64_t hs = a.max_blocks;   // head stride of the workspace scores
  // scores of blocks c0 + u * 256 (u < 4) for this thread: the KV head's own,
  // or (shared) the mean over the heads, summed in head order with up to
  // 8 heads x 4 blocks of loads in flight
  auto scores4 = [&](int c0, int c_end, float (&t)[4]) {
    if (!a.shared) {
#pragma unroll
      for (int u = 0; u < 4; ++u) t[u] = c0 + u * 256 < c_end ? sw[c0 + u * 256] : 0.f;
      return;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) t[u] = 0.f;
    for (int h0 = 0; h0 < a.n_kv_heads; h0 += 8) {
      float x[8][4];
#pragma unroll
      for (int hh = 0; hh < 8; ++hh)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int c = c0 + u * 256;
          x[hh][u] = (h0 + hh < a.n_kv_heads && c < c_end) ? sw[(h0 + hh) * hs + c] : 0.f;
        }
#pragma unroll
      for (int hh = 0; hh < 8; ++hh)
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (h0 + hh < a.n_kv_heads) t[u] += x[hh][u];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) t[u] /= (float)a.n_kv_heads;
  };
  for (int i0 = 0; i0 < nc; i0 += 1024) {
    float t[4];
    scores4(c_lo + i0 + tid, c_lo + nc, t);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i0 + u * 256 + tid < nc) key_s[i0 + u * 256 + tid] = score_key(t[u]);
  }
  if (sc_out != nullptr) {
    for (int c0 = 0; c0 < a.max_blocks; c0 += 1024) {
      float t[4];
      scores4(c0 + tid, a.max_blocks, t);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (c0 + u * 256 + tid < a.max_blocks) sc_out[c0 + u * 256 + tid] = t[u];
    }
  }
  __syncthreads();

  // how many blocks have a score, and how many are chosen
  int nv = 0;
  for (int i = tid; i < nc; i += 256) nv += key_s[i] != 0u;
  int n_valid;
  block_exclusive_sum(nv, red4, &n_valid);
  const int k = min(a.n_select, n_valid);

  // radix select: the k-th largest key (all of them when k == n_valid)
  uint32_t prefix = 0u, mask = 0u;
  int remaining = k;
  if (k > 0 && k < n_valid) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      hist_s[tid] = 0;
      __syncthreads();
      for (int i = tid; i < nc; i += 256) {
        const uint32_t key = key_s[i];
        if (key != 0u && (key & mask) == prefix) atomicAdd(&hist_s[(key >> shift) & 255u], 1);
      }
      __syncthreads();
      if (wave == 0) {
        // lane l holds bins 255 - 4l .. 252 - 4l (descending)
        int h[4], hs = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          h[j] = hist_s[255 - 4 * lane - j];
          hs += h[j];
        }
        int incl = hs;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int y = __shfl_up(incl, o, 64);
          if (lane >= o) incl += y;
        }
        const int excl = incl - hs;   // keys in higher bins than this lane's
        if (excl < remaining && remaining <= incl) {
          int above = excl, d = 255 - 4 * lane;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (above + h[j] >= remaining) {
              d = 255 - 4 * lane - j;
              break;
            }
            above += h[j];
          }
          s_digit = d;
          s_above = above;
        }
      }
      __syncthreads();
      prefix |= (uint32_t)s_digit << shift;
      mask |= 255u << shift;
      remaining -= s_above;
    }
  }
  // chosen: keys above the threshold, then the first `remaining` keys equal
  // to it in block order (every key with a score when k == n_valid); each
  // thread owns a contiguous range of blocks, so block order is thread order
  const bool take_all = k == n_valid;
  const int chunk = (nc + 255) / 256;
  const int ibeg = min(nc, tid * chunk), iend = min(nc, ibeg + chunk);
  auto chosen = [&](uint32_t key, int& eq_rank) -> bool {
    if (k == 0 || key == 0u) return false;
    if (take_all || key > prefix) return true;
    if (key == prefix) return eq_rank++ < remaining;
    return false;
  };
  int n_eq = 0;
  if (!take_all)
    for (int i = ibeg; i < iend; ++i) n_eq += key_s[i] != 0u && key_s[i] == prefix;
  int eq_total;
  const int eq_before = block_exclusive_sum(n_eq, red4, &eq_total);
  int n_take = 0;
  {
    int r = eq_before;
    for (int i = ibeg; i < iend; ++i) n_take += chosen(key_s[i], r);
  }
  int m_total;
  int slot = block_exclusive_sum(n_take, red4, &m_total);
  {
    int r = eq_before;
    for (int i = ibeg; i < iend; ++i)
      if (chosen(key_s[i], r)) sel_s[slot++] = c_lo + i;
  }
  __syncthreads();
  const int m = m_total;

  // segments: 0 = sink, 1..m = chosen blocks (their middle part), then the
  // window in up to kWindowSegs pieces, so that the waves share it
  const int s_end = min(a.n_sink, L);
  const int w_beg = max(a.n_sink, L - a.window);
  const int w_len = L - w_beg;
  const int n_wseg = max(1, min(kWindowSegs, (w_len + 255) / 256));
  const int w_piece = (w_len + n_wseg - 1) / n_wseg;
  const int n_seg = m + 1 + n_wseg;
  const uint8_t* pr = a.pad == nullptr ? nullptr : a.pad + (int64_t)b * a.pad_sb;
  auto seg_range = [&](int sgi, int* lo, int* hi) {
    if (sgi == 0) {
      *lo = 0;
      *hi = s_end;
    } else if (sgi > m) {
      const int k = sgi - m - 1;
      *lo = w_beg + k * w_piece;
      *hi = min(L, *lo + w_piece);
    } else {
      const int c = sel_s[sgi - 1];
      *lo = max(c * a.block, mid_lo);
      *hi = min((c + 1) * a.block, mid_hi);
    }
  };
  for (int sgi = wave; sgi < n_seg; sgi += 4) {
    int lo, hi;
    seg_range(sgi, &lo, &hi);
    int cnt = 0;
    for (int p0 = lo; p0 < hi; p0 += 64) {
      const int p = p0 + lane;
      const bool keep = p < hi && (pr == nullptr || pr[p] == 0);
      cnt += __popcll(__ballot(keep));
    }
    if (lane == 0) segcnt_s[sgi] = cnt;
  }
  __syncthreads();
  {   // segment counts -> offsets (each thread a contiguous run of segments)
    const int nseg = n_seg, sch = (nseg + 255) / 256;
    const int sb = min(nseg, tid * sch), se = min(nseg, sb + sch);
    int local = 0;
    for (int i = sb; i < se; ++i) local += segcnt_s[i];
    int all;
    int run = block_exclusive_sum(local, red4, &all);
    for (int i = sb; i < se; ++i) {
      const int c = segcnt_s[i];
      segcnt_s[i] = run;
      run += c;
    }
    if (tid == 0) s_above = all;
  }
  __syncthreads();
  const int total = s_above;
  for (int sgi = wave; sgi < n_seg; sgi += 4) {
    int lo, hi;
    seg_range(sgi, &lo, &hi);
    int base = segcnt_s[sgi];
    for (int p0 = lo; p0 < hi; p0 += 64) {
      const int p = p0 + lane;
      const bool keep = p < hi && (pr == nullptr || pr[p] == 0);
      const uint64_t bal = __ballot(keep);
      if (keep) out[base + __popcll(bal & ((1ull << lane) - 1ull))] = p;
      base += __popcll(bal);
    }
  }
  for (int i = total + tid; i < a.budget; i += 256) out[i] = -1;
}

}  // namespace

hipError_t launch_block_means(const MeansArgs& a, hipStream_t st) {
  if (a.n_blocks <= 0) return hipSuccess;
  const unsigned gx = (unsigned)((a.n_blocks + kMeanBlocksPerWG - 1) / kMeanBlocksPerWG);
  hipLaunchKernelGGL(block_means_kernel, dim3(gx, (unsigned)a.n_kv_heads, (unsigned)a.batch),
                     dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_select_blocks(const SelectArgs& a, hipStream_t st) {
  const unsigned gx = (unsigned)((a.max_blocks + kScoreBlocksPerWG - 1) / kScoreBlocksPerWG);
  hipLaunchKernelGGL(score_blocks_kernel, dim3(gx, (unsigned)a.n_kv_heads, (unsigned)a.batch),
                     dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(select_blocks_kernel,
                     dim3(a.shared ? 1u : (unsigned)a.n_kv_heads, (unsigned)a.batch), dim3(256), 0,
                     st, a);
  return hipGetLastError();
}

}  // namespace spec
