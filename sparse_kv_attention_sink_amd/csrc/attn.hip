// Draft and verify attention, bf16 inputs, fp32 accumulation (gfx950).
//
// Method.
//  * Draft: "Windowed-MTP: Removing the Full-Context Draft-KV Tax at
//    Million-Token Context" (Pith review), "What carries the argument": the
//    draft reads only the first n_sink cached tokens plus the last W tokens;
//    "BudgetDraft: Acceptance-Aware Multi-View Training for Sparse-KV
//    Speculative Decoding" (Pith review), abstract: the drafter reads a sparse
//    KV view under a fixed budget of positions.
//  * Verify: "SpecMemo: Speculative Decoding is in Your Pocket" (Pith review),
//    "What carries the argument" and Figure 9: the N speculated tree nodes are
//    checked in one pass under a tree attention mask; batched verification
//    pads accepted tokens, remaps position IDs so padding is ignored and gives
//    cached padding slots -inf.
//
// One kernel serves the three key sources.  A workgroup (4 wavefronts) owns
// one (sequence, KV head, row block, split).  Its keys arrive in 32-key tiles
// (K and V rows, D bf16 each) copied straight from HBM into an LDS ring with
// global_load_lds (no register staging); the copies for the next NS-1 tiles
// are in flight while a tile is multiplied.  Both products run on bf16 MFMA
// (v_mfma_f32_16x16x32_bf16) in transposed form:
//     S^T[key][row] = K[key][:] . Q[row][:]
//     O^T[d][row]  += V^T[d][key] . P^T[key][row]
// so a lane owns one query row in both accumulators: the online softmax
// (max, rescale, sum) stays in the lane and P goes from the score registers
// straight into the next MFMA operand.  The V^T operand comes from V's
// natural layout through the LDS transpose read (ds_read_b64_tr_b16).
//
// Two shapes:
//  * many rows (trees: nodes x GQA group > 32): the 4 wavefronts share one
//    ring and each owns 16, 32 or 48 rows (one to three 16-row MFMA tiles,
//    WK = 1);
//  * few rows (chains, drafts): each wavefront streams its own quarter of the
//    workgroup's tiles through a private ring and the four results are merged
//    in LDS at the end (WK = 4).
// Several splits per (sequence, KV head) are merged by the workgroup that
// finishes last, so a call is one launch.
#include "dev_common.h"

namespace spec {

template <int D>
struct Geo {
  static constexpr int ROWB = 2 * D;             // bytes per key row
  static constexpr int CH = ROWB / 16;           // 16-byte chunks per row
  static constexpr int KB = kTileKeys * ROWB;    // K bytes per tile
  static constexpr int SB = 2 * KB;              // stage: K then V
  static constexpr int DPT = SB / 1024;          // 1 KB copy instructions per tile
  static constexpr int RPI = 1024 / ROWB;        // key rows per copy instruction
  static constexpr int ND = D / 32;              // q.k MFMA steps
  static constexpr int NDT = D / 16;             // 16-wide head-dim tiles of O
};

// LDS swizzles (16-byte chunk index XOR a function of the key row) that make
// the K-operand reads (16 rows at one chunk) and the transpose reads of V
// (16 rows x 32 bytes) free of bank conflicts.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int swz_v(int r) {
  return D == 128 ? ((r & 7) << 1) : (((r >> 1) & 3) << 1);
}

__device__ __forceinline__ bf16x8 lds_load_b128(uint32_t addr) {
  return *SPEC_LDS(const bf16x8, (uintptr_t)addr);
}

// Wait until the copies of all but the newest `n` tiles (0 <= n <= MAXN)
// issued by this wavefront have landed.
template <int DPW, int MAXN>
__device__ __forceinline__ void wait_tiles(int n) {
  if constexpr (MAXN <= 0) {
    wait_vm<0>();
  } else {
    if (n >= MAXN) wait_vm<MAXN * DPW>();
    else wait_tiles<DPW, MAXN - 1>(n);
  }
}

// Where the keys of one (sequence, KV head) come from.  Rows are addressed
// with 32-bit byte offsets from the (sequence, KV head)'s first cache row or
// first tree row; the host guarantees they fit.
struct KeySrc {
  const char* k;            // cache K / V rows of this (sequence, KV head)
  const char* v;
  const char* tk;           // tree K / V rows (verify)
  const char* tv;
  const int32_t* idx;       // budget positions staged in LDS (gather), from view v0
  uint32_t rowb, trowb;     // row strides in bytes
  uint32_t kbytes, tbytes;  // addressable bytes from k / tk
  int n_view, cache_tiles, n_tree, s_len, w_start, v0;
  int kv_ring, n_sink;      // window through a ring: slot n_sink + (p - n_sink) % kv_ring
};

// Row of key position p: p itself, or its ring slot when the window is kept
// in a ring after the sink.
__device__ __forceinline__ int ring_row(KeySrc ks, int p) {
  return (ks.kv_ring == 0 || p < ks.n_sink) ? p : ks.n_sink + (p - ks.n_sink) % ks.kv_ring;
}

// Key position of view position v (0 <= v < n_view).
template <int MODE>
__device__ __forceinline__ int view_pos(KeySrc ks, int v) {
  if constexpr (MODE == kDraftWindow) return v < ks.s_len ? v : ks.w_start + (v - ks.s_len);
  else if constexpr (MODE == kDraftGather) return ks.idx[v - ks.v0];
  else return v;
}

__device__ __forceinline__ bool is_tree_tile(KeySrc ks, int t, int mode) {
  return mode == kVerify && t >= ks.cache_tiles;
}

// Row of tile key r (0..31): the segment's row index, clamped to its last
// row (keys past the end re-read it; their scores are masked).
template <int MODE>
__device__ __forceinline__ int tile_row(KeySrc ks, int t, int r) {
  if (!is_tree_tile(ks, t, MODE)) {
    const int p = view_pos<MODE>(ks, min(t * kTileKeys + r, ks.n_view - 1));
    return MODE == kDraftWindow ? ring_row(ks, p) : p;
  }
  return min((t - ks.cache_tiles) * kTileKeys + r, ks.n_tree - 1);
}

// First row of tile t if its 32 rows are consecutive rows of one segment,
// else -1 (budget gathers, a window tile that straddles the sink, and a
// segment's last, partial tile).
template <int MODE>
__device__ __forceinline__ int tile_first_row(KeySrc ks, int t) {
  if (is_tree_tile(ks, t, MODE)) {
    const int j0 = (t - ks.cache_tiles) * kTileKeys;
    return j0 + kTileKeys <= ks.n_tree ? j0 : -1;
  }
  const int v = t * kTileKeys;
  if (v + kTileKeys > ks.n_view) return -1;
  if constexpr (MODE == kDraftWindow) {
    if (v + kTileKeys <= ks.s_len) return v;
    if (v >= ks.s_len) {
      const int p0 = ks.w_start + (v - ks.s_len);
      if (ks.kv_ring == 0 || p0 < ks.n_sink) return p0;
      const int off = (p0 - ks.n_sink) % ks.kv_ring;   // a tile across the ring's end is gathered
      return off + kTileKeys <= ks.kv_ring ? ks.n_sink + off : -1;
    }
    return -1;
  } else if constexpr (MODE == kDraftGather) {
    return -1;
  } else {
    return v;
  }
}

// Issue this wavefront's share (DPW of the tile's 1 KB copies) of tile t into
// the LDS stage at `stage`.  Copy gi covers key rows (gi % (DPT/2)) * RPI ..
// of K (first half) or V (second half); lane l writes 16-byte slot l % CH of
// row l / CH, which holds head-dim chunk (slot XOR swizzle(row)).
template <int MODE, int D, int DPW>
__device__ __forceinline__ void issue_tile(KeySrc ks, int t, uint32_t stage, int wl, int lane) {
  using Ge = Geo<D>;
  const bool tree = is_tree_tile(ks, t, MODE);
  const int j0 = tile_first_row<MODE>(ks, t);
  const bool contig = j0 >= 0;
  const uint32_t rowb = tree ? ks.trowb : ks.rowb;
#pragma unroll
  for (int u = 0; u < DPW; ++u) {
    const int gi = wl * DPW + u;
    const int region = gi / (Ge::DPT / 2);    // 0: K, 1: V
    const int ii = gi % (Ge::DPT / 2);
    const int rl = lane / Ge::CH;
    const int r = ii * Ge::RPI + rl;
    const uint32_t col = (uint32_t)(((lane % Ge::CH) ^ (region ? swz_v<D>(r) : swz_k<D>(r))) * 16);
    const char* seg = tree ? (region ? ks.tv : ks.tk) : (region ? ks.v : ks.k);
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(stage + region * Ge::KB + ii * 1024);
    if (contig) {
      const char* sb = seg + (size_t)(j0 + ii * Ge::RPI) * rowb;   // wave-uniform
      copy16_to_lds_s(sb, (uint32_t)rl * rowb + col, m0);
    } else {
      const int j = tile_row<MODE>(ks, t, r);
      copy16_to_lds(seg + ((uint32_t)j * rowb + col), m0);
    }
  }
}

// Register-staged tile (one wavefront loads all of it): piece gi of the tile
// is K (first half) or V rows (gi % (DPT/2)) * RPI + lane / CH, head-dim
// chunk lane % CH, loaded with coalesced 16-byte buffer loads (streaming
// hint; out-of-range offsets read zeros instead of faulting) ...
template <int MODE, int D>
__device__ __forceinline__ void load_tile_regs(KeySrc ks, int t, int lane, u32x4 (&stg)[Geo<D>::DPT]) {
  using Ge = Geo<D>;
  constexpr int kNt = 2;   // cache policy: non-temporal
  const bool tree = is_tree_tile(ks, t, MODE);
  const int j0 = tile_first_row<MODE>(ks, t);
  const bool contig = j0 >= 0;
  const uint32_t rowb = tree ? ks.trowb : ks.rowb;
  const __amdgpu_buffer_rsrc_t rk = coherent_rsrc(tree ? ks.tk : ks.k, tree ? ks.tbytes : ks.kbytes);
  const __amdgpu_buffer_rsrc_t rv = coherent_rsrc(tree ? ks.tv : ks.v, tree ? ks.tbytes : ks.kbytes);
  const int rl = lane / Ge::CH;
  const uint32_t col = (uint32_t)((lane % Ge::CH) * 16);
  constexpr int H = Ge::DPT / 2;
  // Offsets first (lane offset fixed and row offset in the scalar soffset for
  // a contiguous tile; per-lane rows otherwise), then one burst of loads into
  // the staging registers: a single definition of each register lets the
  // compiler load the next tile in place instead of into temporaries it would
  // have to wait for and copy at the end of the iteration.
  uint32_t voff[Ge::DPT], soff[Ge::DPT];
  if (contig) {
    const uint32_t s0 = (uint32_t)j0 * rowb;
#pragma unroll
    for (int gi = 0; gi < Ge::DPT; ++gi) {
      voff[gi] = (uint32_t)rl * rowb + col;
      soff[gi] = s0 + (uint32_t)((gi % H) * Ge::RPI) * rowb;
    }
  } else {
#pragma unroll
    for (int gi = 0; gi < Ge::DPT; ++gi) {
      voff[gi] = (uint32_t)tile_row<MODE>(ks, t, (gi % H) * Ge::RPI + rl) * rowb + col;
      soff[gi] = 0;
    }
  }
#pragma unroll
  for (int gi = 0; gi < Ge::DPT; ++gi)
    stg[gi] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(gi < H ? rk : rv, voff[gi], soff[gi], kNt));
}
// ... and written to the wavefront's LDS stage at its swizzled slot.
template <int D>
__device__ __forceinline__ void store_tile_lds(uint32_t stage, int lane, const u32x4 (&stg)[Geo<D>::DPT]) {
  using Ge = Geo<D>;
#pragma unroll
  for (int gi = 0; gi < Ge::DPT; ++gi) {
    const int region = gi / (Ge::DPT / 2);
    const int r = (gi % (Ge::DPT / 2)) * Ge::RPI + lane / Ge::CH;
    const int p = (lane % Ge::CH) ^ (region ? swz_v<D>(r) : swz_k<D>(r));
    *SPEC_LDS(u32x4, (uintptr_t)(stage + region * Ge::KB + r * Ge::ROWB + p * 16)) = stg[gi];
  }
}

// Merge n (1..P) partial results of RC rows: partial p of row rl is o
// (normalised by its own softmax sum) at o_rs[((p0 + p) * RC + rl) * D + d]
// and its log2 sum-exp at l_rs[(p0 + p) * RC + rl].  For every (row, 4 head-
// dim values) item of the first `rows` rows, the loads of U items are issued
// before any is used (partials past n re-read the last one and get weight 0),
// and sink(rl, d0, o[4], lse2) receives sum_p 2^(x_p - M) o_p / sum_p 2^(x_p - M)
// and M + log2 sum_p 2^(x_p - M), M = max_p x_p: NaN if any partial is NaN,
// o = 0 and lse = -inf if every partial is empty.
template <int D, int RC, int P, typename Sink>
__device__ __forceinline__ void merge_partials_p(__amdgpu_buffer_rsrc_t o_rs, __amdgpu_buffer_rsrc_t l_rs,
                                                 int p0, int n, int rows, Sink sink) {
  constexpr int kItems = RC * (D / 4);
  constexpr int kPerThread = (kItems + 255) / 256;
  // about 32 partial loads in flight per thread at D = 128, 16 at D = 64
  // (where more registers would cost the main loop occupancy)
  constexpr int kLoads = D == 128 ? 32 : 16;
  constexpr int Uw = kLoads / P > 0 ? kLoads / P : 1;
  constexpr int U = Uw < kPerThread ? Uw : kPerThread;
  for (int i0 = 0; i0 < kPerThread; i0 += U) {
    float x[U][P];
    f32x4 ov[U][P];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int it = (int)threadIdx.x + (i0 + u) * 256;
      const int rl = it / (D / 4), d0 = (it % (D / 4)) * 4;
      const bool live = it < kItems && rl < rows;
      // Short row blocks (drafts, chains: 16 or 32 rows) often have most rows
      // dead (a single query with 4 query heads per KV head uses 4 of 16):
      // a wavefront whose items are all dead skips its loads (a single-query
      // draft over 1M keys: 11.9 -> 11.4 us).  Tree row blocks keep the
      // uniform loads, which measured faster there.
      if constexpr (RC <= 32) {
        const int wfirst = __builtin_amdgcn_readfirstlane((int)(threadIdx.x & ~63u)) + (i0 + u) * 256;
        if (wfirst >= kItems || wfirst / (D / 4) >= rows) continue;
      }
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int pp = p0 + min(p, n - 1);
        // a dead item reads row 0 of the first partial (always in range)
        const int r = live ? rl : 0, dd = live ? d0 : 0;
        x[u][p] = load_sc1_f1(l_rs, (uint32_t)((pp * RC + r) * 4));
        ov[u][p] = load_sc1_f4(o_rs, (uint32_t)(((pp * RC + r) * D + dd) * 4));
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int it = (int)threadIdx.x + (i0 + u) * 256;
      const int rl = it / (D / 4), d0 = (it % (D / 4)) * 4;
      if (it >= kItems || rl >= rows) continue;
      float M = -INFINITY;
      bool nan = false;
#pragma unroll
      for (int p = 0; p < P; ++p)
        if (p < n) {
          nan |= isnan(x[u][p]);
          M = fmaxf(M, x[u][p]);
        }
      float W = 0.f, o[4] = {0.f, 0.f, 0.f, 0.f};
      if (!nan && M != -INFINITY) {
#pragma unroll
        for (int p = 0; p < P; ++p) {
          const float f = p < n ? __builtin_amdgcn_exp2f(x[u][p] - M) : 0.f;
          W += f;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] += f * ov[u][p][e];
        }
      }
      float lse2;
      if (nan) {
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = NAN;
        lse2 = NAN;
      } else if (M == -INFINITY || !(W > 0.f)) {
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = 0.f;
        lse2 = -INFINITY;
      } else {
        const float inv = 1.f / W;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] *= inv;
        lse2 = M + log2f(W);
      }
      sink(rl, d0, o, lse2);
    }
  }
}

// Merge n (1..kMergeFan) partials, loading only as many as there are, to the
// next multiple of 4: most tree verifies merge 4 or fewer.
template <int D, int RC, typename Sink>
__device__ __forceinline__ void merge_partials(__amdgpu_buffer_rsrc_t o_rs, __amdgpu_buffer_rsrc_t l_rs,
                                               int p0, int n, int rows, Sink sink) {
  static_assert(kMergeFan == 16, "merge widths 4, 8 and 16");
  if (n <= 4) merge_partials_p<D, RC, 4>(o_rs, l_rs, p0, n, rows, sink);
  else if (n <= 8) merge_partials_p<D, RC, 8>(o_rs, l_rs, p0, n, rows, sink);
  else merge_partials_p<D, RC, 16>(o_rs, l_rs, p0, n, rows, sink);
}

template <int MODE, int D, int RT, int WK, int NS>
struct AttnCfg {
  static constexpr int WR = 4 / WK;                 // wavefronts per key group
  static constexpr int RCW = RT * 16;               // rows per wavefront
  static constexpr int RC = WR * RCW;               // rows per workgroup
  static constexpr int DPW = Geo<D>::DPT / WR;      // copies per tile per loading wave
  // LDS: one shared ring of NS stages (WK = 1), or one stage per wavefront
  // (WK = 4), which the end-of-split merge of the four wavefronts reuses.
  static constexpr int MERGE = 4 * RC * (D + 2) * 4;
  static constexpr int RING = WK == 1 ? NS * Geo<D>::SB
                                      : (4 * Geo<D>::SB > MERGE ? 4 * Geo<D>::SB : MERGE);
  static_assert(Geo<D>::DPT % WR == 0, "tile copies must split evenly");
  static_assert(WK == 1 || WK == 4, "one shared ring or four private rings");
};

template <int MODE, int D, int RT, int WK, int NS>
__global__ __launch_bounds__(256, ((WK == 4 ? RT == 1 : RT <= 3) && 2 * AttnCfg<MODE, D, RT, WK, NS>::RING <= 136 * 1024) ? 2 : 1)
void attn_bf16_kernel(AttnArgs a) {
  using Cf = AttnCfg<MODE, D, RT, WK, NS>;
  using Ge = Geo<D>;
  constexpr int WR = Cf::WR, RCW = Cf::RCW, RC = Cf::RC, DPW = Cf::DPW;
  constexpr int ND = Ge::ND, NDT = Ge::NDT, ROWB = Ge::ROWB, CH = Ge::CH, KB = Ge::KB,
                SB = Ge::SB, RPI = Ge::RPI;

  __shared__ __attribute__((aligned(1024))) uint8_t ring[Cf::RING];
  // per-tile bits of keys to skip: pad slots (verify), -1 list entries (gather)
  __shared__ uint32_t padbits_s[MODE == kVerify        ? kMaxPadWords
                                : MODE == kDraftGather ? kMaxGatherKeys / kTileKeys
                                                       : 1];
  __shared__ int32_t idx_s[MODE == kDraftGather ? kMaxGatherKeys : 1];
  __shared__ int32_t par_s[MODE == kVerify ? kMaxNodes : 1];
  __shared__ int32_t dep_s[MODE == kVerify ? kMaxNodes : 1];
  __shared__ uint64_t anc_s[MODE == kVerify ? kMaxNodes : 1];
  __shared__ int32_t red_s[4];

  // ---------------------------------------------------------------- who am I
  int unit, z;
  if (a.n_rb == 1) {
    unit = blockIdx.x;
    z = 0;
  } else {
    // The row blocks of one (pair, split) read the same keys: give them
    // consecutive slots on one XCD (workgroups go to XCDs round-robin) so
    // they meet in that XCD's L2.
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    unit = (slot / a.n_rb) * 8 + xcd;
    z = slot % a.n_rb;
    if (unit >= a.units) return;
  }
  int s = unit % a.splits, pair = unit / a.splits;
  // this workgroup's partial slot in its group's buffer, the first slot of
  // its (sequence, KV head), and the split size of the sequence
  int pslot = s, pslot0 = 0, tps_own = a.tps, S_ord = 0;
  if constexpr (MODE == kVerify && WK == 1) {
    if (a.ordered) {
      // Balanced splits, longest first.  Every workgroup reads all the
      // sequences' lengths and derives the same plan: with `conc`
      // workgroups of a (KV head, row block) running at once, a split takes
      // at most T tiles, T the smallest value whose splits, min(S,
      // ceil(tiles_b / T)) for sequence b, number at most conc (so that
      // every split runs in the first round), at most tps_max; sequence b
      // gets that many equal splits, and the splits are numbered as work
      // items in order of size, largest first (ties: smaller sequence
      // index), so that the hardware starts the longest work first.
      // Workgroup j of a KV head takes item j; items past the last split
      // exit.
      // (the tile ring is free until the first copies: it holds the plan)
      static_assert(Cf::RING >= 3 * kMaxOrderBatch * 4, "the ring holds the ordered plan");
      int32_t* const tl_s = reinterpret_cast<int32_t*>(ring);   // tiles per sequence
      int32_t* const ns_s = tl_s + kMaxOrderBatch;              // splits per sequence
      int32_t* const st_s = ns_s + kMaxOrderBatch;              // first item of each sequence
      __shared__ int32_t sel_s[1];
      const int nt = (a.T + kTileKeys - 1) / kTileKeys;   // tree tiles
      int w = 0;
      for (int i = threadIdx.x; i < a.B; i += 256) {
        const int l = a.cache_len[i];
        const int tl = ((l >= 0 && l <= a.capacity) ? (l + kTileKeys - 1) / kTileKeys : 0) + nt;
        tl_s[i] = tl;
        w += tl;
      }
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) w += __shfl_xor(w, m, 64);
      if ((threadIdx.x & 63) == 0) red_s[threadIdx.x >> 6] = w;
      if (threadIdx.x == 0) sel_s[0] = -1;
      __syncthreads();
      const int W = red_s[0] + red_s[1] + red_s[2] + red_s[3];
      // T is sought in [ceil(W / conc), ceil(W / (conc - B))], W the batch's
      // tiles: below the first, uncapped splits would exceed conc, and from
      // the second on ceil() adds at most one split per sequence.  Every wavefront runs the same binary search
      // (a lane holds up to 4 sequences; the split count of a candidate is a
      // wavefront sum), so no barrier is needed.
      int lo = max(1, (W + a.conc - 1) / a.conc);
      int hi = a.conc > a.B ? (W + a.conc - a.B - 1) / (a.conc - a.B) : a.tps_max;
      hi = min(max(hi, lo), a.tps_max);
      lo = min(lo, hi);
      static_assert(kMaxOrderBatch <= 4 * 64, "four sequences per lane");
      int tl_r[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int i = (int)(threadIdx.x & 63) + 64 * k;
        tl_r[k] = i < a.B ? tl_s[i] : 0;
      }
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        int c = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) c += tl_r[k] > 0 ? min(a.splits, (tl_r[k] + mid - 1) / mid) : 0;
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) c += __shfl_xor(c, m, 64);
        if (c <= a.conc) hi = mid;
        else lo = mid + 1;
      }
      const int tgt = lo;
      for (int i = threadIdx.x; i < a.B; i += 256) ns_s[i] = min(a.splits, (tl_s[i] + tgt - 1) / tgt);
      __syncthreads();
      const int item = unit / a.Hkv;
      for (int i = threadIdx.x; i < a.B; i += 256) {
        const int si = (tl_s[i] + ns_s[i] - 1) / ns_s[i];
        int start = 0;
        for (int j = 0; j < a.B; ++j) {
          const int sj = (tl_s[j] + ns_s[j] - 1) / ns_s[j];
          start += (sj > si || (sj == si && j < i)) ? ns_s[j] : 0;
        }
        st_s[i] = start;
        if (item >= start && item < start + ns_s[i]) sel_s[0] = i;   // one sequence matches
      }
      __syncthreads();
      const int bb = sel_s[0];
      if (bb < 0) return;   // past the batch's last split: nothing to do
      pslot0 = st_s[bb];
      s = item - pslot0;
      pslot = item;
      S_ord = ns_s[bb];
      tps_own = (tl_s[bb] + S_ord - 1) / S_ord;
      pair = bb * a.Hkv + unit % a.Hkv;
    }
  }
  const int b = pair / a.Hkv, g = pair % a.Hkv;
  // (the wave index is uniform within a wavefront; saying so keeps
  // everything derived from it, such as a wavefront's tile range and its
  // buffer descriptors, in scalar registers)
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, q4 = lane >> 4;
  const int kgi = WK == 1 ? 0 : wave;   // key group (ring) of this wavefront
  const int rg = WK == 1 ? wave : 0;    // row group of this wavefront
  const bool leader = g == 0 && s == 0 && z == 0;
  const int T = a.T, G = a.G, N = a.T;

  const int L = a.cache_len[b];
  bool bad = MODE == kVerify ? (L < 0 || L > a.capacity)
                             : (L < T || (a.kv_ring == 0 && L > a.capacity));   // a ring keeps the logical length
  if (leader && tid == 0 && bad) raise_error(a.err, SPEC_DEV_CACHE_LEN);
  // Splits of this (sequence, KV head): all of the plan's, or, in the
  // ordered verify, the sequence's own (a sequence with a bad length has
  // one, which writes its poisoned rows).
  int S_own = a.splits;
  if constexpr (MODE == kVerify && WK == 1) {
    if (a.ordered) S_own = S_ord;
  }

  // ---------------------------------------------------------------- tree
  if constexpr (MODE == kVerify) {
    bool bp = false;
    if (tid < N) {
      const int p = a.parents[b * a.par_sb + tid];
      par_s[tid] = p;
      bp = !(p >= -1 && p < tid);
    }
    const bool bad_par = __syncthreads_or(bp);
    if (tid < N) {
      uint64_t m = 0;
      int depth = -1;
      if (!bad_par)
        for (int j = tid; j >= 0; j = par_s[j]) {   // parents precede children: ends
          m |= 1ull << j;
          ++depth;
        }
      anc_s[tid] = m;
      dep_s[tid] = depth;
    }
    if (leader && tid == 0 && bad_par) raise_error(a.err, SPEC_DEV_PARENT);
    bad = bad || bad_par;
    __syncthreads();   // the masks and depths are read by every thread below
  }

  // ---------------------------------------------------------------- key range
  int s_len = 0, w_start = 0, n_view = 0;
  if (!bad) {
    if constexpr (MODE == kDraftWindow) {
      s_len = min(a.n_sink, L);
      w_start = min(max(max(a.n_sink, L - T + 1 - a.window), 0), L);
      n_view = s_len + (L - w_start);
    } else if constexpr (MODE == kDraftGather) {
      n_view = a.budget;
    } else {
      n_view = L;
    }
  }
  const int cache_tiles = (n_view + kTileKeys - 1) / kTileKeys;
  const int tree_tiles = (MODE == kVerify && !bad) ? (N + kTileKeys - 1) / kTileKeys : 0;
  const int total = cache_tiles + tree_tiles;
  int t0, t1;
  split_tiles(total, tps_own, s, t0, t1);
  int k0 = t0, k1 = t1;
  if constexpr (WK == 4) {
    const int per = (t1 - t0 + 3) / 4;
    k0 = min(t1, t0 + kgi * per);
    k1 = min(t1, k0 + per);
  }

  // ---------------------------------------------------------------- rows
  // (the query loads are issued first, so that their latency overlaps the
  // staging loads below and the first tile's loads)
  // erow: a draft row's end position; in verify, the row's tree node (-1
  // past the last row), whose ancestor mask tree tiles read from LDS
  bf16x8 qf[RT][ND];
  int erow[RT];
  const int row0 = z * RC + rg * RCW;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = row0 + rt * 16 + l16;
    erow[rt] = MODE == kVerify ? -1 : 0;
#pragma unroll
    for (int c = 0; c < ND; ++c) qf[rt][c] = bf16x8{};
    if (row < a.R) {
      const int t = row / G, hh = row % G;
      erow[rt] = MODE == kVerify ? t : L - T + t + 1;
      const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) +
                           (((size_t)b * T + t) * a.Hq + g * G + hh) * D + q4 * 8;
#pragma unroll
      for (int c = 0; c < ND; ++c)
        qf[rt][c] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + c * 32));
    }
  }

  // ---------------------------------------------------------------- staging
  bool poison = bad;
  int pad_count = 0;
  if constexpr (MODE == kDraftGather) {
    const int v_end = min(t1 * kTileKeys, n_view);
    const int cnt = max(0, v_end - t0 * kTileKeys);
    const int32_t* ib = a.idx + b * a.idx_sb + g * a.idx_sh + t0 * kTileKeys;
    // -1 entries are padding: they stage row 0 (always addressable) and a
    // set bit in their tile's skip word, one ballot per 64 entries
    bool bi = false;
    for (int i0 = 0; i0 < cnt; i0 += 256) {
      const int i = i0 + tid;
      const int j = i < cnt ? ib[i] : 0;
      if (i < cnt) idx_s[i] = j == -1 ? 0 : j;
      bi |= (j < -1 || j >= L);
      const uint64_t skip = __ballot(i < cnt && j == -1);
      if ((tid & 63) == 0 && i < cnt) {
        padbits_s[i / kTileKeys] = (uint32_t)skip;
        if (i + kTileKeys < cnt) padbits_s[i / kTileKeys + 1] = (uint32_t)(skip >> 32);
      }
    }
    const bool bad_idx = __syncthreads_or(bi);
    if (bad_idx && tid == 0) raise_error(a.err, SPEC_DEV_INDEX);
    poison = poison || bad_idx;
    if (bad_idx) k1 = k0;   // never address a position outside the cache
  } else if constexpr (MODE == kVerify) {
    const int wend = min(t1, cache_tiles);
    int cnt = 0;
    if (a.pad != nullptr) {
      const uint8_t* prow = a.pad + b * a.pad_sb;
      for (int w = t0 + tid; w < wend; w += 256) {
        uint32_t bits = 0;
        const int key0 = w * kTileKeys;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int kk = key0 + 4 * k;
          if (kk < L) {
            const uint32_t d = *reinterpret_cast<const uint32_t*>(prow + kk);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (kk + e < L && ((d >> (8 * e)) & 0xffu)) bits |= 1u << (4 * k + e);
          }
        }
        padbits_s[w - t0] = bits;
        cnt += __popc(bits);
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) cnt += __shfl_xor(cnt, m, 64);
    if (lane == 0) red_s[wave] = cnt;
    __syncthreads();
    pad_count = red_s[0] + red_s[1] + red_s[2] + red_s[3];
  } else {
    __syncthreads();
  }

  // ---------------------------------------------------------------- tile copies
  KeySrc ks;
  ks.k = reinterpret_cast<const char*>(reinterpret_cast<const uint16_t*>(a.k) + b * a.kb + g * a.kh);
  ks.v = reinterpret_cast<const char*>(reinterpret_cast<const uint16_t*>(a.v) + b * a.kb + g * a.kh);
  ks.tk = ks.k;
  ks.tv = ks.v;
  ks.rowb = (uint32_t)(a.kt * 2);
  ks.trowb = ks.rowb;
  ks.kbytes = (uint32_t)min((int64_t)0xffffffff, (int64_t)max(a.capacity - 1, 0) * a.kt * 2 + 2 * D);
  ks.tbytes = ks.kbytes;
  if constexpr (MODE == kVerify) {
    ks.tk = reinterpret_cast<const char*>(reinterpret_cast<const uint16_t*>(a.tk) + b * a.tkb + g * a.tkh);
    ks.tv = reinterpret_cast<const char*>(reinterpret_cast<const uint16_t*>(a.tv) + b * a.tkb + g * a.tkh);
    ks.trowb = (uint32_t)(a.tkt * 2);
    ks.tbytes = (uint32_t)((int64_t)(N - 1) * a.tkt * 2 + 2 * D);
  }
  ks.idx = idx_s;
  ks.n_view = n_view;
  ks.cache_tiles = cache_tiles;
  ks.n_tree = N;
  ks.s_len = s_len;
  ks.w_start = w_start;
  ks.v0 = t0 * kTileKeys;
  ks.kv_ring = MODE == kDraftWindow ? a.kv_ring : 0;
  ks.n_sink = a.n_sink;
  const uint32_t ring_base = lds_addr(ring) + kgi * (WK == 1 ? NS : 1) * SB;
  const int wl = WK == 1 ? wave : 0;   // index of this wavefront among the loaders

  // ---------------------------------------------------------------- main loop
  // m starts at a finite stand-in for -inf: the first visible score of a row
  // then gives exp2(score - m) = +inf, which the growth test catches, while a
  // masked score (-inf) still gives 0 instead of the NaN of -inf - (-inf).
  constexpr float kNoMax = -1e30f;
  f32x4 acc[RT][NDT];
  float m[RT], lsum[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m[rt] = kNoMax;
    lsum[rt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float c2 = a.scale_log2;
  const bool row_masks = MODE != kVerify && T > 1;

  // LDS read addresses of this lane within stage 0 (loop invariant; the stage
  // and the second 16-key half are immediate offsets): K fragment chunk cc of
  // key row l16, and the V^T transpose read of d tile dt for keys 4*q4 + j.
  // Rows r and r + 16 share their swizzle.
  uint32_t koff[ND], voff[NDT];
#pragma unroll
  for (int cc = 0; cc < ND; ++cc)
    koff[cc] = ring_base + l16 * ROWB + (((cc * 4 + q4) ^ swz_k<D>(l16)) * 16);
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    const int r = 4 * q4 + (l16 >> 2);
    const int byte = (dt * 16 + 4 * (l16 & 3)) * 2;
    voff[dt] = ring_base + KB + r * ROWB + (((byte >> 4) ^ swz_v<D>(r)) << 4) + (byte & 15);
  }

  // Copies of a contiguous cache tile: this wavefront's DPW pieces all lie in
  // one region (K or V) and cover rows ii0*RPI .. of the tile, so one scalar
  // base per tile plus loop-invariant lane offsets address them.
  static_assert(WK != 1 || (Ge::DPT / 2) % DPW == 0, "a wavefront's pieces stay in one region");
  const int region = (wl * DPW) / (Ge::DPT / 2), ii0 = (wl * DPW) % (Ge::DPT / 2);
  const char* cbase = region ? ks.v : ks.k;
  const uint32_t m0w = ring_base + region * KB + ii0 * 1024;
  uint32_t vo[DPW];
#pragma unroll
  for (int u = 0; u < DPW; ++u) {
    const int rl = lane / CH, r = (ii0 + u) * RPI + rl;
    vo[u] = (uint32_t)((u * RPI + rl) * ks.rowb) +
            (uint32_t)(((lane % CH) ^ (region ? swz_v<D>(r) : swz_k<D>(r))) * 16);
  }
  // Issue tile tn into stage sn (WK = 1).
  auto issue = [&](int tn, int sn) __attribute__((always_inline)) {
    const int j0 = is_tree_tile(ks, tn, MODE) ? -1 : tile_first_row<MODE>(ks, tn);
    if (j0 >= 0) {
      const char* base = cbase + (size_t)(j0 + ii0 * RPI) * ks.rowb;
#pragma unroll
      for (int u = 0; u < DPW; ++u)
        copy16_to_lds_s(base, vo[u], (uint32_t)(m0w + sn * SB + u * 1024));
    } else {
      issue_tile<MODE, D, DPW>(ks, tn, ring_base + sn * SB, wl, lane);
    }
  };

  // With a shared ring (WK = 1) nothing but ring copies may be in flight
  // from here on.  The wait is the compiler's own intrinsic, so it knows the
  // query loads are complete and inserts no memory-counter wait inside the
  // loop (which, counting the ring copies too, would drain the prefetch
  // pipeline every tile).  The register-staged path (WK = 4) has only loads
  // the compiler tracks, so its first tile load is issued without waiting
  // for the query.
  if constexpr (WK == 1) __builtin_amdgcn_s_waitcnt(0);
  u32x4 stg[WK == 4 ? Ge::DPT : 1];
  if constexpr (WK == 1) {
#pragma unroll
    for (int u = 0; u < NS - 1; ++u)
      if (k0 + u < k1) issue(k0 + u, u);
  }
  // Register-staged splits (WK = 4) of long key ranges: each wave streams a
  // fixed run of about seven eighths of its share, then takes chunks of
  // a.dyn tiles from a pool shared by the (pair, row block) through an
  // arrival-style counter, so that waves on faster XCDs take over work of
  // slower ones.  A wave requests its next chunk right after issuing the
  // loads of its current run's last tile: memory operations complete in
  // order, so a request issued earlier would hold up every later tile wait.
  const bool dyn = WK == 4 && MODE != kDraftGather && a.dyn > 0;
  uint32_t* const c_cnt = a.cnt_chunk + (size_t)pair * a.n_rb + z;
  const int C = dyn ? a.dyn : 1;
  const int n_chunks = (total + C - 1) / C;
  const int wpp = a.splits * 4;                       // waves per (pair, row block)
  const int F = dyn ? (n_chunks * 7 / 8) / wpp : 0;   // fixed chunks per wave
  const int pool0 = wpp * F;                          // first pooled chunk
  int t_first = k0 < k1 ? k0 : -1, run_end = k1, c_next = 0;
  bool pending = false;   // a pool request is on its way
  auto request = [&]() __attribute__((always_inline)) {
    if (lane == 0) c_next = (int)__hip_atomic_fetch_add(c_cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    pending = true;
  };
  // first tile of the requested pool chunk, or -1
  auto take = [&]() __attribute__((always_inline)) -> int {
    const int c = pool0 + __builtin_amdgcn_readfirstlane(c_next);
    pending = false;
    if (c >= n_chunks) return -1;
    run_end = min((c + 1) * C, total);
    return c * C;
  };
  // Interleaved tiles (window drafts and verifies without padding, whose
  // splits stage nothing per key range): wave wi of the (pair, row block)
  // takes tiles wi, wi + wpp, wi + 2 wpp, ... of the fixed part, so that all
  // the waves of a (pair, row block) sweep its keys together and DRAM pages
  // are read by many waves at once (a wave streaming a range of its own
  // reads scattered pages: a plain HBM read runs about 20% slower that way);
  // the pool's chunks follow in memory order.
  const bool ileave = WK == 4 && (MODE == kDraftWindow || (MODE == kVerify && a.pad == nullptr));
  int tstep = 1;
  if (ileave) {
    const int wi = s * 4 + kgi;
    const int fixed_end = dyn ? min(pool0 * C, total) : total;
    tstep = wpp;
    run_end = fixed_end;
    if (wi < fixed_end) {
      t_first = wi;
    } else if (dyn && pool0 < n_chunks) {
      request();
      t_first = take();
      tstep = 1;
    } else {
      t_first = -1;
    }
  } else if (dyn) {
    const int wi = s * 4 + kgi;
    const int a0 = min(wi * F * C, total), a1 = min((wi + 1) * F * C, total);
    if (a0 < a1) {
      t_first = a0;
      run_end = a1;
    } else if (pool0 < n_chunks) {
      request();
      t_first = take();
    } else {
      t_first = -1;
    }
  }

  // One tile: scores, masks, online softmax and P.V for keys of tile t,
  // whose K and V rows sit at stage offset `so` of this wave's ring.
  const uint8_t* const pad_ptr = a.pad;
  const int n_sink_ = a.n_sink, window_ = a.window;
  auto tile_body = [&](const int t, const uint32_t so) __attribute__((always_inline)) {
    const bool tree_tile = MODE == kVerify && t >= cache_tiles;
    // This tile's pad word (verify), read before the fragment reads so that
    // waiting for it never waits for them; it is uniform, so the visibility
    // test below is a scalar branch.
    uint32_t pw = 0u;
    if constexpr (MODE == kVerify) {
      if (!tree_tile && pad_ptr != nullptr) pw = __builtin_amdgcn_readfirstlane(padbits_s[t - t0]);
    } else if constexpr (MODE == kDraftGather) {
      pw = __builtin_amdgcn_readfirstlane(padbits_s[t - t0]);
    }
    bool full = !tree_tile && (t + 1) * kTileKeys <= n_view && pw == 0u;
    if (row_masks) {
      // Several window-draft queries: a tile is visible to every row when
      // its last key precedes the first query (causal) and its window keys
      // lie inside the last query's window (the sink always is); most
      // window tiles are, and skip the per-row masks.  (view positions
      // increase within a tile; uniform scalar tests)
      bool all_rows = false;
      if constexpr (MODE == kDraftWindow) {
        const int v_first = t * kTileKeys, v_last = v_first + kTileKeys - 1;
        const int p_last = v_last < s_len ? v_last : w_start + (v_last - s_len);
        const int v_win = max(v_first, s_len);   // first window key of the tile
        all_rows = p_last < L - T + 1 &&
                   (v_win > v_last || w_start + (v_win - s_len) >= L - window_);
      }
      full = full && all_rows;
    }

    // K fragments (A operand of S^T): key h*16 + l16, head-dim chunk cc*4 + q4;
    // V^T fragments (A operand of O^T) of d tile dt.
    auto read_v = [&](int dt) __attribute__((always_inline)) {
      const s16x4 v0 = lds_read_tr16(voff[dt] + so);
      const s16x4 v1 = lds_read_tr16(voff[dt] + so + 16 * ROWB);
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // With up to two row tiles every fragment of the tile is read at once
    // (the V^T fragments' latency then hides behind the scores and the
    // softmax).  Three row tiles need those registers: K is read one 16-key
    // half at a time and V^T one half of the d tiles at a time, each read
    // issued behind independent MFMAs of the same wavefront.
    constexpr int NV = RT >= 3 ? NDT / 2 : NDT;   // V^T fragments held at once
    bf16x8 vf[NV];
    f32x4 sc[RT][2];
    if constexpr (RT >= 3) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        bf16x8 kh[ND];
#pragma unroll
        for (int cc = 0; cc < ND; ++cc) kh[cc] = lds_load_b128(koff[cc] + so + h * 16 * ROWB);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          f32x4 c = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int cc = 0; cc < ND; ++cc)
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh[cc], qf[rt][cc], c, 0, 0, 0);
          sc[rt][h] = c;
        }
      }
#pragma unroll
      for (int dt = 0; dt < NV; ++dt) vf[dt] = read_v(dt);
    } else {
      bf16x8 kf[2][ND];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int cc = 0; cc < ND; ++cc) kf[h][cc] = lds_load_b128(koff[cc] + so + h * 16 * ROWB);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) vf[dt] = read_v(dt);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          f32x4 c = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int cc = 0; cc < ND; ++cc)
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[h][cc], qf[rt][cc], c, 0, 0, 0);
          sc[rt][h] = c;
        }
    }

    // Visibility of this lane's 8 keys, local index e = h*4 + i, tile key
    // h*16 + q4*4 + i.  `full` tiles (every key visible to every row) skip it.
    uint32_t kmask = 0xffu;
    if (!tree_tile && !full) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kk = (e >> 2) * 16 + q4 * 4 + (e & 3);
        if (t * kTileKeys + kk >= n_view || ((pw >> kk) & 1u)) kmask &= ~(1u << e);
      }
    }
    int jpos[8];
    if (row_masks && !full) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kk = (e >> 2) * 16 + q4 * 4 + (e & 3);
        jpos[e] = view_pos<MODE>(ks, min(t * kTileKeys + kk, n_view - 1));
      }
    }

    // Scores of this lane's row, masked (-inf).
    float x[RT][8];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[rt][e] = sc[rt][e >> 2][e & 3];
      if (!full) {
        uint32_t rm = kmask;
        if (tree_tile) {
          const uint64_t an = erow[rt] >= 0 ? anc_s[erow[rt]] : 0ull;
          const uint32_t aw = (uint32_t)(an >> ((t - cache_tiles) * kTileKeys));
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int kk = (e >> 2) * 16 + q4 * 4 + (e & 3);
            if (!((aw >> kk) & 1u)) rm &= ~(1u << e);
          }
        } else if (row_masks) {
          const int er = erow[rt];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            bool vis = jpos[e] < er;
            if (MODE == kDraftWindow) vis = vis && (jpos[e] < n_sink_ || jpos[e] >= er - window_);
            if (!vis) rm &= ~(1u << e);
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) x[rt][e] = ((rm >> e) & 1u) ? x[rt][e] : -INFINITY;
      }
    }

    // p = 2^(score*c2 - m) against the running maximum m.  Lazy rescale:
    // m is raised only when some p of the wave exceeds 2^8 (a lane's sum
    // of p above 2^8 is the test: it holds whenever one p does), so every
    // p used is at most 2^8, safe in fp32 and bf16; the final o = acc / l
    // is the same either way.  The branch is wave-uniform and rare (at the
    // first visible key of a row and when scores climb by more than 8 in
    // log2 units), so the accumulators stay in the MFMA registers.
    float p[RT][8], ps[RT];
    bool grow = false;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      ps[rt] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[rt][e] = __builtin_amdgcn_exp2f(fmaf(x[rt][e], c2, -m[rt]));
        ps[rt] += p[rt][e];
      }
      grow = grow || ps[rt] > 256.f;
    }
    if (__builtin_expect(__any(grow), 0)) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        float mx = x[rt][0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mx = fmaxf(mx, x[rt][e]);
        mx = fmaxf(mx, shfl_xor(mx, 16));
        mx = fmaxf(mx, shfl_xor(mx, 32));
        const float mn = fmaxf(m[rt], mx * c2);
        const float alpha = __builtin_amdgcn_exp2f(m[rt] - mn);
        m[rt] = mn;
        lsum[rt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) acc[rt][dt] *= alpha;
        ps[rt] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[rt][e] = __builtin_amdgcn_exp2f(fmaf(x[rt][e], c2, -mn));
          ps[rt] += p[rt][e];
        }
      }
    }
    uint32_t pf[RT][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      lsum[rt] += ps[rt];
#pragma unroll
      for (int w = 0; w < 4; ++w) pf[rt][w] = pack_bf16x2(p[rt][2 * w], p[rt][2 * w + 1]);
    }

    // O^T += V^T . P^T (three row tiles: the second half of the V^T
    // fragments is read behind the first half's MFMAs)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      if (NV < NDT && dt == NV) {
#pragma unroll
        for (int d2 = 0; d2 < NV; ++d2) vf[d2] = read_v(NV + d2);
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const bf16x8 pb = __builtin_bit_cast(bf16x8, make_uint4(pf[rt][0], pf[rt][1], pf[rt][2], pf[rt][3]));
        acc[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt % NV], pb, acc[rt][dt], 0, 0, 0);
      }
    }
  };

  if constexpr (WK == 1) {
    // Unrolled by the ring depth, so that a tile's stage is a constant.
    for (int tb = k0; tb < k1; tb += NS) {
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        const int t = tb + st;
        if (t >= k1) break;
        wait_tiles<DPW, NS - 2>(k1 - 1 - t);
        barrier_only();   // every wave's copies of tile t landed; tile t-1 is consumed
        if (t + NS - 1 < k1) issue(t + NS - 1, (st + NS - 1) % NS);
        tile_body(t, st * SB);
      }
    }
  } else {
    // The wave's own stage: LDS operations of a wave execute in order, so
    // the stores of tile t land after the reads of tile t-1 and before its
    // own; the next tile's loads are in flight while tile t is used.
    // (a run's last tile is the one whose successor lies at or past run_end)
    int t = t_first;
    if (t >= 0) load_tile_regs<MODE, D>(ks, t, lane, stg);
    if (dyn && t >= 0 && t + tstep >= run_end && pool0 < n_chunks && !pending) request();
    while (t >= 0) {
      store_tile_lds<D>(ring_base, lane, stg);
      int tn = t + tstep;
      if (tn >= run_end) {
        tn = pending ? take() : -1;
        tstep = 1;   // pool chunks are contiguous
      }
      if (tn >= 0) load_tile_regs<MODE, D>(ks, tn, lane, stg);
      if (dyn && tn >= 0 && tn + tstep >= run_end && pool0 < n_chunks && !pending) request();
      tile_body(t, 0u);
      t = tn;
    }
  }

  // ---------------------------------------------------------------- positions
  if constexpr (MODE == kVerify) {
    if (a.pos_ids != nullptr && g == 0 && z == 0) {
      int n_pad = 0;
      bool write = false;
      if (a.pad == nullptr) {
        write = s == 0;
      } else {
        // every split of head 0 counted its own range; the last one writes
        uint32_t* cnt = a.cnt_pos + 2 * b;
        if (tid == 0 && pad_count)
          __hip_atomic_fetch_add(cnt + 1, (uint32_t)pad_count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        write = arrive_last(cnt, S_own);
        if (write && tid == 0)
          red_s[0] = (int)__hip_atomic_exchange(cnt + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        n_pad = red_s[0];
      }
      if (write && tid < N) a.pos_ids[(size_t)b * N + tid] = bad ? -1 : (L - n_pad) + dep_s[tid];
    }
  }

  // ---------------------------------------------------------------- results
  float lr[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    lr[rt] = lsum[rt];
    lr[rt] += shfl_xor(lr[rt], 16);
    lr[rt] += shfl_xor(lr[rt], 32);
  }
  const int So = S_own;      // splits of this pair that write a partial
  const size_t grp = (size_t)pair * a.n_rb + z;   // counters and block partials
  // split partials: o [S][RC][D], lse [S][RC] (log2 domain) per (pair, row
  // block), or, in the ordered verify, per (KV head, row block) with one
  // slot per work item
  const bool per_item = MODE == kVerify && WK == 1 && a.ordered;
  const int S = per_item ? a.items : a.splits;
  const size_t pgrp = per_item ? (size_t)g * a.n_rb + z : grp;
  const __amdgpu_buffer_rsrc_t o_rs = coherent_rsrc(a.o_part + pgrp * S * RC * D, (uint32_t)(S * RC * D * 4));
  const __amdgpu_buffer_rsrc_t l_rs = coherent_rsrc(a.lse_part + pgrp * S * RC, (uint32_t)(S * RC * 4));
  const int R = a.R, Hq = a.Hq;
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
  float* lse_out = a.lse;

  // store one row's result: final output (S == 1) or this split's partial
  auto store_row = [&](int row_l, int d0, const float* vals, bool lse_lane, float lse2)
                       __attribute__((always_inline)) {
    const int row = z * RC + row_l;
    if (row >= R) return;
    if (So > 1) {
      store_sc1_f4(o_rs, (uint32_t)(((pslot * RC + row_l) * D + d0) * 4), f32x4{vals[0], vals[1], vals[2], vals[3]});
      if (lse_lane) store_sc1_f1(l_rs, (uint32_t)((pslot * RC + row_l) * 4), lse2);
      return;
    }
    const int t = row / G, hh = row % G;
    const size_t oi = ((size_t)b * T + t) * Hq + g * G + hh;
    *reinterpret_cast<uint2*>(out + oi * D + d0) =
        make_uint2(pack_bf16x2(vals[0], vals[1]), pack_bf16x2(vals[2], vals[3]));
    if (lse_lane && lse_out != nullptr) lse_out[oi] = lse2 * kLn2;
  };

  if constexpr (WK == 1) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float inv, lse2;
      if (poison) {
        inv = NAN;
        lse2 = NAN;
      } else if (lr[rt] > 0.f) {
        inv = 1.f / lr[rt];
        lse2 = m[rt] + log2f(lr[rt]);
      } else {
        inv = 0.f;
        lse2 = -INFINITY;
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        float vals[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) vals[e] = poison ? NAN : acc[rt][dt][e] * inv;
        store_row(rg * RCW + rt * 16 + l16, dt * 16 + q4 * 4, vals, q4 == 0 && dt == 0, lse2);
      }
    }
  } else {
    // merge the four wavefronts' running states through LDS (rows past the
    // last one are neither written nor merged)
    __syncthreads();
    float* ms = reinterpret_cast<float*>(ring);   // [4][RC]
    float* ls = ms + 4 * RC;                      // [4][RC]
    float* os = ls + 4 * RC;                      // [4][RC][D]
    const int rows_live = min(RC, a.R - z * RC);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int rl = rt * 16 + l16;
      if (rl >= rows_live) continue;
      if (q4 == 0) {
        ms[wave * RC + rl] = m[rt];
        ls[wave * RC + rl] = lr[rt];
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        *reinterpret_cast<f32x4*>(os + ((size_t)wave * RC + rl) * D + dt * 16 + q4 * 4) = acc[rt][dt];
    }
    __syncthreads();
    for (int it = tid; it < rows_live * (D / 4); it += 256) {
      const int rl = it / (D / 4), d0 = (it % (D / 4)) * 4;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < 4; ++w) M = fmaxf(M, ms[w * RC + rl]);
      float W = 0.f, o[4] = {0.f, 0.f, 0.f, 0.f};
      if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float f = __builtin_amdgcn_exp2f(ms[w * RC + rl] - M);
          W += f * ls[w * RC + rl];
          const f32x4 ov = *reinterpret_cast<const f32x4*>(os + ((size_t)w * RC + rl) * D + d0);
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] += f * ov[e];
        }
      }
      float lse2;
      if (poison) {
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = NAN;
        lse2 = NAN;
      } else if (W > 0.f) {
        const float inv = 1.f / W;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] *= inv;
        lse2 = M + log2f(W);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = 0.f;
        lse2 = -INFINITY;
      }
      store_row(rl, d0, o, d0 == 0, lse2);
    }
  }
  if (So == 1) return;

  // ---------------------------------------------------------------- split merge
  // Two levels: the last of each block of up to kMergeFan splits merges the
  // block; with more than one block, the last block merger merges the block
  // results.  Every merge reads at most kMergeFan partials.
  const int rows = min(RC, a.R - z * RC);
  const int nb = (So + kMergeFan - 1) / kMergeFan;   // merge blocks of this pair
  const int blk = s / kMergeFan, bsz = min(kMergeFan, So - blk * kMergeFan);
  auto final_sink = [&](int rl, int d0, const float* o, float lse2) __attribute__((always_inline)) {
    const int row = z * RC + rl;
    const int t = row / G, hh = row % G;
    const size_t oi = ((size_t)b * T + t) * Hq + g * G + hh;
    *reinterpret_cast<uint2*>(out + oi * D + d0) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
    if (d0 == 0 && lse_out != nullptr) lse_out[oi] = lse2 * kLn2;
  };
  if (!arrive_last(a.cnt_l0 + grp * a.n_blk + blk, bsz)) return;
  // The (pair, row block)'s final merger: every split has arrived, so no
  // wave grabs chunks any more and the chunk counter can start over.
  auto reset_chunks = [&]() __attribute__((always_inline)) {
    if (a.dyn > 0 && tid == 0) __hip_atomic_store(c_cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  if (nb == 1) {
    reset_chunks();
    merge_partials<D, RC>(o_rs, l_rs, pslot0, So, rows, final_sink);
    return;
  }
  const __amdgpu_buffer_rsrc_t o1_rs = coherent_rsrc(a.o_part1 + grp * a.n_blk * RC * D, (uint32_t)(a.n_blk * RC * D * 4));
  const __amdgpu_buffer_rsrc_t l1_rs = coherent_rsrc(a.lse_part1 + grp * a.n_blk * RC, (uint32_t)(a.n_blk * RC * 4));
  merge_partials<D, RC>(o_rs, l_rs, pslot0 + blk * kMergeFan, bsz, rows,
                        [&](int rl, int d0, const float* o, float lse2) __attribute__((always_inline)) {
                          store_sc1_f4(o1_rs, (uint32_t)(((blk * RC + rl) * D + d0) * 4), f32x4{o[0], o[1], o[2], o[3]});
                          if (d0 == 0) store_sc1_f1(l1_rs, (uint32_t)((blk * RC + rl) * 4), lse2);
                        });
  if (!arrive_last(a.cnt_l1 + grp, nb)) return;
  reset_chunks();
  merge_partials<D, RC>(o1_rs, l1_rs, 0, nb, rows, final_sink);
}

// ------------------------------------------------------------------ launch

template <int MODE, int D, int RT, int WK>
static hipError_t launch_shape(const AttnArgs& a, hipStream_t st) {
  constexpr int NS = WK == 1 ? 4 : 1;
  int64_t grid = a.units;
  if (a.n_rb > 1) grid = cdiv(a.units, 8) * 8 * a.n_rb;
  hipLaunchKernelGGL((attn_bf16_kernel<MODE, D, RT, WK, NS>), dim3((unsigned)grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int MODE, int D>
static hipError_t launch_mode(const AttnArgs& a, const Plan& p, hipStream_t st) {
  if (p.wk == 4) {
    if (p.rt == 1) return launch_shape<MODE, D, 1, 4>(a, st);
    return launch_shape<MODE, D, 2, 4>(a, st);
  }
  if (p.rt == 1) return launch_shape<MODE, D, 1, 1>(a, st);
  if (p.rt == 3) return launch_shape<MODE, D, 3, 1>(a, st);
  return launch_shape<MODE, D, 2, 1>(a, st);
}

hipError_t launch_attn_bf16(const AttnArgs& a, int mode, const Plan& p, hipStream_t st) {
  if (a.D == 128) {
    if (mode == kDraftWindow) return launch_mode<kDraftWindow, 128>(a, p, st);
    if (mode == kDraftGather) return launch_mode<kDraftGather, 128>(a, p, st);
    return launch_mode<kVerify, 128>(a, p, st);
  }
  if (mode == kDraftWindow) return launch_mode<kDraftWindow, 64>(a, p, st);
  if (mode == kDraftGather) return launch_mode<kDraftGather, 64>(a, p, st);
  return launch_mode<kVerify, 64>(a, p, st);
}

}  // namespace spec
