// Internal declarations shared by the HIP sources of libspecattn (gfx950).
//
// Work decomposition (all three attention kernels): a "pair" is one
// (sequence b, KV head g).  The query rows that read that KV head are
// r = t*G + hh (draft: query t, head g*G+hh) or r = i*G + hh (verify: node i).
// Rows are cut into row blocks of `rb` rows and the key sequence of a pair
// into `splits` contiguous chunks of `chunk` keys (split-K flash-decode).
// Each (pair, row block, split) is one wavefront; it writes an fp32 partial
// (o normalised by its own softmax sum, and its log2-domain sum-exp) that the
// combine kernel merges.  With a single split the wavefront writes the final
// output directly.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "spec_attn.h"

namespace spec {

constexpr size_t kHeaderBytes = 256;           // [0,4): device error word
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kMaxNodes = 64;                  // one uint64 ancestor mask per node

enum Mode : int { kDraftWindow = 0, kDraftGather = 1, kVerify = 2 };

// Everything a wavefront of an attention kernel needs, passed by value.
struct AttnArgs {
  // tensors
  const void* q;          // [B][T][Hq][D]
  const void* k;          // cache K, strides kb/kh/kt (elements)
  const void* v;
  int64_t kb, kh, kt;
  int32_t capacity;
  const int32_t* cache_len;
  // shape
  int32_t B, Hq, Hkv, G, D, T, R;   // T = Tq (draft) or N (verify); R = T*G
  float scale_log2;                 // softmax_scale * log2(e)
  // draft
  int32_t n_sink, window;
  const int32_t* idx;
  int32_t budget;
  int64_t idx_sb, idx_sh;
  // verify
  const uint8_t* pad;
  int64_t pad_sb;
  const void* tk;
  const void* tv;
  int64_t tkb, tkh, tkt;
  const uint64_t* anc;    // [B][N] ancestor-or-self masks (workspace)
  const int32_t* bad;     // [B] nonzero = sequence rejected by the prep kernel
  // decomposition
  int32_t rb, n_rb, splits, chunk;
  // outputs
  float* o_part;          // [pair][n_rb][splits][rb][D]
  float* lse_part;        // [pair][n_rb][splits][rb]   (log2 domain)
  void* out;              // final output when splits == 1
  float* lse;             // final lse (natural log) or null
  uint32_t* err;          // device error word
};

struct Plan {
  int32_t rows = 0, rb = 0, n_rb = 0, splits = 0, chunk = 0;
  size_t o_off = 0, lse_off = 0, anc_off = 0, bad_off = 0, total = 0;
};

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Split-K plan: enough wavefronts to keep 256 CUs busy, at least `min_keys`
// keys per split, chunk a multiple of `tile`.
inline void plan_splits(Plan& p, int64_t pairs, int64_t keys, int64_t min_keys, int64_t tile,
                        int64_t target_waves) {
  if (keys < 1) keys = 1;
  int64_t units = pairs * p.n_rb;
  int64_t s = cdiv(target_waves, units > 0 ? units : 1);
  int64_t smax = cdiv(keys, min_keys);
  if (s > smax) s = smax;
  if (s < 1) s = 1;
  int64_t chunk = cdiv(cdiv(keys, s), tile) * tile;
  p.chunk = (int32_t)chunk;
  p.splits = (int32_t)cdiv(keys, chunk);
}

inline void plan_partials(Plan& p, int64_t pairs, int D) {
  size_t off = kHeaderBytes;
  if (p.splits > 1) {
    size_t n = (size_t)pairs * p.n_rb * p.splits * p.rb;
    p.o_off = off;
    off = align_up(off + n * D * sizeof(float), 256);
    p.lse_off = off;
    off = align_up(off + n * sizeof(float), 256);
  }
  p.total = off;
}

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error; arguments were validated.
hipError_t launch_draft(const AttnArgs& a, int dtype, hipStream_t st);
hipError_t launch_verify(const AttnArgs& a, int dtype, const int32_t* parents,
                         int64_t parents_sb, int32_t* pos_ids, uint64_t* anc_ws,
                         int32_t* bad_ws, hipStream_t st);
hipError_t launch_combine(const AttnArgs& a, int dtype, hipStream_t st);
hipError_t launch_accept(int B, int N, int V, const float* logits, const int32_t* tokens,
                         const int32_t* parents, int64_t parents_sb, int max_depth,
                         int32_t* accept_len, int32_t* accept_path, int32_t* bonus,
                         void* ws, int vsplits, hipStream_t st, uint32_t* err);

}  // namespace spec
