// Internal declarations shared by the HIP sources of libspecattn (gfx950).
//
// Work decomposition of the attention kernels: a "pair" is one (sequence b,
// KV head g).  The query rows that read that KV head are r = t*G + hh (draft:
// query t, head g*G+hh) or r = i*G + hh (verify: tree node i).  A pair's rows
// are cut into row blocks and its key sequence into `splits` contiguous
// ranges of 32-key tiles (split-K flash-decode).  One workgroup handles one
// (pair, row block, split) and writes an fp32 partial: o normalised by its own
// softmax sum and the log2-domain sum-exp.  The workgroup that finishes a
// (pair, row block) last merges the partials into the final output, so every
// call is a single kernel launch.  With one split the workgroup writes the
// output directly.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "spec_attn.h"

namespace spec {

constexpr size_t kHeaderBytes = 256;           // [0,4): device error word
// Workspace layout shared by every call: the header, then a counter region
// of fixed size (arrival counters, chunk pools; every call leaves the words
// it uses at zero), then the call's own scratch (split partials, scores,
// slice summaries).  Because no call's scratch ever overlaps any call's
// counters, one zero-filled workspace serves any sequence of calls on a
// stream, whatever their shapes and kinds.
constexpr size_t kCounterBytes = size_t(1) << 20;
constexpr size_t kCounterWords = kCounterBytes / 4;
constexpr size_t kScratchOff = kHeaderBytes + kCounterBytes;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kMaxNodes = 64;                  // one uint64 ancestor mask per node
constexpr int kTileKeys = 32;                  // keys per KV tile
constexpr int kMaxGatherKeys = 2048;           // budget indices one workgroup stages in LDS
constexpr int kMaxPadWords = 1024;             // 32-key pad words one workgroup stages in LDS
constexpr int kMergeFan = 16;                  // partials one split-merge step reads
constexpr int kMaxSplits = kMergeFan * kMergeFan;
constexpr int kMinPoolGroups = 8;             // (pair, row block) groups that make a chunk pool pay
constexpr int kChunkTiles = 8;                 // tiles per dynamically taken chunk
constexpr int kMaxOrderBatch = 256;            // tree verify: longest-first work order up to this batch
constexpr int kOrderTiles = 64;                // tree verify (ordered): the finest split the plan allows, in tiles
constexpr int kCompactSlices = 64;             // pad-scan workgroups per sequence (compaction)
constexpr int kCompactScanSlots = 65536;       // compaction: longer pad rows are scanned in slices
constexpr int kMaxSelectBlocks = 8192;         // candidate blocks one selection scores
constexpr int kMaxSelect = 2048;               // blocks one selection may choose
constexpr int kMaxRows = 1 << 16;              // query rows (tokens x GQA group) per (sequence, KV head)

enum Mode : int { kDraftWindow = 0, kDraftGather = 1, kVerify = 2 };

// Everything a workgroup of an attention kernel needs, passed by value.
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
  int32_t kv_ring;                  // > 0: the window is read through a ring of this many slots
  const int32_t* idx;
  int32_t budget;
  int64_t idx_sb, idx_sh;
  // verify
  const uint8_t* pad;
  int64_t pad_sb;
  const void* tk;
  const void* tv;
  int64_t tkb, tkh, tkt;
  const int32_t* parents;
  int64_t par_sb;
  int32_t* pos_ids;
  const uint64_t* anc;    // fp32 path: [B][N] ancestor-or-self masks (workspace)
  const int32_t* bad;     // fp32 path: [B] nonzero = sequence rejected by the prep kernel
  // decomposition
  int32_t rb, n_rb, splits;
  int32_t chunk;          // fp32 path: keys per split
  int32_t tps;            // bf16 path: tiles per split
  int32_t units;          // bf16 path: pairs * splits
  // outputs
  float* o_part;          // [pair][n_rb][splits][rb][D]; ordered: [Hkv][n_rb][items][rb][D]
  float* lse_part;        // [pair][n_rb][splits][rb]   (log2 domain; ordered: by item)
  float* o_part1;         // bf16 path: [pair][n_rb][n_blk][rb][D] block merges
  float* lse_part1;       // bf16 path: [pair][n_rb][n_blk][rb]
  int32_t n_blk;          // bf16 path: ceil(splits / kMergeFan)
  uint32_t* cnt_l0;       // [pair][n_rb][n_blk] arrival counters (zero between calls)
  uint32_t* cnt_l1;       // [pair][n_rb]
  uint32_t* cnt_pos;      // [B][2] pad-count arrival (verify positions)
  uint32_t* cnt_chunk;    // bf16 path: [pair][n_rb] next tile chunk (dynamic splits)
  int32_t dyn;            // bf16 path: tiles per dynamically taken chunk, 0 = fixed ranges
  int32_t ordered;        // bf16 tree verify: balanced splits, longest first (see the kernel)
  int32_t items;          // ordered: work items per (KV head, row block); partial slots per group
  int32_t conc;           // ordered: workgroups per (KV head, row block) that run at once
  int32_t tps_max;        // ordered: the most tiles one split may take (its staged pad words)
  void* out;              // final output
  float* lse;             // final lse (natural log) or null
  uint32_t* err;          // device error word
};

struct Plan {
  int32_t rows = 0, rb = 0, n_rb = 0, splits = 0, chunk = 0, tps = 0;
  int32_t rt = 0, wk = 0;   // bf16 kernel shape: 16-row MFMA tiles per wave, key groups
  size_t cnt_off = 0, o_off = 0, lse_off = 0, o1_off = 0, lse1_off = 0, anc_off = 0, bad_off = 0,
         total = 0;
  int32_t n_blk = 1;
  int32_t dyn = 0;          // tiles per dynamically taken chunk (0: fixed split ranges)
  int32_t ordered = 0;      // tree verify in longest-first order (see AttnArgs)
  int32_t items = 0, conc = 0, tps_max = 0;   // ordered only
};

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Tiles [t0, t1) of split s when a (sequence, KV head) has `total` tiles and
// every split takes `tps` (the attention kernel and the host-side plan
// checker of the debug build compute it the same way).
__host__ __device__ inline void split_tiles(int total, int tps, int s, int& t0, int& t1) {
  t0 = s * tps < total ? s * tps : total;
  t1 = t0 + tps < total ? t0 + tps : total;
}
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Arguments of the KV commit kernel (byte strides; validated by the caller).
struct CommitArgs {
  char* k;
  char* v;
  int64_t c_sb, c_sh, c_st;            // cache strides in bytes
  const char* tk;
  const char* tv;
  int64_t t_sb, t_sh, t_st;            // tree strides in bytes
  int32_t batch, n_kv_heads, row_chunks, capacity, n_nodes, max_depth;
  int32_t* cache_len;
  uint8_t* pad;
  int64_t pad_sb;
  const int32_t* accept_len;
  const int32_t* accept_path;
  int32_t* n_appended;
  uint32_t* err;
};

// Arguments of the compaction kernels (byte strides; validated by the caller).
struct CompactArgs {
  char* k;
  char* v;
  int64_t c_sb, c_sh, c_st;            // cache strides in bytes
  int32_t batch, n_kv_heads, row_chunks, capacity, sliced;
  int32_t* cache_len;
  uint8_t* pad;
  int64_t pad_sb;
  int32_t* summary;                    // [B][kCompactSlices][2] in the workspace: each slice's first pad slot, pad count
  uint32_t* err;
};

// Arguments of the block-mean kernel (byte strides; validated by the caller).
struct MeansArgs {
  const char* k;
  int64_t k_sb, k_sh, k_st;
  int32_t bf16, head_dim, row_chunks, batch, n_kv_heads, capacity;
  int32_t block, first_block, n_blocks, max_blocks;
  const int32_t* cache_len;
  const uint8_t* pad;
  int64_t pad_sb;
  float* means;                        // [B][Hkv][max_blocks][D]
  uint32_t* err;
};

// Arguments of the block selection kernel.
struct SelectArgs {
  const void* q;                       // [B][T][Hq][D]
  int32_t bf16, T, Hq, G, head_dim, batch, n_kv_heads, capacity;
  const float* means;                  // [B][Hkv][max_blocks][D]
  int32_t max_blocks, block, n_sink, window, n_select, budget, shared;
  const int32_t* cache_len;
  const uint8_t* pad;
  int64_t pad_sb;
  int32_t* idx;                        // [B][Hkv][budget]
  float* scores;                       // [B][Hkv][max_blocks] or null
  float* sc_ws;                        // [B][Hkv][max_blocks] workspace scores
  uint32_t* err;
};

// Arguments of the partial-cache gather kernel (byte strides).
struct GatherArgs {
  const char* k;
  const char* v;
  int64_t c_sb, c_sh, c_st;
  char* pk;
  char* pv;
  int64_t p_sb, p_sh, p_st;
  int32_t batch, n_kv_heads, row_chunks, budget, capacity;
  const int32_t* cache_len;
  const int32_t* idx;                  // [B][budget] (one list per sequence)
  int64_t idx_sb;
  int32_t* partial_len;
  uint8_t* partial_pad;
  int64_t pad_sb;
  uint32_t* err;
};

// The tree verify behind spec_attn_verify_tree: validation, planning and
// launches.  With need != NULL the required workspace bytes are stored
// there once the arguments are valid, and a NULL workspace launches nothing.
spec_status verify_impl(const spec_dims* dims, const void* q, int32_t n_nodes,
                        const spec_kv* cache, const int32_t* cache_len,
                        const uint8_t* pad_or_null, int64_t pad_stride_b, const spec_kv* tree,
                        const int32_t* parents, int64_t parents_stride_b, void* out,
                        float* lse_or_null, int32_t* pos_ids_or_null, void* workspace,
                        size_t workspace_bytes, void* stream, size_t* need);

// Sets the thread-local message of spec_last_error() and returns `s`.
spec_status set_error(spec_status s, const char* msg);

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error; arguments were validated.
hipError_t launch_attn_bf16(const AttnArgs& a, int mode, const Plan& p, hipStream_t st);
hipError_t launch_verify_prep(const AttnArgs& a, const int32_t* parents, int64_t parents_sb,
                              int32_t* pos_ids, uint64_t* anc_ws, int32_t* bad_ws,
                              hipStream_t st);
hipError_t launch_attn_f32(const AttnArgs& a, int mode, hipStream_t st);
hipError_t launch_combine(const AttnArgs& a, int dtype, hipStream_t st);
hipError_t launch_accept(int B, int N, int V, const float* logits, const int32_t* tokens,
                         const int32_t* parents, int64_t parents_sb, int max_depth,
                         int32_t* accept_len, int32_t* accept_path, int32_t* bonus,
                         void* ws, int vsplits, int two_level, hipStream_t st, uint32_t* err);
hipError_t launch_kv_commit(const CommitArgs& a, hipStream_t st);
hipError_t launch_kv_compact(const CompactArgs& a, hipStream_t st);
hipError_t launch_block_means(const MeansArgs& a, hipStream_t st);
hipError_t launch_select_blocks(const SelectArgs& a, hipStream_t st);
hipError_t launch_kv_gather(const GatherArgs& a, hipStream_t st);

}  // namespace spec
