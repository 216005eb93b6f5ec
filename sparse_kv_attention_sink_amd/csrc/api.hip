// C ABI of libspecattn: argument validation, split planning and launches.
// Every host-visible argument is checked before the first launch; the
// kernels check the values that live only on the device.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <string>
#include <vector>

#include "spec_internal.h"

using namespace spec;

namespace {

thread_local std::string g_err;

spec_status fail(spec_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

spec_status hip_fail(hipError_t e, const char* what) {
  return fail(SPEC_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int64_t esize(int dtype) { return dtype == SPEC_BF16 ? 2 : 4; }

constexpr int64_t kTargetWaves = 2048;     // 256 CUs x 8 wavefronts
constexpr int64_t kTargetWorkgroups = 512;  // 256 CUs x 2 workgroups of 4 wavefronts
constexpr int64_t kMaxGrid = 0x7fffffff;

spec_status check_dims(const spec_dims* d) {
  if (d == nullptr) return fail(SPEC_E_INVALID, "dims is NULL");
  if (d->batch < 0) return fail(SPEC_E_INVALID, "batch %d < 0", d->batch);
  if (d->n_q_heads < 1 || d->n_kv_heads < 1)
    return fail(SPEC_E_INVALID, "head counts must be >= 1 (Hq=%d, Hkv=%d)", d->n_q_heads, d->n_kv_heads);
  if (d->n_q_heads % d->n_kv_heads != 0)
    return fail(SPEC_E_INVALID, "Hq=%d is not a multiple of Hkv=%d", d->n_q_heads, d->n_kv_heads);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(SPEC_E_UNSUPPORTED, "head_dim %d (supported: 64, 128)", d->head_dim);
  if (d->dtype != SPEC_F32 && d->dtype != SPEC_BF16)
    return fail(SPEC_E_UNSUPPORTED, "dtype %d (supported: SPEC_F32, SPEC_BF16)", d->dtype);
  if (!(d->softmax_scale > 0.f) || !isfinite(d->softmax_scale))
    return fail(SPEC_E_INVALID, "softmax_scale must be finite and > 0");
  if (d->flags & ~(uint32_t)SPEC_FLAG_DETERMINISTIC)
    return fail(SPEC_E_INVALID, "unknown flag bits 0x%x", d->flags & ~(uint32_t)SPEC_FLAG_DETERMINISTIC);
  return SPEC_OK;
}

spec_status check_kv(const spec_kv* kv, const spec_dims* d, const char* name, bool need_cap) {
  if (kv == nullptr) return fail(SPEC_E_INVALID, "%s is NULL", name);
  if (kv->k == nullptr || kv->v == nullptr) return fail(SPEC_E_INVALID, "%s.k / %s.v is NULL", name, name);
  if (!aligned(kv->k, 16) || !aligned(kv->v, 16))
    return fail(SPEC_E_INVALID, "%s.k / %s.v must be 16-byte aligned", name, name);
  const int64_t m = d->dtype == SPEC_BF16 ? 8 : 4;
  if (kv->stride_b < 0 || kv->stride_h < 0 || kv->stride_t < d->head_dim)
    return fail(SPEC_E_INVALID, "%s strides (%lld, %lld, %lld) invalid for head_dim %d", name,
                (long long)kv->stride_b, (long long)kv->stride_h, (long long)kv->stride_t, d->head_dim);
  if (kv->stride_b % m || kv->stride_h % m || kv->stride_t % m)
    return fail(SPEC_E_INVALID, "%s strides must be multiples of %lld elements", name, (long long)m);
  if (need_cap && kv->capacity < 0) return fail(SPEC_E_INVALID, "%s.capacity %d < 0", name, kv->capacity);
  // kernels address a (sequence, head)'s rows with 32-bit byte offsets
  if (kv->stride_t * (int64_t)esize(d->dtype) * 64 > INT32_MAX)
    return fail(SPEC_E_UNSUPPORTED, "%s.stride_t %lld is too large", name, (long long)kv->stride_t);
  if (need_cap && ((int64_t)std::max(kv->capacity, 1) - 1) * kv->stride_t * esize(d->dtype) +
                      (int64_t)d->head_dim * esize(d->dtype) > (int64_t)UINT32_MAX)
    return fail(SPEC_E_UNSUPPORTED, "%s: capacity x stride_t spans more than 4 GiB per head", name);
  return SPEC_OK;
}

// ------------------------------------------------------------ planning

// Shape and split plan of the bf16 attention kernel (and workspace layout).
// `tiles` is the largest number of 32-key tiles a (sequence, KV head) can
// have; `gather` / `verify` bound the per-workgroup key range by what the
// kernel stages in LDS (budget indices, pad bits).
Plan bf16_plan(const spec_dims* d, int32_t T, int64_t tiles, bool gather, bool verify) {
  Plan p;
  const int G = d->n_q_heads / d->n_kv_heads;
  const int64_t pairs = (int64_t)d->batch * d->n_kv_heads;
  if ((int64_t)T * G > kMaxRows) return p;   // total 0: refused
  p.rows = T * G;
  if (p.rows <= 32) {           // few rows: four private rings per workgroup
    p.wk = 4;
    // Up to 32 rows fit one row block (two 16-row tiles per wavefront, one
    // workgroup per CU by registers).  With few (sequence, KV head) pairs the
    // grid is small, and two 16-row blocks, two workgroups per CU, finish
    // sooner (the 4K chain of 5: 19.7 -> 17.1 us); with many pairs, the second
    // block's reads of the same tiles cost more (the 16K batch-8 chain of 5:
    // 112 -> 142 us).
    p.rt = (pairs <= 16) ? 1 : (int32_t)cdiv(p.rows, 16);
    p.rb = 16 * p.rt;
  } else {                      // many rows: one shared ring, 4 x 16*rt rows
    // Up to 128 rows take one or two 16-row tiles per wavefront, more rows
    // row blocks of 128 or 192 (two or three tiles per wavefront; four would
    // need more registers than two wavefronts per SIMD allow).  Every row
    // block reads every tile, and three tiles per wavefront cost more per
    // (row, key) than two (about 17% more cycles per MFMA flop on the
    // ragged batch of 16), so blocks of 192 are taken where
    // they save a block and were measured to pay: 129 to 192 rows (a
    // 44-node tree with 4 query heads per KV head: 176; the 16K batch of 8:
    // 159.4 -> 148.8 us, the ragged batch of 16: 321.7 -> 295.0 us) and 257
    // to 384 rows (44 nodes with 8 query heads per KV head: 352; the 16K
    // batch of 8: 292.8 -> 227.4 us).  512 rows keep four blocks of 128
    // (three of 192: 284.8 -> 390.3 us).
    p.wk = 1;
    if (p.rows <= 128) {
      p.rt = (int32_t)cdiv(p.rows, 64);
    } else {
      p.rt = (p.rows <= 192 || (p.rows > 256 && p.rows <= 384)) ? 3 : 2;
    }
    p.rb = 64 * p.rt;
  }
  p.n_rb = (int32_t)cdiv(p.rows, p.rb);
  if (tiles < 1) tiles = 1;
  const int64_t groups = std::max<int64_t>(1, pairs * p.n_rb);
  // Budget gathers aim at half as many wavefronts: each split stages its own
  // index range and adds a partial to merge, and one workgroup per CU finishes
  // sooner (budgets 1024 / 2048 of the 16K batch of 8: 15.0 -> 14.1 and
  // 20.2 -> 18.8 us per call, device time; a batch-1 budget of 4096 keeps its
  // splits).
  const int64_t waves = gather ? kTargetWaves / 2 : kTargetWaves;
  int64_t S = p.wk == 4 ? std::min(cdiv(waves, groups * 4), cdiv(tiles, 4))
                        : std::min(cdiv(kTargetWorkgroups, groups), tiles);
  // More splits than one merge step reads only when each split streams at
  // least 32 tiles: a second merge level costs a few microseconds, which
  // only a long split amortises.
  S = std::min(S, std::max<int64_t>(kMergeFan, cdiv(tiles, 32)));
  int64_t lo = 1;
  if (gather) lo = std::max(lo, cdiv(tiles, kMaxGatherKeys / kTileKeys));
  if (verify) lo = std::max(lo, cdiv(tiles, kMaxPadWords));
  // A draft whose (sequence, KV head) spans at most 8 tiles runs as one
  // split: its four wavefronts stream up to two tiles each, which costs less
  // than the cross-workgroup merge a second split brings (a budget of 256 of
  // the 16K batch of 8: 10.2 -> 8.0 us per call, device time).  With 16
  // tiles (a budget of 512) four tiles per wavefront cost more than the
  // merge: 11.1 -> 10.2 us split.
  if (p.wk == 4 && !verify && tiles <= 8) S = 1;
  // Window drafts take at most 12 splits: the final merge reads every
  // split's partial, and with 12 splits the deepest wavefront still streams
  // as many tiles as with 16 (the 1M drafts' 129 tiles over 8 KV heads, in
  // device time: 3 queries 13.8 -> 13.3 us, 1 query 10.8 -> 10.7 us; 8, 10,
  // 11 and 14 splits measured slower than 12).
  if (p.wk == 4 && !verify && !gather) S = std::min<int64_t>(S, 12);
  // A tree verify sizes its splits on the device from the sequences' own
  // lengths (see the kernel), at most S per sequence: S allows splits of
  // kOrderTiles tiles over the capacity (up to one merge level of 16), so
  // that a ragged batch's long sequences spread over as many workgroups as
  // balance needs, and at most 384 tiles per split beyond.
  if (verify && p.wk == 1 && d->batch <= kMaxOrderBatch) {
    p.ordered = 1;
    S = std::max({S, std::min<int64_t>(kMergeFan, cdiv(tiles, kOrderTiles)), cdiv(tiles, 384)});
  }
  S = std::min<int64_t>(std::max(S, lo), kMaxSplits);
  if (S < lo) {
    p.total = 0;
    return p;
  }
  // The counters (two per sequence, n_blk + 2 per (pair, row block)) must
  // fit the workspace's fixed counter region; a second merge level is
  // given up before the shape is refused.
  const auto counter_words = [&](int64_t splits) {
    return 2 * (int64_t)std::max(0, d->batch) + groups * (cdiv(splits, kMergeFan) + 2);
  };
  if (counter_words(S) > (int64_t)kCounterWords) S = std::min<int64_t>(S, kMergeFan);
  if (S < lo || counter_words(S) > (int64_t)kCounterWords) {
    p.total = 0;
    return p;
  }
  p.tps = (int32_t)cdiv(tiles, S);
  p.splits = (int32_t)cdiv(tiles, p.tps);
  p.n_blk = (int32_t)cdiv(p.splits, kMergeFan);
  if (p.ordered) {
    // The device takes the smallest T <= tps_max (tiles per split) whose
    // splits, min(splits, ceil(tiles_b / T)) for sequence b, number at most
    // conc, searching up to ceil(W / (conc - B)) (W the batch's tiles), and
    // the largest candidate if none does.  The work items per (KV head, row
    // block) bound those splits from the capacity alone: conc when even
    // T = tps_max gives at most conc splits, or when the search's upper end
    // stays within tps_max (there ceil() adds at most one split per
    // sequence to W / T <= conc - B); conc + B while the batch's tiles stay
    // within conc * tps_max (then W / tps_max + B); otherwise one per
    // (sequence, split).
    p.conc = (int32_t)std::max<int64_t>(1, kTargetWorkgroups / ((int64_t)d->n_kv_heads * p.n_rb));
    p.tps_max = kMaxPadWords;
    const int64_t B = d->batch, all = B * p.splits;
    if (B * std::min<int64_t>(p.splits, cdiv(tiles, p.tps_max)) <= p.conc ||
        (p.conc > B && cdiv(B * tiles, p.conc - B) <= p.tps_max))
      p.items = (int32_t)std::min<int64_t>(all, p.conc);
    else if (B * tiles <= (int64_t)p.conc * p.tps_max)
      p.items = (int32_t)std::min<int64_t>(all, B + p.conc);
    else
      p.items = (int32_t)all;
    // The kernel addresses a (KV head, row block)'s item partials with
    // 32-bit signed byte offsets.  A batch whose items overflow them (only
    // at hundreds of millions of cached keys) keeps the plain split order,
    // whose partials are per (sequence, KV head, row block).
    if ((int64_t)p.items * p.rb * d->head_dim * 4 > INT32_MAX) {
      p.ordered = 0;
      p.items = p.conc = p.tps_max = 0;
    }
  }
  // Long register-staged splits take their tiles in chunks (dynamic
  // balancing across XCDs); budget gathers keep fixed ranges (their indices
  // are staged per range), and so does the deterministic mode (which wave
  // sums which tiles would otherwise depend on timing).  The pool's counter
  // is one address per (pair, row block): with fewer than 8 of them, every
  // wave's requests queue on a few addresses and the pool costs more than it
  // balances (one KV head over 1M keys: 100.3 us pooled, 93.0 us fixed).
  if (p.wk == 4 && !gather && p.splits > 1 && tiles >= (int64_t)p.splits * 32 &&
      groups >= kMinPoolGroups && !(d->flags & SPEC_FLAG_DETERMINISTIC))
    p.dyn = kChunkTiles;
  p.cnt_off = kHeaderBytes;
  size_t off = kScratchOff;
  if (p.splits > 1) {
    // split partials: one slot per (pair, row block, split), or, in the
    // ordered verify, per (KV head, row block, work item)
    const size_t n = p.ordered ? (size_t)d->n_kv_heads * p.n_rb * p.items * p.rb
                               : (size_t)groups * p.splits * p.rb;
    p.o_off = off;
    off = align_up(off + n * d->head_dim * sizeof(float), 256);
    p.lse_off = off;
    off = align_up(off + n * sizeof(float), 256);
  }
  if (p.n_blk > 1) {
    const size_t n = (size_t)groups * p.n_blk * p.rb;
    p.o1_off = off;
    off = align_up(off + n * d->head_dim * sizeof(float), 256);
    p.lse1_off = off;
    off = align_up(off + n * sizeof(float), 256);
  }
  p.total = off;
  return p;
}

// fp32 path: one wavefront per (pair, row, split) and a separate combine.
void f32_splits(Plan& p, int64_t pairs, int64_t keys) {
  if (keys < 1) keys = 1;
  const int64_t units = pairs * p.n_rb;
  int64_t s = cdiv(kTargetWaves, units > 0 ? units : 1);
  s = std::min(s, cdiv(keys, 64));
  if (s < 1) s = 1;
  p.chunk = (int32_t)(cdiv(cdiv(keys, s), 64) * 64);
  p.splits = (int32_t)cdiv(keys, p.chunk);
}

Plan f32_plan(const spec_dims* d, int32_t T, int64_t keys, bool verify) {
  Plan p;
  const int G = d->n_q_heads / d->n_kv_heads;
  const int64_t pairs = (int64_t)d->batch * d->n_kv_heads;
  if ((int64_t)T * G > kMaxRows) return p;   // total 0: refused
  p.rows = T * G;
  p.rb = 1;
  p.n_rb = p.rows;
  f32_splits(p, pairs, keys);
  size_t off = kScratchOff;
  if (p.splits > 1) {
    const size_t n = (size_t)pairs * p.n_rb * p.splits;
    p.o_off = off;
    off = align_up(off + n * d->head_dim * sizeof(float), 256);
    p.lse_off = off;
    off = align_up(off + n * sizeof(float), 256);
  }
  if (verify) {
    p.anc_off = off;
    off = align_up(off + (size_t)d->batch * T * sizeof(uint64_t), 256);
    p.bad_off = off;
    off = align_up(off + (size_t)d->batch * sizeof(int32_t), 256);
  }
  p.total = off;
  return p;
}

Plan draft_plan(const spec_dims* d, int32_t Tq, int64_t max_view, bool gather) {
  if (d->dtype == SPEC_BF16) return bf16_plan(d, Tq, cdiv(std::max<int64_t>(max_view, 1), kTileKeys), gather, false);
  return f32_plan(d, Tq, max_view, false);
}

Plan verify_plan(const spec_dims* d, int32_t N, int32_t capacity) {
  if (d->dtype == SPEC_BF16)
    return bf16_plan(d, N, cdiv(std::max(capacity, 0), kTileKeys) + cdiv(N, kTileKeys), false, true);
  return f32_plan(d, N, std::max(capacity, 1), true);
}

// Slices per logits row: about two rounds of resident blocks (8 blocks of
// 256 threads per CU), at least 4096 values per slice.  (One round, so that
// no straggler round runs alone at the end, took the 16K batch of 8 from 60
// to 52 us with one arrival counter per sequence; with a counter per row,
// two rounds of smaller slices measured 52.2 against 53.9 us there and 94.5
// against 100.2 us on the ragged batch of 16.)
int accept_vsplits(int64_t rows, int64_t V) {
  int64_t vs = kTargetWorkgroups * 8 / (rows > 0 ? rows : 1);
  int64_t vmax = V / 4096;
  if (vmax < 1) vmax = 1;
  if (vs > vmax) vs = vmax;
  if (vs < 1) vs = 1;
  return (int)vs;
}

// header | counter region (unused) | fp32 block scores [B][Hkv][max_blocks]
size_t select_bytes(const spec_dims* d, int32_t max_blocks) {
  return kScratchOff +
         align_up((size_t)std::max(d->batch, 0) * d->n_kv_heads * std::max(max_blocks, 0) * sizeof(float), 256);
}

// header | counter region (one arrival counter per sequence first) |
// (value, index) winner per slice
// Per-row arrival counters (two levels) fit the counter region beside the
// per-sequence ones, and a row's slices fit one wavefront's merge.
bool accept_two_level(int64_t batch, int64_t rows, int vs) {
  return batch + rows <= (int64_t)kCounterWords && vs <= 64;
}

// header | counters | slice winners [rows][vs] | row winners [rows] (8 bytes each)
size_t accept_bytes(int64_t, int64_t rows, int vs) {
  return align_up(kScratchOff + (size_t)rows * (vs + 1) * 8, 256);
}

int64_t draft_max_view(const spec_kv* cache, int32_t Tq, int32_t n_sink, int32_t window,
                       const int32_t* idx, int32_t budget) {
  if (idx != nullptr) return budget;
  int64_t v = (int64_t)n_sink + window + Tq - 1;
  return v < cache->capacity ? v : cache->capacity;
}

// Workgroups (bf16) or wavefronts (fp32) of one attention launch.
int64_t grid_size(const spec_dims* d, const Plan& p) {
  const int64_t units = p.ordered ? (int64_t)p.items * d->n_kv_heads
                                  : (int64_t)d->batch * d->n_kv_heads * p.splits;
  if (d->dtype != SPEC_BF16) return units * p.n_rb;
  return p.n_rb == 1 ? units : cdiv(units, 8) * 8 * p.n_rb;
}

void fill_plan(AttnArgs& a, const Plan& p, void* workspace) {
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  a.rb = p.rb;
  a.n_rb = p.n_rb;
  a.splits = p.splits;
  a.chunk = p.chunk;
  a.tps = p.tps;
  a.units = p.ordered ? p.items * a.Hkv : a.B * a.Hkv * p.splits;
  a.o_part = reinterpret_cast<float*>(ws + p.o_off);
  a.lse_part = reinterpret_cast<float*>(ws + p.lse_off);
  a.o_part1 = reinterpret_cast<float*>(ws + p.o1_off);
  a.lse_part1 = reinterpret_cast<float*>(ws + p.lse1_off);
  a.n_blk = p.n_blk;
  const size_t groups = (size_t)a.B * a.Hkv * p.n_rb;
  a.cnt_l0 = reinterpret_cast<uint32_t*>(ws + p.cnt_off);
  a.cnt_l1 = a.cnt_l0 + groups * p.n_blk;
  a.cnt_pos = a.cnt_l1 + groups;
  a.cnt_chunk = a.cnt_pos + 2 * (size_t)a.B;
  a.dyn = p.dyn;
  a.ordered = p.ordered;
  a.items = p.items;
  a.conc = p.conc;
  a.tps_max = p.tps_max;
  a.err = reinterpret_cast<uint32_t*>(ws);
}

}  // namespace

spec_status spec::set_error(spec_status s, const char* msg) { return fail(s, "%s", msg); }

#pragma GCC visibility push(default)
extern "C" {

int32_t spec_abi_version(void) { return SPEC_ABI_VERSION; }

const char* spec_last_error(void) { return g_err.c_str(); }

const char* spec_status_string(spec_status s) {
  switch (s) {
    case SPEC_OK: return "SPEC_OK";
    case SPEC_E_INVALID: return "SPEC_E_INVALID";
    case SPEC_E_UNSUPPORTED: return "SPEC_E_UNSUPPORTED";
    case SPEC_E_WORKSPACE: return "SPEC_E_WORKSPACE";
    case SPEC_E_HIP: return "SPEC_E_HIP";
    case SPEC_E_DEVICE_RANGE: return "SPEC_E_DEVICE_RANGE";
    default: return "unknown status";
  }
}

size_t spec_draft_workspace_bytes(const spec_dims* dims, int32_t n_q_tokens, int32_t max_view_len) {
  if (check_dims(dims) != SPEC_OK) return 0;
  if (n_q_tokens < 1 || max_view_len < 0) {
    fail(SPEC_E_INVALID, "n_q_tokens must be >= 1 and max_view_len >= 0");
    return 0;
  }
  const size_t n = std::max(draft_plan(dims, n_q_tokens, max_view_len, false).total,
                            draft_plan(dims, n_q_tokens, max_view_len, true).total);
  if (n == 0) fail(SPEC_E_UNSUPPORTED, "no split plan fits this shape");
  return n;
}

size_t spec_verify_workspace_bytes(const spec_dims* dims, int32_t n_nodes, int32_t capacity) {
  if (check_dims(dims) != SPEC_OK) return 0;
  if (n_nodes < 1 || n_nodes > kMaxNodes || capacity < 0) {
    fail(SPEC_E_INVALID, "n_nodes must be in [1, 64] and capacity >= 0");
    return 0;
  }
  const size_t n = verify_plan(dims, n_nodes, capacity).total;
  if (n == 0) fail(SPEC_E_UNSUPPORTED, "no split plan fits this shape");
  return n;
}

size_t spec_accept_workspace_bytes(int32_t batch, int32_t n_nodes, int32_t vocab) {
  if (batch < 0 || n_nodes < 1 || n_nodes > kMaxNodes || vocab < 1) {
    fail(SPEC_E_INVALID, "need batch >= 0, 1 <= n_nodes <= 64, vocab >= 1");
    return 0;
  }
  const int64_t rows = (int64_t)batch * (n_nodes + 1);
  return accept_bytes(batch, rows, accept_vsplits(rows, vocab));
}

// Draft attention; kv_ring > 0 reads the window through a ring of that many
// slots after the sink (validated by the caller).
static spec_status draft_impl(const spec_dims* dims, const void* q, int32_t n_q_tokens,
                              const spec_kv* cache, const int32_t* cache_len, int32_t n_sink,
                              int32_t window, const int32_t* idx, int32_t budget,
                              int64_t idx_stride_b, int64_t idx_stride_h, int32_t kv_ring,
                              void* out, float* lse_or_null, void* workspace,
                              size_t workspace_bytes, void* stream) {
  spec_status st = check_dims(dims);
  if (st != SPEC_OK) return st;
  if (n_q_tokens < 1) return fail(SPEC_E_INVALID, "n_q_tokens %d < 1", n_q_tokens);
  if (dims->batch == 0) return SPEC_OK;   // nothing to read or write; pointers may be NULL
  if ((st = check_kv(cache, dims, "cache", true)) != SPEC_OK) return st;
  if (q == nullptr || out == nullptr || cache_len == nullptr)
    return fail(SPEC_E_INVALID, "q, out and cache_len must not be NULL");
  if (!aligned(q, 16) || !aligned(out, 16)) return fail(SPEC_E_INVALID, "q and out must be 16-byte aligned");
  if (lse_or_null != nullptr && !aligned(lse_or_null, 4)) return fail(SPEC_E_INVALID, "lse must be 4-byte aligned");
  if (!aligned(cache_len, 4)) return fail(SPEC_E_INVALID, "cache_len must be 4-byte aligned");
  int mode;
  if (idx == nullptr) {
    if (n_sink < 0 || window < 1) return fail(SPEC_E_INVALID, "window mode needs n_sink >= 0 and window >= 1");
    mode = kDraftWindow;
  } else {
    if (budget < 1) return fail(SPEC_E_INVALID, "budget %d < 1", budget);
    if (idx_stride_b < 0 || idx_stride_h < 0) return fail(SPEC_E_INVALID, "idx strides must be >= 0");
    if (!aligned(idx, 4)) return fail(SPEC_E_INVALID, "idx must be 4-byte aligned");
    mode = kDraftGather;
  }
  const int64_t max_view = draft_max_view(cache, n_q_tokens, n_sink, window, idx, budget);
  const Plan p = draft_plan(dims, n_q_tokens, max_view, mode == kDraftGather);
  if (p.total == 0) return fail(SPEC_E_UNSUPPORTED, "no split plan fits this shape");
  if (workspace == nullptr || workspace_bytes < p.total)
    return fail(SPEC_E_WORKSPACE, "workspace of %zu bytes needed (got %zu)", p.total,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  if (!aligned(workspace, 256)) return fail(SPEC_E_INVALID, "workspace must be 256-byte aligned");
  if (grid_size(dims, p) > kMaxGrid) return fail(SPEC_E_UNSUPPORTED, "problem too large for one launch");

  AttnArgs a{};
  a.q = q;
  a.k = cache->k;
  a.v = cache->v;
  a.kb = cache->stride_b;
  a.kh = cache->stride_h;
  a.kt = cache->stride_t;
  a.capacity = cache->capacity;
  a.cache_len = cache_len;
  a.B = dims->batch;
  a.Hq = dims->n_q_heads;
  a.Hkv = dims->n_kv_heads;
  a.G = a.Hq / a.Hkv;
  a.D = dims->head_dim;
  a.T = n_q_tokens;
  a.R = p.rows;
  a.scale_log2 = dims->softmax_scale * kLog2e;
  a.n_sink = n_sink;
  a.window = window;
  a.kv_ring = kv_ring;
  a.idx = idx;
  a.budget = budget;
  a.idx_sb = idx_stride_b;
  a.idx_sh = idx_stride_h;
  fill_plan(a, p, workspace);
  a.out = out;
  a.lse = lse_or_null;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (dims->dtype == SPEC_BF16) {
    e = launch_attn_bf16(a, mode, p, s);
    if (e != hipSuccess) return hip_fail(e, "draft launch");
  } else {
    e = launch_attn_f32(a, mode, s);
    if (e != hipSuccess) return hip_fail(e, "draft launch");
    if (p.splits > 1 && (e = launch_combine(a, dims->dtype, s)) != hipSuccess)
      return hip_fail(e, "combine launch");
  }
  return SPEC_OK;
}

spec_status spec_attn_draft_sparse(const spec_dims* dims, const void* q, int32_t n_q_tokens,
                                   const spec_kv* cache, const int32_t* cache_len,
                                   int32_t n_sink, int32_t window, const int32_t* idx,
                                   int32_t budget, int64_t idx_stride_b, int64_t idx_stride_h,
                                   void* out, float* lse_or_null, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  return draft_impl(dims, q, n_q_tokens, cache, cache_len, n_sink, window, idx, budget,
                    idx_stride_b, idx_stride_h, 0, out, lse_or_null, workspace, workspace_bytes,
                    stream);
}

spec_status spec_attn_draft_ring(const spec_dims* dims, const void* q, int32_t n_q_tokens,
                                 const spec_kv* ring_cache, const int32_t* cache_len,
                                 int32_t n_sink, int32_t window, int32_t ring, void* out,
                                 float* lse_or_null, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  spec_status st = check_dims(dims);
  if (st != SPEC_OK) return st;
  if (n_q_tokens < 1) return fail(SPEC_E_INVALID, "n_q_tokens %d < 1", n_q_tokens);
  if (n_sink < 0 || window < 1) return fail(SPEC_E_INVALID, "need n_sink >= 0 and window >= 1");
  if ((int64_t)ring < (int64_t)window + n_q_tokens - 1)
    return fail(SPEC_E_INVALID, "ring %d < window + n_q_tokens - 1 (%lld)", ring,
                (long long)window + n_q_tokens - 1);
  if (ring_cache != nullptr && (int64_t)ring_cache->capacity < (int64_t)n_sink + ring)
    return fail(SPEC_E_INVALID, "ring cache capacity %d < n_sink + ring", ring_cache->capacity);
  return draft_impl(dims, q, n_q_tokens, ring_cache, cache_len, n_sink, window, nullptr, 0, 0, 0,
                    ring, out, lse_or_null, workspace, workspace_bytes, stream);
}

spec_status spec_attn_verify_tree(const spec_dims* dims, const void* q, int32_t n_nodes,
                                  const spec_kv* cache, const int32_t* cache_len,
                                  const uint8_t* pad_or_null, int64_t pad_stride_b,
                                  const spec_kv* tree, const int32_t* parents,
                                  int64_t parents_stride_b, void* out, float* lse_or_null,
                                  int32_t* pos_ids_or_null, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return spec::verify_impl(dims, q, n_nodes, cache, cache_len, pad_or_null, pad_stride_b, tree,
                           parents, parents_stride_b, out, lse_or_null, pos_ids_or_null,
                           workspace, workspace_bytes, stream, nullptr);
}

}  // extern "C"

// Validation, planning and launches of the tree verify.  With `need` set,
// the workspace bytes the call requires are stored there once the
// arguments are known to be valid, and nothing is launched if the
// workspace is NULL (the static-workspace variant asks first).
__attribute__((visibility("hidden")))
spec_status spec::verify_impl(const spec_dims* dims, const void* q, int32_t n_nodes,
                              const spec_kv* cache, const int32_t* cache_len,
                              const uint8_t* pad_or_null, int64_t pad_stride_b,
                              const spec_kv* tree, const int32_t* parents,
                              int64_t parents_stride_b, void* out, float* lse_or_null,
                              int32_t* pos_ids_or_null, void* workspace, size_t workspace_bytes,
                              void* stream, size_t* need) {
  if (need != nullptr) *need = 0;
  spec_status st = check_dims(dims);
  if (st != SPEC_OK) return st;
  if (n_nodes < 1 || n_nodes > kMaxNodes)
    return fail(n_nodes > kMaxNodes ? SPEC_E_UNSUPPORTED : SPEC_E_INVALID,
                "n_nodes %d outside [1, 64]", n_nodes);
  if (dims->batch == 0) return SPEC_OK;   // nothing to read or write; pointers may be NULL
  if ((st = check_kv(cache, dims, "cache", true)) != SPEC_OK) return st;
  if ((st = check_kv(tree, dims, "tree", false)) != SPEC_OK) return st;
  if (q == nullptr || out == nullptr || cache_len == nullptr || parents == nullptr)
    return fail(SPEC_E_INVALID, "q, out, cache_len and parents must not be NULL");
  if (!aligned(q, 16) || !aligned(out, 16)) return fail(SPEC_E_INVALID, "q and out must be 16-byte aligned");
  if (!aligned(cache_len, 4) || !aligned(parents, 4)) return fail(SPEC_E_INVALID, "cache_len and parents must be 4-byte aligned");
  if (lse_or_null != nullptr && !aligned(lse_or_null, 4)) return fail(SPEC_E_INVALID, "lse must be 4-byte aligned");
  if (pos_ids_or_null != nullptr && !aligned(pos_ids_or_null, 4)) return fail(SPEC_E_INVALID, "pos_ids must be 4-byte aligned");
  if (parents_stride_b != 0 && parents_stride_b < n_nodes)
    return fail(SPEC_E_INVALID, "parents_stride_b must be 0 (shared) or >= n_nodes");
  if (pad_or_null != nullptr) {
    if (!aligned(pad_or_null, 4) || pad_stride_b % 4 != 0 || pad_stride_b < cache->capacity)
      return fail(SPEC_E_INVALID, "pad must be 4-byte aligned with pad_stride_b %% 4 == 0 and >= capacity");
  }
  const Plan p = verify_plan(dims, n_nodes, cache->capacity);
  if (p.total == 0) return fail(SPEC_E_UNSUPPORTED, "no split plan fits this shape");
  if (grid_size(dims, p) > kMaxGrid) return fail(SPEC_E_UNSUPPORTED, "problem too large for one launch");
  if (need != nullptr) {
    *need = p.total;
    if (workspace == nullptr) return SPEC_OK;
  }
  if (workspace == nullptr || workspace_bytes < p.total)
    return fail(SPEC_E_WORKSPACE, "workspace of %zu bytes needed (got %zu)", p.total,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  if (!aligned(workspace, 256)) return fail(SPEC_E_INVALID, "workspace must be 256-byte aligned");

  AttnArgs a{};
  a.q = q;
  a.k = cache->k;
  a.v = cache->v;
  a.kb = cache->stride_b;
  a.kh = cache->stride_h;
  a.kt = cache->stride_t;
  a.capacity = cache->capacity;
  a.cache_len = cache_len;
  a.B = dims->batch;
  a.Hq = dims->n_q_heads;
  a.Hkv = dims->n_kv_heads;
  a.G = a.Hq / a.Hkv;
  a.D = dims->head_dim;
  a.T = n_nodes;
  a.R = p.rows;
  a.scale_log2 = dims->softmax_scale * kLog2e;
  a.pad = pad_or_null;
  a.pad_sb = pad_stride_b;
  a.tk = tree->k;
  a.tv = tree->v;
  a.tkb = tree->stride_b;
  a.tkh = tree->stride_h;
  a.tkt = tree->stride_t;
  a.parents = parents;
  a.par_sb = parents_stride_b;
  a.pos_ids = pos_ids_or_null;
  fill_plan(a, p, workspace);
  if (pad_or_null != nullptr) a.dyn = 0;   // pad words are staged per fixed range
  a.out = out;
  a.lse = lse_or_null;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (dims->dtype == SPEC_BF16) {
    e = launch_attn_bf16(a, kVerify, p, s);
    if (e != hipSuccess) return hip_fail(e, "verify launch");
  } else {
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    uint64_t* anc_ws = reinterpret_cast<uint64_t*>(ws + p.anc_off);
    int32_t* bad_ws = reinterpret_cast<int32_t*>(ws + p.bad_off);
    a.anc = anc_ws;
    a.bad = bad_ws;
    e = launch_verify_prep(a, parents, parents_stride_b, pos_ids_or_null, anc_ws, bad_ws, s);
    if (e != hipSuccess) return hip_fail(e, "verify prep launch");
    if ((e = launch_attn_f32(a, kVerify, s)) != hipSuccess) return hip_fail(e, "verify launch");
    if (p.splits > 1 && (e = launch_combine(a, dims->dtype, s)) != hipSuccess)
      return hip_fail(e, "combine launch");
  }
  return SPEC_OK;
}

extern "C" {

spec_status spec_accept_greedy(int32_t batch, int32_t n_nodes, int32_t vocab, const float* logits,
                               const int32_t* draft_tokens, const int32_t* parents,
                               int64_t parents_stride_b, int32_t max_depth, int32_t* accept_len,
                               int32_t* accept_path, int32_t* bonus, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (batch < 0) return fail(SPEC_E_INVALID, "batch %d < 0", batch);
  if (n_nodes < 1 || n_nodes > kMaxNodes)
    return fail(n_nodes > kMaxNodes ? SPEC_E_UNSUPPORTED : SPEC_E_INVALID, "n_nodes %d outside [1, 64]", n_nodes);
  if (vocab < 1) return fail(SPEC_E_INVALID, "vocab %d < 1", vocab);
  if (max_depth < 1) return fail(SPEC_E_INVALID, "max_depth %d < 1", max_depth);
  if (batch == 0) return SPEC_OK;   // nothing to read or write; pointers may be NULL
  if (logits == nullptr || draft_tokens == nullptr || parents == nullptr || accept_len == nullptr ||
      accept_path == nullptr || bonus == nullptr)
    return fail(SPEC_E_INVALID, "a required pointer is NULL");
  if (!aligned(logits, 16)) return fail(SPEC_E_INVALID, "logits must be 16-byte aligned");
  if (!aligned(draft_tokens, 4) || !aligned(parents, 4) || !aligned(accept_len, 4) ||
      !aligned(accept_path, 4) || !aligned(bonus, 4))
    return fail(SPEC_E_INVALID, "int32 arrays must be 4-byte aligned");
  if (parents_stride_b != 0 && parents_stride_b < n_nodes)
    return fail(SPEC_E_INVALID, "parents_stride_b must be 0 (shared) or >= n_nodes");
  if ((size_t)batch > kCounterWords)
    return fail(SPEC_E_UNSUPPORTED, "batch %d exceeds the %zu arrival counters of the workspace", batch,
                kCounterWords);
  const int64_t rows = (int64_t)batch * (n_nodes + 1);
  const int vs = accept_vsplits(rows, vocab);
  const size_t need = accept_bytes(batch, rows, vs);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(SPEC_E_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  if (!aligned(workspace, 256)) return fail(SPEC_E_INVALID, "workspace must be 256-byte aligned");
  if (rows * vs > kMaxGrid) return fail(SPEC_E_UNSUPPORTED, "problem too large for one launch");
  hipError_t e = launch_accept(batch, n_nodes, vocab, logits, draft_tokens, parents, parents_stride_b,
                               max_depth, accept_len, accept_path, bonus, workspace, vs,
                               accept_two_level(batch, rows, vs) ? 1 : 0,
                               static_cast<hipStream_t>(stream), static_cast<uint32_t*>(workspace));
  if (e != hipSuccess) return hip_fail(e, "accept launch");
  return SPEC_OK;
}

spec_status spec_kv_commit(int32_t batch, int32_t n_kv_heads, int32_t head_dim, int32_t dtype,
                           const spec_kv_mut* cache, int32_t* cache_len, uint8_t* pad,
                           int64_t pad_stride_b, const spec_kv* tree, int32_t n_nodes,
                           const int32_t* accept_len, const int32_t* accept_path,
                           int32_t max_depth, int32_t* n_appended_or_null, void* workspace,
                           size_t workspace_bytes, void* stream) {
  const spec_dims d{batch, n_kv_heads, n_kv_heads, head_dim, dtype, 1.f};
  spec_status st = check_dims(&d);
  if (st != SPEC_OK) return st;
  if (n_nodes < 1 || n_nodes > kMaxNodes)
    return fail(n_nodes > kMaxNodes ? SPEC_E_UNSUPPORTED : SPEC_E_INVALID, "n_nodes %d outside [1, 64]", n_nodes);
  if (max_depth < 1) return fail(SPEC_E_INVALID, "max_depth %d < 1", max_depth);
  if (batch == 0) return SPEC_OK;   // nothing to read or write; pointers may be NULL
  if (cache == nullptr) return fail(SPEC_E_INVALID, "cache is NULL");
  const spec_kv c{cache->k, cache->v, cache->stride_b, cache->stride_h, cache->stride_t, cache->capacity};
  if ((st = check_kv(&c, &d, "cache", true)) != SPEC_OK) return st;
  if ((st = check_kv(tree, &d, "tree", false)) != SPEC_OK) return st;
  if (cache_len == nullptr || pad == nullptr || accept_len == nullptr || accept_path == nullptr)
    return fail(SPEC_E_INVALID, "a required pointer is NULL");
  if (!aligned(cache_len, 4) || !aligned(accept_len, 4) || !aligned(accept_path, 4) ||
      (n_appended_or_null != nullptr && !aligned(n_appended_or_null, 4)))
    return fail(SPEC_E_INVALID, "int32 arrays must be 4-byte aligned");
  if (pad_stride_b < cache->capacity)
    return fail(SPEC_E_INVALID, "pad_stride_b %lld < capacity %d", (long long)pad_stride_b, cache->capacity);
  if (workspace == nullptr || workspace_bytes < kHeaderBytes)
    return fail(SPEC_E_WORKSPACE, "workspace of %zu bytes needed (got %zu)", kHeaderBytes,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  if (!aligned(workspace, 256)) return fail(SPEC_E_INVALID, "workspace must be 256-byte aligned");
  const int64_t es = esize(dtype);
  CommitArgs a;
  a.k = static_cast<char*>(cache->k);
  a.v = static_cast<char*>(cache->v);
  a.c_sb = cache->stride_b * es;
  a.c_sh = cache->stride_h * es;
  a.c_st = cache->stride_t * es;
  a.tk = static_cast<const char*>(tree->k);
  a.tv = static_cast<const char*>(tree->v);
  a.t_sb = tree->stride_b * es;
  a.t_sh = tree->stride_h * es;
  a.t_st = tree->stride_t * es;
  a.batch = batch;
  a.n_kv_heads = n_kv_heads;
  a.row_chunks = (int32_t)(head_dim * es / 16);
  a.capacity = cache->capacity;
  a.n_nodes = n_nodes;
  a.max_depth = max_depth;
  a.cache_len = cache_len;
  a.pad = pad;
  a.pad_sb = pad_stride_b;
  a.accept_len = accept_len;
  a.accept_path = accept_path;
  a.n_appended = n_appended_or_null;
  a.err = static_cast<uint32_t*>(workspace);
  hipError_t e = launch_kv_commit(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "kv commit launch");
  return SPEC_OK;
}

size_t spec_commit_workspace_bytes(void) { return kHeaderBytes; }

// header | counter region (unused) | [B][kCompactSlices][2] int32: first pad
// slot and pad count per slice of the pad bytes
size_t spec_compact_workspace_bytes(int32_t batch) {
  return kScratchOff + align_up((size_t)std::max(batch, 0) * kCompactSlices * 2 * sizeof(int32_t), 256);
}

spec_status spec_kv_compact(int32_t batch, int32_t n_kv_heads, int32_t head_dim, int32_t dtype,
                            const spec_kv_mut* cache, int32_t* cache_len, uint8_t* pad,
                            int64_t pad_stride_b, void* workspace, size_t workspace_bytes,
                            void* stream) {
  const spec_dims d{batch, n_kv_heads, n_kv_heads, head_dim, dtype, 1.f};
  spec_status st = check_dims(&d);
  if (st != SPEC_OK) return st;
  if ((int64_t)batch * std::max(n_kv_heads, kCompactSlices) > INT32_MAX)
    return fail(SPEC_E_UNSUPPORTED, "batch x n_kv_heads is too large");
  if (batch == 0) return SPEC_OK;   // nothing to read or write; pointers may be NULL
  if (cache == nullptr) return fail(SPEC_E_INVALID, "cache is NULL");
  const spec_kv c{cache->k, cache->v, cache->stride_b, cache->stride_h, cache->stride_t, cache->capacity};
  if ((st = check_kv(&c, &d, "cache", true)) != SPEC_OK) return st;
  if (cache_len == nullptr || pad == nullptr) return fail(SPEC_E_INVALID, "a required pointer is NULL");
  if (!aligned(cache_len, 4)) return fail(SPEC_E_INVALID, "cache_len must be 4-byte aligned");
  if (!aligned(pad, 4) || pad_stride_b % 4 != 0 || pad_stride_b < cache->capacity)
    return fail(SPEC_E_INVALID, "pad must be 4-byte aligned with pad_stride_b %% 4 == 0 and >= capacity");
  const size_t need = spec_compact_workspace_bytes(batch);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(SPEC_E_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  if (!aligned(workspace, 256)) return fail(SPEC_E_INVALID, "workspace must be 256-byte aligned");
  const int64_t es = esize(dtype);
  CompactArgs a;
  a.k = static_cast<char*>(cache->k);
  a.v = static_cast<char*>(cache->v);
  a.c_sb = cache->stride_b * es;
  a.c_sh = cache->stride_h * es;
  a.c_st = cache->stride_t * es;
  a.batch = batch;
  a.n_kv_heads = n_kv_heads;
  a.row_chunks = (int32_t)(head_dim * es / 16);
  a.capacity = cache->capacity;
  a.cache_len = cache_len;
  a.pad = pad;
  a.pad_sb = pad_stride_b;
  a.summary = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(workspace) + kScratchOff);
  a.sliced = cache->capacity > kCompactScanSlots ? 1 : 0;
  a.err = static_cast<uint32_t*>(workspace);
  hipError_t e = launch_kv_compact(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "kv compact launch");
  return SPEC_OK;
}

spec_status spec_block_means(const spec_dims* dims, const spec_kv* cache, const int32_t* cache_len,
                             const uint8_t* pad_or_null, int64_t pad_stride_b, int32_t block,
                             int32_t first_block, int32_t n_blocks, float* means,
                             int32_t max_blocks, void* workspace, size_t workspace_bytes,
                             void* stream) {
  spec_status st = check_dims(dims);
  if (st != SPEC_OK) return st;
  if (block < 1) return fail(SPEC_E_INVALID, "block %d < 1", block);
  if (first_block < 0 || n_blocks < 0 || max_blocks < 1 ||
      (int64_t)first_block + n_blocks > max_blocks)
    return fail(SPEC_E_INVALID, "need 0 <= first_block, 0 <= n_blocks, first_block + n_blocks <= max_blocks");
  if (dims->batch > 65535 || dims->n_kv_heads > 65535)
    return fail(SPEC_E_UNSUPPORTED, "batch and n_kv_heads must be <= 65535");
  if (dims->batch == 0 || n_blocks == 0) return SPEC_OK;
  if ((st = check_kv(cache, dims, "cache", true)) != SPEC_OK) return st;
  if (cache_len == nullptr || means == nullptr) return fail(SPEC_E_INVALID, "a required pointer is NULL");
  if (!aligned(cache_len, 4) || !aligned(means, 16))
    return fail(SPEC_E_INVALID, "cache_len must be 4-byte and means 16-byte aligned");
  if (pad_or_null != nullptr && pad_stride_b < cache->capacity)
    return fail(SPEC_E_INVALID, "pad_stride_b %lld < capacity %d", (long long)pad_stride_b, cache->capacity);
  if (workspace == nullptr || workspace_bytes < kHeaderBytes)
    return fail(SPEC_E_WORKSPACE, "workspace of %zu bytes needed", kHeaderBytes);
  if (!aligned(workspace, 256)) return fail(SPEC_E_INVALID, "workspace must be 256-byte aligned");
  const int64_t es = esize(dims->dtype);
  MeansArgs a;
  a.k = static_cast<const char*>(cache->k);
  a.k_sb = cache->stride_b * es;
  a.k_sh = cache->stride_h * es;
  a.k_st = cache->stride_t * es;
  a.bf16 = dims->dtype == SPEC_BF16;
  a.head_dim = dims->head_dim;
  a.row_chunks = (int32_t)(dims->head_dim * es / 16);
  a.batch = dims->batch;
  a.n_kv_heads = dims->n_kv_heads;
  a.capacity = cache->capacity;
  a.block = block;
  a.first_block = first_block;
  a.n_blocks = n_blocks;
  a.max_blocks = max_blocks;
  a.cache_len = cache_len;
  a.pad = pad_or_null;
  a.pad_sb = pad_stride_b;
  a.means = means;
  a.err = static_cast<uint32_t*>(workspace);
  hipError_t e = launch_block_means(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "block means launch");
  return SPEC_OK;
}

spec_status spec_select_blocks(const spec_dims* dims, const void* q, int32_t n_q_tokens,
                               const float* means, int32_t max_blocks, int32_t block,
                               const int32_t* cache_len, int32_t capacity,
                               const uint8_t* pad_or_null, int64_t pad_stride_b, int32_t n_sink,
                               int32_t window, int32_t n_select, int32_t shared, int32_t* idx,
                               int32_t budget, float* scores_or_null, void* workspace,
                               size_t workspace_bytes, void* stream) {
  spec_status st = check_dims(dims);
  if (st != SPEC_OK) return st;
  if (n_q_tokens < 1) return fail(SPEC_E_INVALID, "n_q_tokens %d < 1", n_q_tokens);
  if (block < 1 || max_blocks < 1 || capacity < 0)
    return fail(SPEC_E_INVALID, "need block >= 1, max_blocks >= 1, capacity >= 0");
  if (max_blocks > kMaxSelectBlocks)
    return fail(SPEC_E_UNSUPPORTED, "max_blocks %d > %d", max_blocks, kMaxSelectBlocks);
  if ((int64_t)max_blocks * block < capacity)
    return fail(SPEC_E_INVALID, "max_blocks x block (%lld) does not cover capacity %d",
                (long long)max_blocks * block, capacity);
  if (n_sink < 0 || window < 0 || n_select < 0)
    return fail(SPEC_E_INVALID, "n_sink, window and n_select must be >= 0");
  if (n_select > kMaxSelect) return fail(SPEC_E_UNSUPPORTED, "n_select %d > %d", n_select, kMaxSelect);
  if (budget < 1 || (int64_t)budget < (int64_t)n_sink + window + (int64_t)n_select * block)
    return fail(SPEC_E_INVALID, "budget %d < n_sink + window + n_select x block", budget);
  if (dims->batch > 65535 || dims->n_kv_heads > 65535)
    return fail(SPEC_E_UNSUPPORTED, "batch and n_kv_heads must be <= 65535");
  if (dims->batch == 0) return SPEC_OK;
  if (q == nullptr || means == nullptr || cache_len == nullptr || idx == nullptr)
    return fail(SPEC_E_INVALID, "a required pointer is NULL");
  if (!aligned(q, 16) || !aligned(means, 16)) return fail(SPEC_E_INVALID, "q and means must be 16-byte aligned");
  if (!aligned(cache_len, 4) || !aligned(idx, 4) || (scores_or_null != nullptr && !aligned(scores_or_null, 4)))
    return fail(SPEC_E_INVALID, "cache_len, idx and scores must be 4-byte aligned");
  if (pad_or_null != nullptr && pad_stride_b < capacity)
    return fail(SPEC_E_INVALID, "pad_stride_b %lld < capacity %d", (long long)pad_stride_b, capacity);
  const size_t need = select_bytes(dims, max_blocks);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(SPEC_E_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  if (!aligned(workspace, 256)) return fail(SPEC_E_INVALID, "workspace must be 256-byte aligned");
  SelectArgs a;
  a.q = q;
  a.bf16 = dims->dtype == SPEC_BF16;
  a.T = n_q_tokens;
  a.Hq = dims->n_q_heads;
  a.G = dims->n_q_heads / dims->n_kv_heads;
  a.head_dim = dims->head_dim;
  a.batch = dims->batch;
  a.n_kv_heads = dims->n_kv_heads;
  a.capacity = capacity;
  a.means = means;
  a.max_blocks = max_blocks;
  a.block = block;
  a.n_sink = n_sink;
  a.window = window;
  a.n_select = n_select;
  a.budget = budget;
  a.shared = shared != 0;
  a.cache_len = cache_len;
  a.pad = pad_or_null;
  a.pad_sb = pad_stride_b;
  a.idx = idx;
  a.scores = scores_or_null;
  a.sc_ws = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + kScratchOff);
  a.err = static_cast<uint32_t*>(workspace);
  hipError_t e = launch_select_blocks(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "block selection launch");
  return SPEC_OK;
}

spec_status spec_kv_gather(int32_t batch, int32_t n_kv_heads, int32_t head_dim, int32_t dtype,
                           const spec_kv* cache, const int32_t* cache_len, const int32_t* idx,
                           int32_t budget, int64_t idx_stride_b, const spec_kv_mut* partial,
                           int32_t* partial_len, uint8_t* partial_pad,
                           int64_t partial_pad_stride_b, void* workspace, size_t workspace_bytes,
                           void* stream) {
  const spec_dims d{batch, n_kv_heads, n_kv_heads, head_dim, dtype, 1.f};
  spec_status st = check_dims(&d);
  if (st != SPEC_OK) return st;
  if (budget < 1) return fail(SPEC_E_INVALID, "budget %d < 1", budget);
  if (batch > 65535) return fail(SPEC_E_UNSUPPORTED, "batch must be <= 65535");
  if (batch == 0) return SPEC_OK;
  if ((st = check_kv(cache, &d, "cache", true)) != SPEC_OK) return st;
  if (partial == nullptr) return fail(SPEC_E_INVALID, "partial is NULL");
  const spec_kv pc{partial->k, partial->v, partial->stride_b, partial->stride_h, partial->stride_t,
                   partial->capacity};
  if ((st = check_kv(&pc, &d, "partial", true)) != SPEC_OK) return st;
  if (partial->capacity < budget)
    return fail(SPEC_E_INVALID, "partial capacity %d < budget %d", partial->capacity, budget);
  if (cache_len == nullptr || idx == nullptr || partial_len == nullptr || partial_pad == nullptr)
    return fail(SPEC_E_INVALID, "a required pointer is NULL");
  if (!aligned(cache_len, 4) || !aligned(idx, 4) || !aligned(partial_len, 4))
    return fail(SPEC_E_INVALID, "int32 arrays must be 4-byte aligned");
  if (idx_stride_b < budget) return fail(SPEC_E_INVALID, "idx_stride_b %lld < budget %d",
                                         (long long)idx_stride_b, budget);
  if (partial_pad_stride_b < partial->capacity)
    return fail(SPEC_E_INVALID, "partial_pad_stride_b %lld < partial capacity %d",
                (long long)partial_pad_stride_b, partial->capacity);
  if (workspace == nullptr || workspace_bytes < kHeaderBytes)
    return fail(SPEC_E_WORKSPACE, "workspace of %zu bytes needed", kHeaderBytes);
  if (!aligned(workspace, 256)) return fail(SPEC_E_INVALID, "workspace must be 256-byte aligned");
  const int64_t es = esize(dtype);
  GatherArgs a;
  a.k = static_cast<const char*>(cache->k);
  a.v = static_cast<const char*>(cache->v);
  a.c_sb = cache->stride_b * es;
  a.c_sh = cache->stride_h * es;
  a.c_st = cache->stride_t * es;
  a.pk = static_cast<char*>(partial->k);
  a.pv = static_cast<char*>(partial->v);
  a.p_sb = partial->stride_b * es;
  a.p_sh = partial->stride_h * es;
  a.p_st = partial->stride_t * es;
  a.batch = batch;
  a.n_kv_heads = n_kv_heads;
  a.row_chunks = (int32_t)(head_dim * es / 16);
  a.budget = budget;
  a.capacity = cache->capacity;
  a.cache_len = cache_len;
  a.idx = idx;
  a.idx_sb = idx_stride_b;
  a.partial_len = partial_len;
  a.partial_pad = partial_pad;
  a.pad_sb = partial_pad_stride_b;
  a.err = static_cast<uint32_t*>(workspace);
  hipError_t e = launch_kv_gather(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "kv gather launch");
  return SPEC_OK;
}

int32_t spec_verify_mode(int64_t seq_len, int32_t budget, int32_t buffered, int32_t n_nodes,
                         int32_t buffer_capacity) {
  if (seq_len < 0 || budget < 1 || buffered < 0 || n_nodes < 1 || buffer_capacity < 0) {
    fail(SPEC_E_INVALID, "need seq_len >= 0, budget >= 1, buffered >= 0, n_nodes >= 1, "
                         "buffer_capacity >= 0");
    return SPEC_E_INVALID;
  }
  if (seq_len < budget) return SPEC_VERIFY_FULL;
  if ((int64_t)buffered + n_nodes > buffer_capacity) return SPEC_VERIFY_FULL;
  return SPEC_VERIFY_PARTIAL;
}

size_t spec_select_workspace_bytes(const spec_dims* dims, int32_t max_blocks) {
  if (check_dims(dims) != SPEC_OK) return 0;
  if (max_blocks < 0) {
    fail(SPEC_E_INVALID, "max_blocks %d < 0", max_blocks);
    return 0;
  }
  return select_bytes(dims, max_blocks);
}

spec_status spec_device_status(void* workspace, void* stream, uint32_t* bits_or_null) {
  if (workspace == nullptr) return fail(SPEC_E_INVALID, "workspace is NULL");
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  uint32_t bits = 0;
  e = hipMemcpy(&bits, workspace, sizeof bits, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy (read error word)");
  if (bits_or_null) *bits_or_null = bits;
  if (bits == 0) return SPEC_OK;
  const uint32_t zero = 0;
  e = hipMemcpy(workspace, &zero, sizeof zero, hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy (clear error word)");
  return fail(SPEC_E_DEVICE_RANGE, "device range error bits 0x%x", bits);
}

#ifdef SPEC_DEBUG_PLAN
// Debug build only: walks every workgroup of the bf16 attention plan of a
// shape, the way the kernel derives its ranges, and checks that what the
// kernel stages and addresses stays inside its LDS arrays, its counters and
// the workspace.  mode: 0 window draft, 1 budget draft, 2 verify; `extent`
// is the view length (drafts) or the cache capacity (verify).  Returns 0
// (in bounds), 1 (shape refused, nothing to check) or -1 with a message.
int32_t spec_debug_check_plan(const spec_dims* d, int32_t mode, int32_t T, int64_t extent,
                              char* msg, size_t msg_len) {
  auto bad = [&](const char* fmt, auto... args) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Wformat-security"
    snprintf(msg, msg_len, fmt, args...);
#pragma clang diagnostic pop
    return (int32_t)-1;
  };
  if (check_dims(d) != SPEC_OK || d->dtype != SPEC_BF16 || T < 1 || extent < 0) return 1;
  if (mode == 2 && T > kMaxNodes) return 1;
  const bool gather = mode == 1, verify = mode == 2;
  const int64_t tiles = verify ? cdiv(extent, kTileKeys) + cdiv(T, kTileKeys)
                               : cdiv(std::max<int64_t>(extent, 1), kTileKeys);
  if (tiles > INT32_MAX / 2) return 1;
  const Plan p = verify ? verify_plan(d, T, (int32_t)std::min<int64_t>(extent, INT32_MAX))
                        : draft_plan(d, T, extent, gather);
  if (p.total == 0) return 1;
  const int G = d->n_q_heads / d->n_kv_heads;
  const int64_t pairs = (int64_t)d->batch * d->n_kv_heads;
  const int64_t groups = pairs * p.n_rb;
  if ((int64_t)p.rb * p.n_rb < (int64_t)T * G) return bad("row blocks %d x %d miss rows %d", p.n_rb, p.rb, T * G);
  if (p.rb != (p.wk == 4 ? 16 * p.rt : 64 * p.rt)) return bad("row block %d does not match the shape", p.rb);
  if ((int64_t)p.splits * p.tps < tiles || (int64_t)(p.splits - 1) * p.tps >= tiles)
    return bad("splits %d x %d tiles do not cover %lld tiles exactly", p.splits, p.tps, (long long)tiles);
  if (p.splits > kMaxSplits || p.n_blk != cdiv(p.splits, kMergeFan)) return bad("merge plan");
  if (verify && p.ordered && d->batch > kMaxOrderBatch) return bad("ordered verify beyond %d", kMaxOrderBatch);
  // counters: [cnt_l0: groups x n_blk][cnt_l1: groups][cnt_pos: 2B][cnt_chunk: groups]
  const int64_t words = groups * p.n_blk + groups + 2 * (int64_t)d->batch + groups;
  if (p.cnt_off != kHeaderBytes || words > (int64_t)kCounterWords)
    return bad("%lld counter words exceed the region", (long long)words);
  if (p.splits > 1) {
    // one group's slots: a (pair, row block)'s splits, or in the ordered
    // verify a (KV head, row block)'s work items
    const uint64_t slots = p.ordered ? (uint64_t)p.items : (uint64_t)p.splits;
    const uint64_t n_groups = p.ordered ? (uint64_t)d->n_kv_heads * p.n_rb : (uint64_t)groups;
    const uint64_t part = slots * p.rb * d->head_dim * 4;   // one group's o partials
    if (part > UINT32_MAX) return bad("a group's partials exceed a buffer descriptor");
    if (p.o_off < kScratchOff || p.o_off + n_groups * part > p.lse_off ||
        p.lse_off + n_groups * slots * p.rb * 4 > (p.n_blk > 1 ? p.o1_off : p.total))
      return bad("split partials overlap");
  }
  if (p.n_blk > 1 && p.lse1_off + (uint64_t)groups * p.n_blk * p.rb * 4 > p.total)
    return bad("block partials overrun the workspace");
  const int64_t cache_tiles_max = verify ? cdiv(extent, kTileKeys) : tiles;
  for (int s = 0; s < p.splits; ++s) {
    // the largest total a workgroup can meet is the plan's own bound
    int t0, t1;
    split_tiles((int)tiles, p.tps, s, t0, t1);
    if (t0 > t1) return bad("split %d: empty range reversed", s);
    if (gather) {
      const int64_t cnt = std::max<int64_t>(0, std::min<int64_t>((int64_t)t1 * kTileKeys, extent) -
                                                   (int64_t)t0 * kTileKeys);
      if (cnt > kMaxGatherKeys) return bad("split %d stages %lld budget indices", s, (long long)cnt);
    }
    if (verify) {
      const int64_t wend = std::min<int64_t>(t1, cache_tiles_max);
      if (wend - t0 > kMaxPadWords) return bad("split %d stages %lld pad words", s, (long long)(wend - t0));
    }
  }
  if (verify && p.ordered) {
    // the kernel's balanced plan, for a few length patterns: every split
    // must have a work item, stage at most tps_max pad words, and its
    // partial slot must lie inside the split-partial buffer
    if (p.tps_max > kMaxPadWords || p.tps > p.tps_max || p.conc < 1) return bad("ordered bounds");
    if ((int64_t)p.items > (int64_t)d->batch * p.splits) return bad("ordered items");
    if ((int64_t)p.items * p.rb * d->head_dim * 4 > INT32_MAX)
      return bad("%d item partials exceed 32-bit offsets", p.items);
    const int64_t cap_tiles = cdiv(extent, kTileKeys), nt = cdiv(T, kTileKeys);
    // (patterns: all full, all empty, one full, a linear ramp, then
    // pseudo-random lengths: uniform, cubed toward short, and a mix of full
    // and near-empty sequences)
    uint64_t rs = 0x9e3779b97f4a7c15ull ^ ((uint64_t)d->batch << 32) ^ (uint64_t)cap_tiles;
    const auto rnd = [&]() {   // xorshift64, values in [0, 1)
      rs ^= rs << 13;
      rs ^= rs >> 7;
      rs ^= rs << 17;
      return (double)(rs >> 11) / 9007199254740992.0;
    };
    for (int pattern = 0; pattern < 10; ++pattern) {
      int64_t W = 0, n_items = 0;
      std::vector<int64_t> tl(d->batch);
      for (int b = 0; b < d->batch; ++b) {
        const double u = pattern >= 4 ? rnd() : 0.0;
        const int64_t len_tiles = pattern == 0 ? cap_tiles
                                : pattern == 1 ? 0
                                : pattern == 2 ? (b == 0 ? cap_tiles : 0)
                                : pattern == 3 ? (cap_tiles * (b + 1)) / d->batch
                                : pattern % 3 == 1 ? (int64_t)(u * (double)(cap_tiles + 1))
                                : pattern % 3 == 2 ? (int64_t)(u * u * u * (double)(cap_tiles + 1))
                                                   : (u < 0.2 ? cap_tiles : (int64_t)(u * 0.02 * (double)cap_tiles));
        tl[b] = len_tiles + nt;
        W += tl[b];
      }
      // the kernel's search: the smallest T in [lo, hi] whose splits number
      // at most conc
      const auto count = [&](int64_t T) {
        int64_t c = 0;
        for (int b = 0; b < d->batch; ++b) c += std::min<int64_t>(p.splits, cdiv(tl[b], T));
        return c;
      };
      int64_t lo = std::max<int64_t>(1, cdiv(W, p.conc));
      int64_t hi = p.conc > d->batch ? cdiv(W, p.conc - d->batch) : p.tps_max;
      hi = std::min<int64_t>(std::max(hi, lo), p.tps_max);
      lo = std::min(lo, hi);
      while (lo < hi) {
        const int64_t mid = (lo + hi) / 2;
        if (count(mid) <= p.conc) hi = mid;
        else lo = mid + 1;
      }
      const int64_t tgt = lo;
      for (int b = 0; b < d->batch; ++b) {
        const int64_t sb = std::min<int64_t>(p.splits, cdiv(tl[b], tgt));
        if (cdiv(tl[b], sb) > p.tps_max) return bad("ordered split of %lld tiles", (long long)cdiv(tl[b], sb));
        n_items += sb;
      }
      if (n_items > p.items) return bad("%lld splits for %d items", (long long)n_items, p.items);
    }
    if (p.items < 1) return bad("no work items");
  }
  if (grid_size(d, p) > kMaxGrid) return bad("grid");
  return 0;
}
#endif

}  // extern "C"
#pragma GCC visibility pop
