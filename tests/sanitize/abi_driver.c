/* Host-side exercise of libspecattn under AddressSanitizer and
 * UndefinedBehaviorSanitizer (CPU only, no kernel is launched):
 *   1. the split planner of the bf16 attention kernels over a sweep of
 *      shapes, each checked workgroup by workgroup by the debug build's plan
 *      checker (staged indices and pad words within their LDS arrays,
 *      counters within their region, partials within the workspace);
 *   2. every workspace sizer at ordinary and extreme arguments;
 *   3. every entry point with arguments its host-side validation must
 *      reject before launching anything.
 * Prints "abi driver ok: ..." and exits 0, or names the first failure. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "spec_attn.h"
#include "spec_debug.h"

static int failures = 0;

#define EXPECT(cond, ...)                       \
  do {                                          \
    if (!(cond)) {                              \
      fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);             \
      fprintf(stderr, "\n");                    \
      ++failures;                               \
    }                                           \
  } while (0)

static spec_dims dims(int B, int Hq, int Hkv, int D, int dtype) {
  spec_dims d;
  memset(&d, 0, sizeof d);
  d.batch = B;
  d.n_q_heads = Hq;
  d.n_kv_heads = Hkv;
  d.head_dim = D;
  d.dtype = dtype;
  d.softmax_scale = 0.088f;
  d.flags = 0;
  return d;
}

static long plan_sweep(void) {
  static const int Bs[] = {1, 2, 7, 8, 16, 100, 256, 300, 1000};
  static const int Hkvs[] = {1, 8, 32};
  static const int Gs[] = {1, 4, 8};
  static const int Ds[] = {64, 128};
  static const int Ts[] = {1, 3, 5, 8};
  static const int Ns[] = {1, 3, 5, 15, 44, 64};
  static const int64_t views[] = {1, 31, 32, 33, 256, 700, 2048, 2049, 4100, 65536, 524288};
  static const int64_t caps[] = {0, 1, 512, 6000, 16384, 32768, 65536, 1 << 20, (1 << 23) - 64};
  char msg[512];
  long checked = 0;
  for (size_t ib = 0; ib < sizeof Bs / sizeof *Bs; ++ib)
    for (size_t ih = 0; ih < sizeof Hkvs / sizeof *Hkvs; ++ih)
      for (size_t ig = 0; ig < sizeof Gs / sizeof *Gs; ++ig)
        for (size_t id = 0; id < sizeof Ds / sizeof *Ds; ++id)
          for (int det = 0; det < 2; ++det) {
            spec_dims d = dims(Bs[ib], Hkvs[ih] * Gs[ig], Hkvs[ih], Ds[id], SPEC_BF16);
            d.flags = det ? SPEC_FLAG_DETERMINISTIC : 0;
            for (int mode = 0; mode < 2; ++mode)
              for (size_t it = 0; it < sizeof Ts / sizeof *Ts; ++it)
                for (size_t iv = 0; iv < sizeof views / sizeof *views; ++iv) {
                  int rc = spec_debug_check_plan(&d, mode, Ts[it], views[iv], msg, sizeof msg);
                  EXPECT(rc >= 0, "draft mode %d B=%d Hkv=%d G=%d D=%d T=%d view=%lld: %s", mode,
                         d.batch, d.n_kv_heads, Gs[ig], d.head_dim, Ts[it], (long long)views[iv], msg);
                  ++checked;
                }
            for (size_t in = 0; in < sizeof Ns / sizeof *Ns; ++in)
              for (size_t ic = 0; ic < sizeof caps / sizeof *caps; ++ic) {
                int rc = spec_debug_check_plan(&d, 2, Ns[in], caps[ic], msg, sizeof msg);
                EXPECT(rc >= 0, "verify B=%d Hkv=%d G=%d D=%d N=%d cap=%lld: %s", d.batch,
                       d.n_kv_heads, Gs[ig], d.head_dim, Ns[in], (long long)caps[ic], msg);
                ++checked;
              }
          }
  /* the workload shapes themselves must be planned, not refused */
  spec_dims w = dims(1, 32, 8, 128, SPEC_BF16);
  EXPECT(spec_debug_check_plan(&w, 2, 3, 1 << 20, msg, sizeof msg) == 0, "1M verify: %s", msg);
  EXPECT(spec_debug_check_plan(&w, 0, 3, 4102, msg, sizeof msg) == 0, "1M ctx draft: %s", msg);
  w.batch = 8;
  EXPECT(spec_debug_check_plan(&w, 2, 64, 16384, msg, sizeof msg) == 0, "16K verify: %s", msg);
  EXPECT(spec_debug_check_plan(&w, 1, 1, 2048, msg, sizeof msg) == 0, "16K draft: %s", msg);
  w.batch = 16;
  EXPECT(spec_debug_check_plan(&w, 2, 44, 32768, msg, sizeof msg) == 0, "ragged verify: %s", msg);
  return checked;
}

static void sizers(void) {
  spec_dims d = dims(8, 32, 8, 128, SPEC_BF16);
  size_t a = spec_draft_workspace_bytes(&d, 1, 256), b = spec_draft_workspace_bytes(&d, 1, 2048);
  EXPECT(a > 0 && b >= a, "draft sizes %zu %zu", a, b);
  /* a window view has no staging limit; a budget list of 2^31 - 1 does */
  EXPECT(spec_draft_workspace_bytes(&d, 1, 0x7fffffff) > 0, "huge window view");
  char msg[256];
  EXPECT(spec_debug_check_plan(&d, 1, 1, 0x7fffffff, msg, sizeof msg) == 1, "huge budget list refused");
  EXPECT(spec_draft_workspace_bytes(&d, 0, 256) == 0, "zero queries");
  EXPECT(spec_draft_workspace_bytes(&d, 0x7fffffff, 256) == 0, "huge query count refused");
  EXPECT(spec_draft_workspace_bytes(&d, 16384, 256) > 0, "16,384 queries x GQA 4 planned");
  EXPECT(spec_draft_workspace_bytes(NULL, 1, 256) == 0, "null dims");
  EXPECT(spec_verify_workspace_bytes(&d, 64, 0x7fffffff) == 0, "huge capacity must be refused");
  EXPECT(spec_verify_workspace_bytes(&d, 65, 100) == 0, "65 nodes");
  EXPECT(spec_verify_workspace_bytes(&d, 64, 16384) > 0, "16K verify size");
  EXPECT(spec_accept_workspace_bytes(8, 64, 128256) > 0, "accept size");
  EXPECT(spec_accept_workspace_bytes(-1, 64, 10) == 0, "negative batch");
  EXPECT(spec_accept_workspace_bytes(0x7fffffff, 64, 0x7fffffff) > 0, "huge accept sized without overflow");
  EXPECT(spec_compact_workspace_bytes(0x7fffffff) > 0, "huge compact sized");
  EXPECT(spec_select_workspace_bytes(&d, -1) == 0, "negative blocks");
  spec_dims big = dims(0x7fffffff, 0x7fffffff, 1, 128, SPEC_BF16);
  (void)spec_draft_workspace_bytes(&big, 64, 0x7fffffff);
  (void)spec_verify_workspace_bytes(&big, 64, 0x7fffffff);
  (void)spec_select_workspace_bytes(&big, 0x7fffffff);
  spec_dims f = dims(1, 2, 1, 64, SPEC_F32);
  EXPECT(spec_verify_workspace_bytes(&f, 15, 512) > 0, "fp32 verify size");
  EXPECT(spec_draft_workspace_bytes(&f, 1, 68) > 0, "fp32 draft size");
  d.flags = 2;
  EXPECT(spec_draft_workspace_bytes(&d, 1, 256) == 0, "unknown flag");
}

static void rejections(void) {
  /* fake, never dereferenced device addresses: every call below must fail
   * host-side validation before any launch */
  char* p = (char*)(uintptr_t)0x100000;
  void* ws = p;
  int32_t* ip = (int32_t*)p;
  spec_dims d = dims(2, 8, 2, 128, SPEC_BF16);
  spec_kv kv = {p, p, 2 * 1024 * 128, 1024 * 128, 128, 1024};
  spec_kv bad_kv = kv;
  bad_kv.stride_t = 100;
  spec_kv huge = kv;
  huge.stride_t = (int64_t)1 << 40;
  spec_kv over = kv;
  over.capacity = 0x7fffffff;
  over.stride_t = 1 << 20;
  EXPECT(spec_attn_draft_sparse(NULL, p, 1, &kv, ip, 4, 64, NULL, 0, 0, 0, p, NULL, ws, 1 << 30, NULL) != SPEC_OK, "null dims");
  EXPECT(spec_attn_draft_sparse(&d, p, 0, &kv, ip, 4, 64, NULL, 0, 0, 0, p, NULL, ws, 1 << 30, NULL) == SPEC_E_INVALID, "Tq 0");
  EXPECT(spec_attn_draft_sparse(&d, p, 1, &bad_kv, ip, 4, 64, NULL, 0, 0, 0, p, NULL, ws, 1 << 30, NULL) == SPEC_E_INVALID, "stride");
  EXPECT(spec_attn_draft_sparse(&d, p, 1, &huge, ip, 4, 64, NULL, 0, 0, 0, p, NULL, ws, 1 << 30, NULL) != SPEC_OK, "huge stride");
  EXPECT(spec_attn_draft_sparse(&d, p, 1, &over, ip, 4, 64, NULL, 0, 0, 0, p, NULL, ws, 1 << 30, NULL) != SPEC_OK, "4 GiB head");
  EXPECT(spec_attn_draft_sparse(&d, p, 1, &kv, ip, 4, 0, NULL, 0, 0, 0, p, NULL, ws, 1 << 30, NULL) == SPEC_E_INVALID, "window 0");
  EXPECT(spec_attn_draft_sparse(&d, p, 1, &kv, ip, 4, 64, ip, 0, 0, 0, p, NULL, ws, 1 << 30, NULL) == SPEC_E_INVALID, "budget 0");
  EXPECT(spec_attn_draft_sparse(&d, p, 1, &kv, ip, 4, 64, ip, 1 << 30, 0, 0, p, NULL, ws, 1 << 30, NULL) == SPEC_E_UNSUPPORTED, "budget too long");
  EXPECT(spec_attn_draft_sparse(&d, p, 1, &kv, ip, 4, 64, NULL, 0, 0, 0, p, NULL, ws, 16, NULL) == SPEC_E_WORKSPACE, "small workspace");
  EXPECT(spec_attn_draft_sparse(&d, p + 1, 1, &kv, ip, 4, 64, NULL, 0, 0, 0, p, NULL, ws, 1 << 30, NULL) == SPEC_E_INVALID, "q alignment");
  EXPECT(spec_attn_draft_ring(&d, p, 3, &kv, ip, 4, 64, 65, p, NULL, ws, 1 << 30, NULL) == SPEC_E_INVALID, "ring too small");
  EXPECT(spec_attn_verify_tree(&d, p, 65, &kv, ip, NULL, 0, &kv, ip, 0, p, NULL, NULL, ws, 1 << 30, NULL) == SPEC_E_UNSUPPORTED, "65 nodes");
  EXPECT(spec_attn_verify_tree(&d, p, 5, &kv, ip, NULL, 0, &kv, NULL, 0, p, NULL, NULL, ws, 1 << 30, NULL) == SPEC_E_INVALID, "null parents");
  EXPECT(spec_attn_verify_tree(&d, p, 5, &kv, ip, (uint8_t*)p, 3, &kv, ip, 0, p, NULL, NULL, ws, 1 << 30, NULL) == SPEC_E_INVALID, "pad stride");
  EXPECT(spec_attn_verify_tree(&d, p, 5, &kv, ip, NULL, 0, &kv, ip, 3, p, NULL, NULL, ws, 1 << 30, NULL) == SPEC_E_INVALID, "parents stride");
  EXPECT(spec_attn_verify_tree(&d, p, 5, &kv, ip, NULL, 0, &kv, ip, 0, p, NULL, NULL, ws, 16, NULL) == SPEC_E_WORKSPACE, "verify workspace");
  EXPECT(spec_accept_greedy(2, 5, 0, (float*)p, ip, ip, 0, 4, ip, ip, ip, ws, 1 << 30, NULL) == SPEC_E_INVALID, "vocab 0");
  EXPECT(spec_accept_greedy(2, 5, 100, (float*)(p + 4), ip, ip, 0, 4, ip, ip, ip, ws, 1 << 30, NULL) == SPEC_E_INVALID, "logits alignment");
  EXPECT(spec_accept_greedy(2, 5, 100, (float*)p, ip, ip, 0, 0, ip, ip, ip, ws, 1 << 30, NULL) == SPEC_E_INVALID, "max depth 0");
  EXPECT(spec_accept_greedy(2, 5, 100, (float*)p, ip, ip, 0, 4, ip, ip, ip, ws, 16, NULL) == SPEC_E_WORKSPACE, "accept workspace");
  spec_kv_mut mk = {p, p, 2 * 1024 * 128, 1024 * 128, 128, 1024};
  EXPECT(spec_kv_commit(2, 2, 128, SPEC_BF16, &mk, ip, (uint8_t*)p, 10, &kv, 5, ip, ip, 4, NULL, ws, 1 << 30, NULL) == SPEC_E_INVALID, "pad stride < capacity");
  EXPECT(spec_kv_commit(2, 2, 128, SPEC_BF16, NULL, ip, (uint8_t*)p, 1024, &kv, 5, ip, ip, 4, NULL, ws, 1 << 30, NULL) == SPEC_E_INVALID, "null cache");
  EXPECT(spec_kv_compact(2, 2, 128, SPEC_BF16, &mk, ip, (uint8_t*)p, 1022, ws, 1 << 30, NULL) == SPEC_E_INVALID, "compact pad stride");
  EXPECT(spec_block_means(&d, &kv, ip, NULL, 0, 0, 0, 1, (float*)p, 64, ws, 1 << 30, NULL) == SPEC_E_INVALID, "block 0");
  EXPECT(spec_select_blocks(&d, p, 1, (float*)p, 9000, 16, ip, 1024, NULL, 0, 4, 64, 4, 0, ip, 256, NULL, ws, 1 << 30, NULL) == SPEC_E_UNSUPPORTED, "too many blocks");
  EXPECT(spec_select_blocks(&d, p, 1, (float*)p, 64, 16, ip, 1024, NULL, 0, 4, 64, 40, 0, ip, 256, NULL, ws, 1 << 30, NULL) == SPEC_E_INVALID, "budget too small");
  spec_kv_mut pk = {p, p, 2 * 512 * 128, 512 * 128, 128, 100};
  EXPECT(spec_kv_gather(2, 2, 128, SPEC_BF16, &kv, ip, ip, 200, 200, &pk, ip, (uint8_t*)p, 512, ws, 1 << 30, NULL) == SPEC_E_INVALID, "partial capacity");
  EXPECT(spec_verify_mode(-1, 10, 0, 5, 10) == SPEC_E_INVALID, "verify mode");
  EXPECT(spec_verify_mode(100, 200, 0, 5, 64) == SPEC_VERIFY_FULL, "short sequence");
  EXPECT(spec_verify_mode(1000, 200, 60, 5, 64) == SPEC_VERIFY_FULL, "buffer overflow");
  EXPECT(spec_verify_mode(1000, 200, 10, 5, 64) == SPEC_VERIFY_PARTIAL, "partial");
  spec_dims z = dims(0, 8, 2, 128, SPEC_BF16);
  EXPECT(spec_attn_draft_sparse(&z, NULL, 1, NULL, NULL, 4, 64, NULL, 0, 0, 0, NULL, NULL, NULL, 0, NULL) == SPEC_OK, "empty batch");
  EXPECT(spec_attn_verify_tree(&z, NULL, 5, NULL, NULL, NULL, 0, NULL, NULL, 0, NULL, NULL, NULL, NULL, 0, NULL) == SPEC_OK, "empty verify");
  EXPECT(spec_accept_greedy(0, 5, 10, NULL, NULL, NULL, 0, 4, NULL, NULL, NULL, NULL, 0, NULL) == SPEC_OK, "empty accept");
  EXPECT(strlen(spec_last_error()) > 0, "last error set");
  EXPECT(strcmp(spec_status_string(SPEC_E_WORKSPACE), "SPEC_E_WORKSPACE") == 0, "status string");
  EXPECT(spec_abi_version() == SPEC_ABI_VERSION, "abi version");
}

int main(void) {
  long n = plan_sweep();
  sizers();
  rejections();
  if (failures) {
    fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  printf("abi driver ok: %ld plans checked workgroup by workgroup, sizers and rejections clean\n", n);
  return 0;
}
