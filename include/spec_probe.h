/*
 * spec_probe.h -- measurement kernels of libspecprobe (gfx950).
 *
 * Not part of the method: these calls measure the machine the attention
 * kernels run on, so that every rate can be reported against what the GPU
 * delivers, not only against its data-sheet peak.  Windowed-MTP's step cost
 * (Eq. 1 of "Windowed-MTP: Removing the Full-Context Draft-KV Tax at
 * Million-Token Context", Pith review) is a sum of per-call times, so two
 * figures bound a call from below: the HBM read rate a streaming kernel
 * reaches (the ceiling of the long verify reads), and the time of a launch
 * that does no work, or reads a draft-sized buffer once (the floor of the
 * short draft calls).
 *
 * All pointers are device pointers owned by the caller; calls are
 * asynchronous on `stream` (a hipStream_t passed as void*) and return 0 or
 * a negative status (-1 bad argument, -4 HIP error).
 */
#ifndef SPEC_PROBE_H
#define SPEC_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` bytes at `src` once with 16-byte non-temporal buffer loads
 * (the load the register-staged attention path uses), `in_flight` loads per
 * thread before any is used, spread over `workgroups` workgroups of 256
 * threads.  Workgroup w reads the 4 KiB blocks w, w + workgroups, ...; it
 * XORs what it read and writes one word to sink[w], so no load can be
 * dropped.  src 16-byte aligned, bytes a multiple of 4096, workgroups in
 * [1, 2^20], in_flight one of 4, 8, 16. */
int32_t spec_probe_read(const void* src, size_t bytes, int32_t workgroups, int32_t in_flight,
                        uint32_t* sink, void* stream);

/* The same read through global_load_lds_dwordx4, the direct HBM-to-LDS copy
 * of the shared-ring attention path: each workgroup streams its blocks into
 * a ring of `stages` 16 KiB LDS stages (2..8) and XORs one word per block
 * from LDS. */
int32_t spec_probe_read_lds(const void* src, size_t bytes, int32_t workgroups, int32_t stages,
                            uint32_t* sink, void* stream);

/* One launch of `workgroups` workgroups of 256 threads that do nothing but
 * write sink[w] = w: the fixed cost of a launch. */
int32_t spec_probe_empty(int32_t workgroups, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_PROBE_H */
