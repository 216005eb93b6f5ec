/* Test-only entry point of the debug build of libspecattn (compiled with
 * -DSPEC_DEBUG_PLAN): walks every workgroup of the bf16 attention plan of a
 * shape and checks that what the kernel stages (budget indices, pad words,
 * counters, split partials) stays inside its arrays and the workspace.
 * mode: 0 window draft, 1 budget draft, 2 verify; extent: view length or
 * cache capacity.  Returns 0 (in bounds), 1 (shape refused) or -1 (message
 * in msg). */
#ifndef SPEC_DEBUG_H
#define SPEC_DEBUG_H
#include "spec_attn.h"
#ifdef __cplusplus
extern "C" {
#endif
int32_t spec_debug_check_plan(const spec_dims* d, int32_t mode, int32_t T, int64_t extent,
                              char* msg, size_t msg_len);
#ifdef __cplusplus
}
#endif
#endif
