/* Host-side check of libkvpop's argument validation, built and run with
 * AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_abi.py builds
 * the library's C ABI glue with both and links this program against it).
 * Every call below must return its error status before any launch, so no GPU
 * is needed; the sanitizers watch the validation code for out-of-bounds
 * reads, overflow in the size arithmetic and other undefined behaviour.
 * Prints "abi_check ok" and exits 0 when every status matches. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kvpop.h"

static int failures = 0;

#define EXPECT(call, want)                                                          \
  do {                                                                              \
    int got_ = (int)(call);                                                         \
    if (got_ != (int)(want)) {                                                      \
      fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call, got_, \
              (int)(want));                                                         \
      ++failures;                                                                   \
    }                                                                               \
  } while (0)

static kvpop_problem base(void) {
  kvpop_problem p;
  memset(&p, 0, sizeof p);
  p.batch = 1;
  p.n_q_heads = 32;
  p.n_kv_heads = 8;
  p.seq_len = 16384;
  p.head_dim = 128;
  p.sink = 16;
  p.window = 512;
  p.topk = 1520;
  p.softmax_scale = 0.0f;
  p.qkv_dtype = KVPOP_BF16;
  p.out_dtype = KVPOP_BF16;
  return p;
}

int main(void) {
  void* d = (void*)(uintptr_t)0x1000;   /* a non-NULL pointer that is never dereferenced */
  kvpop_problem p = base();
  kvpop_cache c = {d, d, (int32_t*)d, (float*)d, (int32_t*)d};
  const size_t big = (size_t)1 << 40;

  /* workspace sizes: positive for valid problems, 0 for invalid ones and calls */
  for (int call = KVPOP_CALL_THRESHOLDS; call <= KVPOP_CALL_MASKED_BWD; ++call)
    (void)kvpop_workspace_size(call, &p);
  EXPECT(kvpop_workspace_size(-1, &p), 0);
  EXPECT(kvpop_workspace_size(99, &p), 0);
  EXPECT(kvpop_workspace_size(KVPOP_CALL_THRESHOLDS, NULL), 0);
  p.n_q_heads = 30;
  EXPECT(kvpop_workspace_size(KVPOP_CALL_THRESHOLDS, &p), 0);
  p = base();

  /* extreme sizes: the budget and the size arithmetic must not overflow */
  p.sink = 0x7fffffff;
  p.window = 0x7fffffff;
  p.topk = 0x7fffffff;
  EXPECT(kvpop_thresholds(&p, (const float*)d, (int32_t*)d, (int32_t*)d, d, big, NULL),
         KVPOP_ERR_ARG);
  EXPECT(kvpop_workspace_size(KVPOP_CALL_DECODE, &p), 0);
  p = base();
  p.batch = 0x7fffffff;
  p.seq_len = 262144;
  (void)kvpop_workspace_size(KVPOP_CALL_MASKED_FWD, &p);
  (void)kvpop_workspace_size(KVPOP_CALL_MASKED_BWD, &p);
  p = base();
  p.seq_len = 262145;
  EXPECT(kvpop_masked_attn_fwd(&p, d, d, d, (const int32_t*)d, (const int32_t*)d, d, (float*)d, d,
                               big, NULL),
         KVPOP_ERR_UNSUPPORTED);
  p = base();

  /* invalid shapes and values */
  p.n_kv_heads = 0;
  EXPECT(kvpop_thresholds(&p, (const float*)d, (int32_t*)d, (int32_t*)d, d, big, NULL),
         KVPOP_ERR_ARG);
  p = base();
  p.softmax_scale = 1.0f / 0.0f;
  EXPECT(kvpop_future_target(&p, d, d, (const float*)d, (float*)d, NULL, 0, NULL), KVPOP_ERR_ARG);
  p = base();
  p.qkv_dtype = 7;
  EXPECT(kvpop_future_target(&p, d, d, (const float*)d, (float*)d, NULL, 0, NULL), KVPOP_ERR_ARG);
  p = base();
  p.head_dim = 96;
  EXPECT(kvpop_masked_attn_fwd(&p, d, d, d, (const int32_t*)d, (const int32_t*)d, d, (float*)d, d,
                               big, NULL),
         KVPOP_ERR_UNSUPPORTED);
  p = base();
  p.window = 0;
  EXPECT(kvpop_masked_attn_fwd(&p, d, d, d, (const int32_t*)d, (const int32_t*)d, d, (float*)d, d,
                               big, NULL),
         KVPOP_ERR_ARG);
  EXPECT(kvpop_decode_step(&p, &c, (const int32_t*)d, d, d, d, (const float*)d, d, (float*)d, d,
                           big, NULL),
         KVPOP_ERR_ARG);
  p = base();

  /* NULL pointers */
  EXPECT(kvpop_thresholds(&p, NULL, (int32_t*)d, (int32_t*)d, d, big, NULL), KVPOP_ERR_ARG);
  EXPECT(kvpop_decode_step(&p, NULL, (const int32_t*)d, d, d, d, (const float*)d, d, (float*)d, d,
                           big, NULL),
         KVPOP_ERR_ARG);
  EXPECT(kvpop_decode_step_noalloc(&p, &c, NULL, d, d, d, (const float*)d, d, (float*)d, NULL),
         KVPOP_ERR_ARG);
  EXPECT(kvpop_cache_from_prefill(&p, &c, d, d, (const float*)d, NULL, (const int32_t*)d, NULL),
         KVPOP_ERR_ARG);
  EXPECT(kvpop_target_score(&p, NULL, 0.0f, (float*)d, NULL), KVPOP_ERR_ARG);
  EXPECT(kvpop_masked_attn_bwd(&p, d, d, d, d, (const float*)d, (const int32_t*)d,
                               (const int32_t*)d, d, (float*)d, (float*)d, NULL, d, big, NULL),
         KVPOP_ERR_ARG);

  /* short, missing and misaligned workspaces */
  const size_t need = kvpop_workspace_size(KVPOP_CALL_THRESHOLDS, &p);
  EXPECT(kvpop_thresholds(&p, (const float*)d, (int32_t*)d, (int32_t*)d, d, need - 1, NULL),
         KVPOP_ERR_WORKSPACE);
  EXPECT(kvpop_thresholds(&p, (const float*)d, (int32_t*)d, (int32_t*)d, NULL, need, NULL),
         KVPOP_ERR_WORKSPACE);
  EXPECT(kvpop_thresholds(&p, (const float*)d, (int32_t*)d, (int32_t*)d, (char*)d + 4, need, NULL),
         KVPOP_ERR_ARG);

  /* other per-call rules */
  EXPECT(kvpop_target_score(&p, (const float*)d, -1.0f, (float*)d, NULL), KVPOP_ERR_ARG);
  EXPECT(kvpop_boundary_labels(&p, (const float*)d, (const float*)d, 0, (int32_t*)d, (int32_t*)d,
                               NULL),
         KVPOP_ERR_ARG);
  p.seq_len = 32769;
  EXPECT(kvpop_boundary_labels(&p, (const float*)d, (const float*)d, 4, (int32_t*)d, (int32_t*)d,
                               NULL),
         KVPOP_ERR_UNSUPPORTED);
  p = base();
  p.qkv_dtype = KVPOP_F32;
  EXPECT(kvpop_masked_attn_bwd(&p, d, d, d, d, (const float*)d, (const int32_t*)d,
                               (const int32_t*)d, d, (float*)d, (float*)d, (float*)d, d, big, NULL),
         KVPOP_ERR_UNSUPPORTED);
  p = base();
  p.batch = 4;
  p.n_q_heads = 256;
  p.n_kv_heads = 8;
  p.topk = 1 << 16;   /* 16 splits x 1024 query rows exceed the fixed scratch */
  EXPECT(kvpop_decode_step_noalloc(&p, &c, (const int32_t*)d, d, d, d, (const float*)d, d,
                                   (float*)d, NULL),
         KVPOP_ERR_SCRATCH);

  /* status strings and the version */
  for (int st = -1; st <= 6; ++st)
    if (!kvpop_status_string((kvpop_status)st)) ++failures;
  EXPECT(kvpop_abi_version(), KVPOP_ABI_VERSION);

  if (failures) {
    fprintf(stderr, "abi_check: %d failure(s)\n", failures);
    return 1;
  }
  printf("abi_check ok\n");
  return 0;
}
