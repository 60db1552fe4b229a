/* Drives the host side of the C ABI (include/yoco.h) through its helpers and
 * the validation of every entry point, for a host AddressSanitizer /
 * UndefinedBehaviorSanitizer build of api.cpp (tests/test_host_sanitizers.py).
 * No call here passes validation, so nothing is ever launched: the data
 * pointers are placeholders that are never dereferenced.  Exits non-zero
 * on a failed check; the sanitizers abort on any memory or undefined-
 * behaviour error. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "yoco.h"

static int failures = 0;
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); ++failures; } } while (0)
#define FAKE ((void *)0x1000)
#define MIS ((void *)0x1008)

static yoco_kv_cache make_cache(int64_t *lens, int n_seq, int64_t cap, int hkv, int dh, int dtype) {
  yoco_kv_cache c;
  memset(&c, 0, sizeof c);
  c.k = (void *)0x2000;
  c.v = (void *)0x3000;
  c.len_host = lens;
  c.seq_capacity = cap;
  c.n_seq = n_seq;
  c.n_kv_heads = hkv;
  c.head_dim = dh;
  c.dtype = dtype;
  return c;
}

int main(void) {
  CHECK(yoco_abi_version() == YOCO_ABI_VERSION);
  CHECK(strlen(yoco_last_error()) < 512);
  size_t bytes = 0;
  int64_t rs = 0;
  CHECK(yoco_kv_cache_bytes(1, 131072, 8, 128, YOCO_DT_BF16, 0, &bytes) == YOCO_OK && bytes == 268435456u);
  CHECK(yoco_kv_cache_bytes(1, 10, 8, 128, YOCO_DT_BF16, 1023, &bytes) == YOCO_ERR_BAD_SHAPE);
  CHECK(yoco_kv_cache_bytes(0, 10, 8, 128, YOCO_DT_BF16, 0, &bytes) == YOCO_ERR_BAD_SHAPE);
  CHECK(yoco_kv_cache_bytes(1, 10, 8, 128, 9, 0, &bytes) == YOCO_ERR_BAD_DTYPE);
  CHECK(yoco_kv_cache_bytes(1, 10, 8, 128, YOCO_DT_BF16, 0, NULL) == YOCO_ERR_NULL_POINTER);
  CHECK(yoco_kv_cache_row_stride(8, 128, YOCO_DT_BF16, &rs) == YOCO_OK && rs == 1088);
  CHECK(yoco_kv_cache_row_stride(0, 128, YOCO_DT_BF16, &rs) == YOCO_ERR_BAD_SHAPE);
  CHECK(yoco_project_workspace(1, 3072, 1024, 2, YOCO_DT_BF16, &bytes) == YOCO_OK && bytes > YOCO_PROJECT_COUNTER_BYTES);
  CHECK(yoco_project_workspace(33, 3072, 1024, 2, YOCO_DT_BF16, &bytes) == YOCO_OK && bytes == 0);
  CHECK(yoco_project_workspace(1, 3072, 1024, 3, YOCO_DT_BF16, &bytes) == YOCO_ERR_BAD_SHAPE);
  float scale = 0.f;
  CHECK(yoco_default_softmax_scale(128, &scale) == YOCO_OK && scale > 0.0883f && scale < 0.0884f);
  CHECK(yoco_cross_attn_prefill_bwd_workspace(1000, 24, &bytes) == YOCO_OK && bytes == 2u * 1000 * 24 * 4);
  CHECK(yoco_project_bwd_workspace(32768, 3072, 1024, 2, &bytes) == YOCO_OK && bytes > 0);
  CHECK(yoco_project_bwd_workspace(10, 5000, 1024, 2, &bytes) == YOCO_ERR_BAD_SHAPE);
  CHECK(yoco_gret_prefill_workspace(32768, 24, 128, YOCO_DT_BF16, &bytes) == YOCO_OK && bytes > 0);
  CHECK(yoco_gret_prefill_workspace(100, 24, 128, YOCO_DT_F32, &bytes) == YOCO_OK && bytes == 0);

  /* the largest cache descriptor: 256 sequences, every length at capacity */
  static int64_t lens[YOCO_MAX_SEQ];
  for (int b = 0; b < YOCO_MAX_SEQ; ++b) lens[b] = 1 + 37 * b;
  yoco_kv_cache c = make_cache(lens, YOCO_MAX_SEQ, 10000, 8, 128, YOCO_DT_BF16);
  CHECK(yoco_cross_attn_decode_workspace(&c, 24, 0, &bytes) == YOCO_OK && bytes > YOCO_DECODE_COUNTER_BYTES);
  CHECK(yoco_cross_attn_decode_workspace(&c, 24, 256, &bytes) == YOCO_OK);
  CHECK(yoco_cross_attn_decode_workspace(&c, 24, 300, &bytes) == YOCO_ERR_BAD_VALUE);
  CHECK(yoco_cross_attn_decode_workspace(&c, 20, 0, &bytes) == YOCO_ERR_BAD_SHAPE);
  /* rejected calls: lengths must stay untouched */
  CHECK(yoco_cross_attn_decode(FAKE, YOCO_DT_BF16, 24, &c, 0.125f, FAKE, NULL, FAKE, 16, 0, NULL) == YOCO_ERR_WORKSPACE);
  CHECK(yoco_cross_attn_decode(FAKE, YOCO_DT_F32, 24, &c, 0.125f, FAKE, NULL, FAKE, 1u << 30, 0, NULL) == YOCO_ERR_BAD_DTYPE);
  CHECK(yoco_cross_attn_decode(FAKE, YOCO_DT_BF16, 24, &c, -1.f, FAKE, NULL, FAKE, 1u << 30, 0, NULL) == YOCO_ERR_BAD_VALUE);
  CHECK(yoco_cross_attn_decode(NULL, YOCO_DT_BF16, 24, &c, 0.125f, FAKE, NULL, FAKE, 1u << 30, 0, NULL) == YOCO_ERR_NULL_POINTER);
  CHECK(yoco_cross_attn_decode(FAKE, YOCO_DT_BF16, 24, &c, 0.125f, MIS, NULL, FAKE, 1u << 30, 0, NULL) == YOCO_ERR_ALIGNMENT);
  lens[5] = 0;
  CHECK(yoco_cross_attn_decode(FAKE, YOCO_DT_BF16, 24, &c, 0.125f, FAKE, NULL, FAKE, 1u << 30, 0, NULL) == YOCO_ERR_OUT_OF_RANGE);
  lens[5] = 10000;
  CHECK(yoco_kv_append(FAKE, YOCO_DT_BF16, 64, NULL, 1e-6f, FAKE, FAKE, YOCO_DT_BF16, &c, NULL, 0, NULL) == YOCO_ERR_OUT_OF_RANGE);
  CHECK(lens[5] == 10000);
  CHECK(yoco_kv_append(FAKE, YOCO_DT_BF16, 64, NULL, 1e-6f, FAKE, FAKE, YOCO_DT_BF16, &c, FAKE, 16, NULL) == YOCO_ERR_OUT_OF_RANGE);
  lens[5] = 5;
  CHECK(yoco_cross_attn_decode_noalloc(FAKE, YOCO_DT_BF16, 24, &c, 0.125f, FAKE, NULL, 256, NULL) == YOCO_ERR_WORKSPACE);

  int64_t one[1] = {100};
  yoco_kv_cache s1 = make_cache(one, 1, 200, 2, 64, YOCO_DT_BF16);
  CHECK(yoco_kv_project(FAKE, YOCO_DT_BF16, 4, 32, NULL, 1e-6f, FAKE, FAKE, YOCO_DT_BF16, &s1, 0, 198, NULL, 0, NULL) == YOCO_ERR_OUT_OF_RANGE);
  CHECK(yoco_kv_project(FAKE, YOCO_DT_BF16, 4, 32, NULL, -1.f, FAKE, FAKE, YOCO_DT_BF16, &s1, 0, 0, NULL, 0, NULL) == YOCO_ERR_BAD_VALUE);
  CHECK(yoco_kv_project(FAKE, YOCO_DT_BF16, 4, 32, NULL, 1e-6f, FAKE, FAKE, YOCO_DT_BF16, &s1, 0, 0, FAKE, 16, NULL) == YOCO_ERR_WORKSPACE);
  CHECK(yoco_kv_project_rope(FAKE, YOCO_DT_BF16, 4, 32, NULL, 1e-6f, FAKE, FAKE, YOCO_DT_BF16, &s1, 0, 0, 0.5, NULL, 0, NULL) == YOCO_ERR_BAD_VALUE);
  CHECK(yoco_kv_append_rope(FAKE, YOCO_DT_BF16, 32, NULL, 1e-6f, FAKE, FAKE, YOCO_DT_BF16, &s1, HUGE_VAL, NULL, 0, NULL) == YOCO_ERR_BAD_VALUE);
  CHECK(yoco_kv_project(FAKE, YOCO_DT_BF16, 0, 32, NULL, 1e-6f, FAKE, FAKE, YOCO_DT_BF16, &s1, 0, 0, NULL, 0, NULL) == YOCO_OK);
  CHECK(one[0] == 100);
  CHECK(yoco_q_project(FAKE, YOCO_DT_BF16, 4, 32, NULL, 1e-6f, FAKE, YOCO_DT_BF16, 4, 96, FAKE, YOCO_DT_BF16, NULL, 0, NULL) == YOCO_ERR_BAD_SHAPE);
  static int64_t pos[YOCO_MAX_SEQ + 1];
  CHECK(yoco_q_project_rope(FAKE, YOCO_DT_BF16, YOCO_MAX_SEQ + 1, 32, NULL, 1e-6f, FAKE, YOCO_DT_BF16, 4, 64, FAKE,
                            YOCO_DT_BF16, pos, 0, 1e4, NULL, 0, NULL) == YOCO_ERR_BAD_SHAPE);
  pos[2] = -1;
  CHECK(yoco_q_project_rope(FAKE, YOCO_DT_BF16, 3, 32, NULL, 1e-6f, FAKE, YOCO_DT_BF16, 4, 64, FAKE, YOCO_DT_BF16,
                            pos, 0, 1e4, NULL, 0, NULL) == YOCO_ERR_OUT_OF_RANGE);
  CHECK(yoco_cross_attn_prefill(FAKE, YOCO_DT_BF16, 90, 11, 4, &s1, 0, 0.125f, FAKE, YOCO_DT_F32, NULL, NULL) == YOCO_ERR_OUT_OF_RANGE);
  CHECK(yoco_cross_attn_prefill(FAKE, YOCO_DT_BF16, 0, 4, 5, &s1, 0, 0.125f, FAKE, YOCO_DT_F32, NULL, NULL) == YOCO_ERR_BAD_SHAPE);
  CHECK(yoco_cross_attn_prefill(FAKE, YOCO_DT_BF16, 0, 0, 4, &s1, 0, 0.125f, FAKE, YOCO_DT_F32, NULL, NULL) == YOCO_OK);
  CHECK(yoco_cross_attn_prefill_bwd(FAKE, FAKE, YOCO_DT_F32, FAKE, FAKE, 0, 4, 4, &s1, 0, 0.125f, FAKE, FAKE, FAKE,
                                    FAKE, 8, NULL) == YOCO_ERR_WORKSPACE);
  CHECK(yoco_kv_project_bwd(FAKE, YOCO_DT_BF16, 4, 32, NULL, 1e-6f, FAKE, FAKE, YOCO_DT_BF16, 2, 64, FAKE, FAKE,
                            YOCO_DT_F32, FAKE, FAKE, FAKE, NULL, FAKE, 0, NULL) == YOCO_ERR_WORKSPACE);
  CHECK(yoco_q_project_bwd(FAKE, YOCO_DT_BF16, 4, 32, NULL, 1e-6f, FAKE, YOCO_DT_BF16, 4, 96, FAKE, YOCO_DT_F32,
                           FAKE, FAKE, NULL, FAKE, 1u << 20, NULL) == YOCO_ERR_BAD_SHAPE);
  CHECK(yoco_gret_prefill(FAKE, FAKE, FAKE, YOCO_DT_BF16, FAKE, 0.f, 100, 4, 128, NULL, FAKE, NULL, FAKE, 1u << 30,
                          NULL) == YOCO_ERR_BAD_VALUE);
  CHECK(yoco_gret_prefill(FAKE, FAKE, FAKE, YOCO_DT_BF16, FAKE, 16.f, 1000, 4, 128, NULL, FAKE, NULL, FAKE, 8,
                          NULL) == YOCO_ERR_WORKSPACE);
  CHECK(yoco_gret_decode(FAKE, FAKE, FAKE, YOCO_DT_BF16, FAKE, 16.f, 2, 4, 128, NULL, FAKE, NULL) == YOCO_ERR_NULL_POINTER);
  CHECK(strlen(yoco_last_error()) > 0);

  if (failures) fprintf(stderr, "%d checks failed\n", failures);
  else printf("ABI driver: every host path ran clean\n");
  return failures ? 1 : 0;
}
