/*
 * Host-only exercise of libtpshard's C ABI under AddressSanitizer and
 * UndefinedBehaviorSanitizer (the host half of the library is built with
 * them; no GPU is touched).  Every call below either is host-only
 * (accounting, shard splits, options, status strings) or carries an
 * argument the validation rejects before anything is enqueued, so each
 * return code is checked and no kernel is launched.  Fake device addresses
 * are never dereferenced.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "tp_shard.h"

static int failures = 0;
#define EXPECT(cond)                                                    \
  do {                                                                  \
    if (!(cond)) {                                                      \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                       \
    }                                                                   \
  } while (0)

#define A16 ((void*)(uintptr_t)0x10000)
#define MIS ((void*)(uintptr_t)0x10002)

int main(void) {
  /* host-only accounting and shard splits */
  tp_comm c;
  EXPECT(tp_comm_bytes(8192, 8192, 8, 2, &c) == TP_OK && c.payload_bytes == 134217728ull);
  EXPECT(tp_comm_bytes(-1, 8, 2, 2, &c) == TP_EINVAL);
  EXPECT(tp_comm_bytes(8, 8, 0, 2, &c) == TP_EINVAL);
  EXPECT(tp_comm_bytes(8, 8, 2, 2, NULL) == TP_EINVAL);
  int64_t f = 0, c0 = 0;
  for (int32_t t = 1; t <= 64; ++t)
    for (int32_t r = 0; r < t; ++r) EXPECT(tp_mlp_shard_cols(11008, t, r, TP_BF16, &f, &c0) == TP_OK);
  EXPECT(tp_mlp_shard_cols(11008, 3, 3, TP_BF16, &f, &c0) == TP_EINVAL);
  EXPECT(tp_mlp_shard_cols(11004, 3, 0, TP_BF16, &f, &c0) == TP_EALIGN);
  EXPECT(tp_mlp_shard_cols(INT64_MAX, 1, 0, TP_F32, &f, &c0) == TP_EALIGN);
  EXPECT(tp_mlp_shard_cols(INT64_MAX - 3, 1, 0, TP_F32, &f, &c0) == TP_OK && f == INT64_MAX - 3 && c0 == 0);
  EXPECT(tp_mlp_shard_cols(INT64_MAX - 7, 64, 63, TP_BF16, &f, &c0) == TP_OK && c0 + f == INT64_MAX - 7);
  int32_t q, kv, q0, kv0;
  for (int32_t t = 1; t <= 64; ++t)
    for (int32_t r = 0; r < t; ++r) tp_attn_shard_heads(64, 8, t, r, &q, &kv, &q0, &kv0);
  EXPECT(tp_attn_shard_heads(63, 8, 8, 0, &q, &kv, &q0, &kv0) == TP_ENOTDIV);
  EXPECT(tp_attn_shard_heads(64, 8, 8, 0, NULL, &kv, &q0, &kv0) == TP_EINVAL);
  for (int s = -8; s <= 1; ++s) EXPECT(strlen(tp_status_string(s)) > 0);

  /* options and the profiling hook */
  int32_t tile = -1, split = -1;
  EXPECT(tp_get_options(&tile, &split) == TP_OK && tile == TP_TILE_AUTO && split == 1);
  EXPECT(tp_set_options(TP_TILE_TINY + 1, 1) == TP_EINVAL);
  EXPECT(tp_set_options(TP_TILE_SMALL, 0) == TP_OK);
  EXPECT(tp_set_options(TP_TILE_AUTO, 1) == TP_OK);
  void* ev[2] = {A16, NULL};
  EXPECT(tp_profile_arm(ev, 2) == TP_EINVAL);
  EXPECT(tp_profile_arm(ev, 3) == TP_EINVAL);
  EXPECT(tp_profile_arm(NULL, 0) == TP_OK);

  /* MLP entry points: rejected before launch */
  tp_mlp_desc m = {64, 128, 512, 2, 0, TP_BF16, TP_GELU};
  EXPECT(tp_mlp_shard_fwd(NULL, A16, A16, NULL, NULL, A16, A16, A16, A16, NULL) == TP_EINVAL);
  EXPECT(tp_mlp_shard_fwd(&m, MIS, A16, NULL, NULL, A16, A16, A16, A16, NULL) == TP_EALIGN);
  EXPECT(tp_mlp_shard_fwd(&m, NULL, A16, NULL, NULL, A16, A16, A16, A16, NULL) == TP_EINVAL);
  EXPECT(tp_mlp_shard_fwd(&m, A16, A16, A16, NULL, A16, A16, A16, A16, NULL) == TP_EINVAL);
  tp_mlp_desc bad = m;
  bad.rank = 2;
  EXPECT(tp_mlp_shard_fwd(&bad, A16, A16, NULL, NULL, A16, A16, A16, A16, NULL) == TP_EINVAL);
  bad = m;
  bad.dtype = 7;
  EXPECT(tp_mlp_shard_fwd(&bad, A16, A16, NULL, NULL, A16, A16, A16, A16, NULL) == TP_EDTYPE);
  bad = m;
  bad.h = 130;
  EXPECT(tp_mlp_shard_fwd(&bad, A16, A16, NULL, NULL, A16, A16, A16, A16, NULL) == TP_EALIGN);
  bad = m;
  bad.tokens = (int64_t)1 << 40;
  EXPECT(tp_mlp_shard_fwd(&bad, A16, A16, NULL, NULL, A16, A16, A16, A16, NULL) == TP_EINVAL);
  EXPECT(tp_mlp_shard_bwd(&m, A16, 1.5f, 0, A16, A16, NULL, A16, A16, A16, A16, NULL, A16, (float*)A16, NULL,
                          (float*)A16, A16, NULL) == TP_EINVAL);
  EXPECT(tp_mlp_shard_bwd(&m, A16, 0.1f, 0, A16, A16, NULL, A16, A16, A16, NULL, NULL, A16, (float*)A16, NULL,
                          (float*)A16, A16, NULL) == TP_EINVAL);

  /* attention entry points */
  tp_attn_desc d = {2, 128, 256, 8, 2, 128, 2, 0, TP_BF16, 1};
  tp_attn_desc da = d;
  da.d = 96;
  EXPECT(tp_attn_shard_fwd(&da, A16, A16, A16, A16, A16, NULL, A16, NULL) == TP_EUNSUPPORTED);
  da = d;
  da.n_q = 7;
  EXPECT(tp_attn_shard_fwd(&da, A16, A16, A16, A16, A16, NULL, A16, NULL) == TP_ENOTDIV);
  da = d;
  da.dtype = TP_F32;
  EXPECT(tp_attn_shard_fwd(&da, A16, A16, A16, A16, A16, NULL, A16, NULL) == TP_EDTYPE);
  EXPECT(tp_attn_shard_fwd(&d, A16, A16, A16, A16, MIS, NULL, A16, NULL) == TP_EALIGN);
  EXPECT(tp_attn_shard_bwd(&d, A16, A16, A16, A16, A16, A16, (float*)A16, A16, NULL, A16, (float*)A16, (float*)A16,
                           A16, NULL) == TP_EINVAL);
  tp_attn_desc big = {8, 65536, 1024, 2, 2, 64, 1, 0, TP_BF16, 1};
  EXPECT(tp_attn_shard_bwd_noalloc(&big, A16, A16, A16, A16, A16, A16, (float*)A16, A16, A16, (float*)A16,
                                   (float*)A16, A16, NULL) == TP_ENOSCRATCH);

  /* all-reduce family */
  const void* parts[64];
  for (int i = 0; i < 64; ++i) parts[i] = A16;
  EXPECT(tp_sum_partials(16, 64, 65, TP_BF16, parts, NULL, 0.0f, 0, A16, NULL) == TP_EUNSUPPORTED);
  EXPECT(tp_sum_partials(16, 60, 4, TP_BF16, parts, NULL, 0.0f, 0, A16, NULL) == TP_EALIGN);
  EXPECT(tp_sum_partials(16, 64, 4, TP_BF16, NULL, NULL, 0.0f, 0, A16, NULL) == TP_EINVAL);
  EXPECT(tp_sum_partials(16, 64, 4, TP_BF16, parts, NULL, -0.1f, 0, A16, NULL) == TP_EINVAL);
  EXPECT(tp_sum_partials_residual(16, 64, 4, TP_BF16, parts, MIS, 0.0f, 0, NULL, A16, NULL) == TP_EALIGN);
  EXPECT(tp_reduce_scatter(15, 64, 4, 0, TP_BF16, parts, NULL, 0.0f, 0, NULL, A16, NULL) == TP_ENOTDIV);
  EXPECT(tp_reduce_scatter(16, 64, 4, 4, TP_BF16, parts, NULL, 0.0f, 0, NULL, A16, NULL) == TP_EINVAL);
  EXPECT(tp_sum_partials_norm(16, 64, 4, TP_BF16, parts, NULL, 0.0f, 0, NULL, 5, NULL, NULL, 1e-5f, A16, A16,
                              NULL) == TP_EINVAL);
  EXPECT(tp_sum_partials_norm(16, 32776, 4, TP_BF16, parts, NULL, 0.0f, 0, NULL, TP_NORM_RMS, NULL, NULL, 1e-5f,
                              A16, A16, NULL) == TP_EUNSUPPORTED);
  EXPECT(tp_reduce_scatter_norm(16, 64, 4, 1, TP_BF16, parts, NULL, 0.0f, 0, NULL, TP_NORM_RMS, NULL, A16, 1e-5f,
                                A16, A16, NULL) == TP_EINVAL);
  EXPECT(tp_all_gather(4, 60, 4, TP_BF16, parts, A16, NULL) == TP_EALIGN);
  EXPECT(tp_all_gather(4, 64, 0, TP_BF16, parts, A16, NULL) == TP_EINVAL);
  EXPECT(tp_sum_partials(0, 64, 4, TP_BF16, parts, NULL, 0.0f, 0, A16, NULL) == TP_OK); /* empty: no launch */

  if (failures) {
    fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  printf("abi_driver: all expectations hold\n");
  return 0;
}
