/* Host-side paths of libgqa.so driven from plain C, for a build whose host code carries
 * AddressSanitizer and UndefinedBehaviorSanitizer (the CPU test builds both).  Every call
 * here is answered by the host checks or by pure host arithmetic, so no GPU is needed:
 * rejected arguments of every entry point, workspace sizes, the decode split rule, the RoPE
 * frequency tables, status strings.  Fake device addresses are only looked at, never
 * dereferenced; host arrays (the frequency table) are real.  Prints "host checks: OK" and
 * returns 0 when every answer is the expected one. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "gqa.h"

static int failures = 0;

#define EXPECT(cond)                                                       \
  do {                                                                     \
    if (!(cond)) {                                                         \
      fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                          \
    }                                                                      \
  } while (0)

#define DEV(x) ((void *)(uintptr_t)(x))

int main(void) {
  void *A = DEV(0x10000), *MIS = DEV(0x10008);
  const int32_t *IA = (const int32_t *)DEV(0x20000);
  gqa_params p;
  gqa_params_init(&p);
  EXPECT(p.dtype == GQA_BF16 && p.rope_theta == 1e6 && p.workspace == NULL);

  /* prefill: bad sizes, heads, alignment, workspace, masks, frequency tables */
  p.workspace = A;
  p.workspace_bytes = 1u << 30;
  EXPECT(gqa_prefill(A, A, A, NULL, A, -1, 8, 8, 8, 128, 1, &p) == GQA_EINVAL);
  EXPECT(gqa_prefill(A, A, A, NULL, A, 1, 8, 6, 4, 128, 1, &p) == GQA_EINVAL);
  EXPECT(gqa_prefill(A, A, A, NULL, A, 1, 8, 8, 8, 96, 1, &p) == GQA_ENOTSUP);
  EXPECT(gqa_prefill(MIS, A, A, NULL, A, 1, 8, 8, 8, 128, 1, &p) == GQA_EINVAL);
  EXPECT(gqa_prefill(A, A, A, NULL, NULL, 1, 8, 8, 8, 128, 1, &p) == GQA_EINVAL);
  EXPECT(gqa_prefill(A, A, A, NULL, A, 1, 8, 8, 8, 128, 2, &p) == GQA_EINVAL);
  EXPECT(gqa_prefill(A, A, A, NULL, A, 0, 8, 8, 8, 128, 1, &p) == GQA_OK);
  EXPECT(gqa_prefill(A, A, A, NULL, A, 1, 8, 8, 8, 128, 1, NULL) == GQA_EINVAL);
  p.workspace_bytes = 16;
  EXPECT(gqa_prefill(A, A, A, NULL, A, 1, 4096, 16, 8, 128, 1, &p) == GQA_EWORKSPACE);
  p.workspace_bytes = 1u << 30;
  p.window = 8;
  EXPECT(gqa_prefill(A, A, A, NULL, A, 1, 8, 8, 8, 128, 0, &p) == GQA_EINVAL);
  p.window = -1;
  EXPECT(gqa_prefill(A, A, A, NULL, A, 1, 8, 8, 8, 128, 1, &p) == GQA_EINVAL);
  p.window = 0;
  p.block_mask = (const uint32_t *)DEV(0x30000);
  p.block_mask_words = 0;
  EXPECT(gqa_prefill(A, A, A, NULL, A, 1, 8, 8, 8, 128, 1, &p) == GQA_EINVAL);
  p.block_mask = NULL;
  double table[64];
  for (int j = 0; j < 64; ++j) table[j] = 0.5;
  table[63] = NAN;
  p.rope_inv_freq = table;
  EXPECT(gqa_prefill(A, A, A, NULL, A, 1, 8, 8, 8, 128, 1, &p) == GQA_EINVAL);
  table[63] = 0.5;
  table[31] = INFINITY;
  EXPECT(gqa_prefill(A, A, A, NULL, A, 1, 8, 8, 8, 64, 1, &p) == GQA_EINVAL);
  p.rope_inv_freq = NULL;
  p.eps = -1.f;
  EXPECT(gqa_prefill(A, A, A, NULL, A, 1, 8, 8, 8, 128, 1, &p) == GQA_EINVAL);
  p.eps = 1e-6f;
  p.dtype = (gqa_dtype)7;
  EXPECT(gqa_prefill(A, A, A, NULL, A, 1, 8, 8, 8, 128, 1, &p) == GQA_ENOTSUP);
  p.dtype = GQA_BF16;

  /* cached prefill */
  EXPECT(gqa_prefill_cached(A, A, A, A, A, IA, NULL, A, 1, 8, 8, 8, 128, 0, 1, &p) ==
         GQA_EINVAL);
  EXPECT(gqa_prefill_cached(A, A, A, A, A, NULL, NULL, A, 1, 8, 8, 8, 128, 64, 1, &p) ==
         GQA_EINVAL);
  p.dtype = GQA_F32;
  EXPECT(gqa_prefill_cached(A, A, A, A, A, IA, NULL, A, 1, 8, 8, 8, 128, 64, 1, &p) ==
         GQA_ENOTSUP);
  p.dtype = GQA_BF16;

  /* decode and the decode graph */
  EXPECT(gqa_decode(A, A, A, IA, A, 2, 8, 8, 128, 0, &p) == GQA_EINVAL);
  EXPECT(gqa_decode(A, A, A, NULL, A, 2, 8, 8, 128, 64, &p) == GQA_EINVAL);
  EXPECT(gqa_decode(A, A, A, IA, A, 70000, 8, 8, 128, 64, &p) == GQA_ENOTSUP);
  p.k_new = A;
  EXPECT(gqa_decode(A, A, A, IA, A, 2, 8, 8, 128, 64, &p) == GQA_EINVAL); /* k_new without v_new */
  p.k_new = NULL;
  p.workspace_bytes = 8;
  EXPECT(gqa_decode(A, A, A, IA, A, 2, 8, 8, 128, 64, &p) == GQA_EWORKSPACE);
  p.workspace_bytes = 1u << 30;
  p.window = 16;
  EXPECT(gqa_decode(A, A, A, IA, A, 2, 8, 8, 128, 64, &p) == GQA_ENOTSUP);
  p.window = 0;
  EXPECT(gqa_decode(A, A, A, IA, A, 0, 8, 8, 128, 64, &p) == GQA_OK);
  gqa_decode_graph *g = (gqa_decode_graph *)DEV(1);
  EXPECT(gqa_decode_graph_create(A, A, A, (int32_t *)IA, A, 2, 8, 8, 128, 64, &p, &g) ==
         GQA_EINVAL); /* no k_new / v_new */
  EXPECT(g == NULL);
  EXPECT(gqa_decode_graph_create(A, A, A, (int32_t *)IA, A, 2, 8, 8, 128, 64, &p, NULL) ==
         GQA_EINVAL);
  EXPECT(gqa_decode_graph_create_steps(A, A, A, (int32_t *)IA, A, 2, 8, 8, 128, 64, 0, &p, &g) ==
         GQA_EINVAL); /* steps < 1 */
  EXPECT(gqa_decode_graph_create_steps(A, A, A, (int32_t *)IA, A, 2, 8, 8, 128, 64, 257, &p, &g) ==
         GQA_EINVAL); /* steps > 256 */
  EXPECT(g == NULL);
  EXPECT(gqa_decode_graph_launch(NULL, NULL) == GQA_EINVAL);
  EXPECT(gqa_decode_graph_destroy(NULL) == GQA_OK);

  /* the prologue alone */
  EXPECT(gqa_qk_norm_rope(A, A, NULL, A, NULL, 8, 8, 8, 128, &p) == GQA_EINVAL);
  EXPECT(gqa_qk_norm_rope(A, NULL, NULL, A, NULL, -1, 8, 8, 128, &p) == GQA_EINVAL);
  EXPECT(gqa_qk_norm_rope(A, NULL, NULL, A, NULL, 0, 8, 8, 128, &p) == GQA_OK);

  /* sizes and rules */
  EXPECT(gqa_workspace_bytes(GQA_OP_PREFILL, 1, 4096, 16, 8, 128, GQA_BF16) ==
         (size_t)4096 * 8 * 128 * 2 + 1280 + (size_t)256 * 2 * (128 * 128 + 256) * 4);
  EXPECT(gqa_workspace_bytes(GQA_OP_PREFILL, 1, 8, 6, 4, 128, GQA_BF16) == 0);
  EXPECT(gqa_workspace_bytes(99, 1, 8, 8, 8, 128, GQA_BF16) == 0);
  EXPECT(gqa_decode_split_keys(64, 32, 8, 32768) == 1024);
  EXPECT(gqa_decode_split_keys(0, 32, 8, 32768) == 0);
  for (int s = 0; s <= 5; ++s) EXPECT(gqa_status_str((gqa_status)s) != NULL);
  EXPECT(strncmp(gqa_status_str(GQA_EHIP), "GQA_EHIP", 8) == 0);

  /* frequency tables: values of the base rule, and refusals that write nothing */
  double w[64];
  EXPECT(gqa_rope_freq_table(GQA_ROPE_BASE, 128, 1e6, 0, 0, 0, 0, w) == GQA_OK);
  EXPECT(w[0] == 1.0 && fabs(w[32] - 1e-3) < 1e-15 && w[63] > 0.0);
  EXPECT(gqa_rope_freq_table(GQA_ROPE_YARN, 128, 1e6, 0, 32768, 131072, 1.0, w) == GQA_OK);
  EXPECT(w[0] == 1.0 && w[63] < 0.0); /* s = 2: 1 - 2 * 126/128 < 0 */
  EXPECT(gqa_rope_freq_table(GQA_ROPE_NTK, 128, 1e6, 8.0, 0, 0, 0, w) == GQA_OK);
  for (int j = 0; j < 64; ++j) w[j] = -7.0;
  EXPECT(gqa_rope_freq_table(GQA_ROPE_LINEAR, 128, 1e6, 0.0, 0, 0, 0, w) == GQA_EINVAL);
  EXPECT(gqa_rope_freq_table(9, 128, 1e6, 1.0, 0, 0, 0, w) == GQA_EINVAL);
  EXPECT(gqa_rope_freq_table(GQA_ROPE_BASE, 130, 1e6, 1.0, 0, 0, 0, w) == GQA_EINVAL);
  EXPECT(gqa_rope_freq_table(GQA_ROPE_BASE, 128, 1e6, 1.0, 0, 0, 0, NULL) == GQA_EINVAL);
  EXPECT(w[0] == -7.0 && w[63] == -7.0);

  if (failures) {
    fprintf(stderr, "host checks: %d failures\n", failures);
    return 1;
  }
  printf("host checks: OK\n");
  return 0;
}
