/* Host-only driver for the C-ABI validation layer, linked against a copy of
 * the library's host code built with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_abi_sanitize.py builds and runs it).
 * Every call below is rejected by validation before any HIP call, so it needs
 * no GPU: the point is that the checks themselves read no byte outside the
 * caller's arrays (the decay array is exactly `heads` doubles of heap memory)
 * and overflow no integer, whatever the shape. Exit status 0 and "ok" on
 * success; the first wrong status prints the case and exits 1. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "retention.h"

static int failures = 0;

static void expect(const char *what, int got, int want) {
  if (got != want) {
    printf("FAIL %s: status %d, want %d\n", what, got, want);
    ++failures;
  }
}

/* fake device addresses: validation only compares and aligns them */
#define A(i) ((void *)(uintptr_t)((uint64_t)(i) << 32))

static ret_desc_t desc(int b, int n, int h, int d, int dtype, const double *gam) {
  ret_desc_t r;
  r.batch = b;
  r.seqlen = n;
  r.heads = h;
  r.dk = d;
  r.dv = d;
  r.dtype = dtype;
  r.gamma = gam;
  r.rotary_base = 0.0;
  r.pos_offset = 0;
  r.gn_eps = 1e-5f;
  return r;
}

int main(void) {
  const int H = 16;
  /* exactly H decays on the heap: any read past them is reported */
  double *gam = (double *)malloc(H * sizeof(double));
  for (int h = 0; h < H; ++h) gam[h] = 1.0 - ldexp(1.0, -5 - h);
  ret_desc_t d = desc(2, 8192, H, 256, RET_BF16, gam);

  /* NULL descriptor and NULL tensors */
  expect("parallel NULL desc", retention_parallel_fwd(NULL, A(1), A(2), A(3), NULL, A(4), NULL, 0, NULL),
         RET_ERR_NULL);
  expect("chunkwise NULL q",
         retention_chunkwise_fwd(&d, 512, NULL, A(2), A(3), NULL, A(4), NULL, NULL, A(8), 1u << 30, NULL),
         RET_ERR_NULL);
  ret_desc_t d1 = d;
  d1.seqlen = 1;
  expect("step NULL state", retention_recurrent_step(&d1, A(1), A(2), A(3), NULL, A(4), NULL, NULL), RET_ERR_NULL);

  /* shapes */
  ret_desc_t s = d;
  s.heads = 129;
  expect("heads 129", retention_parallel_fwd(&s, A(1), A(2), A(3), NULL, A(4), NULL, 0, NULL), RET_ERR_SHAPE);
  s = d;
  s.batch = INT32_MAX;
  s.seqlen = INT32_MAX;
  expect("grid overflow", retention_chunkwise_fwd(&s, 512, A(1), A(2), A(3), NULL, A(4), NULL, NULL, A(8), 0, NULL),
         RET_ERR_SHAPE);
  expect("grid overflow size", (int)retention_chunkwise_workspace_bytes(&s, 512), 0);
  expect("grid overflow bwd size", (int)retention_chunkwise_bwd_workspace_bytes(&s, 512, 1), 0);
  expect("chunk 0", retention_chunkwise_fwd(&d, 0, A(1), A(2), A(3), NULL, A(4), NULL, NULL, A(8), 0, NULL),
         RET_ERR_SHAPE);
  expect("chunk -5 size", (int)retention_chunkwise_workspace_bytes(&d, -5), 0);
  s = d;
  s.dk = 96;
  s.dv = 96;
  expect("d 96", retention_parallel_fwd(&s, A(1), A(2), A(3), NULL, A(4), NULL, 0, NULL), RET_ERR_UNSUPPORTED);
  s = d;
  s.dtype = 7;
  expect("dtype 7", retention_parallel_fwd(&s, A(1), A(2), A(3), NULL, A(4), NULL, 0, NULL), RET_ERR_UNSUPPORTED);

  /* decays, rotation, eps */
  gam[H - 1] = 1.5;
  expect("gamma 1.5", retention_parallel_fwd(&d, A(1), A(2), A(3), NULL, A(4), NULL, 0, NULL), RET_ERR_GAMMA);
  gam[H - 1] = NAN;
  expect("gamma nan", retention_parallel_fwd(&d, A(1), A(2), A(3), NULL, A(4), NULL, 0, NULL), RET_ERR_GAMMA);
  gam[H - 1] = 0.0;
  expect("gamma 0", retention_parallel_fwd(&d, A(1), A(2), A(3), NULL, A(4), NULL, 0, NULL), RET_ERR_GAMMA);
  gam[H - 1] = 1.0 - ldexp(1.0, -5 - (H - 1));
  s = d;
  s.rotary_base = -1.0;
  expect("base -1", retention_parallel_fwd(&s, A(1), A(2), A(3), NULL, A(4), NULL, 0, NULL), RET_ERR_ARG);
  s = d;
  s.pos_offset = -1;
  expect("pos -1", retention_parallel_fwd(&s, A(1), A(2), A(3), NULL, A(4), NULL, 0, NULL), RET_ERR_ARG);
  s = d;
  s.gn_eps = 0.0f;
  expect("eps 0 with gate", retention_parallel_fwd(&s, A(1), A(2), A(3), A(5), A(4), NULL, 0, NULL), RET_ERR_ARG);

  /* alignment, aliasing, workspace */
  expect("k misaligned", retention_parallel_fwd(&d, A(1), (char *)A(2) + 8, A(3), NULL, A(4), NULL, 0, NULL),
         RET_ERR_ALIGN);
  expect("o inside q", retention_parallel_fwd(&d, A(1), A(2), A(3), NULL, (char *)A(1) + 256, NULL, 0, NULL),
         RET_ERR_ALIAS);
  const size_t need = retention_chunkwise_workspace_bytes(&d, 512);
  expect("workspace size", need > 0, 1);
  expect("workspace short",
         retention_chunkwise_fwd(&d, 512, A(1), A(2), A(3), NULL, A(4), NULL, NULL, A(8), need - 1, NULL),
         RET_ERR_WORKSPACE);
  expect("state_out inside q",
         retention_chunkwise_fwd(&d, 512, A(1), A(2), A(3), NULL, A(4), NULL, (float *)((char *)A(1) + 4096), A(8),
                                 need, NULL),
         RET_ERR_ALIAS);
  expect("timed short",
         retention_chunkwise_fwd_timed(&d, 512, A(1), A(2), A(3), NULL, A(4), NULL, NULL, A(8), need - 1, NULL, NULL,
                                       NULL),
         RET_ERR_WORKSPACE);
  int32_t word = 0;
  expect("noalloc NULL o",
         retention_chunkwise_fwd_noalloc(&d, 512, A(1), A(2), A(3), NULL, NULL, NULL, NULL, &word, NULL),
         RET_ERR_NULL);
  expect("error word, short workspace", retention_chunkwise_error(A(8), 4, &word, NULL), RET_ERR_WORKSPACE);
  expect("error word, NULL out", retention_chunkwise_error(A(8), 64, NULL, NULL), RET_ERR_NULL);

  /* packed sequences: more rows than batch * seqlen, misaligned offsets */
  const size_t vneed = retention_chunkwise_varlen_workspace_bytes(&d, 512);
  expect("varlen total",
         retention_chunkwise_varlen_fwd(&d, 512, (const int32_t *)A(9), (int64_t)2 * 8192 + 1, A(1), A(2), A(3), NULL,
                                        A(4), NULL, NULL, A(8), vneed, NULL),
         RET_ERR_SHAPE);
  expect("varlen cu misaligned",
         retention_chunkwise_varlen_fwd(&d, 512, (const int32_t *)((char *)A(9) + 2), 100, A(1), A(2), A(3), NULL,
                                        A(4), NULL, NULL, A(8), vneed, NULL),
         RET_ERR_ALIGN);

  /* decode step: seqlen must be 1; positions aligned */
  expect("step seqlen", retention_recurrent_step(&d, A(1), A(2), A(3), NULL, A(4), (float *)A(5), NULL),
         RET_ERR_SHAPE);
  s = d;
  s.seqlen = 1;
  expect("step positions misaligned",
         retention_recurrent_step_positions(&s, A(1), A(2), A(3), NULL, A(4), (float *)A(5),
                                            (const int64_t *)((char *)A(6) + 4), NULL),
         RET_ERR_ALIGN);

  /* backward and score map */
  const size_t bneed = retention_parallel_bwd_workspace_bytes(&d, 1);
  expect("parallel bwd short",
         retention_parallel_bwd(&d, A(1), A(2), A(3), A(5), A(6), A(7), A(10), A(11), A(12), A(13), bneed - 1, NULL),
         RET_ERR_WORKSPACE);
  const size_t cneed = retention_chunkwise_bwd_state_workspace_bytes(&d, 512, 0);
  expect("chunkwise bwd state NULL dq",
         retention_chunkwise_bwd_state(&d, 512, A(1), A(2), A(3), NULL, A(6), NULL, NULL, NULL, A(10), A(11), NULL,
                                       NULL, A(13), cneed, NULL),
         RET_ERR_NULL);
  expect("score map query past end",
         retention_score_map(&d, A(1), A(2), 8192, (float *)A(3), NULL, 0, NULL), RET_ERR_ARG);

  /* every status has a message, also out of range */
  for (int c = -3; c < 16; ++c)
    if (!retention_status_string((ret_status_t)c)) {
      printf("FAIL status string %d\n", c);
      ++failures;
    }
  expect("abi version", retention_abi_version(), 1);

  free(gam);
  if (failures) return 1;
  printf("ok\n");
  return 0;
}
