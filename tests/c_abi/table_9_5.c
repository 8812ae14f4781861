/* The C ABI used from C, with no Python in between: the two-step tree of
 * "llm_internals" section 9.2.2 (Table 9-5, Figure 9-3) on the GPU, checked
 * against the values the page prints.
 *
 * Step 1 probabilities A 0.5, B 0.4, C 0.1; step 2 conditionals after A:
 * x 0.40, y 0.35, z 0.25, after B: x 0.90, y 0.06, z 0.04; W = 2, no length
 * penalty. Logits are the natural logs of the probabilities (token ids:
 * A/x = 0, B/y = 1, C/z = 2). The page keeps B x (-1.022) and A x (-1.609),
 * i.e. beam_idx = [1, 0]: a swap, which the in-place KV reorder must apply.
 * Exit status 0 and "ok" when every check holds. */
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "beamstep.h"

static int failures = 0;

#define CHECK(cond, ...)                 \
  do {                                   \
    if (!(cond)) {                       \
      fprintf(stderr, "FAIL: ");         \
      fprintf(stderr, __VA_ARGS__);      \
      fprintf(stderr, "\n");             \
      ++failures;                        \
    }                                    \
  } while (0)

#define HIP(call)                                                        \
  do {                                                                   \
    hipError_t e_ = (call);                                              \
    if (e_ != hipSuccess) {                                              \
      fprintf(stderr, "HIP error %d at %s\n", (int)e_, #call);           \
      return 2;                                                          \
    }                                                                    \
  } while (0)

#define BS(call)                                                         \
  do {                                                                   \
    int s_ = (call);                                                     \
    if (s_ != BS_OK) {                                                   \
      fprintf(stderr, "%s: %s\n", #call, bs_strerror(s_));               \
      return 3;                                                          \
    }                                                                    \
  } while (0)

int main(void) {
  hipStream_t stream;
  HIP(hipStreamCreate(&stream));

  bs_config cfg;
  memset(&cfg, 0, sizeof cfg);
  cfg.batch = 1;
  cfg.beam = 2;
  cfg.vocab = 3;
  cfg.max_steps = 2;
  cfg.eos_id = -1;
  cfg.pad_id = -1;
  cfg.logits_dtype = BS_F32;
  cfg.lp = BS_LP_NONE;
  cfg.alpha = 0.0;
  cfg.stop = BS_STOP_HEURISTIC;
  cfg.num_return = 1;
  cfg.tile_elems = 0;
  cfg.prune = BS_PRUNE_TOPW;
  cfg.select = BS_SELECT_FUSED;
  bs_state *h = NULL;
  BS(bs_create(&cfg, stream, &h));

  /* device buffers: logits [2][3], outputs, two KV planes [2 rows][1 position][4 words] */
  float *logits, *scores, *norms;
  int32_t *beam_idx, *token_id, *tokens, *lengths;
  uint8_t *done;
  int32_t *planes[2];
  HIP(hipMalloc((void **)&logits, 6 * sizeof(float)));
  HIP(hipMalloc((void **)&scores, 2 * sizeof(float)));
  HIP(hipMalloc((void **)&norms, sizeof(float)));
  HIP(hipMalloc((void **)&beam_idx, 2 * sizeof(int32_t)));
  HIP(hipMalloc((void **)&token_id, 2 * sizeof(int32_t)));
  HIP(hipMalloc((void **)&tokens, 2 * sizeof(int32_t)));
  HIP(hipMalloc((void **)&lengths, sizeof(int32_t)));
  HIP(hipMalloc((void **)&done, 1));
  for (int p = 0; p < 2; ++p) HIP(hipMalloc((void **)&planes[p], 8 * sizeof(int32_t)));

  /* step 1: only slot 0 is live (scores start at [0, -inf]) */
  const float step1[6] = {logf(0.5f), logf(0.4f), logf(0.1f), logf(0.5f), logf(0.4f), logf(0.1f)};
  HIP(hipMemcpy(logits, step1, sizeof step1, hipMemcpyHostToDevice));
  BS(bs_step(h, logits, 3, beam_idx, token_id, scores, done));
  int32_t bi[2], tk[2];
  float sc[2];
  HIP(hipStreamSynchronize(stream));
  HIP(hipMemcpy(bi, beam_idx, sizeof bi, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(tk, token_id, sizeof tk, hipMemcpyDeviceToHost));
  CHECK(bi[0] == 0 && bi[1] == 0, "step 1 beam_idx %d %d, expected 0 0", bi[0], bi[1]);
  CHECK(tk[0] == 0 && tk[1] == 1, "step 1 tokens %d %d, expected A B (0 1)", tk[0], tk[1]);

  /* the forward of step 2 writes position 0 of both rows: A's row, then B's */
  const int32_t kv0[8] = {11, 12, 13, 14, 21, 22, 23, 24};
  for (int p = 0; p < 2; ++p) HIP(hipMemcpy(planes[p], kv0, sizeof kv0, hipMemcpyHostToDevice));

  /* step 2: row 0 continues A, row 1 continues B */
  const float step2[6] = {logf(0.40f), logf(0.35f), logf(0.25f),
                          logf(0.90f), logf(0.06f), logf(0.04f)};
  HIP(hipMemcpy(logits, step2, sizeof step2, hipMemcpyHostToDevice));
  BS(bs_step(h, logits, 3, beam_idx, token_id, scores, done));
  bs_kv_desc kv;
  void *ptrs[2] = {planes[0], planes[1]};
  kv.n_planes = 2;
  kv.planes = ptrs;
  kv.row_stride = 4 * sizeof(int32_t);
  kv.pos_stride = 4 * sizeof(int32_t);
  kv.pos_offset = 0;
  kv.bytes_per_pos = 4 * sizeof(int32_t);
  BS(bs_reorder_kv(h, &kv, 1));
  BS(bs_finalize(h, tokens, lengths, norms));
  HIP(hipStreamSynchronize(stream));

  HIP(hipMemcpy(bi, beam_idx, sizeof bi, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(tk, token_id, sizeof tk, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(sc, scores, sizeof sc, hipMemcpyDeviceToHost));
  CHECK(bi[0] == 1 && bi[1] == 0, "step 2 beam_idx %d %d, expected [B, A] = 1 0", bi[0], bi[1]);
  CHECK(tk[0] == 0 && tk[1] == 0, "step 2 tokens %d %d, expected x x (0 0)", tk[0], tk[1]);
  /* the page prints three decimals (its B x entry rounded in the last digit) */
  CHECK(fabsf(sc[0] - (-1.022f)) < 1e-3f, "score of B x %.5f, the page gives -1.022", sc[0]);
  CHECK(fabsf(sc[1] - (-1.609f)) < 1e-3f, "score of A x %.5f, the page gives -1.609", sc[1]);
  for (int p = 0; p < 2; ++p) {
    int32_t got[8];
    HIP(hipMemcpy(got, planes[p], sizeof got, hipMemcpyDeviceToHost));
    const int32_t want[8] = {21, 22, 23, 24, 11, 12, 13, 14};  /* the swap, in place */
    CHECK(memcmp(got, want, sizeof want) == 0, "plane %d after the reorder: rows not swapped", p);
  }
  int32_t tok[2], len;
  HIP(hipMemcpy(tok, tokens, sizeof tok, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(&len, lengths, sizeof len, hipMemcpyDeviceToHost));
  CHECK(len == 2 && tok[0] == 1 && tok[1] == 0, "best hypothesis %d %d (length %d), expected B x",
        tok[0], tok[1], len);

  bs_destroy(h);
  for (int p = 0; p < 2; ++p) (void)hipFree(planes[p]);
  (void)hipFree(logits);
  (void)hipFree(scores);
  (void)hipFree(norms);
  (void)hipFree(beam_idx);
  (void)hipFree(token_id);
  (void)hipFree(tokens);
  (void)hipFree(lengths);
  (void)hipFree(done);
  (void)hipStreamDestroy(stream);
  if (failures) return 1;
  printf("ok\n");
  return 0;
}
