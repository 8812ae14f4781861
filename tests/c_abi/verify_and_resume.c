/* More of the C ABI used from C, with no Python in between.
 *
 * 1. The verify step of "Blockwise Parallel Decoding" (section 3, Figure 1):
 *    the proposals "in the bus" against the greedy choices "in the car"
 *    (vocabulary in=0 the=1 bus=2 car=3) accept two tokens. Checked through
 *    bs_verify (a handle), bs_verify_noalloc (no handle, no allocation) and
 *    bs_verify_ex (section 5.1 top-k acceptance, section 5.3 minimum block).
 * 2. Checkpoint and resume on the two-step tree of "llm_internals" section
 *    9.2.2 (Table 9-5): the state saved after step 1 and loaded into a new
 *    handle gives the page's step-2 result, B x (-1.022) and A x (-1.609).
 * Exit status 0 and "ok" when every check holds. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
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

static int verify_figure_1(hipStream_t stream) {
  enum { K = 3, V = 4 };
  /* position i: the greedy model's choice carries the only large logit */
  const int greedy[K] = {0, 1, 3};
  const int32_t proposals[K] = {0, 1, 2};
  float host[K * V];
  for (int i = 0; i < K * V; ++i) host[i] = 0.0f;
  for (int i = 0; i < K; ++i) host[i * V + greedy[i]] = 5.0f;

  float *logits;
  int32_t *prop, *accept, *argmax, *rank;
  HIP(hipMalloc((void **)&logits, sizeof host));
  HIP(hipMalloc((void **)&prop, sizeof proposals));
  HIP(hipMalloc((void **)&accept, sizeof(int32_t)));
  HIP(hipMalloc((void **)&argmax, K * sizeof(int32_t)));
  HIP(hipMalloc((void **)&rank, K * sizeof(int32_t)));
  HIP(hipMemcpy(logits, host, sizeof host, hipMemcpyHostToDevice));
  HIP(hipMemcpy(prop, proposals, sizeof proposals, hipMemcpyHostToDevice));

  bs_verify_state *vh = NULL;
  BS(bs_verify_create(1, K, V, BS_F32, stream, &vh));
  int32_t acc, am[K], rk[K];

  BS(bs_verify(vh, logits, V, prop, accept, argmax));
  HIP(hipStreamSynchronize(stream));
  HIP(hipMemcpy(&acc, accept, sizeof acc, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(am, argmax, sizeof am, hipMemcpyDeviceToHost));
  CHECK(acc == 2, "bs_verify accepted %d, Figure 1 accepts 2 (in, the)", acc);
  CHECK(am[0] == 0 && am[1] == 1 && am[2] == 3, "greedy %d %d %d, expected in the car (0 1 3)",
        am[0], am[1], am[2]);

  HIP(hipMemset(accept, 0, sizeof(int32_t)));
  BS(bs_verify_noalloc(stream, logits, BS_F32, 1, K, V, V, prop, accept, argmax));
  HIP(hipStreamSynchronize(stream));
  HIP(hipMemcpy(&acc, accept, sizeof acc, hipMemcpyDeviceToHost));
  CHECK(acc == 2, "bs_verify_noalloc accepted %d, expected 2", acc);

  /* top-k: "bus" at position 2 is beaten by car (larger) and by in and the
   * (equal logits at lower indices): rank 3, so top_k = 4 accepts all three */
  BS(bs_verify_ex(vh, logits, V, prop, 4, 0, accept, argmax, rank));
  HIP(hipStreamSynchronize(stream));
  HIP(hipMemcpy(&acc, accept, sizeof acc, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(rk, rank, sizeof rk, hipMemcpyDeviceToHost));
  CHECK(rk[0] == 0 && rk[1] == 0 && rk[2] == 3, "proposal ranks %d %d %d, expected 0 0 3", rk[0],
        rk[1], rk[2]);
  CHECK(acc == 3, "top_k = 4 accepted %d, expected 3", acc);
  BS(bs_verify_ex(vh, logits, V, prop, 3, 0, accept, argmax, NULL));
  HIP(hipStreamSynchronize(stream));
  HIP(hipMemcpy(&acc, accept, sizeof acc, hipMemcpyDeviceToHost));
  CHECK(acc == 2, "top_k = 3 accepted %d, expected 2", acc);
  /* minimum block size: at least three tokens are taken */
  BS(bs_verify_ex(vh, logits, V, prop, 1, 3, accept, argmax, NULL));
  HIP(hipStreamSynchronize(stream));
  HIP(hipMemcpy(&acc, accept, sizeof acc, hipMemcpyDeviceToHost));
  CHECK(acc == 3, "min_block = 3 accepted %d, expected 3", acc);
  CHECK(bs_verify_ex(vh, logits, V, prop, 0, 0, accept, argmax, NULL) == BS_EINVAL,
        "top_k = 0 must be refused");

  bs_verify_destroy(vh);
  (void)hipFree(logits);
  (void)hipFree(prop);
  (void)hipFree(accept);
  (void)hipFree(argmax);
  (void)hipFree(rank);
  return 0;
}

static bs_config tree_config(void) {
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
  cfg.prune = BS_PRUNE_TOPW;
  cfg.select = BS_SELECT_FUSED;
  return cfg;
}

static int resume_table_9_5(hipStream_t stream) {
  const bs_config cfg = tree_config();
  float *logits, *scores;
  int32_t *beam_idx, *token_id;
  uint8_t *done;
  HIP(hipMalloc((void **)&logits, 6 * sizeof(float)));
  HIP(hipMalloc((void **)&scores, 2 * sizeof(float)));
  HIP(hipMalloc((void **)&beam_idx, 2 * sizeof(int32_t)));
  HIP(hipMalloc((void **)&token_id, 2 * sizeof(int32_t)));
  HIP(hipMalloc((void **)&done, 1));

  /* step 1 on a first handle, then its state saved (A 0.5, B 0.4, C 0.1) */
  bs_state *h = NULL;
  BS(bs_create(&cfg, stream, &h));
  const float step1[6] = {logf(0.5f), logf(0.4f), logf(0.1f), logf(0.5f), logf(0.4f), logf(0.1f)};
  HIP(hipMemcpy(logits, step1, sizeof step1, hipMemcpyHostToDevice));
  BS(bs_step(h, logits, 3, beam_idx, token_id, scores, done));
  int64_t size = 0;
  BS(bs_state_size(h, &size));
  CHECK(size > 0, "snapshot size %lld", (long long)size);
  void *snap = malloc((size_t)size);
  if (!snap) return 4;
  BS(bs_state_save(h, snap, size));
  CHECK(bs_state_save(h, snap, size - 1) == BS_EINVAL, "a short buffer must be refused");
  bs_destroy(h);

  /* a new handle of the same configuration resumes at step 2 */
  bs_state *g = NULL;
  BS(bs_create(&cfg, stream, &g));
  BS(bs_state_load(g, snap, size));
  CHECK(bs_steps_taken(g) == 1, "steps taken after the load: %d, expected 1", bs_steps_taken(g));
  const float step2[6] = {logf(0.40f), logf(0.35f), logf(0.25f),
                          logf(0.90f), logf(0.06f), logf(0.04f)};
  HIP(hipMemcpy(logits, step2, sizeof step2, hipMemcpyHostToDevice));
  BS(bs_step(g, logits, 3, beam_idx, token_id, scores, done));
  HIP(hipStreamSynchronize(stream));
  int32_t bi[2], tk[2];
  float sc[2];
  HIP(hipMemcpy(bi, beam_idx, sizeof bi, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(tk, token_id, sizeof tk, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(sc, scores, sizeof sc, hipMemcpyDeviceToHost));
  CHECK(bi[0] == 1 && bi[1] == 0, "resumed step 2 beam_idx %d %d, expected [B, A] = 1 0", bi[0],
        bi[1]);
  CHECK(tk[0] == 0 && tk[1] == 0, "resumed step 2 tokens %d %d, expected x x", tk[0], tk[1]);
  CHECK(fabsf(sc[0] - (-1.022f)) < 1e-3f, "score of B x %.5f, the page gives -1.022", sc[0]);
  CHECK(fabsf(sc[1] - (-1.609f)) < 1e-3f, "score of A x %.5f, the page gives -1.609", sc[1]);

  /* a handle of another configuration refuses the snapshot */
  bs_config other = cfg;
  other.vocab = 4;
  bs_state *o = NULL;
  BS(bs_create(&other, stream, &o));
  CHECK(bs_state_load(o, snap, size) == BS_EINVAL, "a snapshot of another configuration must be refused");
  bs_destroy(o);

  free(snap);
  bs_destroy(g);
  (void)hipFree(logits);
  (void)hipFree(scores);
  (void)hipFree(beam_idx);
  (void)hipFree(token_id);
  (void)hipFree(done);
  return 0;
}

int main(void) {
  hipStream_t stream;
  HIP(hipStreamCreate(&stream));
  int rc = verify_figure_1(stream);
  if (rc == 0) rc = resume_table_9_5(stream);
  (void)hipStreamDestroy(stream);
  if (rc) return rc;
  if (failures) return 1;
  printf("ok\n");
  return 0;
}
