/*
 * beam_oracle.c -- plain, slow, single-threaded CPU oracle of the batched
 * beam-search decode step.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this library. The product
 * path (the HIP library) shares no code, header, table or helper with it.
 *
 * What it computes, and where each step comes from:
 *   - "llm_internals" 9.2.2 (one beam step: expand, score, prune, finalize):
 *     row log-softmax of the logits, add the running score of each
 *     hypothesis, take the W best of the W*V flattened candidates of a batch
 *     item (parent = integer quotient of the flat index by V, token = the
 *     remainder), move EOS selections into the finished set.
 *   - "Transformers中的Beam Search高效实现", batched section: rows are
 *     b*W+w, the running scores start at [0, -inf, ...] per item so the first
 *     step only expands row 0, and each item keeps a finished-hypothesis set
 *     of capacity W (BeamHypotheses: insert while not full, else replace the
 *     worst when strictly better; is_done compares the worst kept score with
 *     the best current score normalised at the current length). At the end,
 *     unfinished live beams are added to the set and the best are returned,
 *     padded.
 *   - "llm_internals" 9.2.3: GNMT length penalty ((5+|y|)/6)^alpha and the
 *     plain |y|^alpha form (Hugging Face's length_penalty exponent); the
 *     normalised score is log P / lp.
 *   - "llm_internals" 9.2.2, KV-cache paragraph: the cache rows follow
 *     beam_idx; a parent chosen twice is copied twice.
 *   - "Blockwise Parallel Decoding" section 3 (verify sub-step): greedy
 *     argmax per position, then the longest prefix where proposals agree.
 *
 * Precision. The pages' batched code works in fp32 (log_softmax, add, top-k
 * on fp32 tensors), so decisions are taken on fp32 candidate scores:
 *     lse32  = fp32(m + ln sum_v exp(x_v - m))     (sum and log in double)
 *     cand32 = fp32(s32 + fp32(x32 - lse32))
 * Ties in cand32 go to the lower flat index j. Logits given as bf16 are
 * widened exactly to fp32 first. Length penalties are evaluated in double and
 * the normalised score is fp32(raw / lp).
 *
 * Hugging Face variant (or_set_prune, mode 1): the pages' batched code ranks
 * 2W candidates and skips an EOS ranked W or below ("Transformers中的Beam
 * Search高效实现", batched section: the rank >= num_beams test and the
 * break once num_beams beams are filled), which only makes sense with 2W
 * candidates. Here: take the best 2W; in rank order, an EOS of rank < W
 * enters the finished set, an EOS of rank >= W is dropped, any other
 * candidate becomes the next live slot until W slots are filled.
 *
 * Readings where the pages are silent or disagree (each one is listed with its
 * reason in the design notes): top-W candidates by default; an EOS selection
 * leaves a dead slot (score -inf) and live selections are compacted in rank
 * order; |y| counts generated tokens including EOS; the stop test runs once
 * per item per step after that step's inserts; "best" in the heuristic test
 * is the rank-0 selection of the step; finished-set order is (normalised
 * score desc, step asc, rank asc); done items and dead slots report
 * beam_idx = own slot, token = pad, score = -inf.
 *
 * Pins (what ties this file to something other than itself) are in the test
 * suite: the two-step tree of "llm_internals" Table 9-5, the length-penalty
 * Table 9-6, the blockwise Figure 1 example, exhaustive search over all |V|^n
 * paths on tiny inputs, W=1 against greedy argmax, and torch CPU
 * log_softmax/topk/index_select special cases, and a search that never stops
 * early: the "never" mode (any length penalty) and the heuristic mode (no
 * length penalty) must return what that search reaches at the maximum length.
 * The exact stopping step of both modes beyond hand-built cases, and the
 * heuristic mode's result under a length penalty (where it may differ from the
 * full search), are parity unpinned.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_BF16 = 1 };
enum { OR_LP_NONE = 0, OR_LP_GNMT = 1, OR_LP_POW = 2 };
enum { OR_STOP_TRUE = 0, OR_STOP_HEURISTIC = 1, OR_STOP_NEVER = 2 };

/* ------------------------------------------------------------------ */
/* small helpers                                                       */
/* ------------------------------------------------------------------ */

static float widen_bf16(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* element v of row r of a [rows][row_stride] logits array */
static float logit_at(const void *logits, int dtype, int64_t row_stride,
                      int64_t r, int64_t v)
{
    if (dtype == OR_BF16)
        return widen_bf16(((const uint16_t *)logits)[r * row_stride + v]);
    return ((const float *)logits)[r * row_stride + v];
}

/* "llm_internals" 9.2.3: lp = ((5+|y|)/6)^alpha (GNMT) or |y|^alpha */
double or_length_penalty(int kind, double alpha, int len)
{
    if (kind == OR_LP_GNMT)
        return pow((5.0 + (double)len) / 6.0, alpha);
    if (kind == OR_LP_POW)
        return pow((double)len, alpha);
    return 1.0;
}

float or_normalise(int kind, double alpha, float raw, int len)
{
    return (float)((double)raw / or_length_penalty(kind, alpha, len));
}

/* "llm_internals" 9.2.2 step 1: the log-sum-exp of one row, in double,
 * rounded once to fp32. A row that is entirely -inf has lse = -inf. */
float or_row_lse(const void *logits, int dtype, int64_t row_stride,
                 int64_t r, int64_t V)
{
    double m = -INFINITY;
    for (int64_t v = 0; v < V; ++v) {
        double x = logit_at(logits, dtype, row_stride, r, v);
        if (x > m)
            m = x;
    }
    if (m == -INFINITY)
        return -INFINITY;
    double sum = 0.0;
    for (int64_t v = 0; v < V; ++v)
        sum += exp((double)logit_at(logits, dtype, row_stride, r, v) - m);
    return (float)(m + log(sum));
}

/* "llm_internals" 9.2.2 step 2: the candidate's score in fp32 */
static float cand_score(float s, float x, float lse)
{
    volatile float logp = x - lse; /* fp32 rounding of the log-prob */
    volatile float c = s + logp;   /* fp32 rounding of the sum      */
    return c;
}

typedef struct {
    float c;
    int64_t j;
} or_cand;

/* selection order: score descending, then the lower flat index */
static int cand_cmp(const void *pa, const void *pb)
{
    const or_cand *a = (const or_cand *)pa, *b = (const or_cand *)pb;
    if (a->c > b->c)
        return -1;
    if (a->c < b->c)
        return 1;
    return (a->j < b->j) ? -1 : (a->j > b->j);
}

/* ------------------------------------------------------------------ */
/* search state: explicit token sequences, no backpointers             */
/* ------------------------------------------------------------------ */

typedef struct {
    float norm, raw;
    int32_t len, step, rank;
} or_hyp;

typedef struct or_search {
    int B, W, V, T, eos, pad, dtype, lp, stop;
    int K;               /* candidates ranked per item: W, or 2W       */
    double alpha;
    int t;               /* steps taken so far                        */
    int finished;        /* or_finish has run                         */
    float *s;            /* [B*W] running score, -inf = dead slot     */
    int32_t *seq;        /* [B*W][T] tokens of each slot's sequence   */
    int32_t *slot_rank;  /* [B*W] rank of the slot's last selection   */
    uint8_t *done;       /* [B]                                       */
    or_hyp *hyp;         /* [B][W] finished set                       */
    int32_t *hyp_tok;    /* [B][W][T] tokens of the finished set      */
    int32_t *hyp_n;      /* [B]                                       */
    float *lse;          /* [B*W] lse32 of the last select            */
    int32_t *sel_n;      /* [B] number of finite candidates (<= K+1)  */
    int64_t *sel_j;      /* [B][K+1] ranked selection                 */
    float *sel_c;        /* [B][K+1]                                  */
    or_cand *scratch;    /* W*V candidates of one item                */
    int32_t *tmp_seq;    /* [W][T]                                    */
} or_search;

void or_destroy(or_search *o)
{
    if (!o)
        return;
    free(o->s);
    free(o->seq);
    free(o->slot_rank);
    free(o->done);
    free(o->hyp);
    free(o->hyp_tok);
    free(o->hyp_n);
    free(o->lse);
    free(o->sel_n);
    free(o->sel_j);
    free(o->sel_c);
    free(o->scratch);
    free(o->tmp_seq);
    free(o);
}

or_search *or_create(int B, int W, int V, int T, int eos, int pad, int dtype,
                     int lp, double alpha, int stop)
{
    if (B < 1 || W < 1 || V < 1 || T < 1)
        return NULL;
    or_search *o = (or_search *)calloc(1, sizeof *o);
    if (!o)
        return NULL;
    o->B = B; o->W = W; o->V = V; o->T = T; o->eos = eos; o->pad = pad;
    o->dtype = dtype; o->lp = lp; o->alpha = alpha; o->stop = stop;
    o->K = W;
    size_t R = (size_t)B * W;
    o->s = (float *)malloc(R * sizeof(float));
    o->seq = (int32_t *)calloc(R * T, sizeof(int32_t));
    o->slot_rank = (int32_t *)calloc(R, sizeof(int32_t));
    o->done = (uint8_t *)calloc(B, 1);
    o->hyp = (or_hyp *)calloc(R, sizeof(or_hyp));
    o->hyp_tok = (int32_t *)calloc(R * T, sizeof(int32_t));
    o->hyp_n = (int32_t *)calloc(B, sizeof(int32_t));
    o->lse = (float *)calloc(R, sizeof(float));
    o->sel_n = (int32_t *)calloc(B, sizeof(int32_t));
    o->sel_j = (int64_t *)calloc((size_t)B * (2 * W + 1), sizeof(int64_t));
    o->sel_c = (float *)calloc((size_t)B * (2 * W + 1), sizeof(float));
    o->scratch = (or_cand *)malloc((size_t)W * V * sizeof(or_cand));
    o->tmp_seq = (int32_t *)calloc((size_t)W * T, sizeof(int32_t));
    if (!o->s || !o->seq || !o->slot_rank || !o->done || !o->hyp ||
        !o->hyp_tok || !o->hyp_n || !o->lse || !o->sel_n || !o->sel_j ||
        !o->sel_c || !o->scratch || !o->tmp_seq) {
        or_destroy(o);
        return NULL;
    }
    /* batched section: beam_scores[:, 1:] = -inf so that step 1 only
     * expands row 0 of every item */
    for (int b = 0; b < B; ++b)
        for (int w = 0; w < W; ++w)
            o->s[b * W + w] = (w == 0) ? 0.0f : -INFINITY;
    return o;
}

/* Candidates ranked per step: mode 0 the W best (the default), mode 1 the
 * 2W best with the Hugging Face fill rule (see the header). Only before the
 * first step. */
int or_set_prune(or_search *o, int mode)
{
    if (o->t != 0 || (mode != 0 && mode != 1))
        return -1;
    o->K = mode ? 2 * o->W : o->W;
    return 0;
}

/* finished-set order: normalised score desc, then step asc, then rank asc */
static int hyp_better(const or_hyp *a, const or_hyp *b)
{
    if (a->norm != b->norm)
        return a->norm > b->norm;
    if (a->step != b->step)
        return a->step < b->step;
    return a->rank < b->rank;
}

/* BeamHypotheses.add: insert while fewer than W are kept; otherwise replace
 * the worst kept hypothesis when the new one is strictly better. */
static void hyp_add(or_search *o, int b, float raw, int len, int step, int rank,
                    const int32_t *tokens)
{
    int W = o->W, T = o->T;
    or_hyp h;
    h.raw = raw;
    h.len = len;
    h.step = step;
    h.rank = rank;
    h.norm = or_normalise(o->lp, o->alpha, raw, len);
    or_hyp *set = o->hyp + (size_t)b * W;
    int32_t *tok = o->hyp_tok + (size_t)b * W * T;
    int slot;
    if (o->hyp_n[b] < W) {
        slot = o->hyp_n[b]++;
    } else {
        int worst = 0;
        for (int i = 1; i < W; ++i)
            if (hyp_better(&set[worst], &set[i]))
                worst = i;
        if (!hyp_better(&h, &set[worst]))
            return;
        slot = worst;
    }
    set[slot] = h;
    for (int i = 0; i < T; ++i)
        tok[(size_t)slot * T + i] = (i < len) ? tokens[i] : o->pad;
}

static float hyp_worst_norm(const or_search *o, int b)
{
    const or_hyp *set = o->hyp + (size_t)b * o->W;
    float w = INFINITY;
    for (int i = 0; i < o->hyp_n[b]; ++i)
        if (set[i].norm < w)
            w = set[i].norm;
    return w;
}

/* ------------------------------------------------------------------ */
/* prune: the W best of the W*V candidates of every live item          */
/* ------------------------------------------------------------------ */

/* Fills the ranked selection (top K+1, the extra one for near-tie
 * diagnostics) of every item that is not done. Candidates with score -inf
 * (dead rows, -inf logits) are not candidates. */
int or_select(or_search *o, const void *logits, int64_t row_stride)
{
    int B = o->B, W = o->W, K = o->K;
    int64_t V = o->V;
    for (int b = 0; b < B; ++b) {
        o->sel_n[b] = 0;
        for (int k = 0; k <= K; ++k) {
            o->sel_j[(size_t)b * (K + 1) + k] = -1;
            o->sel_c[(size_t)b * (K + 1) + k] = -INFINITY;
        }
        if (o->done[b])
            continue;
        size_t n = 0;
        for (int w = 0; w < W; ++w) {
            int64_t r = (int64_t)b * W + w;
            float s = o->s[r];
            if (s == -INFINITY) {
                o->lse[r] = -INFINITY;
                continue;
            }
            float lse = or_row_lse(logits, o->dtype, row_stride, r, V);
            o->lse[r] = lse;
            if (lse == -INFINITY)
                continue;
            for (int64_t v = 0; v < V; ++v) {
                float c = cand_score(s, logit_at(logits, o->dtype, row_stride, r, v), lse);
                if (c == -INFINITY)
                    continue;
                o->scratch[n].c = c;
                o->scratch[n].j = (int64_t)w * V + v;
                ++n;
            }
        }
        qsort(o->scratch, n, sizeof(or_cand), cand_cmp);
        int keep = (n < (size_t)(K + 1)) ? (int)n : K + 1;
        o->sel_n[b] = keep;
        for (int k = 0; k < keep; ++k) {
            o->sel_j[(size_t)b * (K + 1) + k] = o->scratch[k].j;
            o->sel_c[(size_t)b * (K + 1) + k] = o->scratch[k].c;
        }
    }
    return 0;
}

/* ranked selection of the last or_select: [B][K+1] flat indices and scores */
void or_get_selection(const or_search *o, int64_t *sel_j, float *sel_c,
                      int32_t *sel_n)
{
    size_t n = (size_t)o->B * (o->K + 1);
    memcpy(sel_j, o->sel_j, n * sizeof(int64_t));
    memcpy(sel_c, o->sel_c, n * sizeof(float));
    memcpy(sel_n, o->sel_n, (size_t)o->B * sizeof(int32_t));
}

/* The oracle's fp32 score of arbitrary flat candidates j of item b, using the
 * lse of the last or_select (for judging near-ties). Dead rows give -inf. */
void or_cand_scores(const or_search *o, const void *logits, int64_t row_stride,
                    int b, int n, const int64_t *js, float *out)
{
    for (int i = 0; i < n; ++i) {
        int64_t j = js[i];
        if (j < 0 || j >= (int64_t)o->W * o->V) {
            out[i] = NAN;
            continue;
        }
        int64_t w = j / o->V, v = j % o->V;
        int64_t r = (int64_t)b * o->W + w;
        float s = o->s[r], lse = o->lse[r];
        if (s == -INFINITY || lse == -INFINITY) {
            out[i] = -INFINITY;
            continue;
        }
        out[i] = cand_score(s, logit_at(logits, o->dtype, row_stride, r, v), lse);
    }
}

/* ------------------------------------------------------------------ */
/* finalize: apply a ranked selection                                  */
/* ------------------------------------------------------------------ */

/* Applies the ranked selection sel_j/sel_c ([B][K], flat index and fp32
 * score; j < 0 or score -inf means "no candidate") as the next step. Used
 * with the oracle's own selection, or with another implementation's so that
 * both continue from the same state. Outputs are [B][W] and [B]. */
int or_apply(or_search *o, const int64_t *sel_j, const float *sel_c,
             int32_t *beam_idx, int32_t *token, float *scores, uint8_t *done_out)
{
    int B = o->B, W = o->W, T = o->T, K = o->K;
    int64_t V = o->V;
    if (o->t >= T || o->finished)
        return -4;
    int t = o->t + 1; /* 1-based step; generated length after this step */
    for (int b = 0; b < B; ++b) {
        int32_t *bi = beam_idx + (size_t)b * W;
        int32_t *tk = token + (size_t)b * W;
        float *sc = scores + (size_t)b * W;
        if (o->done[b]) {
            for (int i = 0; i < W; ++i) {
                bi[i] = i;
                tk[i] = o->pad;
                sc[i] = -INFINITY;
            }
            done_out[b] = 1;
            continue;
        }
        int live = 0;
        float new_s[W];
        int32_t new_rank[W];
        float best_raw = -INFINITY;
        for (int k = 0; k < K && live < W; ++k) {
            int64_t j = sel_j[(size_t)b * K + k];
            float c = sel_c[(size_t)b * K + k];
            if (j < 0 || !(c > -INFINITY))
                continue;
            if (best_raw == -INFINITY)
                best_raw = c; /* rank-0 selection of this step */
            int p = (int)(j / V);
            int32_t tok = (int32_t)(j % V);
            const int32_t *pseq = o->seq + ((size_t)b * W + p) * T;
            if (o->eos >= 0 && tok == o->eos) {
                if (k >= W)
                    continue; /* 2W variant: an EOS ranked W or below is dropped */
                int32_t hyp[T];
                memcpy(hyp, pseq, (size_t)(t - 1) * sizeof(int32_t));
                hyp[t - 1] = tok;
                hyp_add(o, b, c, t, t, k, hyp);
            } else {
                int32_t *ns = o->tmp_seq + (size_t)live * T;
                memcpy(ns, pseq, (size_t)(t - 1) * sizeof(int32_t));
                ns[t - 1] = tok;
                for (int i = t; i < T; ++i)
                    ns[i] = 0;
                new_s[live] = c;
                new_rank[live] = k;
                bi[live] = p;
                tk[live] = tok;
                sc[live] = c;
                ++live;
            }
        }
        for (int i = 0; i < live; ++i) {
            memcpy(o->seq + ((size_t)b * W + i) * T, o->tmp_seq + (size_t)i * T,
                   (size_t)T * sizeof(int32_t));
            o->s[b * W + i] = new_s[i];
            o->slot_rank[b * W + i] = new_rank[i];
        }
        for (int i = live; i < W; ++i) {
            o->s[b * W + i] = -INFINITY;
            o->slot_rank[b * W + i] = W;
            bi[i] = i;
            tk[i] = o->pad;
            sc[i] = -INFINITY;
        }
        /* stop test, once per item after this step's inserts */
        int d = 0;
        if (live == 0) {
            d = 1;
        } else if (o->hyp_n[b] == W) {
            float worst = hyp_worst_norm(o, b);
            if (o->stop == OR_STOP_TRUE) {
                d = 1;
            } else if (o->stop == OR_STOP_HEURISTIC) {
                d = worst >= or_normalise(o->lp, o->alpha, best_raw, t);
            } else { /* never: no live beam can still beat the worst kept */
                float best_live = new_s[0];
                int len = (o->alpha > 0.0 && best_live <= 0.0f) ? T : t;
                d = worst >= or_normalise(o->lp, o->alpha, best_live, len);
            }
        }
        o->done[b] = (uint8_t)d;
        done_out[b] = (uint8_t)d;
    }
    o->t = t;
    return 0;
}

/* one whole step with the oracle's own selection */
int or_step(or_search *o, const void *logits, int64_t row_stride,
            int32_t *beam_idx, int32_t *token, float *scores, uint8_t *done_out)
{
    if (o->t >= o->T || o->finished)
        return -4;
    or_select(o, logits, row_stride);
    int B = o->B, K = o->K;
    int64_t *j = (int64_t *)malloc((size_t)B * K * sizeof(int64_t));
    float *c = (float *)malloc((size_t)B * K * sizeof(float));
    if (!j || !c) {
        free(j);
        free(c);
        return -2;
    }
    for (int b = 0; b < B; ++b)
        for (int k = 0; k < K; ++k) {
            j[b * K + k] = o->sel_j[(size_t)b * (K + 1) + k];
            c[b * K + k] = o->sel_c[(size_t)b * (K + 1) + k];
        }
    int rc = or_apply(o, j, c, beam_idx, token, scores, done_out);
    free(j);
    free(c);
    return rc;
}

/* ------------------------------------------------------------------ */
/* final selection                                                     */
/* ------------------------------------------------------------------ */

/* Adds every live beam of every unfinished item to its finished set at the
 * current length, then writes the best num_return hypotheses per item in
 * finished-set order: tokens [B][R][T] pad-filled (EOS included when the
 * hypothesis ended with it), lengths [B][R], normalised scores [B][R].
 * Missing entries get length 0, score -inf, all pad. Requires at least one
 * step; adding the live beams happens once. */
int or_finish(or_search *o, int num_return, int32_t *tokens, int32_t *lengths,
              float *norms)
{
    int B = o->B, W = o->W, T = o->T;
    if (num_return < 1 || num_return > W)
        return -1;
    if (o->t == 0)
        return -4; /* the final selection follows at least one decode step */
    if (!o->finished) {
        for (int b = 0; b < B; ++b) {
            if (o->done[b])
                continue;
            for (int i = 0; i < W; ++i) {
                float s = o->s[b * W + i];
                if (s == -INFINITY)
                    continue;
                hyp_add(o, b, s, o->t, o->t, o->slot_rank[b * W + i],
                        o->seq + ((size_t)b * W + i) * T);
            }
        }
        o->finished = 1;
    }
    for (int b = 0; b < B; ++b) {
        int n = o->hyp_n[b];
        int order[W];
        for (int i = 0; i < n; ++i)
            order[i] = i;
        /* insertion sort of at most W entries, best first */
        for (int i = 1; i < n; ++i) {
            int x = order[i], k = i;
            while (k > 0 && hyp_better(&o->hyp[(size_t)b * W + x],
                                       &o->hyp[(size_t)b * W + order[k - 1]])) {
                order[k] = order[k - 1];
                --k;
            }
            order[k] = x;
        }
        for (int r = 0; r < num_return; ++r) {
            int32_t *dst = tokens + ((size_t)b * num_return + r) * T;
            if (r < n) {
                const or_hyp *h = &o->hyp[(size_t)b * W + order[r]];
                memcpy(dst, o->hyp_tok + ((size_t)b * W + order[r]) * T,
                       (size_t)T * sizeof(int32_t));
                lengths[b * num_return + r] = h->len;
                norms[b * num_return + r] = h->norm;
            } else {
                for (int i = 0; i < T; ++i)
                    dst[i] = o->pad;
                lengths[b * num_return + r] = 0;
                norms[b * num_return + r] = -INFINITY;
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* state getters                                                       */
/* ------------------------------------------------------------------ */

int or_steps(const or_search *o) { return o->t; }

void or_get_scores(const or_search *o, float *s)
{
    memcpy(s, o->s, (size_t)o->B * o->W * sizeof(float));
}

void or_get_done(const or_search *o, uint8_t *d)
{
    memcpy(d, o->done, (size_t)o->B);
}

void or_get_lse(const or_search *o, float *lse)
{
    memcpy(lse, o->lse, (size_t)o->B * o->W * sizeof(float));
}

/* tokens of every slot's sequence: [B*W][T] */
void or_get_seqs(const or_search *o, int32_t *seq)
{
    memcpy(seq, o->seq, (size_t)o->B * o->W * o->T * sizeof(int32_t));
}

/* finished set of item b, in storage order: returns its size */
int or_get_hyps(const or_search *o, int b, float *norm, float *raw,
                int32_t *len, int32_t *step, int32_t *rank, int32_t *tokens)
{
    int n = o->hyp_n[b];
    for (int i = 0; i < n; ++i) {
        const or_hyp *h = &o->hyp[(size_t)b * o->W + i];
        norm[i] = h->norm;
        raw[i] = h->raw;
        len[i] = h->len;
        step[i] = h->step;
        rank[i] = h->rank;
        memcpy(tokens + (size_t)i * o->T,
               o->hyp_tok + ((size_t)b * o->W + i) * o->T,
               (size_t)o->T * sizeof(int32_t));
    }
    return n;
}

/* ------------------------------------------------------------------ */
/* KV-cache reorder ("llm_internals" 9.2.2, KV-cache paragraph)        */
/* ------------------------------------------------------------------ */

/* For every plane (one (layer, K|V) buffer), every item that is not done and
 * every slot i whose beam_idx differs from i: positions
 * [pos_offset, pos_offset + gen_len) of row b*W+i become those of row
 * b*W+beam_idx before the reorder. Plain: snapshot the item's rows, then
 * gather. Strides are in bytes. */
int or_kv_reorder(int n_planes, uint8_t *const *planes, int64_t row_stride,
                  int64_t pos_stride, int64_t pos_offset, int64_t bytes_per_pos,
                  int B, int W, int gen_len, const int32_t *beam_idx,
                  const uint8_t *done)
{
    if (gen_len <= 0)
        return 0;
    size_t row_bytes = (size_t)gen_len * (size_t)bytes_per_pos;
    uint8_t *snap = (uint8_t *)malloc((size_t)W * row_bytes);
    if (!snap)
        return -2;
    for (int pl = 0; pl < n_planes; ++pl) {
        for (int b = 0; b < B; ++b) {
            if (done[b])
                continue;
            for (int w = 0; w < W; ++w)
                for (int p = 0; p < gen_len; ++p)
                    memcpy(snap + (size_t)w * row_bytes + (size_t)p * bytes_per_pos,
                           planes[pl] + (int64_t)(b * W + w) * row_stride +
                               (pos_offset + p) * pos_stride,
                           (size_t)bytes_per_pos);
            for (int i = 0; i < W; ++i) {
                int src = beam_idx[b * W + i];
                if (src == i)
                    continue;
                for (int p = 0; p < gen_len; ++p)
                    memcpy(planes[pl] + (int64_t)(b * W + i) * row_stride +
                               (pos_offset + p) * pos_stride,
                           snap + (size_t)src * row_bytes + (size_t)p * bytes_per_pos,
                           (size_t)bytes_per_pos);
            }
        }
    }
    free(snap);
    return 0;
}

/* ------------------------------------------------------------------ */
/* blockwise verify ("Blockwise Parallel Decoding" section 3)          */
/* ------------------------------------------------------------------ */

/* argmax[b][i] = first index of the largest logit of position i (greedy needs
 * no softmax, "llm_internals" 9.2.1); accept_len[b] = the largest k' such
 * that proposals[b][i] == argmax[b][i] for every i < k'. When proposals[b][0]
 * is the base model's own greedy token, accept_len >= 1. */
int or_verify(const void *logits, int dtype, int B, int k, int V,
              int64_t row_stride, const int32_t *proposals, int32_t *accept_len,
              int32_t *argmax)
{
    for (int b = 0; b < B; ++b) {
        for (int i = 0; i < k; ++i) {
            int64_t r = (int64_t)b * k + i;
            float best = logit_at(logits, dtype, row_stride, r, 0);
            int32_t arg = 0;
            for (int v = 1; v < V; ++v) {
                float x = logit_at(logits, dtype, row_stride, r, v);
                if (x > best) {
                    best = x;
                    arg = v;
                }
            }
            argmax[r] = arg;
        }
        int a = 0;
        while (a < k && proposals[b * k + a] == argmax[b * k + a])
            ++a;
        accept_len[b] = a;
    }
    return 0;
}

/* Approximate verify ("Blockwise Parallel Decoding" section 5.1, top-k
 * selection, and section 5.3, minimum block size): position i passes while
 * the rank of proposals[b][i] among the logits of row b*k+i is below top_k,
 * the rank being the number of logits that beat the proposal's (larger, or
 * equal at a lower index), so that top_k = 1 is the exact greedy check;
 * accept_len = max(longest passing prefix, min(min_block, k)). A proposal
 * outside [0, V) has rank V. rank may be NULL. */
int or_verify_ex(const void *logits, int dtype, int B, int k, int V,
                 int64_t row_stride, const int32_t *proposals, int top_k,
                 int min_block, int32_t *accept_len, int32_t *argmax,
                 int32_t *rank)
{
    if (top_k < 1 || min_block < 0 || min_block > k)
        return -1;
    or_verify(logits, dtype, B, k, V, row_stride, proposals, accept_len, argmax);
    for (int b = 0; b < B; ++b) {
        int a = 0, passing = 1;
        for (int i = 0; i < k; ++i) {
            int64_t r = (int64_t)b * k + i;
            int32_t p = proposals[r];
            int32_t rk = V;
            if (p >= 0 && p < V) {
                float xp = logit_at(logits, dtype, row_stride, r, p);
                rk = 0;
                for (int v = 0; v < V; ++v) {
                    float x = logit_at(logits, dtype, row_stride, r, v);
                    if (x > xp || (x == xp && v < p))
                        ++rk;
                }
            }
            if (rank)
                rank[r] = rk;
            if (passing && rk < top_k)
                ++a;
            else
                passing = 0;
        }
        accept_len[b] = a > min_block ? a : min_block;
    }
    return 0;
}

