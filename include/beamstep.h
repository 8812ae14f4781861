/*
 * beamstep.h -- C ABI of libbeamstep.so, a batched beam-search decode step
 * for AMD Instinct MI355X (gfx950).
 *
 * One decode step of beam search, as described in "llm_internals" section
 * 9.2.2 (the four sub-steps expand, score, prune, finalize) and in the
 * batched section of "Transformers中的Beam Search高效实现" (rows b*W+w,
 * running scores initialised to [0, -inf, ...] per item, a finished set of
 * capacity W per item, early stopping), followed by the KV-cache reorder by
 * beam_idx ("llm_internals" 9.2.2, KV-cache paragraph) and, separately, the
 * verify sub-step of blockwise parallel decoding ("Blockwise Parallel
 * Decoding for Deep Autoregressive Models", section 3).
 *
 * Conventions shared by every entry point:
 *   - Pointers documented as "device" point to memory the caller allocated on
 *     the GPU the handle was created on (for example torch tensors); the
 *     library never frees them. Pointers documented as "host" are plain CPU
 *     memory, read during the call only.
 *   - Every call is enqueued on the handle's HIP stream and returns without
 *     waiting for the GPU, except where stated. Results are valid once the
 *     stream reaches them.
 *   - Every call returns a bs_status. BS_EINVAL and BS_ESTATE are decided on
 *     the host before anything is enqueued: such a call has enqueued nothing
 *     and left the handle unchanged. BS_EDEVICE reports a HIP error seen at a
 *     launch. The launches the same call issued before that one may already
 *     be enqueued (bs_step's first kernel, the earlier plane groups of a KV
 *     reorder, a paged reorder's table update), so after BS_EDEVICE the
 *     handle's search state and every buffer the call writes (outputs, KV
 *     planes or pools) are undefined: bs_reset the handle and rebuild the
 *     cache before using them again.
 *   - A handle is not thread-safe; use one handle per stream.
 *   - Logits must not contain NaN or +inf (behaviour is undefined); -inf is
 *     allowed and means "impossible token".
 */
#ifndef BEAMSTEP_H
#define BEAMSTEP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BS_OK = 0,
    BS_EINVAL = -1,  /* invalid argument or configuration            */
    BS_ENOMEM = -2,  /* device allocation failed (the create calls)  */
    BS_EDEVICE = -3, /* HIP runtime error                            */
    BS_ESTATE = -4   /* call not valid in the handle's current state */
} bs_status;

typedef enum { BS_F32 = 0, BS_BF16 = 1 } bs_dtype;

/* Length normalisation, "llm_internals" 9.2.3: the normalised score of a
 * finished hypothesis is log P / lp(|y|) with
 *   BS_LP_GNMT: lp = ((5 + |y|) / 6)^alpha
 *   BS_LP_POW : lp = |y|^alpha        (Hugging Face's length_penalty)
 *   BS_LP_NONE: lp = 1
 * |y| counts the generated tokens whose log-probabilities are in the score,
 * EOS included. lp is evaluated in double; the normalised score is
 * fp32(raw / lp). */
typedef enum { BS_LP_NONE = 0, BS_LP_GNMT = 1, BS_LP_POW = 2 } bs_lp;

/* When an item stops ("llm_internals" 9.2.2, "when to stop"; the is_done
 * test of the batched section). Checked once per item per step, after the
 * step's EOS hypotheses entered the finished set; an item with no live beam
 * left is always done.
 *   BS_STOP_TRUE     : done once W hypotheses are finished.
 *   BS_STOP_HEURISTIC: done once W are finished and the worst kept normalised
 *                      score >= fp32(best / lp(t)), best being the score of
 *                      the step's rank-0 selection and t the step.
 *   BS_STOP_NEVER    : done once W are finished and the worst kept normalised
 *                      score >= the best any live beam can still reach:
 *                      s / lp(max_steps) when alpha > 0 and s <= 0, else
 *                      s / lp(t), s being the best live score. */
typedef enum { BS_STOP_TRUE = 0, BS_STOP_HEURISTIC = 1, BS_STOP_NEVER = 2 } bs_stop;

/* Candidates ranked per item and step.
 *   BS_PRUNE_TOPW : the W best of the W*V ("llm_internals" 9.2.2 step 3).
 *   BS_PRUNE_TOP2W: the Hugging Face form of the batched section of
 *                   "Transformers中的Beam Search高效实现": the 2W best are
 *                   ranked; in rank order an EOS of rank < W is finished, an
 *                   EOS of rank >= W is dropped, and any other candidate fills
 *                   the next live slot until W are filled. Needs W <= 8. */
typedef enum { BS_PRUNE_TOPW = 0, BS_PRUNE_TOP2W = 1 } bs_prune;

/* How the K candidates of each item are found (the result is the same):
 *   BS_SELECT_FUSED   : one pass over the logits; every tile keeps its own
 *                       best K and (max, sum exp); the lists are merged.
 *   BS_SELECT_TWO_PASS: the coarse-to-fine selection of the LightSeq article
 *                       ("层级式解码计算"): a first pass takes, per row, the
 *                       maxima of KP >= K groups of logits (KP a power of
 *                       two) and the log-sum-exp; the K-th largest of the
 *                       group maxima, R, is at most the row's K-th best
 *                       logit. A second pass queues every logit >= R with
 *                       its candidate score s + (x - lse) (the article's
 *                       queue value leaves out the running score s; it is
 *                       needed to rank the candidates of an item), and the
 *                       queue is sorted. It reads the logits twice. */
typedef enum { BS_SELECT_FUSED = 0, BS_SELECT_TWO_PASS = 1 } bs_select;

typedef struct {
    int32_t batch;        /* B >= 1, with B*W <= 65535                     */
    int32_t beam;         /* W, 1..16                                      */
    int32_t vocab;        /* V >= 1, with W*V < 2^31                       */
    int32_t max_steps;    /* T >= 1: decode steps, the longest hypothesis  */
    int32_t eos_id;       /* EOS token, or < 0 for none                    */
    int32_t pad_id;       /* token reported for dead slots and padding     */
    int32_t logits_dtype; /* bs_dtype                                      */
    int32_t lp;           /* bs_lp                                         */
    double alpha;         /* length-penalty exponent, finite               */
    int32_t stop;         /* bs_stop                                       */
    int32_t num_return;   /* hypotheses returned per item, 1..W            */
    int32_t tile_elems;   /* logits per thread in the streaming pass:
                             16, 32 or 64; 0 picks one from B, W, V       */
    int32_t prune;        /* bs_prune                                      */
    int32_t select;       /* bs_select                                     */
} bs_config;

typedef struct bs_state bs_state;

/* Creates a handle for one batched search on the current HIP device and
 * allocates, once, every buffer the search needs at its maximum shapes
 * (running scores, per-tile partial results, finished sets, backpointers
 * [T][B][W], done flags, the reorder plan), following the static-shape
 * memory reuse of the LightSeq article ("动态显存复用"): no later call
 * allocates. Initialises the running scores to [0, -inf, ..., -inf] per item.
 *   cfg        host, read only
 *   hip_stream a hipStream_t (NULL: the null stream) that every later call on
 *              this handle is ordered on
 *   out        host; receives the handle
 * Errors: BS_EINVAL (bad config), BS_ENOMEM, BS_EDEVICE. Synchronises the
 * stream before returning. */
int bs_create(const bs_config *cfg, void *hip_stream, bs_state **out);

/* Starts a new search on the same handle: scores back to [0, -inf, ...],
 * finished sets emptied, done flags cleared, step counter to 0. */
int bs_reset(bs_state *h);

/* One decode step t = (steps taken) + 1, "llm_internals" 9.2.2:
 *   expand   lse_r = ln sum_v exp(x[r][v]) per live row r (fp32 arithmetic,
 *            logits read once; the log-probabilities are never stored),
 *   score    cand = fp32(s_r + fp32(x[r][v] - lse_r)) for j = w*V + v,
 *   prune    the W best candidates of each item over its W*V flattened
 *            candidates, ordered by (cand desc, j asc); parent w = j / V,
 *            token = j % V (integer quotient and remainder),
 *   finalize in rank order, an EOS selection enters the item's finished set
 *            with |y| = t; every other selection becomes the next live slot.
 *            Live slots are compacted in rank order; remaining slots are dead
 *            (score -inf). Then the stop rule runs (see bs_stop).
 * Rows of items that are done, and dead rows (score -inf), are not read:
 * their logits may hold anything, and need not be valid memory. At step 1
 * only slot 0 of each item is live, so only rows b*W are read.
 *   logits           device, [B*W][row_stride_elems] of fp32 or bf16 (as
 *                    configured); row r = b*W + w; only the first V of each
 *                    row are read
 *   row_stride_elems >= V
 *   beam_idx         device int32 [B][W], written: local parent slot
 *                    (0..W-1) of each new slot; own slot for dead slots and
 *                    for items already done before this step
 *   token_id         device int32 [B][W], written: the new token; pad_id for
 *                    dead slots and done items
 *   scores           device fp32 [B][W], written: the new running score; -inf
 *                    for dead slots and done items
 *   done             device uint8 [B], written: 1 if the item is done after
 *                    this step
 * Errors: BS_EINVAL (NULL pointer, stride < V); BS_ESTATE if max_steps steps
 * were already taken; BS_EDEVICE. */
int bs_step(bs_state *h, const void *logits, int64_t row_stride_elems,
            int32_t *beam_idx, int32_t *token_id, float *scores, uint8_t *done);

/* KV-cache layout for bs_reorder_kv: n_planes planes (one per layer and K or
 * V), each holding rows b*W+w of positions of bytes_per_pos contiguous bytes. */
typedef struct {
    int32_t n_planes;        /* >= 1                                          */
    void *const *planes;     /* host array of n_planes device pointers        */
    int64_t row_stride;      /* bytes between row r and row r+1 of a plane    */
    int64_t pos_stride;      /* bytes between position p and p+1 of a row     */
    int64_t pos_offset;      /* first position the reorder touches: a prompt
                                kept before it is shared and never moved      */
    int64_t bytes_per_pos;   /* bytes of one position of one row              */
} bs_kv_desc;

/* The cache reorder that follows the last bs_step ("llm_internals" 9.2.2,
 * KV-cache paragraph: a new slot reads its parent's cache, and a parent chosen
 * by several slots is copied to each). For every item not done after that
 * step and every live slot i whose parent p = beam_idx[b][i] differs from i,
 * positions [pos_offset, pos_offset + gen_len) of row b*W+i of every plane
 * become what row b*W+p held before the call, bit for bit. Rows of slots that
 * keep their parent, dead slots and done items are not touched. Every
 * distinct parent is read once per position; the copy is in place and safe
 * for swaps and cycles.
 *   kv       host descriptor; planes are device pointers
 *   gen_len  number of positions to move (>= 0; 0 is a no-op)
 * Each plane goes through one call per step: a second call on the same plane
 * applies the step's permutation again. Planes may be split over several calls
 * (different layouts, more planes than one launch takes).
 * Requires bytes_per_pos, row_stride, pos_stride, pos_offset*pos_stride and
 * every plane address to be multiples of 4 bytes (16 for the fast path), and
 * a row's gen_len * bytes_per_pos to be under 2^32 copy words (of 16 bytes on
 * the fast path, 4 otherwise). The moved (row, position) pairs of a plane
 * must not share bytes: bytes_per_pos <= pos_stride, and either rows lie a
 * whole moved span apart, (gen_len-1)*pos_stride + bytes_per_pos <=
 * row_stride (rows outermost), or positions lie all rows apart,
 * (B*W-1)*row_stride + bytes_per_pos <= pos_stride with bytes_per_pos <=
 * row_stride (positions outermost); other layouts are refused.
 * Errors: BS_EINVAL; BS_ESTATE before the first bs_step; BS_EDEVICE. */
int bs_reorder_kv(bs_state *h, const bs_kv_desc *kv, int32_t gen_len);

/* bs_reorder_kv, timed: for callers that measure the reorder's own duration
 * (benchmarks) without adding records to the stream. start_event and
 * stop_event are hipEvent_t handles created by the caller (either may be
 * NULL; the caller keeps ownership). They are attached to the call's first
 * and last kernel dispatch (hipExtLaunchKernel), so they take the time at
 * which the reorder kernels start and end, as a kernel trace does. A call
 * that launches nothing (gen_len 0) records both on the stream back to back.
 * Errors: as bs_reorder_kv; BS_EDEVICE also if an event cannot be used. */
int bs_reorder_kv_timed(bs_state *h, const bs_kv_desc *kv, int32_t gen_len,
                        void *start_event, void *stop_event);

/* Paged KV cache ("llm_internals" 9.2.2, KV-cache paragraph: with a paged
 * cache the reorder becomes a rewrite of block-table entries, and a block is
 * copied only when a shared block is about to be written, i.e. copy on
 * write; 9.2.4: the generated parts' common prefixes are then shared too).
 *
 * The generated positions of every row live in blocks of block_size
 * positions in block pools owned by the caller, one pool per layer and K or
 * V, all indexed by the same block ids. Row r = b*W+w maps its logical block
 * k (positions k*block_size .. (k+1)*block_size-1) to the physical block
 * table[r][k], or -1 for none. Item b owns the physical blocks
 * [b*blocks_per_item, (b+1)*blocks_per_item): rows share blocks only within
 * an item, and a block shared by two live rows is never written. The handle
 * owns the table, the reference counts and each item's free list. */
typedef struct bs_kv_paged bs_kv_paged;

/* Every pool holds B * blocks_per_item blocks of block_size positions. */
typedef struct {
    int32_t n_planes;        /* >= 1                                          */
    void *const *pools;      /* host array of n_planes device pointers        */
    int64_t block_stride;    /* bytes between physical block k and k+1        */
    int64_t pos_stride;      /* bytes between positions p and p+1 of a block  */
    int64_t bytes_per_pos;   /* bytes of one position of one row              */
} bs_kv_pool;

/* Creates the paged tables for handle h (B items, W beams, T = max_steps):
 * the table [B*W][max_blocks] with max_blocks = T / block_size + 1 (blocks
 * for positions 0..T), and per item blocks_per_item reference counts and a
 * free list. Then resets them as bs_kv_paged_reset does. Synchronises.
 * The first cache created on a handle is attached to it: while every step of
 * the search has been reordered, in order, bs_step runs the table part of
 * the next reorder (see bs_kv_paged_reorder) in its own launch when it uses
 * the fused selection and a row spans at most 64 tiles of its streaming pass
 * (V <= 64 * 256 * the logits per thread, tile_elems or the library's
 * choice), and bs_kv_paged_reorder then only makes the copies. The table
 * therefore shows step t's blocks from that bs_step on. A cache whose
 * handle is destroyed first is orphaned: every later call on it returns
 * BS_ESTATE, except bs_kv_paged_destroy, which frees it.
 *   block_size       positions per block, >= 1
 *   blocks_per_item  W <= blocks_per_item <= 4096; W * max_blocks always
 *                    suffices, fewer relies on shared prefixes
 * Limit: W * max_blocks <= 2048.
 * Errors: BS_EINVAL; BS_ENOMEM; BS_EDEVICE. */
int bs_kv_paged_create(bs_state *h, int32_t block_size, int32_t blocks_per_item,
                       bs_kv_paged **out);

/* Every row gets a private block for its logical block 0, so position 0 of
 * every row is writable; every other block of the item is free. Call it
 * together with bs_reset, before the first bs_step of a search. */
int bs_kv_paged_reset(bs_kv_paged *p);

/* The device table, int32 [B*W][max_blocks] (row r at table + r*max_blocks),
 * valid until bs_kv_paged_destroy; the caller reads it to address the pools
 * and must not write it. */
int bs_kv_paged_table(const bs_kv_paged *p, int32_t **table, int32_t *max_blocks);

/* The reorder that follows the bs_step of step t, with gen_len = t positions
 * [0, t) written:
 *  (1) for every live slot i of an item not done after the step whose parent
 *      p = beam_idx[b][i] differs from i, row i's blocks 0..ceil(t/block_size)-1
 *      become row p's (block ids are copied, not data); blocks no live row of
 *      an item still running references any more (those of overwritten rows,
 *      of dead slots and of items that are done) return to the free list;
 *  (2) position t is made writable for every live slot of an item not done:
 *      at a block boundary (t % block_size == 0) the slot gets a fresh block;
 *      otherwise, where live slots share the block holding position t, every
 *      slot but the lowest gets a private copy of that block's first
 *      t % block_size positions in every pool (the copy on write).
 * Afterwards every live row's positions [0, t), read through the table, hold
 * what its parent's held before the call, bit for bit. For the cache attached
 * to the handle, (1) and the block assignment of (2) may already have run in
 * bs_step (see bs_kv_paged_create); the result after this call is the same.
 *   pool     host descriptor of the caller's pools; block_stride, pos_stride,
 *            bytes_per_pos and every pool address must be multiples of 4 bytes
 *            (16 for the fast path)
 *   gen_len  must equal the steps taken: one call after every bs_step, in
 *            order, starting at step 1 after bs_kv_paged_reset
 * An item that runs out of free blocks leaves the slot's entry at -1 and sets
 * the overflow flag read by bs_kv_paged_status.
 * Errors: BS_EINVAL; BS_ESTATE (gen_len is not the steps taken, or the
 * previous step was not reordered, or this one already was); BS_EDEVICE. */
int bs_kv_paged_reorder(bs_kv_paged *p, const bs_kv_pool *pool, int32_t gen_len);

/* Synchronises the handle's stream, then reports whether any item ran out of
 * free blocks since the last reset (*overflow, host int32) and, when
 * free_blocks is not NULL, each item's free block count (host int32 [B]). */
int bs_kv_paged_status(bs_kv_paged *p, int32_t *overflow, int32_t *free_blocks);

/* Frees the tables after synchronising the stream. */
void bs_kv_paged_destroy(bs_kv_paged *p);

/* Final selection (batched section of "Transformers中的Beam Search高效实现",
 * after the decode loop): every live beam of an item that is not done joins
 * a copy of its finished set with |y| = steps taken; the best num_return
 * hypotheses per item, ordered by (normalised score desc, step asc, rank
 * asc), are written out. Does not change the handle; may be called again.
 *   tokens       device int32 [B][num_return][max_steps]: the generated
 *                tokens (EOS included when the hypothesis ended with it),
 *                pad_id after the end
 *   lengths      device int32 [B][num_return]: |y|; 0 for a missing entry
 *   norm_scores  device fp32 [B][num_return]: normalised score; -inf for a
 *                missing entry
 * Errors: BS_EINVAL; BS_ESTATE before the first bs_step; BS_EDEVICE. */
int bs_finalize(bs_state *h, int32_t *tokens, int32_t *lengths, float *norm_scores);

/* The ranked selection of the last bs_step, before compaction ("prune"
 * output): flat index j (= parent*V + token) and fp32 candidate score, for
 * ranks 0..K-1 of each item, K = W (BS_PRUNE_TOPW) or 2W (BS_PRUNE_TOP2W);
 * j = -1 and score -inf where an item had fewer than K finite candidates or
 * was already done.
 *   flat_idx  device int32 [B][K];  cand_score  device fp32 [B][K]
 * Errors: BS_EINVAL; BS_ESTATE before the first bs_step. */
int bs_last_selection(bs_state *h, int32_t *flat_idx, float *cand_score);

/* Each item's finished set as it stands (storage order, unsorted):
 *   norm, raw  device fp32 [B][W]; len, step, rank  device int32 [B][W];
 *   count      device int32 [B]  (entries at index >= count are undefined) */
int bs_get_finished(bs_state *h, float *norm, float *raw, int32_t *len,
                    int32_t *step, int32_t *rank, int32_t *count);

/* Steps taken since bs_create or bs_reset (host value, no GPU work). */
int bs_steps_taken(const bs_state *h);

/* Checkpoint and resume (a search moved to another handle, process or device):
 * a snapshot holds the search state -- running scores, slot ranks, done flags,
 * finished sets, the backpointers of the steps taken, the last selection and
 * the reorder plan -- behind a header naming the configuration and the steps
 * taken. It holds values only (no addresses), in host memory the caller owns.
 * bs_state_size: the snapshot's size in bytes (host int64).
 * bs_state_save: synchronises the handle's stream and copies the snapshot into
 *   dst (host, at least bs_state_size bytes); does not change the handle.
 * bs_state_load: restores a snapshot into a handle created with the same
 *   bs_config (every field; the device may differ), then synchronises; the
 *   next bs_step is step (steps taken in the snapshot) + 1, and bs_reorder_kv
 *   uses the snapshot's last plan. The KV cache itself is the caller's (save
 *   it alongside); a paged cache attached to the handle is not part of the
 *   snapshot: after a load it refuses reorders (BS_ESTATE), and bs_step leaves
 *   its tables alone, until bs_kv_paged_reset.
 * Errors: BS_EINVAL (NULL pointer, too small a buffer, a snapshot of another
 * configuration or a corrupt header); BS_EDEVICE. */
int bs_state_size(const bs_state *h, int64_t *bytes);
int bs_state_save(bs_state *h, void *dst, int64_t capacity);
int bs_state_load(bs_state *h, const void *src, int64_t size);

/* Frees the handle's device buffers after synchronising its stream. */
void bs_destroy(bs_state *h);

/* Blockwise-parallel verify ("Blockwise Parallel Decoding", section 3, the
 * verify sub-step, and Figure 1): for each item b and position i < k,
 * argmax[b][i] is the first index of the largest logit of row b*k+i (greedy
 * needs no softmax, "llm_internals" 9.2.1), and accept_len[b] is the largest
 * k' <= k with proposals[b][i] == argmax[b][i] for every i < k'. When
 * proposals[b][0] is the base model's own greedy token, accept_len >= 1. */
typedef struct bs_verify_state bs_verify_state;

/* Allocates the per-tile partial results for logits [B][k][V] once.
 *   batch >= 1, k in 1..64, batch*k <= 65535, vocab >= 1; logits_dtype a
 *   bs_dtype. */
int bs_verify_create(int32_t batch, int32_t k, int32_t vocab, int32_t logits_dtype,
                     void *hip_stream, bs_verify_state **out);

/*   logits      device [B*k][row_stride_elems] (row b*k+i), fp32 or bf16
 *   proposals   device int32 [B][k]
 *   accept_len  device int32 [B], written
 *   argmax      device int32 [B][k], written
 * Errors: BS_EINVAL (NULL pointer, stride < V); BS_EDEVICE. */
int bs_verify(bs_verify_state *h, const void *logits, int64_t row_stride_elems,
              const int32_t *proposals, int32_t *accept_len, int32_t *argmax);

/* Approximate verify ("Blockwise Parallel Decoding", section 5.1 top-k
 * selection and section 5.3 minimum block size). Position i passes while the
 * rank of proposals[b][i] among the logits of row b*k+i is below top_k, the
 * rank being the number of logits that beat the proposal's (larger, or equal
 * at a lower index); top_k = 1 is the exact greedy check of bs_verify.
 * accept_len[b] = max(longest passing prefix, min_block). A proposal outside
 * [0, V) has rank V and never passes; it is not read.
 *   top_k      >= 1
 *   min_block  0..k (0 and 1: no minimum beyond the pages' k^ >= 1)
 *   prop_rank  device int32 [B][k], written when not NULL
 * Other arguments as for bs_verify.
 * Errors: BS_EINVAL (NULL pointer, stride < V, top_k < 1, min_block outside
 * 0..k); BS_EDEVICE. */
int bs_verify_ex(bs_verify_state *h, const void *logits, int64_t row_stride_elems,
                 const int32_t *proposals, int32_t top_k, int32_t min_block,
                 int32_t *accept_len, int32_t *argmax, int32_t *prop_rank);

/* bs_verify without a handle and without allocating, for callers that cannot
 * allocate device memory: code under HIP graph capture, serving loops,
 * harnesses that forbid hipMalloc. Computes what bs_verify computes (the
 * exact criterion) for logits [batch][k][vocab] of logits_dtype, on
 * hip_stream (NULL: the null stream). Its per-segment partials live in a
 * static device array of the library, 4 MiB on each GPU, held until the
 * process ends and shared by every bs_verify_noalloc call on that GPU:
 * calls that overlap on one GPU (other streams, other threads) race, so
 * order them on one stream. Nothing in the array needs clearing between
 * calls. The first call on a device looks up the array's address there
 * (hipGetSymbolAddress): make it outside graph capture.
 *   logits, proposals, accept_len, argmax, row_stride_elems: as bs_verify
 *   Limits: batch >= 1, k in 1..64, batch*k <= 65535 (as bs_verify_create),
 *   and the partials within the array: batch*k*S <= 524288, S being the
 *   segments of a row, ceil(vocab / 4096) when batch*k < 256 and at most 4
 *   otherwise (so every shape with batch*k >= 256 fits).
 * Errors: BS_EINVAL (NULL pointer, stride < vocab, a shape out of range or
 * beyond the array); BS_EDEVICE. */
int bs_verify_noalloc(void *hip_stream, const void *logits, int32_t logits_dtype,
                      int32_t batch, int32_t k, int32_t vocab, int64_t row_stride_elems,
                      const int32_t *proposals, int32_t *accept_len, int32_t *argmax);

void bs_verify_destroy(bs_verify_state *h);

/* Static description of a status code. */
const char *bs_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* BEAMSTEP_H */
