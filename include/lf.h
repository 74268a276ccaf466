/*
 * lf.h - C ABI of the LongFlow-style fused decode step for AMD MI355X (gfx950).
 *
 * One call of lf_decode_step runs, for every sequence b and KV head g of a
 * static fixed-budget KV cache, in one kernel launch:
 *   (a) GQA decode attention of the query heads of group g over the cached
 *       slots plus the incoming token,
 *   (b) the history-free importance of every cached slot: the softmax weight
 *       that this step's attention gives it, summed over the group's query
 *       heads (LF_SCORE_ATTN), or that sum times the L1 norm of the slot's
 *       value vector (LF_SCORE_VL1, the LongFlowScore equation of the LongFlow
 *       summary on gist.science, section 2.B),
 *   (c) the argmin over the slots outside the sink and recent windows,
 *   (d) the in-place overwrite of that slot with the incoming K/V,
 * so the cache never holds more than its budget.  The fusion of attention,
 * importance and eviction into a single operator over a statically
 * pre-allocated cache is the design of the LongFlow summary, section 2.C, and
 * of the LongFlow blog post (denisavetisyan.com), section on fused kernels.
 *
 * Conventions shared by every entry point:
 *  - Device buffers are caller-owned and passed as plain device pointers
 *    (for example torch tensors' data_ptr()).  The library allocates only the
 *    small host-side lf_cache handle; it never allocates device memory.
 *  - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *  - Errors are returned as lf_status, never thrown across the ABI; the text of
 *    the last error of the calling thread is available from lf_last_error().
 *  - Layouts are dense row-major.  Element type is lf_config.dtype everywhere
 *    (q, k_new, v_new, out, k_cache, v_cache).
 *  - Query head h belongs to KV head h / G with G = n_q_heads / n_kv_heads
 *    (contiguous groups).
 */
#ifndef LF_H_
#define LF_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LF_ABI_VERSION 2

typedef enum lf_status {
  LF_OK = 0,
  LF_ERR_ARG = 1,         /* invalid argument (null pointer, shape, window, size) */
  LF_ERR_UNSUPPORTED = 2, /* well-formed but not built: head_dim, group size, dtype */
  LF_ERR_STATE = 3,       /* handle is not a live lf_cache */
  LF_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
} lf_status;

typedef enum lf_dtype { LF_F32 = 0, LF_BF16 = 1 } lf_dtype;

typedef enum lf_score {
  LF_SCORE_ATTN = 0, /* I_i = sum over the group's query heads of alpha_{h,i} */
  LF_SCORE_VL1 = 1,  /* I_i = (sum_h alpha_{h,i}) * sum_l |v_i[l]|            */
  LF_SCORE_NONE = 2  /* full-cache comparator: attention (a) only, no importance
                      * and no eviction.  The incoming token is appended while
                      * the cache has room; once it is full the token is
                      * attended but not stored (evict_idx = -2).  This is the
                      * uncompressed cache the pages compare LongFlow against
                      * (LongFlow summary, section 3), run by the same streaming
                      * kernel; size max_budget for the longest context.      */
} lf_score;

typedef struct lf_config {
  int32_t batch;         /* B >= 1                                                */
  int32_t n_q_heads;     /* Hq, a multiple of n_kv_heads                          */
  int32_t n_kv_heads;    /* Hkv >= 1; G = Hq / Hkv must be in [1, 8]              */
  int32_t head_dim;      /* d: 64 or 128                                          */
  int32_t max_budget;    /* slot stride of k_cache/v_cache; every budget <= this, */
                         /* at most 65536                                         */
  int32_t sink;          /* slots [0, sink) hold positions 0..sink-1, never evicted */
  int32_t recent;        /* the `recent` newest cached tokens are never evicted   */
  int32_t dtype;         /* lf_dtype                                              */
  int32_t score;         /* lf_score                                              */
  float softmax_scale;   /* logit scale; <= 0 selects 1/sqrt(head_dim)            */
  int32_t chunk_slots;   /* split-KV chunk length in slots; 0 = automatic         */
  int32_t reserved;      /* must be 0                                             */
} lf_config;

typedef struct lf_cache lf_cache; /* opaque host handle */

/* lf_init_cache flag: keep the device state as it is (resume from a saved copy
 * of k_cache, v_cache and state); only the host handle is rebuilt. */
#define LF_INIT_ATTACH 1

/*
 * lf_state_bytes - size of the device `state` buffer lf_init_cache needs.
 *   cfg      host, validated as in lf_init_cache.
 *   budgets  host int32[B], per-sequence budget (1 <= budget <= max_budget and
 *            budget > sink + recent), or NULL for max_budget everywhere.
 *   bytes    host, receives the size.
 * Pure host computation; no HIP call.  Errors: LF_ERR_ARG, LF_ERR_UNSUPPORTED.
 */
lf_status lf_state_bytes(const lf_config* cfg, const int32_t* budgets, size_t* bytes);

/*
 * lf_init_cache - bind a filled static cache and build the device state.
 *   budgets  host int32[B] or NULL (= max_budget).
 *   seq_len  host int64[B]: tokens seen so far per sequence (0 <= seq_len < 2^31).
 *            Contract on the cache contents: slots [0, min(seq_len, budget))
 *            hold the cached tokens in increasing position order, slots
 *            [0, sink) hold positions 0..sink-1, and when seq_len >= budget the
 *            last `recent` slots hold positions seq_len-recent .. seq_len-1.
 *   k_cache, v_cache  device [B][Hkv][max_budget][d]; must stay valid until
 *            lf_free.  Only the slots of the first step's eviction are ever
 *            written.
 *   state, state_bytes  device buffer of at least lf_state_bytes() bytes,
 *            caller-owned, 256-byte aligned, kept for the cache's lifetime.
 *            Holds the per-(sequence, KV head) step counter, fill level, ring
 *            of recent slots, the split-KV work list and the partial results.
 *   flags    0, or LF_INIT_ATTACH to reuse a state written by an earlier
 *            lf_init_cache + lf_decode_step sequence with the same cfg/budgets.
 *   stream   the state upload is ordered on this stream; the call waits for it.
 *   out      host, receives the handle.
 * Errors: LF_ERR_ARG (any bad size, window, budget, pointer or alignment),
 * LF_ERR_UNSUPPORTED (head_dim, G, dtype), LF_ERR_HIP.
 */
lf_status lf_init_cache(const lf_config* cfg, const int32_t* budgets, const int64_t* seq_len,
                        void* k_cache, void* v_cache, void* state, size_t state_bytes,
                        int32_t flags, void* stream, lf_cache** out);

/*
 * lf_decode_step - one fused decode step (attention + importance + argmin +
 * in-place overwrite) for the whole batch, one kernel launch on `stream`.
 *   q          device [B][Hq][d]
 *   k_new      device [B][Hkv][d]   incoming token's keys
 *   v_new      device [B][Hkv][d]   incoming token's values
 *   out        device [B][Hq][d]    attention output over cache + new token,
 *              rounded to nearest-even when dtype is bf16
 *   evict_idx  device int32 [B][Hkv]: slot overwritten by the new token, or -1
 *              when the cache was not yet full and the token was appended,
 *              or -2 when the token was not stored (LF_SCORE_NONE, full).
 * Asynchronous and stream-ordered; no host synchronisation, no allocation.
 * Calls on one handle must be ordered on one stream.  Validation is limited to
 * null pointers and the handle (a handle from lf_init_cache: one layer);
 * errors: LF_ERR_ARG, LF_ERR_STATE, LF_ERR_HIP.
 */
lf_status lf_decode_step(const void* q, const void* k_new, const void* v_new, lf_cache* cache,
                         void* out, int32_t* evict_idx, void* stream);

/*
 * lf_decode_step_dbg - lf_decode_step that also exports its intermediates.
 *   scores  device float [B][Hkv][max_budget] or NULL: importance of every
 *           cached slot i < fill level, before the window mask (other entries
 *           are left untouched; nothing is written under LF_SCORE_NONE).
 *   lse     device float [B][Hq] or NULL: natural-log softmax normaliser
 *           log(sum_i exp(scale q.k_i)) over cache + new token.
 * Same semantics and errors as lf_decode_step otherwise.
 */
lf_status lf_decode_step_dbg(const void* q, const void* k_new, const void* v_new, lf_cache* cache,
                             void* out, int32_t* evict_idx, float* scores, float* lse, void* stream);

/*
 * lf_state_bytes_layers - size of the state buffer of lf_init_layers:
 * n_layers (1 .. 4096) times lf_state_bytes.  Errors as lf_state_bytes.
 */
lf_status lf_state_bytes_layers(const lf_config* cfg, const int32_t* budgets, int32_t n_layers, size_t* bytes);

/*
 * lf_init_layers - one handle over the n_layers layer caches of a model (the
 * statically pre-allocated cache of the LongFlow summary, section 2.C, for
 * every layer; memory management across the layers is what section 4 credits
 * for the larger batches).  Every layer shares cfg, budgets and seq_len;
 * layer l's state occupies bytes [l * S, (l + 1) * S) of `state` with
 * S = state_bytes / n_layers rounded down to a multiple of 256, which must be
 * at least lf_state_bytes (the same S again when attaching with
 * LF_INIT_ATTACH, so pass the same state_bytes).
 *   k_caches, v_caches  host arrays of n_layers device pointers, each a
 *            [B][Hkv][max_budget][d] cache laid out as lf_init_cache describes.
 * Other arguments, the cache contract and errors as lf_init_cache.  The
 * resets (lf_reset_sequences, lf_reset_sequences_budget), lf_set_split_wait and
 * lf_check_state act on every layer of the handle; steps run per layer with
 * lf_decode_step_layer (lf_decode_step rejects a handle of several layers).
 */
lf_status lf_init_layers(const lf_config* cfg, int32_t n_layers, const int32_t* budgets, const int64_t* seq_len,
                         void* const* k_caches, void* const* v_caches, void* state, size_t state_bytes,
                         int32_t flags, void* stream, lf_cache** out);

/*
 * lf_decode_step_layer - lf_decode_step on layer `layer` (0 .. n_layers - 1)
 * of a handle, with that layer's q, k_new, v_new, out and evict_idx.  Layers
 * are independent: their steps may run in any order, each layer's steps in
 * sequence on one stream.  Errors: LF_ERR_ARG (also a layer out of range),
 * LF_ERR_STATE, LF_ERR_HIP.
 */
lf_status lf_decode_step_layer(const void* q, const void* k_new, const void* v_new, lf_cache* cache, int32_t layer,
                               void* out, int32_t* evict_idx, void* stream);

/* lf_decode_step_layer_dbg - lf_decode_step_dbg on one layer of a handle. */
lf_status lf_decode_step_layer_dbg(const void* q, const void* k_new, const void* v_new, lf_cache* cache,
                                   int32_t layer, void* out, int32_t* evict_idx, float* scores, float* lse,
                                   void* stream);

/*
 * lf_set_split_wait - how long a chunk of a split (sequence, KV head) pair
 * waits, after streaming its rows, for the pair's other chunks to publish
 * their softmax statistics; with them it scores its own slots from on-chip
 * logits.  A chunk that stops waiting (or never waits) hands its logits over
 * through the state buffer and the pair's last chunk scores them: results are
 * bit-identical either way, only slower (lf_check_state counts such chunks,
 * together with the chunks whose logits never stay on chip: fp32 caches and
 * chunks longer than the on-chip buffers).  Waiting pays when the pair's
 * chunks run at the same time, which a step whose work items fit the GPU at
 * once gives.
 *   cache        live handle.
 *   max_wait_us  0 .. 1000000 microseconds; 0: never wait.  Default 100.
 * Takes effect for the steps launched after the call.  Errors: LF_ERR_ARG,
 * LF_ERR_STATE.
 */
lf_status lf_set_split_wait(lf_cache* cache, int32_t max_wait_us);

/* Result of lf_check_state. */
typedef struct {
  uint32_t deferred; /* split chunks that handed their logits over through memory, since init (all layers) */
  int32_t n_pairs;   /* batch * n_kv_heads (per layer) */
  int32_t bad_pair;  /* first pair that failed a check, or -1 */
  int32_t bad_layer; /* layer of the failed check, or -1 */
} lf_state_report;

/*
 * lf_check_state - read the state back (after the steps queued on `stream`)
 * and check its invariants, in every layer of the handle: the header matches
 * the handle and no wait hit its safety bound; per pair the
 * layout fields are the handle's, the fill level is min(position, budget),
 * the epoch is non-zero, no chunk counter is left over from a step, and the
 * slots of the `recent` newest positions are distinct filled slots.
 *   report  host: filled on LF_OK and on LF_ERR_STATE (bad_pair names the pair).
 * Synchronous (a device-to-host copy); errors: LF_ERR_ARG, LF_ERR_STATE
 * (a broken invariant, described by lf_last_error), LF_ERR_HIP.
 */
lf_status lf_check_state(const lf_cache* cache, void* stream, lf_state_report* report);

/*
 * lf_reset_sequences - restart some sequences of the batch in place (a finished
 * request's place taken by a new one under continuous batching) while the
 * others keep their state.  On a handle over several layers
 * (lf_init_layers) the listed sequences restart in every layer.  The decode step runs over a static, pre-allocated
 * cache (LongFlow summary, section 2.C); this only re-initialises the listed
 * sequences' position, fill level and recent-window ring, exactly as
 * lf_init_cache does for the whole batch.
 *   cache    live handle.
 *   n        number of listed sequences (0: nothing to do).
 *   seqs     host int32[n]: distinct sequence indices in [0, B).
 *   seq_len  host int64[n]: tokens the new request has seen; its cached tokens
 *            are already in the sequence's k_cache/v_cache rows, laid out as
 *            lf_init_cache describes (for example by lf_prefill_compress).
 * Budgets and the split of work stay as at init.  The metadata is written by
 * small uploads ordered on `stream` after the steps already queued there; the
 * call returns once they completed.  Errors: LF_ERR_ARG, LF_ERR_STATE,
 * LF_ERR_HIP.
 */
lf_status lf_reset_sequences(lf_cache* cache, int32_t n, const int32_t* seqs, const int64_t* seq_len,
                             void* stream);

/*
 * lf_reset_sequences_budget - lf_reset_sequences that also gives the listed
 * sequences new slot budgets (a new request with another memory allowance
 * takes a finished one's place).  Every other sequence keeps its state and
 * budget.  The split of work and the workspace layout follow the new budgets,
 * so the call reads the metadata and rings back from the device after the
 * steps queued on `stream`, keeps the other sequences' positions, fill levels
 * and rings, restarts the listed ones as lf_reset_sequences does, and writes
 * the whole metadata and work list back; it returns once that completed.
 *   budgets  host int32[n]: new budget of each listed sequence, in
 *            (sink + recent, max_budget]; the listed sequence's cached tokens
 *            (seq_len, capped at the new budget) are already laid out in its
 *            k_cache/v_cache rows as lf_init_cache describes.
 * On a handle over several layers the listed sequences restart, with their
 * new budgets, in every layer.  The state buffer passed at init (its
 * state_bytes, divided by the number of layers) must hold the layout of the
 * new budgets (lf_state_bytes with them); otherwise LF_ERR_ARG and nothing
 * changes.  Errors: LF_ERR_ARG, LF_ERR_STATE, LF_ERR_HIP.
 */
lf_status lf_reset_sequences_budget(lf_cache* cache, int32_t n, const int32_t* seqs, const int64_t* seq_len,
                                    const int32_t* budgets, void* stream);

/*
 * lf_prefill_work_bytes - size of the device scratch lf_prefill_compress needs
 * (importance and the group's logits of every prefill position of every
 * (sequence, KV head), per-chunk statistics, plus the prefill lengths and
 * budgets).  cfg validated as in lf_init_cache.
 */
lf_status lf_prefill_work_bytes(const lf_config* cfg, int32_t max_prefill, size_t* bytes);

/*
 * lf_prefill_compress - one-shot compression of a prefill longer than the
 * budget, run once before decoding (the step before the decode path).  For
 * every sequence b and KV head g the last prefill query attends over all P_b
 * prefill tokens; a token's importance is the softmax weight it receives
 * summed over the group's query heads (the decode step's LF_SCORE_ATTN
 * importance: from the current query only, LongFlow summary, section 2.A).
 * Kept: positions [0, sink), the `recent` last positions [P_b - recent, P_b),
 * and the budget_b - sink - recent middle positions of largest importance
 * (equal importance: the lower position).  The pages leave long prefill to
 * other methods (summary, section 5); this selection is a reading.  When
 * P_b <= budget_b every token is kept.
 *   cfg          host; shapes, dtype, sink, recent, softmax_scale as for
 *                lf_init_cache (score and chunk_slots are not used).
 *   budgets      host int32[B] or NULL (max_budget), validated as in lf_init_cache.
 *   prefill      host int32[B]: P_b in [1, max_prefill]; max_prefill <= 65536.
 *   q_last       device [B][Hq][d]: the query of each sequence's last prefill token.
 *   k_pre, v_pre device [B][Hkv][max_prefill][d]: prefill K/V, position p in row p.
 *   k_cache, v_cache  device [B][Hkv][max_budget][d]: slots 0 .. min(P_b, budget_b)-1
 *                receive the kept tokens in increasing position order; other
 *                slots are untouched.  Then call lf_init_cache with
 *                seq_len[b] = P_b (the recent window is the last slots).
 *   kept         device int32 [B][Hkv][max_budget]: the kept positions, same order.
 *   work         device scratch of work_bytes >= lf_prefill_work_bytes(); on
 *                return it holds the importance [B][Hkv][max_prefill] (float).
 * All device pointers 16-byte aligned; k_pre/v_pre must not overlap k_cache/v_cache.
 * Asynchronous on `stream`; batches of more than 128 sequences first upload
 * their lengths with a small copy that waits for the stream.
 * Errors: LF_ERR_ARG, LF_ERR_UNSUPPORTED, LF_ERR_HIP.
 */
lf_status lf_prefill_compress(const lf_config* cfg, const int32_t* budgets, const int32_t* prefill,
                              int32_t max_prefill, const void* q_last, const void* k_pre, const void* v_pre,
                              void* k_cache, void* v_cache, int32_t* kept, void* work, size_t work_bytes,
                              void* stream);

/*
 * lf_prefill_compress_noalloc - lf_prefill_compress without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * scratch is a static device array inside the library, LF_PREFILL_SCRATCH_BYTES
 * (64 MiB) per GPU, held by every GPU the library runs on until the process
 * ends; its address is looked up once per device.  The call allocates nothing.
 * Arguments, results and errors as lf_prefill_compress; batches whose
 * lf_prefill_work_bytes() exceeds LF_PREFILL_SCRATCH_BYTES are rejected with
 * LF_ERR_ARG (use lf_prefill_compress with a workspace instead).  All calls on
 * one GPU share its scratch: calls that overlap on one GPU (different streams,
 * different threads) race and must be serialised by the caller.
 */
#define LF_PREFILL_SCRATCH_BYTES ((size_t)64 << 20)
lf_status lf_prefill_compress_noalloc(const lf_config* cfg, const int32_t* budgets, const int32_t* prefill,
                                      int32_t max_prefill, const void* q_last, const void* k_pre,
                                      const void* v_pre, void* k_cache, void* v_cache, int32_t* kept,
                                      void* stream);

/* lf_free - release the host handle (NULL-safe).  Device buffers stay the caller's. */
void lf_free(lf_cache* cache);

/* lf_last_error - message of the last failed call on this thread ("" if none). */
const char* lf_last_error(void);

/* lf_abi_version - LF_ABI_VERSION of the built library. */
int32_t lf_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LF_H_ */
