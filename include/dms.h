/*
 * dms.h — C ABI of the DMS (Dynamic Memory Sparsification) inference hot path
 * for AMD Instinct MI355X (gfx950).
 *
 * What the library computes (pages cited by title and section):
 *   - the per-KV-head keep/evict decision: logit = Linear(RMSNorm(h)) * scale
 *     - offset, or the repurposed last element of the first query head of each
 *     KV group times scale minus offset; a token is evicted when logit > 0
 *     ("基于 DMS 的 KV Cache 压缩实战" walkthrough, sections 决策来源一,
 *     决策来源二, 决策粒度, and the inference hard threshold in the Gumbel
 *     section);
 *   - delayed eviction into a per-head paged KV store: a marked token stays
 *     visible until it leaves the sliding window w, then the token w positions
 *     later overwrites its slot in place (same walkthrough, 延迟驱逐 and
 *     推理模式);
 *   - GQA decode attention and chunked-prefill attention over the resulting
 *     ragged per-head cache (推理模式; 高级选项 Chunked Prefill; the exact
 *     prefill with the eviction mask in the repository tree).
 *
 * Key j is visible to query i iff j <= i and (j is kept or i - j < w).
 *
 * Conventions for every call:
 *   - Returns 0 (DMS_OK) or a negative dms_status.  Argument and configuration
 *     errors are detected on the host before anything is launched; the
 *     message is available from dms_last_error() (thread-local).
 *   - Conditions only the device can see (page pool exhausted, a sequence
 *     past its preallocated capacity, a sequence id out of range) set bits of
 *     a sticky device status word and skip the affected writes; read it with
 *     dms_cache_status().  After a nonzero device status the cache contents
 *     are unspecified until the affected sequences are reset.
 *   - All tensor pointers are device pointers owned by the caller, contiguous
 *     row-major, unless stated otherwise.  The library allocates no device
 *     memory: the cache lives in one caller-allocated buffer.
 *   - Calls are asynchronous on the given stream (a hipStream_t passed as
 *     void*; NULL is the null stream).  One cache handle must be used from one
 *     stream at a time.
 *   - "act" dtype is the dtype of hidden states, Q/K/V inputs and outputs:
 *     float32 when kv_dtype is DMS_F32, bfloat16 otherwise.
 */
#ifndef DMS_H
#define DMS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dms_status {
  DMS_OK = 0,
  DMS_ERR_ARG = -1,          /* null pointer, bad size, bad sequence id list */
  DMS_ERR_CONFIG = -2,       /* configuration rejected by dms_config_validate */
  DMS_ERR_CAPACITY = -3,     /* buffer too small, B or T above the configured maximum */
  DMS_ERR_POOL = -4,         /* reserved: pool exhaustion is reported by the device status */
  DMS_ERR_HIP = -5,          /* a HIP runtime call failed */
  DMS_ERR_UNSUPPORTED = -6   /* shape/dtype combination without a kernel */
} dms_status;

/* Bits of the sticky device status word (dms_cache_status). */
#define DMS_DEV_POOL_EXHAUSTED 0x1  /* an append needed a page and the pool was empty */
#define DMS_DEV_CAPACITY 0x2        /* an append would pass max_tokens_per_seq */
#define DMS_DEV_BAD_SEQ 0x4         /* a sequence id outside [0, max_batch) */
#define DMS_DEV_STEP_SYNC 0x8       /* a one-launch decode step gave up waiting for its attention
                                       workgroups and did not commit: positions, lengths, ring and
                                       page tables are as before the call, but the rows it would have
                                       placed may already be written; clear the status
                                       (dms_cache_clear_status), then repeat the same step */

typedef enum dms_dtype { DMS_F32 = 0, DMS_BF16 = 1, DMS_FP8_E4M3 = 2 } dms_dtype;
typedef enum dms_decide_mode { DMS_DECIDE_LINEAR = 0, DMS_DECIDE_QNEURON = 1 } dms_decide_mode;
typedef enum dms_alpha_per { DMS_ALPHA_PER_HEAD = 0, DMS_ALPHA_PER_LAYER = 1 } dms_alpha_per;

/*
 * Configuration of one layer's cache (walkthrough, Qwen3ConfigDMS parameter
 * table and hard constraints: block_size > 0 and window > block_size).
 */
typedef struct dms_config {
  int32_t max_batch;           /* sequence slots (ids 0..max_batch-1) */
  int32_t num_q_heads;         /* Hq */
  int32_t num_kv_heads;        /* Hkv; Hq / Hkv must be 1, 2, 4 or 8 */
  int32_t head_dim;            /* D: 32, 64 or 128 */
  int32_t hidden;              /* H of the hidden states fed to the linear adapter (multiple of 4) */
  int32_t window;              /* w: sliding window of delayed eviction (dms_window_size) */
  int32_t block_size;          /* P: slots per page (dms_paged_attention_block_size) */
  int32_t max_tokens_per_seq;  /* preallocated positions per sequence (dms_preallocate_for_tokens) */
  int32_t pool_pages;          /* pages in the shared pool, over all sequences and heads */
  int32_t max_chunk;           /* largest T of one append or prefill call (dms_chunked_prefill) */
  int32_t kv_dtype;            /* dms_dtype of the pages */
  int32_t decide_mode;         /* dms_decide_mode (dms_separate_alpha True -> LINEAR) */
  int32_t alpha_per;           /* dms_alpha_per (dms_alpha_per) */
  int32_t disable_eviction;    /* nonzero: every decision is "keep" (dms_disable_eviction) */
  float alpha_scale;           /* dms_alpha_scale (100) */
  float rms_eps;               /* RMSNorm epsilon of the adapter norm */
  float softmax_scale;         /* 0 means 1/sqrt(head_dim) */
} dms_config;

typedef struct dms_cache dms_cache;

/* Host-side copies of the cache tables (dms_cache_dump).  Any pointer may be NULL. */
typedef struct dms_dump {
  int32_t* lengths;      /* [max_batch][Hkv] live slots per head */
  int32_t* page_table;   /* [max_batch][Hkv][max_pages_per_seq] page ids, -1 unused */
  int32_t* slot_meta;    /* [pool_pages][block_size] position | (evict << 31) of each slot's token */
  int32_t* ring;         /* [max_batch][Hkv][window] slot | (evict << 31) of position p at p % window */
  int32_t* positions;    /* [max_batch] tokens appended per sequence */
  int32_t* free_stack;   /* [pool_pages] free page ids, next pop at free_count-1 */
  int32_t* free_count;   /* [1] */
  void* k_pages;         /* [pool_pages][block_size][D] raw page bytes (kv dtype) */
  void* v_pages;         /* same for V */
  float* page_scales;    /* [pool_pages][2] fp8 K/V scales */
} dms_dump;

typedef struct dms_stats {
  int64_t tokens;            /* sum over sequences and KV heads of appended tokens */
  int64_t live_slots;        /* sum of per-head lengths */
  int64_t pages_in_use;      /* pool pages held by sequences */
  int64_t bytes_live;        /* K+V bytes of live slots */
  int64_t bytes_allocated;   /* K+V bytes of held pages */
  double cache_cr;           /* tokens / live_slots */
} dms_stats;

/* Validates a configuration.  DMS_ERR_CONFIG (with a message) when block_size
 * <= 0, window <= block_size, Hq % Hkv != 0, an unsupported head_dim, group
 * size or dtype, a bad enum, or a nonpositive size. */
int dms_config_validate(const dms_config* cfg);

/* Bytes of the single device buffer a cache with this configuration needs
 * (walkthrough, 高级选项 预分配: the cache is preallocated for
 * dms_preallocate_for_tokens positions, here max_tokens_per_seq per sequence,
 * with pool_pages pages shared by all sequences and heads).  It holds the K/V
 * pages, the fp8 scales, the slot/page/ring tables, the free-page stack and
 * small control words; decode scratch is the caller's workspace
 * (dms_decode_workspace_bytes), not part of the cache. */
int dms_cache_bytes(const dms_config* cfg, size_t* bytes);

/* Bytes of the workspace dms_decode_attn and dms_decode_step need for a call
 * of B rows on the current device: the partial (o, max, sum) records of the
 * (row, KV head) units whose live slots are split over several workgroups
 * (two per attention workgroup plus one per unit, Hq / Hkv * (head_dim + 2)
 * floats each).  DMS_ERR_ARG for B outside [1, max_batch]. */
int dms_decode_workspace_bytes(const dms_config* cfg, int B, size_t* bytes);

/* Pages a sequence may hold per KV head: ceil(max_tokens_per_seq / block_size). */
int dms_max_pages_per_seq(const dms_config* cfg, int32_t* pages);

/*
 * Creates a cache inside dev_buf (device memory of at least
 * dms_cache_bytes(cfg), 256-byte aligned, owned by the caller and kept alive
 * until dms_cache_destroy) and initialises it on `stream`: every sequence
 * empty, the free stack ordered so pops return pages 0, 1, 2, ..., status 0
 * (walkthrough, 高级选项 预分配: all cache memory is reserved up front; no call
 * allocates afterwards).  The host handle (*out) owns no device memory.
 */
int dms_cache_create(const dms_config* cfg, void* dev_buf, size_t bytes, void* stream, dms_cache** out);

/* Frees the host handle.  The device buffer stays the caller's. */
int dms_cache_destroy(dms_cache* cache);

/* Copy of the configuration the cache was created with. */
int dms_cache_config(const dms_cache* cache, dms_config* cfg);

/*
 * Decision for B x T tokens (walkthrough, 决策来源一 / 决策来源二 / 决策粒度).
 * LINEAR: hidden [B][T][H] (act dtype), rms_gamma [H] f32, W [Hkv][H] f32,
 *   bias [Hkv] f32 or NULL, offsets [Hkv] f32.  Computes
 *   z = W . (h / sqrt(mean(h^2) + eps) * gamma) (+ bias) in fp32,
 *   logit = alpha_scale * z - offset.  q_inout is ignored (may be NULL).
 * QNEURON: q_inout [B][T][Hq][D] (act dtype), offsets [Hkv] f32;
 *   logit[b][k][t] = alpha_scale * q[b][t][k*g][D-1] - offset[k], after which
 *   that element is set to 0 in place.  hidden/gamma/W/bias are ignored.
 * alpha_per LAYER: every head takes head 0's logit (all k*g neurons are still
 * zeroed).  evict = disable_eviction ? 0 : logit > 0.
 * Outputs: logits_out [B][Hkv][T] f32 (may be NULL), evict_out [B][Hkv][T] u8.
 * Pure function of its inputs; does not touch the cache state.
 */
int dms_decide(dms_cache* cache, const void* hidden, const float* rms_gamma, const float* W,
               const float* bias, const float* offsets, void* q_inout, int B, int T,
               float* logits_out, uint8_t* evict_out, void* stream);

/*
 * Appends T tokens to each of B sequences (walkthrough, 推理模式: if the token
 * w positions back was marked, the new token overwrites its slot in place;
 * otherwise it takes the next free slot, opening a page from the shared pool
 * when the head's length is a multiple of block_size).
 * seq_ids [B] int32 device array (NULL: row b is sequence b); ids in one call
 * must be distinct.  k, v [B][T][Hkv][D] act dtype; evict [B][Hkv][T] u8.
 * Token positions continue from each sequence's count of appended tokens.
 * T == 1 is the decode append; T > 1 (<= max_chunk) gives exactly the slot
 * table of T single-token appends and writes only each slot's final occupant.
 * Pages are handed out in (row, head) row-major order, then token order.
 * fp8 pages: a page's K and V scales are set when it is opened, from the
 * largest magnitude the opening call writes into it (power of two with two
 * binades of headroom); values are stored as e4m3 (nearest even, saturating).
 * Device-side: DMS_DEV_CAPACITY, DMS_DEV_POOL_EXHAUSTED, DMS_DEV_BAD_SEQ.
 * Order: after dms_prefill_attn for a prefill chunk, before dms_decode_attn
 * for a decode token.
 */
int dms_append_evict(dms_cache* cache, const int32_t* seq_ids, const void* k, const void* v,
                     const uint8_t* evict, int B, int T, void* stream);

/*
 * One decode token per row: the decision (dms_decide with T = 1) followed by
 * the append (dms_append_evict with T = 1) of the same tokens, in one call, so
 * a layer's decode step is dms_decode_prepare -> dms_decode_attn.  Results are
 * identical to calling the two functions in turn.
 * hidden [B][H] (LINEAR) or q_inout [B][Hq][D] (QNEURON, neuron zeroed in
 * place); k, v [B][Hkv][D]; logits_out [B][Hkv] (may be NULL), evict_out
 * [B][Hkv] u8 (written, then read by the append).  B <= max_batch.
 * Device-side errors as in dms_append_evict.
 */
int dms_decode_prepare(dms_cache* cache, const int32_t* seq_ids, const void* hidden, const float* rms_gamma,
                       const float* W, const float* bias, const float* offsets, void* q_inout, const void* k,
                       const void* v, int B, float* logits_out, uint8_t* evict_out, void* stream);

/*
 * Decode attention (walkthrough, 推理模式: attention over the per-head paged
 * cache).  For each row b and query head h (KV head h / g):
 *   out[b][h] = softmax_s(scale * <q[b][h], K_s>) V_s over all live slots s of
 *   that head — after the append of the current token the live slots are
 *   exactly the visible keys, so no mask is applied.
 * q [B][Hq][D], out [B][Hq][D] act dtype; seq_ids as in dms_append_evict.
 * A head with no live slot gets zeros.  fp32 accumulation.
 * workspace: device memory of at least dms_decode_workspace_bytes(cfg, B)
 * bytes, 256-byte aligned, owned by the caller, overwritten (no contents are
 * kept between calls, so one workspace can serve every layer's cache in turn
 * on one stream; calls that overlap in time need workspaces of their own).
 * DMS_ERR_CAPACITY for a missing or short workspace, before any launch.
 */
int dms_decode_attn(dms_cache* cache, const int32_t* seq_ids, const void* q, void* out, int B,
                    void* workspace, size_t ws_bytes, void* stream);

/*
 * dms_decode_attn for callers that cannot allocate device memory (code under
 * HIP graph capture, serving loops and harnesses that must not call hipMalloc
 * or bring a workspace): the same kernels and results, with the partial
 * records in a static 8 MiB array held by each GPU for the life of the
 * process, instead of a caller workspace.  Calls no allocating routine.
 * Arguments as in dms_decode_attn; the cache's device must be current.
 * DMS_ERR_CAPACITY (before any launch) when the call needs more than 8 MiB of
 * records (dms_decode_workspace_bytes(cfg, B) > 8 MiB: with head_dim 128 at
 * the default 512 workgroups, 4 query heads per KV head fit every call of up
 * to 2048 (row, KV head) units, 8 query heads up to about 990).  All calls on
 * one GPU share the array: calls that overlap in time on one GPU (other
 * streams, other threads) race and must not be issued.
 */
int dms_decode_attn_noalloc(dms_cache* cache, const int32_t* seq_ids, const void* q, void* out, int B,
                            void* stream);

/*
 * A layer's whole decode step in one call: the decision and append of
 * dms_decode_prepare and the attention of dms_decode_attn for one token per
 * row (walkthrough, 推理模式, and the FastDMS post's fused decode path).
 * Results equal those of the two calls in turn, up to the order of the
 * floating-point sums in the attention.
 * Arguments as in dms_decode_prepare; q_inout [B][Hq][D] is also the query of
 * the attention (QNEURON: its decision neuron is zeroed in place and plays no
 * part); out [B][Hq][D] act dtype.
 * bf16 or fp8 pages (fast decode shapes, 16-byte aligned q_inout, k, v, out
 * and, LINEAR, hidden, rms_gamma, W with hidden a multiple of 8) run as one
 * launch when all of its workgroups (B * Hkv that prepare a (row, KV head)
 * pair, plus the attention's) can be resident at once: the attention takes
 * the current token from k/v (fp8: quantised with the scale its page has or
 * gets, as the append stores it) and masks the slot it overwrites; the last
 * preparing workgroup commits the append once every attention workgroup has
 * read the shared tables, and leaves the next step of the same rows a plan
 * of its attention split (kept in the cache; any other call that changes
 * the cache drops it).  Other configurations and larger steps call
 * dms_decode_prepare, then dms_decode_attn (the environment variable
 * DMS_DECODE_STEP_FUSE, read at cache creation, forces one (1) or two (0)
 * launches; DMS_DECODE_STEP_ROWS=1, read at every call, prepares one batch
 * row per workgroup instead of one pair).  workspace / ws_bytes as in
 * dms_decode_attn.  Device-side
 * errors as in dms_append_evict, and DMS_DEV_STEP_SYNC if the commit's
 * bounded wait for the attention workgroups ran out (only when far more
 * workgroups than the GPU holds at once queue behind it; the environment
 * variable DMS_STEP_SPIN_LIMIT, read at every call, sets the bound in polls,
 * 0 giving up at once).
 */
int dms_decode_step(dms_cache* cache, const int32_t* seq_ids, const void* hidden, const float* rms_gamma,
                    const float* W, const float* bias, const float* offsets, void* q_inout, const void* k,
                    const void* v, void* out, int B, float* logits_out, uint8_t* evict_out, void* workspace,
                    size_t ws_bytes, void* stream);

/*
 * The decode step of every layer of a model in one launch (the FastDMS post's
 * subsystem table, Decode kernel row: keep/evict, the retention window and
 * the compact append at every decode step, here for all layers at once).
 *
 * dms_step_layers_create binds n_layers (1..512) distinct caches of one shape
 * (head counts, head_dim, window, block size, kv dtype, decision source,
 * max_batch and device) and, per layer, the device buffers of its step,
 * io[l], with the meaning, layout and dtype of the same-named arguments of
 * dms_decode_step.  The pointers are copied: the buffers must stay valid, and
 * each call reads and writes them (the serving-loop pattern of static
 * per-layer buffers).  Allocates a small device buffer (the per-layer
 * arguments and a barrier counter) on the caches' device, which must be
 * current.  *out receives the binding.  DMS_ERR_ARG for NULL, duplicate or
 * mismatched caches and missing buffers.
 *
 * dms_step_layers_run runs one decode step of rows seq_ids[0..B) through
 * layers 0, 1, ..., n_layers - 1 in order; results equal n_layers
 * dms_decode_step calls in that order, up to the order of the attention's
 * floating-point sums.  When the one-launch step applies (as in
 * dms_decode_step: fast decode shapes, 16-byte aligned buffers) and all of a
 * layer's workgroups can be resident at once, it is one launch: each layer's
 * step as in dms_decode_step, and a grid-wide barrier after each layer's
 * attention, so that no workgroup starts layer l + 1 before every output of
 * layer l is written (a model computes layer l + 1's inputs from them).
 * Otherwise it makes the n_layers dms_decode_step calls.  workspace / ws_bytes
 * as in dms_decode_attn (one workspace serves all layers).  Calls on one
 * binding are ordered by their stream and must not overlap.  Device-side
 * errors as in dms_decode_step (per layer's cache); DMS_DEV_STEP_SYNC also
 * when the barrier's bounded wait ran out (DMS_STEP_SPIN_LIMIT as there).
 *
 * dms_step_layers_one_launch tells (*one_launch = 1) whether a run of B rows
 * is one launch.  dms_step_layers_destroy frees a binding (NULL is a no-op).
 */
typedef struct dms_step_layers dms_step_layers;
typedef struct dms_layer_io {
  const void* hidden;      /* [B][hidden] act dtype (LINEAR), else NULL */
  const float* rms_gamma;  /* [hidden] (LINEAR) */
  const float* W;          /* [Hkv][hidden] (LINEAR) */
  const float* bias;       /* [Hkv] or NULL */
  const float* offsets;    /* decision offsets, as in dms_decode_prepare */
  void* q_inout;           /* [B][Hq][D] act dtype */
  const void* k;           /* [B][Hkv][D] act dtype */
  const void* v;           /* [B][Hkv][D] act dtype */
  void* out;               /* [B][Hq][D] act dtype */
  float* logits_out;       /* [B][Hkv] or NULL */
  uint8_t* evict_out;      /* [B][Hkv] */
} dms_layer_io;
int dms_step_layers_create(dms_cache* const* caches, const dms_layer_io* io, int n_layers, dms_step_layers** out);
int dms_step_layers_run(dms_step_layers* layers, const int32_t* seq_ids, int B, void* workspace, size_t ws_bytes,
                        void* stream);
int dms_step_layers_one_launch(const dms_step_layers* layers, int B, int32_t* one_launch);
int dms_step_layers_destroy(dms_step_layers* layers);

/* ---- training mode (walkthrough, Gumbel 噪声与可微门控 and 注意力 / 训练模式) ---- */

/*
 * Forward of the training-time gating: y = (logits + noise) / tau,
 * probs = sigmoid(y), hard = 1 where probs > 1/2 (taken as y > 0), else 0
 * (the forward value of the straight-through decision).  The noise (the
 * Gumbel / logistic sample the trainer draws) is an input; NULL means none.
 * All arrays are n device floats; any output may be NULL.  tau > 0.
 */
int dms_train_gate(const float* logits, const float* noise, float tau, int64_t n, float* y_out,
                   float* probs_out, float* hard_out, void* stream);

/*
 * Backward of dms_train_gate (walkthrough, Gumbel 噪声与可微门控): the gradient
 * to the decision logits given the loss's gradients with respect to y (dy,
 * e.g. dms_train_attn_bwd's), to the straight-through decision (dhard: its
 * forward value is the hard threshold, its gradient that of probs) and to
 * probs (dprobs):
 *   dlogits = (dy + (dhard + dprobs) * probs * (1 - probs)) / tau,
 * probs = sigmoid((logits + noise) / tau) recomputed from the same logits,
 * noise and tau as the forward.  All arrays are n device floats; dy, dhard,
 * dprobs and noise may be NULL (zero); logits and dlogits_out are required.
 */
int dms_train_gate_bwd(const float* logits, const float* noise, float tau, int64_t n, const float* dy,
                       const float* dhard, const float* dprobs, float* dlogits_out, void* stream);

/*
 * Forward of the training-mode attention (walkthrough, 训练模式): causal
 * attention over the whole sequence in which key j keeps its score for
 * queries closer than `window` and gets logsigmoid(-y[j]) added for queries
 * at distance window or more (y = the key's gate logit, e.g. dms_train_gate's
 * y_out; a re-indexing such as the pages' shift by one is the caller's).
 * Non-causal keys get no weight (the pages' -50000 mask value).
 *   q [B][T][Hq][D], k, v [B][T][Hkv][D] bf16 (16-byte aligned);
 *   gate_logits [B][Hkv][T] f32; out [B][T][Hq][D] bf16;
 *   lse [B][Hq][T] f32: natural log of the softmax normaliser per query
 *   (what a backward pass needs).
 * Query head h uses KV head h / (Hq / Hkv).  head_dim 64 or 128, Hq / Hkv in
 * {1, 2, 4}; softmax_scale <= 0 means 1 / sqrt(head_dim).  Needs no cache.
 */
int dms_train_attn_fwd(int B, int T, int num_q_heads, int num_kv_heads, int head_dim, int window,
                       float softmax_scale, const void* q, const void* k, const void* v,
                       const float* gate_logits, void* out, float* lse, void* stream);

/*
 * Prefill attention for one chunk of C new tokens per sequence (walkthrough,
 * 高级选项 Chunked Prefill, and the exact prefill with the eviction mask),
 * computed against the cache state *before* the chunk is appended.  Query i
 * (position pos+i) sees cached slot s iff its token is kept or i - pos_s < w,
 * and chunk key j iff j <= i and (evict[j] == 0 or i - j < w).
 * q [B][C][Hq][D], k/v [B][C][Hkv][D], out [B][C][Hq][D] act dtype;
 * evict [B][Hkv][C] u8.  C <= max_chunk.
 */
int dms_prefill_attn(dms_cache* cache, const int32_t* seq_ids, const void* q, const void* k,
                     const void* v, const uint8_t* evict, void* out, int B, int C, void* stream);

/*
 * Empties the listed sequences (walkthrough, 当前限制: the cache is reset
 * between independent sequences).  Pages return to the pool in reverse
 * page-table order, sequences and heads in reverse order, so the next pops
 * return them in their original order.  seq_ids [n] device array, or NULL to
 * reset sequences 0..n-1.
 */
int dms_seq_reset(dms_cache* cache, const int32_t* seq_ids, int n, void* stream);

/* Synchronises `stream` and returns the sticky device status bits in *device_status. */
int dms_cache_status(dms_cache* cache, void* stream, int32_t* device_status);

/* Clears the sticky device status word and resets the one-launch decode
 * step's arrival counters (asynchronous). */
int dms_cache_clear_status(dms_cache* cache, void* stream);

/* Synchronises `stream` and copies the tables into host buffers. */
int dms_cache_dump(dms_cache* cache, void* stream, const dms_dump* out);

/* Debug check of the cache's structural invariants (walkthrough, 推理模式:
 * the delayed-eviction slot rule that keeps the live slots equal to the keys
 * the last query may see; the shared page pool).  Synchronises `stream`,
 * copies the tables to the host and checks there: per (sequence, head),
 * min(position, window) <= L <= position; live slots 0..L-1 each hold one
 * distinct token, kept or inside the window of the last position; the
 * window entries of the last `window` positions name the slots holding
 * those tokens (slot, evict flag and page row); the current page is the page
 * of slot L - 1; page ids lie in the pool, each page is held by one head or
 * free, and held + free = pool.  *violations gets a bit mask (0 =
 * consistent): 0x1 length, 0x2 page id, 0x4 page ownership, 0x8 slot
 * occupants, 0x10 window entries, 0x20 current page, 0x40 free stack;
 * *first_unit (may be NULL) the first sequence * Hkv + head found wrong, or
 * -1.  Returns DMS_ERR_ARG for NULL cache or violations. */
int dms_cache_check(dms_cache* cache, void* stream, uint32_t* violations, int32_t* first_unit);

/* Synchronises `stream` and summarises occupancy (walkthrough, 损失函数与压缩比调度:
 * realised compression; here tokens / live slots). */
int dms_cache_stats(dms_cache* cache, void* stream, dms_stats* out);

/*
 * Backward of dms_train_attn_fwd (walkthrough, 训练模式): given the forward's
 * inputs, its output `out` and log-sum-exp `lse`, and the output gradient
 * `dout`, writes
 *   dq [B][T][Hq][D], dk, dv [B][T][Hkv][D]   float32 (dk, dv summed over the
 *                                               query heads of each KV head)
 *   dgate [B][Hkv][T] float32: the gradient of the gate logits y, through
 *                      the penalty logsigmoid(-y) of the scores at distance
 *                      >= window: -sigmoid(y_j) * sum of those scores' gradients.
 * q, k, v, out, dout bf16 in the forward's layouts (16-byte aligned);
 * gate_logits [B][Hkv][T] and lse [B][Hq][T] float32 as given to / returned
 * by the forward.  workspace: device memory of at least
 * dms_train_attn_bwd_workspace_bytes bytes (overwritten).  head_dim 64 or
 * 128, Hq / Hkv in {1, 2, 4}; softmax_scale <= 0 means 1 / sqrt(head_dim).
 * DMS_ERR_ARG for NULL tensors or bad sizes, DMS_ERR_CAPACITY for a short
 * workspace.  Needs no cache.
 */
int dms_train_attn_bwd(int B, int T, int num_q_heads, int num_kv_heads, int head_dim, int window,
                       float softmax_scale, const void* q, const void* k, const void* v, const void* out,
                       const void* dout, const float* gate_logits, const float* lse, void* dq, void* dk,
                       void* dv, float* dgate, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of dms_train_attn_bwd (two floats per query row and head: the
 * rows' rowsum(dO * O), then the keys' penalties). */
int dms_train_attn_bwd_workspace_bytes(int B, int T, int num_q_heads, size_t* bytes);

/* ---- KVzap scorers ("动态内存稀疏化（DMS）策略：KVzap-linear-Llama-3.1-8B-Instruct的核心创新点",
 * KVzap-linear的技术架构; "革命性LLM加速技术：NVIDIA KVzap-mlp-Qwen3-8B如何实现高效KV缓存修剪？",
 * 模型架构 and 工作流程) ---- */

/* Scores every token's KV pairs from the layer's hidden state and applies the
 * pruning threshold, for B x T tokens:
 *   linear (Hm == 0):  s[b][k][t] = W1[k] . h[b][t] + b1[k]
 *   MLP    (Hm >  0):  s[b][k][t] = W2[k] . gelu(W1 . h[b][t] + b1) + b2[k]   (exact erf GELU)
 *   evict[b][k][t] = s[b][k][t] < threshold   (the pages' default threshold is -4)
 * The decisions feed dms_append_evict / dms_prefill_attn of a cache whose
 * window is the pages' 128 tokens: a token with a score below the threshold
 * leaves the cache once it is 128 positions old, the others stay.
 *   hidden     device [B][T][H], float32 (act_dtype DMS_F32) or bfloat16 (DMS_BF16), 16-byte aligned
 *   W1         device float32, linear [Hkv][H], MLP [Hm][H], 16-byte aligned
 *   b1         device float32, linear [Hkv], MLP [Hm], or NULL (no bias)
 *   W2, b2     device float32 [Hkv][Hm], [Hkv] (b2 may be NULL); MLP only, ignored for linear
 *   scores_out device float32 [B][Hkv][T], or NULL
 *   evict_out  device uint8 [B][Hkv][T]
 *   workspace  MLP only: device memory of at least dms_kvzap_workspace_bytes(B, T, Hkv, Hm)
 *              bytes, owned by the caller, overwritten (the inner-unit workgroups' shares of
 *              the second layer, added in a fixed order: scores are deterministic); ignored
 *              (may be NULL) for linear
 * Limits: H a multiple of 32, 1 <= Hkv <= 16, Hm a multiple of 64
 * (DMS_ERR_UNSUPPORTED otherwise).  Asynchronous on `stream`; needs no cache.
 * DMS_ERR_ARG for NULL required pointers, negative sizes or a non-finite
 * threshold; DMS_ERR_CAPACITY for a missing or short MLP workspace. */
int dms_kvzap_score(int B, int T, int H, int Hkv, int Hm, int act_dtype, const void* hidden, const float* W1,
                    const float* b1, const float* W2, const float* b2, float threshold, float* scores_out,
                    uint8_t* evict_out, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes dms_kvzap_score needs for B x T tokens (0 for Hm == 0). */
int dms_kvzap_workspace_bytes(int B, int T, int Hkv, int Hm, size_t* bytes);

/* ---- serving accounting (FastDMS post, subsystem table: the scheduler admits
 * requests by compact KV capacity, continuous batching accounts surviving
 * tokens rather than logical length; walkthrough, 当前限制: interleaved
 * prefill / generate turns on one sequence need no reset here) ---- */

typedef struct dms_seq_info {
  int32_t position;         /* tokens appended so far (logical length) */
  int32_t live_slots;       /* surviving tokens: sum over KV heads of live slots */
  int32_t max_head_slots;   /* largest per-head length */
  int32_t pages;            /* pool pages the sequence holds */
} dms_seq_info;

/* Synchronises `stream`; per listed sequence (seq_ids host array of n ids, or
 * NULL for 0..n-1) fills out[i] (host).  DMS_ERR_ARG for an id outside
 * [0, max_batch). */
int dms_seq_info_get(dms_cache* cache, const int32_t* seq_ids, int n, void* stream, dms_seq_info* out);

/* Synchronises `stream`; the most pool pages that appending n_new[i] more
 * tokens to sequence seq_ids[i] can take, whatever the new tokens' decisions:
 * every new token is taken as kept, except that the first w of them
 * overwrite in place the slots of already-marked tokens in the window
 * (walkthrough, 推理模式).  pages_out[i] = -1 when the sequence would pass
 * max_tokens_per_seq.  *free_pages (may be NULL) = pages left in the pool.
 * Host arrays; admit when the sum of pages_out fits in *free_pages. */
int dms_pages_needed(dms_cache* cache, const int32_t* seq_ids, const int32_t* n_new, int n, void* stream,
                     int64_t* pages_out, int64_t* free_pages);

/* Last error message of this thread ("" if none). */
const char* dms_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DMS_H */
