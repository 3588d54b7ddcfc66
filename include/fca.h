/*
 * fca.h -- Forest Cascade Attention decode on gfx950 (MI355X), C ABI.
 *
 * Batched single-token decode attention over a paged bf16 KV cache, split the
 * way the ZoRRo Inference & Forest Cascade Attention page describes it
 * ("Overview" and "Core Mechanism"):
 *
 *   1. discover the groups of requests whose block tables share a prefix of
 *      physical block IDs (fca_plan_create);
 *   2. read each shared prefix block once per group in a grouped pass,
 *   3. read each request's own suffix blocks in a per-request pass, and
 *   4. combine the partial results exactly by log-sum-exp weighting
 *      (fca_decode runs 2-4).
 *
 * The result equals standard per-request softmax attention (the page states
 * the method is mathematically equivalent to it), up to floating-point
 * rounding: bf16 inputs, fp32 accumulation, bf16 output.
 *
 * Conventions for every entry point:
 *   - Pointers named *_dev are device pointers; everything else is host.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *   - The caller owns every buffer it passes in.  The library never frees
 *     caller memory and never keeps a pointer to it past the call, except
 *     the plan workspace, which must outlive the plan.
 *   - Nothing throws or aborts across this boundary.  Every call returns an
 *     fca_status; on failure fca_last_error() gives a message (per thread).
 */
#ifndef FCA_H_
#define FCA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fca_status {
  FCA_OK = 0,
  FCA_ERR_INVALID_ARG = 1, /* null pointer, negative size, inconsistent shape */
  FCA_ERR_UNSUPPORTED = 2, /* head dims / block size / ratio not built */
  FCA_ERR_WORKSPACE = 3,   /* workspace too small or misaligned */
  FCA_ERR_BAD_TABLE = 4,   /* found on the device: block ID outside the pool
                              in a used slot, or seq_len outside
                              [0, max_blocks * block_size] */
  FCA_ERR_HIP = 5,         /* a HIP runtime call failed */
  FCA_ERR_HOST_ALLOC = 6   /* host memory for the plan could not be had */
} fca_status;

/* fca_attn_desc.flags */
#define FCA_PLAN_DISABLE_CASCADE 1u /* no groups: every request is read whole
                                       by the per-request pass (the
                                       non-cascade paged-decode baseline) */
#define FCA_PLAN_SEPARATE_PASSES 2u /* launch the grouped pass and the
                                       per-request pass one after the other
                                       (for per-pass timing).  By default one
                                       launch of persistent workgroups runs
                                       the work items of both passes (GQA);
                                       latent caches always use two. */
#define FCA_PLAN_AUTO_FOLD 8u       /* activation heuristic (GQA caches),
                                       on by default (this bit is accepted
                                       and changes nothing): a group whose
                                       shared blocks would save fewer bytes
                                       than its partial rows cost to write
                                       and merge is read per request instead
                                       (folded into its members' suffixes);
                                       groups are folded from the leaves up.
                                       When every group folds, the plan is
                                       the non-cascade one (the cascade is
                                       bypassed).  Latent caches keep every
                                       group (their passes are bound by the
                                       matrix products, which a fold leaves
                                       unchanged). */
#define FCA_PLAN_KEEP_GROUPS 16u    /* no activation heuristic: every
                                       discovered group is read once for all
                                       its members */
#define FCA_PLAN_OUT_F32 4u         /* fca_decode writes `out` as float32
                                       (an attention state that
                                       fca_merge_states can combine without
                                       a bf16 rounding in between) */

/*
 * Shape and cache layout of one attention layer.
 *
 * Cache layout (bf16, elements, d = head-dim index, t = slot in the block).
 * Two layouts are read; k_stride_token chooses:
 *
 *   tiles (k_stride_token = v_stride_token = 0):
 *     key  (blk, h, t, d) at k_cache[blk*k_stride_block + h*k_stride_head
 *                                    + (d/8)*(block_size*8) + t*8 + d%8]
 *     value(blk, h, t, d) at v_cache[blk*v_stride_block + h*v_stride_head
 *                                    + d*block_size + t]
 *     i.e. inside one (block, head) tile keys are stored in 16-byte chunks
 *     of 8 head dims, chunk-major, and values transposed (one row of
 *     block_size tokens per value dim).  A tile must not straddle strides
 *     (k_stride_head >= head_dim_qk*block_size, and so on).
 *
 *   token rows (k_stride_token > 0): each (block, head, slot) holds one row
 *   of head dims with unit stride,
 *     key  (blk, h, t, d) at k_cache[blk*k_stride_block + h*k_stride_head
 *                                    + t*k_stride_token + d]
 *     value(blk, h, t, d) at v_cache[blk*v_stride_block + h*v_stride_head
 *                                    + t*v_stride_token + d]
 *     e.g. [num_blocks][block_size][num_kv_heads][head_dim] (token stride
 *     num_kv_heads*head_dim, head stride head_dim) or
 *     [num_blocks][num_kv_heads][block_size][head_dim] (token stride
 *     head_dim, head stride block_size*head_dim).  Both token strides are
 *     set (GQA), and every stride is at least the row width (GQA: token,
 *     head and block strides >= 128; latent: token stride in
 *     [576, 2^20], block stride >= 576, head stride >= 0); the caller keeps
 *     rows of different (block, head, slot) from overlapping.  All
 *     block_size rows of a referenced block are read, also past a
 *     request's length.  The kernels gather the rows into the tile
 *     arrangement on the way into LDS; fca_kv_append writes rows.
 *
 * With v_aliases_k = 1 (latent caches) the values are the first head_dim_v
 * key dims of the same tile or row, and v_cache, v_stride_* are ignored.
 * Strides are in elements and must be multiples of 8 (every tile and every
 * row starts on a 16-byte boundary, as must the pools).
 *
 * Supported (others return FCA_ERR_UNSUPPORTED):
 *   - GQA:  head_dim_qk = head_dim_v = 128, block_size = 16,
 *           num_q_heads / num_kv_heads in [1, 16], v_aliases_k = 0.
 *   - MLA:  head_dim_qk = 576, head_dim_v = 512, block_size = 64,
 *           num_kv_heads = 1, v_aliases_k = 1.  The value products run in
 *           fp16 (probabilities to 11 bits), so the value columns (the first
 *           512 dims) must stay below 65504 in magnitude; larger values are
 *           not representable there and give wrong results.
 *
 * Query head h reads KV head h / (num_q_heads / num_kv_heads).
 * `scale` multiplies q.k before the softmax.
 */
typedef struct fca_attn_desc {
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim_qk;
  int32_t head_dim_v;
  int32_t block_size;
  int32_t num_blocks; /* pool size: valid block IDs are [0, num_blocks) */
  int64_t k_stride_block;
  int64_t k_stride_head;
  int64_t v_stride_block;
  int64_t v_stride_head;
  int64_t k_stride_token; /* 0: tile layout; > 0: token rows (see above) */
  int64_t v_stride_token; /* 0 with k_stride_token = 0; ignored when v_aliases_k */
  int32_t v_aliases_k;
  float scale;
  uint32_t flags; /* FCA_PLAN_* */
  int32_t reserved; /* must be 0 */
} fca_attn_desc;

typedef struct fca_plan_s* fca_plan; /* opaque, host-side */

/* Counts of a built plan. */
typedef struct fca_plan_info {
  int32_t batch;
  int32_t num_groups;        /* groups found by discovery */
  int32_t max_depth;         /* deepest group depth (roots are 0), -1 if none */
  int32_t num_grouped_items; /* work items of the grouped pass */
  int32_t num_suffix_items;  /* work items of the per-request pass */
  int32_t num_merge_sources; /* partial triples the merge reads, summed over
                                (request, query head) */
  int64_t num_partial_rows;  /* (o, m, l) rows written per decode */
  int64_t logical_tokens;    /* sum of seq_lens */
  int64_t unique_tokens;     /* group ranges once + every suffix */
  size_t decode_workspace_bytes; /* bytes fca_decode needs */
  int32_t num_folded_groups; /* groups read per request (FCA_PLAN_AUTO_FOLD) */
} fca_plan_info;

/*
 * Bytes of device workspace fca_plan_create needs for a batch of `batch`
 * requests with block tables `max_blocks` wide.  Depends only on the
 * arguments.  Returns FCA_ERR_INVALID_ARG / FCA_ERR_UNSUPPORTED for a bad
 * descriptor or sizes (batch in [0, 8192], max_blocks in [1, 2^20]).
 */
fca_status fca_plan_workspace_size(int32_t batch, int32_t max_blocks, const fca_attn_desc* desc,
                                   size_t* bytes);

/*
 * Discover the prefix forest of a batch and build the decode schedule
 * (the "discovers groups of requests sharing a KV-cache prefix" step of
 * "Core Mechanism").
 *
 *   block_tables_dev  int32 [batch, >= max_blocks], row stride bt_row_stride
 *                     (elements).  Row i maps request i's logical block j to
 *                     a physical block; only j < ceil(seq_lens[i]/block_size)
 *                     is read, the rest may hold anything.
 *   seq_lens_dev      int32 [batch]: cached tokens of each request, the
 *                     decode token's own key/value included.
 *   workspace_dev     >= fca_plan_workspace_size bytes, 256-byte aligned;
 *                     owned by the caller, must outlive the plan.
 *
 * Enqueues the discovery kernels on `stream`, then waits once for a small
 * read-back (group records, counts and the device error flag), then enqueues
 * the upload of the schedule (one copy and one small kernel) on `stream`:
 * decodes on another stream must be ordered after this point of `stream`.
 * The plan copies the tables and lengths it needs into the workspace: the
 * caller may change or free block_tables_dev / seq_lens_dev once this
 * returns.  `stream` must outlive the plan (fca_plan_destroy records an
 * event on it).  batch == 0 gives a valid, empty plan.  *out is set only on
 * FCA_OK.
 */
fca_status fca_plan_create(const int32_t* block_tables_dev, int64_t bt_row_stride, const int32_t* seq_lens_dev,
                           int32_t batch, int32_t max_blocks, const fca_attn_desc* desc, void* workspace_dev,
                           size_t workspace_bytes, void* stream, fca_plan* out);

fca_status fca_plan_get_info(fca_plan plan, fca_plan_info* info);

/*
 * Decode attention for the planned batch (grouped pass, per-request pass,
 * exact log-sum-exp merge; "Core Mechanism", steps 2-3).
 *
 *   q_dev        bf16 [batch, num_q_heads, head_dim_qk], contiguous.
 *   k_cache_dev  bf16 pool, layout above.  v_cache_dev likewise (ignored
 *                when v_aliases_k).
 *   out_dev      bf16 [batch, num_q_heads, head_dim_v], contiguous (float32
 *                with FCA_PLAN_OUT_F32); row i is request i.  A request with
 *                seq_len 0 gets zeros.
 *   lse_dev      float [batch, num_q_heads] natural-log sum of exp(scores),
 *                or NULL.  -inf for seq_len 0.
 *   workspace_dev >= info.decode_workspace_bytes, 256-byte aligned: holds the
 *                partial (o, max, denominator) triples of this call.
 *
 * Asynchronous on `stream`: no host synchronisation and no allocation.
 * Calls that share a decode workspace must not overlap.  Calls on one plan
 * may target different streams if each has its own decode workspace; with
 * profiling enabled they must come from one host thread at a time.
 */
fca_status fca_decode(fca_plan plan, const void* q_dev, const void* k_cache_dev, const void* v_cache_dev,
                      void* out_dev, float* lse_dev, void* workspace_dev, size_t workspace_bytes, void* stream);

/*
 * fca_decode without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the partial (o, max, denominator) rows go to a
 * scratch array that the library keeps in each device's memory (64 MiB per
 * device, for the life of the process).  Same arguments, layout, results and
 * launches as fca_decode, bit for bit.  The call allocates nothing (no
 * hipMalloc, no host allocation of device memory) and does not record
 * profiling events; its first call on a device looks up that device's
 * scratch address once.
 *
 * Every call on one device shares that device's scratch and leaves its rows
 * there: calls that may overlap on one device (other streams, other host
 * threads) race and must be ordered by the caller.  The plan must have been
 * made on the current device (FCA_ERR_INVALID_ARG otherwise).  A plan whose
 * info.decode_workspace_bytes exceeds 64 MiB is rejected with
 * FCA_ERR_WORKSPACE before anything is launched.
 */
fca_status fca_decode_no_alloc(fca_plan plan, const void* q_dev, const void* k_cache_dev, const void* v_cache_dev,
                               void* out_dev, float* lse_dev, void* stream);

/*
 * The decode of several layers that share one batch and so one plan (the
 * plan is made once for each decode batch and serves every layer: "Core
 * Mechanism").  Layer l reads q_dev[l], k_caches_dev[l], v_caches_dev[l] and
 * writes out_dev[l], lse_dev[l], each as for fca_decode; the arrays are host
 * arrays of n_layers device pointers (v_caches_dev may be NULL when
 * v_aliases_k; lse_dev may be NULL, or hold NULL entries).  The layers run in
 * order on `stream` and share one decode workspace (>=
 * info.decode_workspace_bytes), which is safe because each layer's launches
 * are queued after the previous layer's.  Every layer's arguments are checked
 * before anything is launched; an error names the layer.  Asynchronous, no
 * allocation on the device, no host synchronisation; it can be captured in a
 * HIP graph.  Profiling (fca_profile_enable) does not record these launches.
 */
fca_status fca_decode_layers(fca_plan plan, int32_t n_layers, const void* const* q_dev, const void* const* k_caches_dev,
                             const void* const* v_caches_dev, void* const* out_dev, float* const* lse_dev,
                             void* workspace_dev, size_t workspace_bytes, void* stream);

/* One discovered group, canonical order: sorted by (smallest member, depth). */
typedef struct fca_group_record {
  int32_t depth;        /* number of groups strictly above; roots are 0 */
  int32_t parent;       /* canonical index of the nearest group above, or -1 */
  int32_t block_begin;  /* logical block range [block_begin, block_end) */
  int32_t block_end;
  int32_t member_begin; /* offset of its ascending member list in `members` */
  int32_t member_count;
} fca_group_record;

/*
 * Canonical form of the plan's grouping, for tests and tools (host copies):
 *   groups   [num_groups]
 *   members  [sum of member_count]  request indices
 *   requests [batch * 3]  per request: suffix_block_begin, suffix_tokens,
 *                         deepest group (canonical index) or -1, as read by
 *                         the per-request pass (with FCA_PLAN_AUTO_FOLD a
 *                         folded group's range belongs to its members'
 *                         suffixes and the deepest group is the nearest
 *                         one kept)
 * Any pointer may be NULL to skip that part.
 */
fca_status fca_plan_export(fca_plan plan, fca_group_record* groups, int32_t* members, int32_t* requests);

/* folded [num_groups]: 1 for a group read per request (FCA_PLAN_AUTO_FOLD),
 * else 0, in canonical order (host copy). */
fca_status fca_plan_export_folded(fca_plan plan, int32_t* folded);

/* One unit of work of the grouped or per-request pass (host copy). */
typedef struct fca_work_item {
  int32_t request;    /* block-table row the item's block IDs come from */
  int32_t tok_begin;  /* logical token range [tok_begin, tok_end) */
  int32_t tok_end;
  int32_t kv_head;
  int32_t member_off; /* grouped: offset of the group's range in the
                         depth-first member order; -1: suffix item */
  int32_t ncols;      /* query rows of the unit: members * (Hq/Hkv) */
  int32_t col0;       /* query rows [col0, col1) of the unit */
  int32_t col1;
  int32_t part_base;  /* partial row of (kv_head, col0) of the item; head h,
                         row n is part_base + (h - kv_head)*(col1 - col0)
                         + (n - col0) */
  int32_t kv_heads;   /* the item covers KV heads kv_head .. kv_head+kv_heads-1 */
  int32_t stripes;    /* block stripes S: stripe t takes blocks t, t+S, ... of
                         the range and writes rows part_base + t*kv_heads*
                         (col1 - col0) + (as above) */
  int32_t flags;      /* bit 0: every tile of the item has exactly one reader
                         (a suffix of a cascade plan, or a group whose query
                         rows fit one wave), so the GQA kernel loads it with
                         the non-temporal cache policy */
} fca_work_item;

/*
 * The decode schedule, for tests and tools (host copies):
 *   grouped [num_grouped_items], suffix [num_suffix_items]
 *   src_off [batch * num_q_heads + 1], src [num_merge_sources]
 * Query head h of request i merges the partial rows
 *   src[s], s in [src_off[i * num_q_heads + h], src_off[i * num_q_heads + h + 1]).
 * src_off and src are copied from the tables the merge reads, which the
 * plan builds on the device: asking for them waits for the plan's stream.
 * num_merge_sources equals num_partial_rows (every row is read by exactly
 * one (request, head)).
 */
fca_status fca_plan_export_schedule(fca_plan plan, fca_work_item* grouped, fca_work_item* suffix,
                                    int32_t* src_off, int32_t* src);

/* Summed GPU time of the launches of profiled fca_decode calls. */
typedef struct fca_profile {
  double attention_ms; /* all attention launches (grouped and per-request passes) */
  double grouped_ms;   /* the launch of the grouped pass alone, when the plan
                          launches the passes separately (else 0) */
  double suffix_ms;    /* the launch of the per-request pass alone, likewise */
  double merge_ms;     /* log-sum-exp merge */
  double decode_ms;    /* whole call, first launch to last */
  int64_t calls;
} fca_profile;

/*
 * Measurement hook.  While enabled, every fca_decode on this plan records HIP
 * events on its stream before and after each launch.  fca_profile_read waits
 * for the recorded events, returns the sums since the previous read and
 * resets them.  Events are created on first use and freed with the plan.
 * Not thread-safe; meant for benchmarks and profilers, not serving loops.
 */
fca_status fca_profile_enable(fca_plan plan, int32_t enable);
fca_status fca_profile_read(fca_plan plan, fca_profile* out);

/*
 * Measurement hook: average GPU time of each launch of a decode, free of the
 * per-launch event overhead of fca_profile_enable.  Each launch kind of the
 * plan (the attention launch, or the grouped then the per-request launch,
 * then the merge) is issued repeats * n_caches times back to back between two
 * HIP events on `stream`, cycling over the caches (so that one cache does not
 * stay in the last-level cache between launches).
 *
 *   k_caches, v_caches  host arrays of n_caches device pointers, layout as for
 *                       fca_decode (v_caches ignored, may be NULL, when
 *                       v_aliases_k).
 *   q_dev, out_dev, lse_dev, workspace_dev  as for fca_decode; out / lse end
 *                       up holding the decode of the last cache.
 *   result              per-launch averages in ms (attention_ms sums the
 *                       plan's attention launches; grouped_ms / suffix_ms are
 *                       set when the plan launches the passes separately, as
 *                       on latent caches;
 *                       decode_ms = attention_ms + merge_ms); calls =
 *                       repeats * n_caches.
 *
 * Blocks the host until the launches finish.  FCA_ERR_INVALID_ARG for NULL
 * arguments or n_caches / repeats < 1, FCA_ERR_WORKSPACE as fca_decode,
 * FCA_ERR_HIP if a launch or event call fails.
 */
fca_status fca_time_launches(fca_plan plan, const void* q_dev, const void* const* k_caches,
                             const void* const* v_caches, int32_t n_caches, int32_t repeats, void* out_dev,
                             float* lse_dev, void* workspace_dev, size_t workspace_bytes, void* stream,
                             fca_profile* result);

/*
 * Measurement hook: the HBM read rate of a plain streaming kernel on this
 * device, the practical ceiling next to the published peak.  Each of the
 * n_bufs buffers (device, 16-byte aligned, `bytes` each, a positive multiple
 * of 16; bytes well above the 256 MB last-level cache) is read once untimed,
 * then repeats * n_bufs reads cycling over the buffers run back to back
 * between two HIP events on `stream`, for each of two launch shapes of the
 * kernel; *gbps = bytes read / elapsed time of the faster shape (1e9 bytes
 * per second).  Nothing is written.  Blocks the host until the
 * reads finish.  FCA_ERR_INVALID_ARG for NULL or misaligned pointers or bad
 * sizes, FCA_ERR_HIP if a launch or event call fails.
 */
fca_status fca_measure_read_bandwidth(const void* const* bufs_dev, int32_t n_bufs, size_t bytes, int32_t repeats,
                                      void* stream, double* gbps);

/* Operand types of fca_measure_mfma_rate. */
#define FCA_MFMA_BF16 0
#define FCA_MFMA_F16 1

/*
 * Measurement hook: the matrix-core rate a plain loop of independent dense
 * products reaches on this device, the practical ceiling next to the
 * published dense peak (2.5 PFLOP/s bf16 and fp16 on MI355X) that the
 * latent-cache kernels' roofline fractions are quoted against.  One
 * workgroup of 8 waves per compute unit; each wave issues iters x 32
 * v_mfma_f32_16x16x32 products (dtype FCA_MFMA_BF16 or FCA_MFMA_F16) into
 * 32 independent accumulators, the operand shape of the value products.
 * One untimed launch, then one timed between two HIP events on `stream`;
 * *tflops = 2 x 16 x 16 x 32 flops per product / elapsed time (1e12 per
 * second).  Nothing is read or written in device memory.  Blocks the host
 * until the launch ends.  FCA_ERR_INVALID_ARG for NULL tflops, another dtype
 * or iters outside [1, 2^20], FCA_ERR_HIP if a launch or event call fails.
 */
fca_status fca_measure_mfma_rate(int32_t dtype, int32_t iters, void* stream, double* tflops);

/*
 * Exact combination of attention states over disjoint key sets: state j of
 * (request i, head h) is a normalised output o_j (float32) and its natural
 * log-sum-exp lse_j, as fca_decode writes them with FCA_PLAN_OUT_F32 and an
 * lse buffer.  The result is
 *   w_j = exp(lse_j - max_j lse_j),  out = sum_j w_j o_j / sum_j w_j,
 *   lse = max_j lse_j + ln sum_j w_j,
 * attention over the union of the key sets.  This is the merge half of
 * routing the query to the holder of a part of the cache ("Move the Query,
 * Not the Cache", Metodologia: partial attention computed where the blocks
 * live, combined by the online-softmax merge) and the same weighting as the
 * exact reduction of "Core Mechanism", step 3.  States with lse = -inf (no
 * keys) carry no weight; if all do, out = 0 and lse = -inf.
 *
 *   outs      host array of n_states device pointers, float32
 *             [batch, num_heads, head_dim], contiguous.
 *   lses      host array of n_states device pointers, float32
 *             [batch, num_heads].
 *   out_dev   [batch, num_heads, head_dim]: bf16, or float32 with
 *             FCA_MERGE_OUT_F32 in `flags`; may alias outs[0] when float32.
 *   lse_dev   float32 [batch, num_heads], or NULL; may alias lses[0].
 *
 * n_states in [1, 16], head_dim in {128, 512}, batch * num_heads in
 * [0, 2^31).  Asynchronous on `stream`; no allocation.
 * FCA_ERR_INVALID_ARG for NULL pointers or sizes out of range,
 * FCA_ERR_UNSUPPORTED for another head_dim, FCA_ERR_HIP if the launch fails.
 */
#define FCA_MERGE_OUT_F32 1u
fca_status fca_merge_states(int32_t n_states, const float* const* outs, const float* const* lses, int32_t batch,
                            int32_t num_heads, int32_t head_dim, void* out_dev, float* lse_dev, uint32_t flags,
                            void* stream);

/*
 * Append one decode token per request to the paged cache, copying a shared
 * block first when asked (copy-on-write).  A paged cache grows by filling
 * fixed-size blocks that the block table lists; requests forked from one
 * prompt reference the same physical blocks, and the one that writes into a
 * shared block is given its own copy so the others keep the old contents
 * (PagedAttention vs. RadixAttention page, "How PagedAttention Works",
 * steps 3 and 4).  Run before fca_plan_create / fca_decode of the step that
 * reads the new token; then the plan keeps the invariant it relies on, that
 * a block two requests share holds the same tokens for both.
 *
 * For request i with L = seq_lens_dev[i] cached tokens, let
 * j = L / block_size and t = L % block_size:
 *   - if cow_dst_dev is not NULL and c = cow_dst_dev[i] >= 0 (and c differs
 *     from block_tables_dev[i][j]), the request's tokens of block
 *     block_tables_dev[i][j] (slots 0 .. t-1, every KV head, keys and
 *     values) are copied to block c and block_tables_dev[i][j] is set to c;
 *     slots after t of block c keep what they held (in the source they may
 *     be a longer sharer's tokens);
 *   - the new key (and value) is written at slot t of block
 *     block_tables_dev[i][j], in the cache layout fca_decode reads
 *     (desc's strides).
 * seq_lens are not changed: the caller's next plan uses L + 1.  The caller
 * fills block_tables_dev[i][j] with a fresh block when L is a multiple of
 * block_size (a new block starts).
 *
 *   desc          as for fca_plan_create (shape, strides, num_blocks; flags
 *                 are checked but unused).
 *   k_new_dev     bf16 [batch][num_kv_heads][head_dim_qk], contiguous.
 *   v_new_dev     bf16 [batch][num_kv_heads][head_dim_v]; ignored (may be
 *                 NULL) when desc->v_aliases_k.
 *   k_cache_dev, v_cache_dev  the pools (v ignored when v_aliases_k); 16-byte
 *                 aligned.
 *   block_tables_dev int32, row i at block_tables_dev + i * bt_row_stride,
 *                 max_blocks entries used; entry j of a copied request is
 *                 rewritten.
 *   seq_lens_dev  int32 [batch].
 *   cow_dst_dev   int32 [batch] or NULL; negative = no copy.
 *   status_dev    int32 or NULL.  A request whose L is outside
 *                 [0, max_blocks * block_size), whose block entry is outside
 *                 [0, num_blocks), or whose cow target is >= num_blocks is
 *                 skipped and ORs FCA_APPEND_BAD_LEN / _BAD_BLOCK / _BAD_COW
 *                 into *status_dev; the caller zeroes it beforehand and reads
 *                 it when it wants to know.
 *
 * A request may write in place only into a slot no other request holds a
 * token in: of the requests sharing a partly filled last block, at most one
 * of those with the most tokens in it goes without a cow target.  Cow
 * targets must differ from each other and from every block a request of the
 * call reads; overlapping calls race.  Returns
 * FCA_ERR_INVALID_ARG for NULL or misaligned pointers, batch outside
 * [0, 8192], max_blocks outside [1, 2^20] or bt_row_stride < max_blocks;
 * FCA_ERR_UNSUPPORTED as fca_plan_create; FCA_ERR_HIP if the launch fails.
 * Asynchronous on `stream`.
 *
 * This call covers one layer's pool.  When several layers share the block
 * table (as they share the plan), use fca_kv_append_layers: appending layer
 * by layer with this call would rewrite a copied request's table entry after
 * the first layer, and the later layers would then write in place into the
 * copy without copying their own tokens.
 */
#define FCA_APPEND_BAD_LEN 1
#define FCA_APPEND_BAD_BLOCK 2
#define FCA_APPEND_BAD_COW 4
fca_status fca_kv_append(const fca_attn_desc* desc, const void* k_new_dev, const void* v_new_dev, void* k_cache_dev,
                         void* v_cache_dev, int32_t* block_tables_dev, int64_t bt_row_stride, int32_t max_blocks,
                         const int32_t* seq_lens_dev, const int32_t* cow_dst_dev, int32_t* status_dev, int32_t batch,
                         void* stream);

/*
 * fca_kv_append for n_layers layers that share one block table (each layer
 * its own pool with the same block IDs): k_new_dev[l], v_new_dev[l],
 * k_caches_dev[l], v_caches_dev[l] are host arrays of device pointers, one
 * entry per layer, each as for fca_kv_append (v arrays may be NULL when
 * v_aliases_k).  Every layer's copy reads block_tables_dev as the caller
 * left it; the entries of copied requests are rewritten once, after every
 * layer's copy (so a copy target receives the request's tokens in every
 * layer).  Status bits are ORed once per skipped request.  Same contract and
 * errors as fca_kv_append, plus FCA_ERR_INVALID_ARG for n_layers < 0 or a
 * NULL / misaligned layer pointer (the error names the layer).  n_layers == 0
 * or batch == 0 does nothing.  Asynchronous on `stream`: a few launches, no
 * allocation.
 */
fca_status fca_kv_append_layers(const fca_attn_desc* desc, int32_t n_layers, const void* const* k_new_dev,
                                const void* const* v_new_dev, void* const* k_caches_dev, void* const* v_caches_dev,
                                int32_t* block_tables_dev, int64_t bt_row_stride, int32_t max_blocks,
                                const int32_t* seq_lens_dev, const int32_t* cow_dst_dev, int32_t* status_dev,
                                int32_t batch, void* stream);

/*
 * Frees the plan without waiting for the device.  Its device schedule is
 * kept by the library (a few buffers per process) and reused by a later plan
 * once the stream the plan was created with has passed the point of this
 * call: decodes of the plan queued on other streams must be complete, or
 * ordered before that point, when it is called.  The workspace stays the
 * caller's.  NULL is ok.
 */
void fca_plan_destroy(fca_plan plan);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* fca_last_error(void);

/* Library version, e.g. "0.1.0". */
const char* fca_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FCA_H_ */
