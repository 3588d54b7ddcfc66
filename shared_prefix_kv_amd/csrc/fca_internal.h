// Internal declarations shared by the host library and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "fca.h"
#include "plan_types.h"

namespace fca {

// Device arrays of the discovery step (all inside the plan workspace).
struct DiscoveryPtrs {
  int32_t* header;     // [kHdrWords]   -- read back
  int32_t* lens;       // [B]           -- read back
  int32_t* deepest;    // [B] device group id, -1   -- read back
  int32_t* sfx_begin;  // [B] first suffix block    -- read back
  int32_t* records;    // [B * kRecordInts]         -- read back
  int32_t* bt;         // [B * W4] copy of the used table entries (-1 elsewhere), rows 16-byte aligned
  int32_t* nfull;
  int32_t* root;
  int32_t* depth_at;   // current node's first block
  int32_t* node;
  int32_t* gdepth;
  int32_t* gparent;
  int32_t* active;
  int32_t* lcp0;       // common prefix (full blocks) of each request with its tree's root
  int32_t* ngid;
  int32_t* first;      // first block ID of each request with a full block, else -1
};

// W: table width (entries per row the caller's tables use); W4: row stride of
// the copy in the workspace (W rounded up to a multiple of 4).
hipError_t launch_discovery(const int32_t* bt_in, int64_t bt_stride, const int32_t* lens_in, int B, int W, int W4,
                            int block_size, int num_blocks, bool cascade, const DiscoveryPtrs& p, hipStream_t s);

// Partial (o, m, l) rows: o unnormalised w.r.t. its own running max m
// (log2 domain), l the matching denominator.
struct PartialPtrs {
  float* o;
  float* m;
  float* l;
};

struct GqaParams {
  const WorkItem* items;    // grouped by bin
  const BinHead* bins;      // one per workgroup
  const int32_t* perm;
  const int32_t* bt;
  int32_t W;  // row stride of bt (the workspace copy)
  int32_t Hq;
  int32_t r;
  float scale_log2;
  const void* q;
  const void* k;
  const void* v;
  int64_t k_stride_block, k_stride_head, v_stride_block, v_stride_head;
  int64_t k_stride_token, v_stride_token;  // 0: tile layout; > 0: token rows
  PartialPtrs part;
};

// Grouped and per-request work items, one persistent workgroup per bin
// (bins [0, n_bins) of p.bins).  `passes` names the launch's passes; it
// picks the kernel entry the launch is traced under (same code).
hipError_t launch_attention(const GqaParams& p, int n_bins, PassSet passes, hipStream_t s);

// The same for a latent cache (576-wide keys, values = first 512 dims,
// 64-token blocks): items of up to 128 query rows of one head.  `grouped_pass`
// picks the kernel entry the launch is traced under (same code).
hipError_t launch_mla(const GqaParams& p, int n_bins, bool grouped_pass, hipStream_t s);

// Device tables built at plan time (plan_tables.hip), in one launch:
//   * merge tables from the planner's metadata: src_span [B * Hq] (start,
//     count) into src_row.  With stride > 0 pair q's rows start at q * stride
//     and the rest of its stride holds -1 (every pair has at most stride
//     rows); with stride 0 they are packed, placed through *total (zero
//     before the launch), which ends at the number of rows;
//   * id[] of every bin head: the first block IDs of its first item, from
//     the block-table copy bt (row stride W4, block size bs).
struct TableParams {
  const ReqMeta* req;
  const GroupMeta* grp;
  const LaneMeta* lanes;
  int32_t B, Hq, r, item_cols;
  int2* src_span;
  int32_t* src_row;
  int32_t* total;
  int32_t stride;
  BinHead* heads;
  int32_t n_bins;
  const int32_t* bt;
  int32_t W4, bs;
};

hipError_t launch_plan_tables(const TableParams& p, hipStream_t s);

struct MergeParams {
  // Partial rows of (request i, query head h), in merge order (deepest
  // group's splits, then its ancestors', then the suffix's):
  // src_row[s.x .. s.x + s.y), s = src_span[i * Hq + h].  With
  // src_stride > 0 (at most 64), s.x = (i * Hq + h) * src_stride and the
  // entries after s.y hold -1 up to the stride, so the merge reads the rows
  // without the span.
  const int2* src_span;
  const int32_t* src_row;
  int32_t src_stride;
  int32_t B, Hq, Dv;
  PartialPtrs part;
  void* out;
  float* lse;
  int32_t out_f32;  // out is float32 (else bf16)
};

hipError_t launch_merge(const MergeParams& p, hipStream_t s);

// Combination of attention states (normalised float32 outputs and their
// natural log-sum-exp) over disjoint key sets.
constexpr int kMaxStates = 16;
struct StatesParams {
  const float* outs[kMaxStates];
  const float* lses[kMaxStates];
  int32_t n, pairs, D;
  void* out;
  float* lse;
  int32_t out_f32;
};

hipError_t launch_merge_states(const StatesParams& p, hipStream_t s);

// Decode-token append (kv_append.hip).  Element strides as fca_attn_desc.
// One launch handles up to kAppendLayers layers of one block table; the
// table entries of copied blocks are rewritten by a separate commit launch
// after every layer's copy has read them.
constexpr int kAppendLayers = 32;
struct AppendParams {
  const uint16_t* k_new[kAppendLayers];  // [batch][num_kv_heads][head_dim_qk] bf16 per layer
  const uint16_t* v_new[kAppendLayers];  // [batch][num_kv_heads][head_dim_v] bf16 (unused for latent caches)
  uint16_t* k_cache[kAppendLayers];
  uint16_t* v_cache[kAppendLayers];
  int32_t n_layers;                      // layers of this launch
  const int32_t* block_tables;           // read only here
  int64_t bt_row_stride;
  const int32_t* seq_lens;
  const int32_t* cow_dst;  // may be null
  int64_t k_stride_block, k_stride_head, v_stride_block, v_stride_head;
  int64_t k_stride_token, v_stride_token;  // 0: tile layout; > 0: token rows
  int32_t batch, num_kv_heads, max_blocks, num_blocks;
};

// Copies / in-place writes of every layer in p (block tables unchanged).
hipError_t launch_append(const AppendParams& p, bool latent, hipStream_t s);
// Points block_tables[i][L / bs] at cow_dst[i] where the append copied, and
// ORs FCA_APPEND_BAD_* bits into *status for skipped requests.
hipError_t launch_append_commit(int32_t* block_tables, int64_t bt_row_stride, const int32_t* seq_lens,
                                const int32_t* cow_dst, int32_t* status, int batch, int max_blocks, int block_size,
                                int num_blocks, hipStream_t s);

// Streaming-read probe (measure.hip): reads `bytes` (multiple of 16) from src
// with launch shape 0 (512 threads x 4 loads) or 1 (256 threads x 8 loads).
constexpr int kReadShapes = 2;
hipError_t launch_stream_read(const void* src, size_t bytes, int n_cu, int shape, hipStream_t s);
// MFMA-rate probe: one workgroup of kMfmaThreads per compute unit, each wave
// issuing 32 x iters 16x16x32 products (bf16, else fp16).
constexpr int kMfmaThreads = 512;
constexpr int kMfmaPerIter = 32;
hipError_t launch_mfma_rate(bool bf16, int iters, int n_cu, hipStream_t s);

}  // namespace fca
