// Internal declarations shared by the host library and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "fca.h"

namespace fca {

constexpr int kMaxBatch = 8192;
constexpr int kMaxTableWidth = 1 << 20;
constexpr int kAttnLgWaves = 2;                 // log2 of the waves of an attention workgroup
constexpr int kAttnWaves = 1 << kAttnLgWaves;   // waves that share one work item
constexpr int kItemColsGqa = 64;                // query rows of one GQA work item at most

// A unit of work of the grouped or per-request pass; same layout as the
// public fca_work_item.
struct WorkItem {
  int32_t request;
  int32_t tok_begin;
  int32_t tok_end;
  int32_t kv_head;
  int32_t member_off;
  int32_t ncols;
  int32_t col0;
  int32_t col1;
  int32_t part_base;
  int32_t kv_heads;  // KV heads the item covers: kv_head .. kv_head + kv_heads - 1
  int32_t stripes;   // block stripes (the kernel derives them; exported for tests)
  int32_t flags;     // kItemStream: tiles with one reader (non-temporal loads)
};
constexpr int32_t kItemStream = 1;
static_assert(sizeof(WorkItem) == sizeof(fca_work_item), "work item layout");

// Per-request data the merge reads.
struct ReqMeta {
  int32_t pos;         // position in the depth-first member order
  int32_t deepest;     // canonical index of the deepest group, -1 if none
  int32_t sfx_lane;    // first lane of the suffix (-1: no suffix tokens); the
  int32_t sfx_H;       //   lane of (kv head h, query row n) is
  int32_t sfx_chunks;  //   sfx_lane + (h / sfx_H) * sfx_chunks + n / item_cols
  int32_t pad0, pad1, pad2;
};

// Per-group data the merge reads (canonical order).
struct GroupMeta {
  int32_t parent;  // canonical index or -1
  int32_t r0;      // first position of the group's members in `perm`
  int32_t ncols;   // members * (Hq / Hkv)
  int32_t lane0;   // lane of (head block 0, column chunk 0)
  int32_t H;       // KV heads per lane; lane of (kv head h, column n) is
  int32_t chunks;  //   lane0 + (h / H) * chunks + n / item_cols
  int32_t pad0, pad1;
};

// One (unit, head block, column chunk) stream of a pass and its partial
// rows: token split s, KV head h, column n is row
//   base + s * H * ccols + (h - kv0) * ccols + (n - col0).
struct LaneMeta {
  int32_t base;
  int32_t splits;
  int32_t kv0;
  int32_t H;
  int32_t col0;
  int32_t ccols;
  int32_t pad0, pad1;
};

// Discovery header words.
enum { kHdrGroups = 0, kHdrErr = 1, kHdrBadReq = 2, kHdrWords = 64 };
enum { kErrBadBlock = 1, kErrBadLen = 2 };
constexpr int kRecordInts = 8;  // leader, depth, parent gid, begin, end, count, 0, 0

// Device arrays of the discovery step (all inside the plan workspace).
struct DiscoveryPtrs {
  int32_t* header;     // [kHdrWords]   -- read back
  int32_t* lens;       // [B]           -- read back
  int32_t* deepest;    // [B] device group id, -1   -- read back
  int32_t* sfx_begin;  // [B] first suffix block    -- read back
  int32_t* records;    // [B * kRecordInts]         -- read back
  int32_t* bt;         // [B * W] copy of the used table entries (-1 elsewhere)
  int32_t* nfull;
  int32_t* root;
  int32_t* depth_at;   // current node's first block
  int32_t* node;
  int32_t* gdepth;
  int32_t* gparent;
  int32_t* active;
  int32_t* ndstar;
  int32_t* ncount;
  int32_t* ngid;
  int32_t* newnode;
};

hipError_t launch_discovery(const int32_t* bt_in, int64_t bt_stride, const int32_t* lens_in, int B, int W,
                            int block_size, int num_blocks, bool cascade, const DiscoveryPtrs& p, hipStream_t s);

// Partial (o, m, l) rows: o unnormalised w.r.t. its own running max m
// (log2 domain), l the matching denominator.
struct PartialPtrs {
  float* o;
  float* m;
  float* l;
};

// What a persistent attention workgroup needs first, in one 128-byte line:
// its range of items, the first item, and the block IDs of that item's
// first four blocks (each wave's first tile), so that the first copies go
// out after a single memory round trip.
struct BinHead {
  int32_t i_begin, i_end;  // items of the bin: [i_begin, i_end) of the item array
  int32_t id[4];           // block IDs of blocks 0..3 of the first item (0 past its end)
  int32_t pad0, pad1;
  WorkItem first;          // item i_begin
  int32_t pad2[12];
};
static_assert(sizeof(BinHead) == 128, "bin head layout");

// Fills id[] of every bin head from the block-table copy (plan time).
hipError_t launch_bin_heads(BinHead* heads, int n_bins, const int32_t* bt, int W, int bs, hipStream_t s);

struct GqaParams {
  const WorkItem* items;    // grouped by bin
  const BinHead* bins;      // one per workgroup
  const int32_t* perm;
  const int32_t* bt;
  int32_t W;
  int32_t Hq;
  int32_t r;
  float scale_log2;
  const void* q;
  const void* k;
  const void* v;
  int64_t k_stride_block, k_stride_head, v_stride_block, v_stride_head;
  PartialPtrs part;
};

// Grouped and per-request work items, one persistent workgroup per bin
// (bins [0, n_bins) of p.bins).
hipError_t launch_attention(const GqaParams& p, int n_bins, hipStream_t s);

// The same for a latent cache (576-wide keys, values = first 512 dims,
// 64-token blocks): items of up to 128 query rows of one head.  `grouped_pass`
// picks the kernel entry the launch is traced under (same code).
hipError_t launch_mla(const GqaParams& p, int n_bins, bool grouped_pass, hipStream_t s);

struct MergeParams {
  // Partial rows of (request i, query head h), in merge order (deepest
  // group's splits, then its ancestors', then the suffix's):
  // src_row[src_off[i * Hq + h] .. src_off[i * Hq + h + 1]).
  const int32_t* src_off;
  const int32_t* src_row;
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

}  // namespace fca
