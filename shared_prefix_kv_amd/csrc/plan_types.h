// Plain data shared by the host planner and the gfx950 kernels: work items,
// merge metadata, the discovery read-back, and the planner's interface.
// No HIP here: the planner (planner.cpp) builds as ordinary host C++.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "fca.h"

namespace fca {

constexpr int kMaxBatch = 8192;
constexpr int kMaxTableWidth = 1 << 20;
// Entries of the plan workspace after the last row of the block-table copy:
// the common-prefix step of discovery reads up to one span of 4 x lanes x
// loads entries (at most 128) past the compared range.
constexpr int kLcpTail = 256;
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

// Alignment of the regions inside workspaces.
constexpr size_t kWsAlign = 256;
inline size_t ws_align_up(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }

// ---- Planner (planner.cpp) ----

enum Kind { kGqa = 0, kMla = 1 };

// Attention launches of a plan: bins [bin0, bin0 + n_bins) of the plan's
// bins, holding the work items of both passes or of one.
enum PassSet { kBothPasses = 0, kGroupedPass = 1, kSuffixPass = 2 };
struct Launch {
  int bin0, n_bins;
  PassSet passes;
};

// What fca_plan_create reads back from the discovery kernels (host copies).
struct DiscoveryView {
  const int32_t* header;     // [kHdrWords]
  const int32_t* lens;       // [B] validated lengths
  const int32_t* deepest;    // [B] discovery group id or -1
  const int32_t* sfx_begin;  // [B] first suffix block
  const int32_t* records;    // [B * kRecordInts]: leader, depth, parent id, begin, end, count
};

// The host side of a plan: the canonical grouping, the schedule of both
// passes and the merge tables.  fca_plan_create uploads it.
struct PlanHost {
  fca_attn_desc desc;
  Kind kind = kGqa;
  int B = 0, W = 0, r = 1;
  std::vector<fca_group_record> groups;
  std::vector<int32_t> members;   // ascending per group
  std::vector<int32_t> folded;    // per group: read per request (activation heuristic)
  std::vector<int32_t> req3;      // per request: suffix_block_begin, suffix_tokens, deepest
  std::vector<WorkItem> items;             // what the device runs: all launches' items (in bin order)
  std::vector<int32_t> bins;               // bin b runs items [bins[b], bins[b + 1])
  std::vector<Launch> launches;            // one (both passes) or two (grouped, suffix)
  std::vector<int32_t> perm;
  std::vector<ReqMeta> req;
  std::vector<GroupMeta> grp;
  std::vector<LaneMeta> lanes;  // grouped lanes, then suffix lanes
  int item_cols = kItemColsGqa;  // query rows per column chunk
  int64_t max_pair_sources = 0;  // upper bound of the partial rows one (request, head) merges
  fca_plan_info info{};
};

// The grouped items (member_off >= 0) or the per-request items of a plan, in
// bin order (what the export reports for each pass).
inline std::vector<WorkItem> pass_items(const PlanHost& P, bool grouped) {
  std::vector<WorkItem> v;
  for (const WorkItem& it : P.items)
    if ((it.member_off >= 0) == grouped) v.push_back(it);
  return v;
}

// Builds P's grouping and schedule from a discovery read-back, for a device
// with n_cu compute units.  P.desc, P.kind, P.B, P.W and P.r must be set.
// The read-back is checked (ranges, nesting, member counts) before it is
// used; an inconsistent one gives FCA_ERR_HIP.  On failure *err holds the
// message.  May throw std::bad_alloc.
fca_status build_plan(PlanHost& P, const DiscoveryView& d, int n_cu, std::string* err);

// Partial rows request i merges for query head h, in the merge's order:
// every split of the deepest group's lane, then of its ancestors' lanes, then
// of the suffix lane.
template <class F>
void for_each_source(const PlanHost& P, int i, int h, F&& f) {
  const int r = P.r;
  const int kvh = h / r, rr = h % r;
  const ReqMeta& rq = P.req[i];
  auto lane_rows = [&](int lane, int col) {
    const LaneMeta& L = P.lanes[lane];
    for (int s = 0; s < L.splits; ++s)
      f((int64_t)L.base + (int64_t)s * L.H * L.ccols + (int64_t)(kvh - L.kv0) * L.ccols + (col - L.col0));
  };
  for (int g = rq.deepest; g >= 0; g = P.grp[g].parent) {
    const GroupMeta& gm = P.grp[g];
    const int col = (rq.pos - gm.r0) * r + rr;
    lane_rows(gm.lane0 + (kvh / gm.H) * gm.chunks + col / P.item_cols, col);
  }
  if (rq.sfx_lane >= 0) lane_rows(rq.sfx_lane + (kvh / rq.sfx_H) * rq.sfx_chunks + rr / P.item_cols, rr);
}

}  // namespace fca
