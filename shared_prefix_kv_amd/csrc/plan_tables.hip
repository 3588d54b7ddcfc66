// Merge tables of a plan, built on the device at plan time (gfx950).
//
// The exact combination of "Core Mechanism" step 3 (ZoRRo Inference &
// Forest Cascade Attention page) reads, for request i and query head h, the
// partial rows of every token split of every group on i's path (deepest
// group first, then its parents) and of i's own suffix.  The merge kernel
// takes them from a flat table: (start, count) = src_span[i * Hq + h] gives
// src_row[start .. start + count).  The host planner lays out the lanes
// (LaneMeta: base row, splits, head block, column range of one (unit, head
// block, column chunk) stream) and the per-request and per-group metadata;
// one kernel turns them into the table -- a thread per (request, head)
// counts its rows and writes them -- instead of the host walking B x Hq paths
// at every plan.  When the host has bounded every pair's count by a stride of
// at most 64, pair q's rows sit at q * stride, padded with -1 (the merge then
// reads them without the span); otherwise each wave takes room for its
// threads' rows with one atomic add on a counter, so where a pair's rows sit
// depends on the order in which waves reach it; what they are, and their
// order, does not.  The same launch fills the first block IDs of every
// workgroup's bin head (its last blocks, one thread per bin), so the plan's
// device tables cost one launch after the upload.

#include <algorithm>
#include <climits>

#include "fca_internal.h"

namespace fca {
namespace {

constexpr int kTableThreads = 256;

// Calls f(lane, column) for the units on the path of (request i, head h), in
// merge order.
template <class F>
__device__ __forceinline__ void path_units(const TableParams& p, int i, int h, F&& f) {
  const int kvh = h / p.r, rr = h - kvh * p.r;
  const ReqMeta rq = p.req[i];
  for (int g = rq.deepest; g >= 0;) {
    const GroupMeta gm = p.grp[g];
    const int col = (rq.pos - gm.r0) * p.r + rr;
    f(gm.lane0 + (kvh / gm.H) * gm.chunks + col / p.item_cols, col);
    g = gm.parent;
  }
  if (rq.sfx_lane >= 0) f(rq.sfx_lane + (kvh / rq.sfx_H) * rq.sfx_chunks + rr / p.item_cols, rr);
}

// Blocks [0, table_blocks) build the merge tables, the rest the bin heads.
__global__ __launch_bounds__(kTableThreads) void k_plan_tables(TableParams p, int table_blocks) {
  if ((int)blockIdx.x >= table_blocks) {
    // Block IDs of blocks 0..3 of the bin's first item (validated by
    // discovery), 0 past its end.
    const int b = ((int)blockIdx.x - table_blocks) * kTableThreads + threadIdx.x;
    if (b >= p.n_bins) return;
    BinHead& h = p.heads[b];
    const WorkItem& it = h.first;
    const int nblk = (it.tok_end - it.tok_begin + p.bs - 1) / p.bs;
    for (int j = 0; j < 4; ++j)
      h.id[j] = j < nblk ? p.bt[(int64_t)it.request * p.W4 + it.tok_begin / p.bs + j] : 0;
    return;
  }
  const int64_t pair = (int64_t)blockIdx.x * kTableThreads + threadIdx.x;
  const int64_t n = (int64_t)p.B * p.Hq;
  const int lane = threadIdx.x & 63;
  int i = 0, h = 0, cnt = 0;
  if (pair < n) {
    i = (int)(pair / p.Hq);
    h = (int)(pair - (int64_t)i * p.Hq);
    path_units(p, i, h, [&](int lane_id, int) { cnt += p.lanes[lane_id].splits; });
  }
  int start;
  if (p.stride > 0) {
    // fixed stride: the pair's rows, then -1 up to the stride
    if (pair >= n) return;
    start = (int)(pair * p.stride);
    for (int k = cnt; k < p.stride; ++k) p.src_row[start + k] = -1;
  } else {
    // packed: inclusive prefix sum of the counts over the wave, one atomic
    // add per wave for its room
    int incl = cnt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d);
      if (lane >= d) incl += v;
    }
    int base = 0;
    if (lane == 63) base = atomicAdd(p.total, incl);
    base = __shfl(base, 63);
    if (pair >= n) return;
    start = base + incl - cnt;
  }
  p.src_span[pair] = make_int2(start, p.stride > 0 ? min(cnt, (int)p.stride) : cnt);
  const int kvh = h / p.r;
  int32_t* out = p.src_row + start;
  // the pair's room: its count (packed) or the stride, which the host sizes
  // to a bound of every pair's count; never written past
  const int32_t* const room = out + (p.stride > 0 ? p.stride : cnt);
  path_units(p, i, h, [&](int lane_id, int col) {
    const LaneMeta L = p.lanes[lane_id];
    const int step = L.H * L.ccols;
    int row = L.base + (kvh - L.kv0) * L.ccols + (col - L.col0);
    for (int s = 0; s < L.splits && out < room; ++s, row += step) *out++ = row;
  });
}

}  // namespace

hipError_t launch_plan_tables(const TableParams& p, hipStream_t s) {
  const int64_t n = (int64_t)p.B * p.Hq;
  const int64_t table_blocks = (n + kTableThreads - 1) / kTableThreads;
  const int64_t head_blocks = ((int64_t)std::max(p.n_bins, 0) + kTableThreads - 1) / kTableThreads;
  if (table_blocks + head_blocks == 0) return hipSuccess;
  if (table_blocks + head_blocks > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_plan_tables, dim3((unsigned)(table_blocks + head_blocks)), dim3(kTableThreads), 0, s, p,
                     (int)table_blocks);
  return hipGetLastError();
}

}  // namespace fca
