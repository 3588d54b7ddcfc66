// Host side of the C ABI: validation, plan construction, launches.
//
// fca_plan_create runs the discovery kernels, reads back one small region
// (counters, error flags, group records, per-request deepest group and
// suffix start), and turns it into:
//   * the canonical group order (smallest member, depth),
//   * a depth-first member order in which every group is a contiguous range,
//   * the split schedule of the grouped and per-request passes,
//   * the per-request / per-group metadata the merge walks.
// These are uploaded into the caller's plan workspace.  fca_decode only
// launches kernels.

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <cstdlib>
#include <mutex>
#include <new>
#include <queue>
#include <stdexcept>
#include <string>
#include <vector>

#include "fca_internal.h"

using namespace fca;

namespace {

thread_local std::string g_last_error;

fca_status fail(fca_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

fca_status hip_fail(hipError_t e, const char* what) {
  return fail(FCA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int env_int(const char* name, int dflt) {
  const char* s = getenv(name);
  if (!s || !*s) return dflt;
  const int v = atoi(s);
  return v > 0 ? v : dflt;
}

// Split-schedule targets (developer tuning knobs).
struct Tuning {
  int bins_per_cu;  // attention workgroups per compute unit (the dispatcher balances them)
};

Tuning tuning() {
  Tuning t;
  t.bins_per_cu = env_int("FCA_TUNE_BINS_PER_CU", 2);
  return t;
}

constexpr int kXcds = 8;  // accelerator dies per device; workgroup b is dispatched to die b mod 8
constexpr int kItemColsMla = 64;   // query rows of one latent-cache work item at most
constexpr int kItemWaves = kAttnWaves;  // waves per work item: heads x column groups x block stripes
constexpr int kWaveCols = 32;  // query rows one wave covers at most

enum Kind { kGqa = 0, kMla = 1 };

fca_status check_desc(const fca_attn_desc* d, Kind* kind) {
  if (!d) return fail(FCA_ERR_INVALID_ARG, "desc is NULL");
  if (d->reserved != 0) return fail(FCA_ERR_INVALID_ARG, "desc.reserved must be 0");
  if (d->num_q_heads <= 0 || d->num_kv_heads <= 0 || d->num_q_heads % d->num_kv_heads)
    return fail(FCA_ERR_INVALID_ARG, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                d->num_q_heads, d->num_kv_heads);
  if (d->num_blocks <= 0) return fail(FCA_ERR_INVALID_ARG, "num_blocks must be positive");
  if (!(d->scale > 0.f) || !std::isfinite(d->scale)) return fail(FCA_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (d->flags & ~(FCA_PLAN_DISABLE_CASCADE | FCA_PLAN_SEPARATE_PASSES | FCA_PLAN_OUT_F32 | FCA_PLAN_AUTO_FOLD))
    return fail(FCA_ERR_INVALID_ARG, "unknown flag bits 0x%x", d->flags);
  const int r = d->num_q_heads / d->num_kv_heads;
  if (d->head_dim_qk == 128 && d->head_dim_v == 128 && d->block_size == 16 && !d->v_aliases_k) {
    if (r > 16) return fail(FCA_ERR_UNSUPPORTED, "GQA ratio %d > 16 is not built", r);
    if (d->k_stride_head < 128 * 16 || d->v_stride_head < 128 * 16 ||
        d->k_stride_block < (int64_t)d->num_kv_heads * d->k_stride_head ||
        d->v_stride_block < (int64_t)d->num_kv_heads * d->v_stride_head)
      return fail(FCA_ERR_INVALID_ARG, "cache strides overlap tiles");
    if ((d->k_stride_head | d->k_stride_block | d->v_stride_head | d->v_stride_block) % 8)
      return fail(FCA_ERR_INVALID_ARG, "cache strides must keep 16-byte tile alignment");
    *kind = kGqa;
    return FCA_OK;
  }
  if (d->head_dim_qk == 576 && d->head_dim_v == 512 && d->block_size == 64 && d->v_aliases_k) {
    if (d->k_stride_head < 576 * 64 || d->k_stride_block < (int64_t)d->num_kv_heads * d->k_stride_head)
      return fail(FCA_ERR_INVALID_ARG, "cache strides overlap tiles");
    if ((d->k_stride_head | d->k_stride_block) % 8)
      return fail(FCA_ERR_INVALID_ARG, "cache strides must keep 16-byte tile alignment");
    *kind = kMla;
    return FCA_OK;
  }
  return fail(FCA_ERR_UNSUPPORTED, "unsupported shape: head_dim_qk=%d head_dim_v=%d block_size=%d v_aliases_k=%d",
              d->head_dim_qk, d->head_dim_v, d->block_size, d->v_aliases_k);
}

// Caller-owned plan workspace: discovery read-back region, table copy and
// discovery state.  Its size depends only on (batch, max_blocks).
struct Layout {
  size_t header, lens, deepest, sfx_begin, records, readback_bytes;
  size_t bt, state;
  size_t total;
};

Layout make_layout(int B, int W) {
  Layout L{};
  const size_t b = (size_t)B;
  L.header = 0;
  L.lens = L.header + kHdrWords * 4;
  L.deepest = L.lens + b * 4;
  L.sfx_begin = L.deepest + b * 4;
  L.records = L.sfx_begin + b * 4;
  L.readback_bytes = L.records + b * kRecordInts * 4 - L.header;
  size_t off = align_up(L.header + L.readback_bytes);
  L.bt = off;
  off = align_up(off + b * (size_t)W * 4);
  L.state = off;
  off = align_up(off + 11 * b * 4);
  L.total = off;
  return L;
}

// Plan-owned device buffer holding the schedule.
struct SchedLayout {
  size_t items, heads, perm, src_off, src_row, total;
};

// One launch of the attention kernel: bins [bin0, bin0 + n_bins) of the
// plan's bins, holding the work items of both passes or of one.
enum PassSet { kBothPasses = 0, kGroupedPass = 1, kSuffixPass = 2 };
struct Launch {
  int bin0, n_bins;
  PassSet passes;
};

DiscoveryPtrs discovery_ptrs(char* ws, const Layout& L, int B) {
  DiscoveryPtrs p;
  p.header = reinterpret_cast<int32_t*>(ws + L.header);
  p.lens = reinterpret_cast<int32_t*>(ws + L.lens);
  p.deepest = reinterpret_cast<int32_t*>(ws + L.deepest);
  p.sfx_begin = reinterpret_cast<int32_t*>(ws + L.sfx_begin);
  p.records = reinterpret_cast<int32_t*>(ws + L.records);
  p.bt = reinterpret_cast<int32_t*>(ws + L.bt);
  int32_t* st = reinterpret_cast<int32_t*>(ws + L.state);
  int32_t** arr[] = {&p.nfull,  &p.root,   &p.depth_at, &p.node, &p.gdepth, &p.gparent,
                     &p.active, &p.ndstar, &p.ncount,   &p.ngid, &p.newnode};
  for (int a = 0; a < 11; ++a) *arr[a] = st + (size_t)a * B;
  return p;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t m) { return ceil_div(a, m) * m; }

}  // namespace

namespace {

// Schedule buffers of destroyed plans, kept for later plans of the same
// device: hipFree waits for the whole device and a fresh hipMalloc is slow,
// once per decode step each.  A buffer carries an event recorded on its
// plan's stream when the plan was destroyed; it is reused once that event
// has completed (every decode of the plan is ordered before it).
struct SchedBuf {
  char* ptr;
  size_t cap;
  int dev;
  hipEvent_t done;
};
std::mutex g_sched_mu;
std::vector<SchedBuf> g_sched_free;
constexpr size_t kSchedKeep = 8;  // buffers kept at most

// A kept buffer of at least `bytes` on `dev` whose plan's work is done, or
// none (ptr == nullptr).
SchedBuf sched_take(int dev, size_t bytes) {
  std::lock_guard<std::mutex> lock(g_sched_mu);
  int best = -1;
  for (int i = 0; i < (int)g_sched_free.size(); ++i) {
    const SchedBuf& b = g_sched_free[i];
    if (b.dev != dev || b.cap < bytes || (best >= 0 && b.cap >= g_sched_free[best].cap)) continue;
    if (hipEventQuery(b.done) != hipSuccess) {
      (void)hipGetLastError();  // not ready: no error for later calls to see
      continue;
    }
    best = i;
  }
  if (best < 0) return SchedBuf{nullptr, 0, dev, nullptr};
  const SchedBuf b = g_sched_free[best];
  g_sched_free.erase(g_sched_free.begin() + best);
  return b;
}

void sched_give(SchedBuf b) {
  SchedBuf drop{nullptr, 0, 0, nullptr};
  {
    std::lock_guard<std::mutex> lock(g_sched_mu);
    g_sched_free.push_back(b);
    if (g_sched_free.size() > kSchedKeep) {
      drop = g_sched_free.front();
      g_sched_free.erase(g_sched_free.begin());
    }
  }
  if (drop.ptr) {
    (void)hipFree(drop.ptr);
    (void)hipEventDestroy(drop.done);
  }
}

}  // namespace

struct fca_plan_s {
  fca_attn_desc desc;
  Kind kind;
  int B, W, r;
  char* ws;
  Layout L;
  // host copies
  std::vector<fca_group_record> groups;
  std::vector<int32_t> members;   // ascending per group
  std::vector<int32_t> folded;    // per group: read per request (FCA_PLAN_AUTO_FOLD)
  std::vector<int32_t> req3;      // per request: suffix_block_begin, suffix_tokens, deepest
  std::vector<WorkItem> items_g, items_s;  // host copies of each pass's items, in bin order
  std::vector<WorkItem> items;             // what the device runs: all launches' items
  std::vector<int32_t> bins;               // bin b runs items [bins[b], bins[b + 1])
  std::vector<Launch> launches;            // one (both passes) or two (grouped, suffix)
  std::vector<int32_t> perm;
  std::vector<ReqMeta> req;
  std::vector<GroupMeta> grp;
  std::vector<LaneMeta> lanes;  // grouped lanes, then suffix lanes
  std::vector<int32_t> src_off, src_row;  // merge sources per (request, query head), CSR
  int item_cols = kItemColsGqa;  // query rows per column chunk
  fca_plan_info info;
  // plan-owned device copy of the schedule (a buffer of sched_cap bytes on
  // device `dev`, created with `stream`), handed to later plans when this one
  // is destroyed
  char* sched = nullptr;
  size_t sched_cap = 0;
  int dev = 0;
  hipStream_t stream = nullptr;
  hipEvent_t sched_done = nullptr;
  SchedLayout SL{};
  // measurement hook
  bool profiling = false;
  std::vector<hipEvent_t> event_pool;
  std::vector<hipEvent_t> pending;  // kProfEvents per profiled call
  ~fca_plan_s() {
    if (sched) {
      hipEvent_t ev = sched_done;
      hipError_t e = ev ? hipSuccess : hipEventCreateWithFlags(&ev, hipEventDisableTiming);
      if (e == hipSuccess) e = hipEventRecord(ev, stream);
      if (e == hipSuccess) {
        sched_give(SchedBuf{sched, sched_cap, dev, ev});
      } else {
        (void)hipGetLastError();
        if (ev) (void)hipEventDestroy(ev);
        (void)hipFree(sched);
      }
    } else if (sched_done) {
      (void)hipEventDestroy(sched_done);
    }
    for (hipEvent_t e : pending) (void)hipEventDestroy(e);
    for (hipEvent_t e : event_pool) (void)hipEventDestroy(e);
  }
};

namespace {

// Pinned host staging for a plan's read-back and schedule upload, one buffer
// per host thread, grown on demand and kept until the process ends.  An
// upload from it may still be in flight when the thread's next plan needs it;
// `busy` (recorded after that upload) orders the reuse.
struct Staging {
  char* ptr = nullptr;
  size_t cap = 0;
  hipEvent_t busy = nullptr;
  bool pending = false;
};
thread_local Staging t_stage;

hipError_t stage_acquire(size_t bytes, char** out) {
  Staging& st = t_stage;
  hipError_t e = hipSuccess;
  if (st.pending) {
    e = hipEventSynchronize(st.busy);
    if (e != hipSuccess) return e;
    st.pending = false;
  }
  if (st.cap < bytes) {
    if (st.ptr) {
      e = hipHostFree(st.ptr);
      st.ptr = nullptr;
      st.cap = 0;
      if (e != hipSuccess) return e;
    }
    const size_t cap = std::max<size_t>(bytes + bytes / 2, (size_t)64 << 10);
    e = hipHostMalloc(reinterpret_cast<void**>(&st.ptr), cap, hipHostMallocDefault);
    if (e != hipSuccess) {
      st.ptr = nullptr;
      return e;
    }
    st.cap = cap;
  }
  *out = st.ptr;
  return hipSuccess;
}

// The staging buffer is read by work queued on `s`.
hipError_t stage_in_use(hipStream_t s) {
  Staging& st = t_stage;
  hipError_t e = hipSuccess;
  if (!st.busy) e = hipEventCreateWithFlags(&st.busy, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventRecord(st.busy, s);
  if (e == hipSuccess) st.pending = true;
  return e;
}

}  // namespace

// Partial rows request i merges for query head h, in the merge's order:
// every split of the deepest group's lane, then of its ancestors' lanes, then
// of the suffix lane.
template <class F>
void for_each_source(const fca_plan_s& P, int i, int h, F&& f) {
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

int64_t count_sources(const fca_plan_s& P, int i, int h) {
  int64_t n = 0;
  for_each_source(P, i, h, [&](int64_t) { ++n; });
  return n;
}

extern "C" {

const char* fca_last_error(void) { return g_last_error.c_str(); }

const char* fca_version(void) { return "0.1.0"; }

fca_status fca_plan_workspace_size(int32_t batch, int32_t max_blocks, const fca_attn_desc* desc, size_t* bytes) {
  try {
    if (!bytes) return fail(FCA_ERR_INVALID_ARG, "bytes is NULL");
    Kind kind;
    fca_status st = check_desc(desc, &kind);
    if (st != FCA_OK) return st;
    if (batch < 0 || batch > kMaxBatch) return fail(FCA_ERR_INVALID_ARG, "batch %d outside [0, %d]", batch, kMaxBatch);
    if (max_blocks < 1 || max_blocks > kMaxTableWidth)
      return fail(FCA_ERR_INVALID_ARG, "max_blocks %d outside [1, %d]", max_blocks, kMaxTableWidth);
    *bytes = make_layout(batch, max_blocks).total;
    return FCA_OK;
  } catch (...) {
    return fail(FCA_ERR_HOST_ALLOC, "host allocation failed");
  }
}

static fca_status build_plan(fca_plan_s* P, const std::vector<int32_t>& rb, int n_cu_) {
  const int B = P->B;
  const int bs = P->desc.block_size;
  const int hkv = P->desc.num_kv_heads;
  const int hq = P->desc.num_q_heads;
  const int r = P->r;
  const Layout& L = P->L;
  const int32_t* hdr = rb.data();
  const int32_t* lens = hdr + (L.lens - L.header) / 4;
  const int32_t* deep = hdr + (L.deepest - L.header) / 4;
  const int32_t* sfxb = hdr + (L.sfx_begin - L.header) / 4;
  const int32_t* rec = hdr + (L.records - L.header) / 4;
  const int G = hdr[kHdrGroups];
  if (G < 0 || G > std::max(B - 1, 0)) return fail(FCA_ERR_HIP, "discovery produced %d groups for %d requests", G, B);

  // Canonical order: (leader = smallest member, depth).
  std::vector<int> order(G);
  for (int g = 0; g < G; ++g) order[g] = g;
  std::sort(order.begin(), order.end(), [&](int a, int b) {
    const int32_t* ra = rec + (size_t)a * kRecordInts;
    const int32_t* rb2 = rec + (size_t)b * kRecordInts;
    return ra[0] != rb2[0] ? ra[0] < rb2[0] : ra[1] < rb2[1];
  });
  std::vector<int> canon(G);
  for (int c = 0; c < G; ++c) canon[order[c]] = c;

  P->groups.assign(G, fca_group_record{});
  P->grp.assign(G, GroupMeta{});
  std::vector<int> count(G);
  std::vector<std::vector<int>> children(G), direct(G);
  std::vector<int> roots;
  int max_depth = -1;
  for (int c = 0; c < G; ++c) {
    const int32_t* x = rec + (size_t)order[c] * kRecordInts;
    fca_group_record& gr = P->groups[c];
    gr.depth = x[1];
    gr.parent = x[2] >= 0 ? canon[x[2]] : -1;
    gr.block_begin = x[3];
    gr.block_end = x[4];
    count[c] = x[5];
    max_depth = std::max(max_depth, gr.depth);
    if (gr.parent >= 0)
      children[gr.parent].push_back(c);
    else
      roots.push_back(c);
  }
  std::vector<int> deepest_c(B);
  for (int i = 0; i < B; ++i) {
    deepest_c[i] = deep[i] >= 0 ? canon[deep[i]] : -1;
    if (deepest_c[i] >= 0) direct[deepest_c[i]].push_back(i);
  }

  // Depth-first member order: every group is the contiguous range [r0, r1).
  P->perm.clear();
  P->perm.reserve(B);
  std::vector<int> r0(G), r1(G);
  {
    std::vector<std::pair<int, size_t>> stack;  // (group, next child)
    for (int root : roots) {
      stack.push_back({root, 0});
      r0[root] = (int)P->perm.size();
      for (int i : direct[root]) P->perm.push_back(i);
      while (!stack.empty()) {
        auto& top = stack.back();
        const int c = top.first;
        if (top.second < children[c].size()) {
          const int ch = children[c][top.second++];
          r0[ch] = (int)P->perm.size();
          for (int i : direct[ch]) P->perm.push_back(i);
          stack.push_back({ch, 0});
        } else {
          r1[c] = (int)P->perm.size();
          stack.pop_back();
        }
      }
    }
    for (int i = 0; i < B; ++i)
      if (deepest_c[i] < 0) P->perm.push_back(i);
  }
  if ((int)P->perm.size() != B) return fail(FCA_ERR_HIP, "inconsistent discovery output (member order)");
  std::vector<int> pos(B);
  for (int k = 0; k < B; ++k) pos[P->perm[k]] = k;

  P->members.clear();
  for (int c = 0; c < G; ++c) {
    if (r1[c] - r0[c] != count[c] || count[c] < 2)
      return fail(FCA_ERR_HIP, "inconsistent discovery output (group %d: %d members, range %d)", c, count[c],
                  r1[c] - r0[c]);
    P->groups[c].member_begin = (int32_t)P->members.size();
    P->groups[c].member_count = count[c];
    std::vector<int> m(P->perm.begin() + r0[c], P->perm.begin() + r1[c]);
    std::sort(m.begin(), m.end());
    P->members.insert(P->members.end(), m.begin(), m.end());
  }

  // Activation (FCA_PLAN_AUTO_FOLD, GQA caches): a group is read once for
  // all members only if that saves more bytes than its partial rows cost.
  // Reading a group of n members over T tokens once instead of n times
  // saves (n - 1) T t bytes (t: KV bytes per token); in exchange, each of
  // its token pieces writes n Hq partial rows that the merge reads back, and
  // a written byte costs about three read bytes here, so 4 (4 Dv + 8) bytes
  // per row.  The pieces are estimated as the group's bytes over one
  // workgroup's share of all unique bytes.  Leaves first: a group is folded
  // only when all its children are.
  P->folded.assign(G, 0);
  int n_folded = 0;
  std::vector<int> eff_deep(deepest_c);
  std::vector<int> eff_sb(sfxb, sfxb + B);
  if ((P->desc.flags & FCA_PLAN_AUTO_FOLD) && P->kind == kGqa && G > 0) {
    const Tuning tf = tuning();
    const double tok_bytes = (double)hkv * (P->desc.head_dim_qk + P->desc.head_dim_v) * 2;
    double unique_tok = 0;
    for (int i = 0; i < B; ++i) unique_tok += lens[i] - bs * sfxb[i];
    for (int c = 0; c < G; ++c) unique_tok += (double)(P->groups[c].block_end - P->groups[c].block_begin) * bs;
    const double share = std::max(unique_tok * tok_bytes / ((double)n_cu_ * tf.bins_per_cu), 1.0);
    const double row_cost = 4.0 * (4.0 * P->desc.head_dim_v + 8.0);
    for (int c = G - 1; c >= 0; --c) {  // children come after their parents
      bool leaves_folded = true;
      for (int ch : children[c]) leaves_folded = leaves_folded && P->folded[ch];
      if (!leaves_folded) continue;
      const double T = (double)(P->groups[c].block_end - P->groups[c].block_begin) * bs;
      const double saved = (count[c] - 1) * T * tok_bytes;
      const double pieces = std::max(1.0, std::ceil(T * tok_bytes / share));
      const double cost = pieces * count[c] * hq * row_cost;
      if (saved < cost) {
        P->folded[c] = 1;
        ++n_folded;
      }
    }
    for (int i = 0; i < B; ++i)
      while (eff_deep[i] >= 0 && P->folded[eff_deep[i]]) {
        eff_sb[i] = P->groups[eff_deep[i]].block_begin;
        eff_deep[i] = P->groups[eff_deep[i]].parent;
      }
  }

  P->req3.assign((size_t)B * 3, 0);
  int64_t logical = 0, unique = 0;
  std::vector<int> sfx_tokens(B);
  for (int i = 0; i < B; ++i) {
    const int sb = eff_sb[i];
    sfx_tokens[i] = lens[i] - bs * sb;
    P->req3[3 * i + 0] = sb;
    P->req3[3 * i + 1] = sfx_tokens[i];
    P->req3[3 * i + 2] = eff_deep[i];
    logical += lens[i];
    unique += sfx_tokens[i];
    if (sfx_tokens[i] < 0) return fail(FCA_ERR_HIP, "inconsistent discovery output (suffix of request %d)", i);
  }

  // ---- Work items ----
  // A lane is one (unit, head block, column chunk) stream of stages: a unit
  // is a group's prefix range or a request's suffix, a head block H KV heads,
  // a column chunk up to 64 query rows.  The 4 waves of a workgroup take an
  // item's H heads x C column groups (C = 2 for chunks wider than 32 rows) x
  // S = 4 / (H C) block stripes, so one stage is S blocks of each head.  H is
  // the largest power of two that divides Hkv with H x C <= 4 for the unit's
  // widest chunk.  The lanes are laid end to end and the stream is cut into
  // one equal run of stages per persistent workgroup; a lane cut k times
  // yields k + 1 items (token pieces), and every piece has S stripe splits,
  // each with its own partial rows.
  const Tuning t = tuning();
  const bool mla = P->kind == kMla;
  P->item_cols = mla ? kItemColsMla : kItemColsGqa;
  const int H_div = hkv % 8 == 0 ? 8 : hkv % 4 == 0 ? 4 : hkv % 2 == 0 ? 2 : 1;
  struct Lane {
    int request, member_off, ncols, tok0, tok_end;
    int kv0, H, col0, col1;
    int S;       // block stripes
    int stream;  // kItemStream when every tile of the lane has one reader
    int64_t stages;
    int64_t base;
    int splits;
  };
  // Appends the lanes of one unit; returns the index of its first lane.
  auto add_lanes = [&](std::vector<Lane>& lanes, int tok0, int tok_end, int request, int member_off,
                       int ncols, bool one_reader, int* H_out, int* chunks_out) {
    const int first = (int)lanes.size();
    const int icols = P->item_cols;
    const int cmax = std::min(ncols, icols) > kWaveCols ? 2 : 1;
    // Latent cache: one head per item, its 4 waves split the item's up to
    // 128 query rows and share every block (no stripes).
    const int H = mla ? 1 : std::min(H_div, kItemWaves / cmax);
    const int chunks = (int)ceil_div(ncols, icols);
    const int64_t nblk = ceil_div((int64_t)tok_end - tok0, bs);
    for (int hb = 0; hb < hkv / H; ++hb)
      for (int c = 0; c < chunks; ++c) {
        const int col0 = c * icols, col1 = std::min(ncols, (c + 1) * icols);
        const int S = mla ? 1 : kItemWaves / (H * (col1 - col0 > kWaveCols ? 2 : 1));
        lanes.push_back(Lane{request, member_off, ncols, tok0, tok_end, hb * H, H, col0, col1, S,
                             one_reader ? kItemStream : 0, ceil_div(nblk, S), 0, 0});
      }
    *H_out = H;
    *chunks_out = chunks;
    return first;
  };
  // Cuts lanes [l0, l1) of `all` into one launch: its bins are appended to
  // P->bins / P->items.  An item's part_base holds its piece index until the
  // lane bases are known.
  std::vector<Lane> all;
  std::vector<int> item_lane;
  P->items.clear();
  P->bins.assign(1, 0);
  P->launches.clear();
  auto cut = [&](size_t l0, size_t l1, PassSet passes) {
    int64_t W = 0;
    for (size_t k = l0; k < l1; ++k) {
      W += all[k].stages;
    }
    const int64_t nb = std::min<int64_t>(W, (int64_t)n_cu_ * t.bins_per_cu);
    if (nb == 0) return;
    P->launches.push_back(Launch{(int)P->bins.size() - 1, (int)nb, passes});
    size_t li = l0;
    int64_t lpos = 0, pos = 0;
    for (int64_t b = 0; b < nb; ++b) {
      const int64_t end = (b + 1) * W / nb;
      while (pos < end) {
        Lane& L = all[li];
        const int64_t take = std::min(L.stages - lpos, end - pos);
        const int64_t stok = (int64_t)L.S * bs;  // tokens per stage
        WorkItem it{};
        it.request = L.request;
        it.tok_begin = (int)(L.tok0 + lpos * stok);
        it.tok_end = (int)std::min<int64_t>(L.tok0 + (lpos + take) * stok, L.tok_end);
        it.kv_head = L.kv0;
        it.kv_heads = L.H;
        it.member_off = L.member_off;
        it.ncols = L.ncols;
        it.col0 = L.col0;
        it.col1 = L.col1;
        it.part_base = L.splits++;
        it.stripes = L.S;
        it.flags = L.stream;
        P->items.push_back(it);
        item_lane.push_back((int)li);
        pos += take;
        lpos += take;
        if (lpos == L.stages) {
          ++li;
          lpos = 0;
        }
      }
      P->bins.push_back((int32_t)P->items.size());
      if (P->bins.back() == P->bins[P->bins.size() - 2]) throw std::logic_error("empty bin");
    }
  };

  // Latent cache: one persistent workgroup per compute unit, and the column
  // chunks of one large unit are cut at the same token boundaries and placed
  // on bins of one die (bin b runs on die b mod kXcds), so the chunks that
  // read the same key tiles at the same time share that die's L2: the
  // grouped pass then fetches each prefix block from HBM about once instead
  // of once per chunk.  Large units (several chunks, at least half the mean
  // bin load) go first, largest first, in pieces of about the mean bin load
  // on the least loaded bins; the other lanes are then poured in order into
  // the bins up to a common makespan.  Bins left empty are dropped.
  auto place = [&](size_t l0, size_t l1, PassSet passes) {
    int64_t W = 0;
    for (size_t k = l0; k < l1; ++k) W += all[k].stages;
    if (W == 0) return;
    const int nb = (int)std::min<int64_t>(W, n_cu_);
    const double T = (double)W / nb;
    struct Unit {
      size_t l0, l1;
    };
    std::vector<Unit> units;
    for (size_t k = l0; k < l1;) {
      size_t e = k + 1;
      while (e < l1 && all[e].request == all[k].request && all[e].member_off == all[k].member_off &&
             all[e].tok0 == all[k].tok0 && all[e].tok_end == all[k].tok_end)
        ++e;
      units.push_back(Unit{k, e});
      k = e;
    }
    auto large = [&](const Unit& u) { return u.l1 - u.l0 >= 2 && 2.0 * all[u.l0].stages >= T; };
    std::stable_partition(units.begin(), units.end(), large);
    const size_t n_large = std::count_if(units.begin(), units.end(), large);
    std::stable_sort(units.begin(), units.begin() + n_large, [&](const Unit& a, const Unit& b) {
      return all[a.l0].stages * (int64_t)(a.l1 - a.l0) > all[b.l0].stages * (int64_t)(b.l1 - b.l0);
    });
    std::vector<std::vector<std::pair<int, std::pair<int64_t, int64_t>>>> bin(nb);  // (lane, stages)
    std::vector<int64_t> load(nb, 0);
    const int per_die = (nb + kXcds - 1) / kXcds;
    std::vector<int> cand;
    for (size_t ui = 0; ui < n_large; ++ui) {
      const Unit& u = units[ui];
      const int64_t n = all[u.l0].stages;
      const int64_t pieces = std::max<int64_t>(1, std::min<int64_t>(n, std::llround(n / T)));
      const int C = (int)(u.l1 - u.l0);
      for (int64_t p = 0; p < pieces; ++p) {
        const int64_t s0 = p * n / pieces, s1 = (p + 1) * n / pieces;
        for (int c0 = 0; c0 < C; c0 += per_die) {
          const int cn = std::min(per_die, C - c0);
          // The die whose cn least loaded bins carry the least work.
          int best_x = 0;
          int64_t best = INT64_MAX;
          for (int x = 0; x < kXcds && x < nb; ++x) {
            cand.clear();
            for (int b = x; b < nb; b += kXcds) cand.push_back(b);
            if ((int)cand.size() < cn) continue;
            std::partial_sort(cand.begin(), cand.begin() + cn, cand.end(),
                              [&](int a, int b) { return load[a] < load[b]; });
            int64_t sum = 0;
            for (int j = 0; j < cn; ++j) sum += load[cand[j]];
            if (sum < best) {
              best = sum;
              best_x = x;
            }
          }
          cand.clear();
          for (int b = best_x; b < nb; b += kXcds) cand.push_back(b);
          const int take = std::min<int>(cn, (int)cand.size());
          std::partial_sort(cand.begin(), cand.begin() + take, cand.end(),
                            [&](int a, int b) { return load[a] < load[b]; });
          for (int j = 0; j < cn; ++j) {
            const int b = cand[j % take];
            bin[b].push_back({(int)(u.l0 + c0 + j), {s0, s1}});
            load[b] += s1 - s0;
          }
        }
      }
    }
    // Pour the other lanes, in order, into the room left under the makespan.
    int64_t M = (W + nb - 1) / nb;
    for (int b = 0; b < nb; ++b) M = std::max(M, load[b]);
    int fb = 0;
    for (size_t ui = n_large; ui < units.size(); ++ui)
      for (size_t k = units[ui].l0; k < units[ui].l1; ++k) {
        int64_t s0 = 0;
        const int64_t n = all[k].stages;
        while (s0 < n) {
          while (fb < nb && load[fb] >= M) ++fb;  // the room under M covers what is left
          if (fb == nb) throw std::logic_error("placement overflow");
          const int64_t take = std::min(n - s0, M - load[fb]);
          bin[fb].push_back({(int)k, {s0, s0 + take}});
          load[fb] += take;
          s0 += take;
        }
      }
    const int first = (int)P->bins.size() - 1;
    int used = 0;
    for (int b = 0; b < nb; ++b) {
      if (bin[b].empty()) continue;
      for (const auto& e : bin[b]) {
        Lane& L = all[e.first];
        const int64_t stok = (int64_t)L.S * bs;
        WorkItem it{};
        it.request = L.request;
        it.tok_begin = (int)(L.tok0 + e.second.first * stok);
        it.tok_end = (int)std::min<int64_t>(L.tok0 + e.second.second * stok, L.tok_end);
        it.kv_head = L.kv0;
        it.kv_heads = L.H;
        it.member_off = L.member_off;
        it.ncols = L.ncols;
        it.col0 = L.col0;
        it.col1 = L.col1;
        it.part_base = L.splits++;
        it.stripes = L.S;
        it.flags = L.stream;
        P->items.push_back(it);
        item_lane.push_back(e.first);
      }
      P->bins.push_back((int32_t)P->items.size());
      ++used;
    }
    if (used) P->launches.push_back(Launch{first, used, passes});
  };

  int64_t row = 0;
  for (int c = 0; c < G; ++c) {
    const fca_group_record& gr = P->groups[c];
    GroupMeta& gm = P->grp[c];
    gm.parent = gr.parent;
    gm.r0 = r0[c];
    gm.ncols = count[c] * r;
    gm.lane0 = -1;
    gm.H = 1;
    gm.chunks = 0;
    if (P->folded[c]) continue;  // read per request: no grouped work, on no merge path
    // The group's tiles have one reader when its query rows fit one wave
    // (one column chunk, one column group).
    gm.lane0 = add_lanes(all, gr.block_begin * bs, gr.block_end * bs, P->perm[r0[c]], r0[c], count[c] * r,
                         count[c] * r <= kWaveCols, &gm.H, &gm.chunks);
    unique += (int64_t)(gr.block_end - gr.block_begin) * bs;
  }
  const size_t n_glanes = all.size();
  P->req.assign(B, ReqMeta{});
  for (int i = 0; i < B; ++i) {
    ReqMeta& rq = P->req[i];
    rq.pos = pos[i];
    rq.deepest = eff_deep[i];
    rq.sfx_lane = -1;
    rq.sfx_H = 1;
    rq.sfx_chunks = 1;
    // A suffix has one reader in a cascade plan unless it took in a folded
    // group's blocks; without the cascade, shared prefixes are in every
    // member's suffix.
    const bool one_reader = !(P->desc.flags & FCA_PLAN_DISABLE_CASCADE) && eff_sb[i] == sfxb[i];
    if (sfx_tokens[i] > 0)
      rq.sfx_lane = add_lanes(all, P->req3[3 * i] * bs, lens[i], i, -1, r, one_reader, &rq.sfx_H, &rq.sfx_chunks);
  }
  auto schedule = [&](size_t l0, size_t l1, PassSet passes) {
    if (mla)
      place(l0, l1, passes);
    else
      cut(l0, l1, passes);
  };
  // Latent caches always launch the two passes one after the other: the
  // grouped pass then runs its die-aligned pieces alone, and the suffix
  // pieces are not left to the tails of the grouped bins (measured faster).
  if ((P->desc.flags & FCA_PLAN_SEPARATE_PASSES) || mla) {
    schedule(0, n_glanes, kGroupedPass);
    schedule(n_glanes, all.size(), kSuffixPass);
  } else {
    schedule(0, all.size(), kBothPasses);
  }
  for (Lane& L : all) {
    L.splits *= L.S;  // stripe splits of every piece
    L.base = row;
    row += (int64_t)L.splits * L.H * (L.col1 - L.col0);
  }
  if (row > INT32_MAX) return fail(FCA_ERR_UNSUPPORTED, "too many partial rows");
  P->items_g.clear();
  P->items_s.clear();
  for (size_t k = 0; k < P->items.size(); ++k) {
    WorkItem& it = P->items[k];
    const Lane& L = all[item_lane[k]];
    it.part_base = (int32_t)(L.base + (int64_t)it.part_base * L.S * L.H * (L.col1 - L.col0));
    (it.member_off >= 0 ? P->items_g : P->items_s).push_back(it);
  }
  P->lanes.clear();
  for (const Lane& L : all)
    P->lanes.push_back(LaneMeta{(int32_t)L.base, L.splits, L.kv0, L.H, L.col0, L.col1 - L.col0, 0, 0});

  // Merge sources: one per (request, query head, token split on its path),
  // as a flat table of partial-row indices the merge reads directly.
  P->src_off.assign((size_t)B * hq + 1, 0);
  P->src_row.clear();
  for (int i = 0; i < B; ++i)
    for (int h = 0; h < hq; ++h) {
      for_each_source(*P, i, h, [&](int64_t rw) { P->src_row.push_back((int32_t)rw); });
      if (P->src_row.size() > (size_t)INT32_MAX) return fail(FCA_ERR_UNSUPPORTED, "too many merge sources");
      P->src_off[(size_t)i * hq + h + 1] = (int32_t)P->src_row.size();
    }
  const int64_t sources = (int64_t)P->src_row.size();

  fca_plan_info& info = P->info;
  info.batch = B;
  info.num_groups = G;
  info.max_depth = max_depth;
  info.num_grouped_items = (int32_t)P->items_g.size();
  info.num_suffix_items = (int32_t)P->items_s.size();
  info.num_merge_sources = (int32_t)std::min<int64_t>(sources, INT32_MAX);
  info.num_partial_rows = row;
  info.logical_tokens = logical;
  info.unique_tokens = unique;
  info.num_folded_groups = n_folded;
  const size_t dv = (size_t)P->desc.head_dim_v;
  info.decode_workspace_bytes = align_up((size_t)row * dv * 4) + 2 * align_up((size_t)row * 4) + kAlign;
  return FCA_OK;
}

fca_status fca_plan_create(const int32_t* block_tables_dev, int64_t bt_row_stride, const int32_t* seq_lens_dev,
                           int32_t batch, int32_t max_blocks, const fca_attn_desc* desc, void* workspace_dev,
                           size_t workspace_bytes, void* stream, fca_plan* out) {
  fca_plan_s* P = nullptr;
  try {
    if (!out) return fail(FCA_ERR_INVALID_ARG, "out is NULL");
    Kind kind;
    fca_status st = check_desc(desc, &kind);
    if (st != FCA_OK) return st;
    if (batch < 0 || batch > kMaxBatch) return fail(FCA_ERR_INVALID_ARG, "batch %d outside [0, %d]", batch, kMaxBatch);
    if (max_blocks < 1 || max_blocks > kMaxTableWidth)
      return fail(FCA_ERR_INVALID_ARG, "max_blocks %d outside [1, %d]", max_blocks, kMaxTableWidth);
    if (batch > 0 && (!block_tables_dev || !seq_lens_dev))
      return fail(FCA_ERR_INVALID_ARG, "block_tables / seq_lens is NULL");
    if (batch > 0 && bt_row_stride < max_blocks)
      return fail(FCA_ERR_INVALID_ARG, "bt_row_stride %lld < max_blocks %d", (long long)bt_row_stride, max_blocks);
    if (!workspace_dev) return fail(FCA_ERR_INVALID_ARG, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(workspace_dev) % kAlign)
      return fail(FCA_ERR_WORKSPACE, "workspace must be %zu-byte aligned", kAlign);
    const Layout L = make_layout(batch, max_blocks);
    if (workspace_bytes < L.total)
      return fail(FCA_ERR_WORKSPACE, "plan workspace has %zu bytes, needs %zu", workspace_bytes, L.total);

    P = new fca_plan_s();
    P->desc = *desc;
    P->kind = kind;
    P->B = batch;
    P->W = max_blocks;
    P->r = desc->num_q_heads / desc->num_kv_heads;
    P->ws = static_cast<char*>(workspace_dev);
    P->L = L;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool cascade = !(desc->flags & FCA_PLAN_DISABLE_CASCADE);
    DiscoveryPtrs dp = discovery_ptrs(P->ws, L, batch);
    hipError_t e = launch_discovery(block_tables_dev, bt_row_stride, seq_lens_dev, batch, max_blocks,
                                    desc->block_size, desc->num_blocks, cascade, dp, s);
    if (e != hipSuccess) {
      delete P;
      return hip_fail(e, "discovery launch");
    }
    std::vector<int32_t> rb(L.readback_bytes / 4);
    char* stage = nullptr;
    e = stage_acquire(L.readback_bytes, &stage);
    if (e == hipSuccess) e = hipMemcpyAsync(stage, P->ws + L.header, L.readback_bytes, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
      delete P;
      return hip_fail(e, "discovery read-back");
    }
    std::memcpy(rb.data(), stage, L.readback_bytes);
    if (rb[kHdrErr]) {
      const int bad = rb[kHdrBadReq];
      const int err = rb[kHdrErr];
      delete P;
      return fail(FCA_ERR_BAD_TABLE, "request %d: %s", bad,
                  (err & kErrBadLen) ? "seq_len outside [0, max_blocks * block_size]"
                                     : "block ID outside [0, num_blocks) in a used slot");
    }
    int dev = 0, n_cu = 0;
    e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess || n_cu <= 0) {
      delete P;
      return hip_fail(e, "compute-unit count");
    }
    st = build_plan(P, rb, n_cu);
    if (st != FCA_OK) {
      delete P;
      return st;
    }
    // Plan-owned device copy of the schedule, packed in the pinned staging
    // buffer and uploaded with one copy.
    SchedLayout& S = P->SL;
    size_t off = 0;
    auto place = [&](size_t bytes) {
      const size_t at = off;
      off = align_up(off + std::max<size_t>(bytes, 1));
      return at;
    };
    const size_t n_heads = P->bins.size() - 1;
    S.items = place(P->items.size() * sizeof(WorkItem));
    S.heads = place(n_heads * sizeof(BinHead));
    S.perm = place(P->perm.size() * 4);
    S.src_off = place(P->src_off.size() * 4);
    S.src_row = place(P->src_row.size() * 4);
    S.total = off;
    P->dev = dev;
    P->stream = s;
    const SchedBuf kept = sched_take(dev, S.total);
    if (kept.ptr) {
      P->sched = kept.ptr;
      P->sched_cap = kept.cap;
      P->sched_done = kept.done;
    } else {
      const size_t cap = align_up(S.total + S.total / 4);
      e = hipMalloc(&P->sched, cap);
      if (e != hipSuccess) {
        P->sched = nullptr;
        delete P;
        return hip_fail(e, "schedule buffer");
      }
      P->sched_cap = cap;
    }
    e = stage_acquire(S.total, &stage);
    if (e != hipSuccess) {
      delete P;
      return hip_fail(e, "schedule staging");
    }
    std::memset(stage, 0, S.total);
    std::memcpy(stage + S.items, P->items.data(), P->items.size() * sizeof(WorkItem));
    BinHead* heads = reinterpret_cast<BinHead*>(stage + S.heads);
    for (size_t b = 0; b < n_heads; ++b) {
      heads[b].i_begin = P->bins[b];
      heads[b].i_end = P->bins[b + 1];
      heads[b].first = P->items[P->bins[b]];
    }
    std::memcpy(stage + S.perm, P->perm.data(), P->perm.size() * 4);
    std::memcpy(stage + S.src_off, P->src_off.data(), P->src_off.size() * 4);
    std::memcpy(stage + S.src_row, P->src_row.data(), P->src_row.size() * 4);
    e = hipMemcpyAsync(P->sched, stage, S.total, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = stage_in_use(s);
    if (e != hipSuccess) {
      delete P;
      return hip_fail(e, "schedule upload");
    }
    e = launch_bin_heads(reinterpret_cast<BinHead*>(P->sched + S.heads), (int)n_heads,
                         reinterpret_cast<const int32_t*>(P->ws + P->L.bt), P->W, P->desc.block_size, s);
    if (e != hipSuccess) {
      delete P;
      return hip_fail(e, "bin heads");
    }
    *out = P;
    return FCA_OK;
  } catch (const std::bad_alloc&) {
    delete P;
    return fail(FCA_ERR_HOST_ALLOC, "host allocation failed");
  } catch (const std::logic_error& x) {
    delete P;
    return fail(FCA_ERR_HIP, "internal planner error: %s", x.what());
  } catch (...) {
    delete P;
    return fail(FCA_ERR_HOST_ALLOC, "unexpected host exception");
  }
}

fca_status fca_plan_get_info(fca_plan plan, fca_plan_info* info) {
  if (!plan || !info) return fail(FCA_ERR_INVALID_ARG, "plan / info is NULL");
  *info = plan->info;
  return FCA_OK;
}

}  // extern "C"

namespace {

// Kernel arguments of one decode call: the attention launches' and the
// merge's.  Checks the caller's pointers and workspace.
fca_status decode_params(const fca_plan_s* P, const void* q_dev, const void* k_cache_dev, const void* v_cache_dev,
                         void* out_dev, float* lse_dev, void* workspace_dev, size_t workspace_bytes, GqaParams* gp,
                         MergeParams* mp) {
  if (!q_dev || !k_cache_dev || !out_dev || (!P->desc.v_aliases_k && !v_cache_dev))
    return fail(FCA_ERR_INVALID_ARG, "q / k_cache / v_cache / out is NULL");
  if (P->info.num_partial_rows > 0) {
    if (!workspace_dev) return fail(FCA_ERR_INVALID_ARG, "decode workspace is NULL");
    if (reinterpret_cast<uintptr_t>(workspace_dev) % kAlign)
      return fail(FCA_ERR_WORKSPACE, "decode workspace must be %zu-byte aligned", kAlign);
    if (workspace_bytes < P->info.decode_workspace_bytes)
      return fail(FCA_ERR_WORKSPACE, "decode workspace has %zu bytes, needs %zu", workspace_bytes,
                  P->info.decode_workspace_bytes);
  }
  const int64_t rows = P->info.num_partial_rows;
  const size_t dv = (size_t)P->desc.head_dim_v;
  char* w = static_cast<char*>(workspace_dev);
  PartialPtrs part;
  part.o = reinterpret_cast<float*>(w);
  part.m = reinterpret_cast<float*>(w + align_up((size_t)rows * dv * 4));
  part.l = reinterpret_cast<float*>(w + align_up((size_t)rows * dv * 4) + align_up((size_t)rows * 4));

  const Layout& L = P->L;
  const SchedLayout& S = P->SL;
  gp->perm = reinterpret_cast<const int32_t*>(P->sched + S.perm);
  gp->bt = reinterpret_cast<const int32_t*>(P->ws + L.bt);
  gp->W = P->W;
  gp->Hq = P->desc.num_q_heads;
  gp->r = P->r;
  gp->scale_log2 = P->desc.scale * 1.4426950408889634f;
  gp->q = q_dev;
  gp->k = k_cache_dev;
  gp->v = v_cache_dev;
  gp->k_stride_block = P->desc.k_stride_block;
  gp->k_stride_head = P->desc.k_stride_head;
  gp->v_stride_block = P->desc.v_stride_block;
  gp->v_stride_head = P->desc.v_stride_head;
  gp->part = part;
  gp->items = reinterpret_cast<const WorkItem*>(P->sched + S.items);
  gp->bins = nullptr;

  mp->src_off = reinterpret_cast<const int32_t*>(P->sched + S.src_off);
  mp->src_row = reinterpret_cast<const int32_t*>(P->sched + S.src_row);
  mp->B = P->B;
  mp->Hq = P->desc.num_q_heads;
  mp->Dv = P->desc.head_dim_v;
  mp->part = part;
  mp->out = out_dev;
  mp->lse = lse_dev;
  mp->out_f32 = (P->desc.flags & FCA_PLAN_OUT_F32) ? 1 : 0;
  return FCA_OK;
}

// Attention launch `k` of the plan.
hipError_t launch_pass(const fca_plan_s* P, GqaParams gp, int k, hipStream_t s) {
  const Launch& ln = P->launches[k];
  gp.bins = reinterpret_cast<const BinHead*>(P->sched + P->SL.heads) + ln.bin0;
  return P->kind == kMla ? launch_mla(gp, ln.n_bins, ln.passes == kGroupedPass, s)
                         : launch_attention(gp, ln.n_bins, s);
}

// Adds the time of attention launch `k` to the profile's per-pass sums.
void add_pass_time(const fca_plan_s* P, int k, double ms, fca_profile* acc) {
  acc->attention_ms += ms;
  if (P->launches[k].passes == kGroupedPass) acc->grouped_ms += ms;
  if (P->launches[k].passes == kSuffixPass) acc->suffix_ms += ms;
}

// Timing-only events: no system-scope fence when they complete, which keeps
// them from adding cache write-back to the launches they bracket.
hipError_t timing_event(hipEvent_t* ev) { return hipEventCreateWithFlags(ev, hipEventDisableSystemFence); }

}  // namespace

extern "C" {

fca_status fca_decode(fca_plan plan, const void* q_dev, const void* k_cache_dev, const void* v_cache_dev,
                      void* out_dev, float* lse_dev, void* workspace_dev, size_t workspace_bytes, void* stream) {
  if (!plan) return fail(FCA_ERR_INVALID_ARG, "plan is NULL");
  const fca_plan_s* P = plan;
  if (P->B == 0) return FCA_OK;
  GqaParams gp;
  MergeParams mp;
  fca_status st = decode_params(P, q_dev, k_cache_dev, v_cache_dev, out_dev, lse_dev, workspace_dev, workspace_bytes,
                                &gp, &mp);
  if (st != FCA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  fca_plan_s* M = plan;
  // Profiling events: start, then begin/end of each attention launch (up to
  // two), then begin/end of the merge.
  constexpr int kProf = 7;
  hipEvent_t ev[kProf] = {};
  if (P->profiling) {
    for (int j = 0; j < kProf; ++j) {
      if (M->event_pool.empty()) {
        e = timing_event(&ev[j]);
        if (e != hipSuccess) return hip_fail(e, "profiling event");
      } else {
        ev[j] = M->event_pool.back();
        M->event_pool.pop_back();
      }
      M->pending.push_back(ev[j]);
    }
  }
  auto mark = [&](int j) -> hipError_t { return ev[j] ? hipEventRecord(ev[j], s) : hipSuccess; };
#define FCA_TRY(expr, what)             \
  do {                                  \
    e = (expr);                         \
    if (e != hipSuccess) return hip_fail(e, what); \
  } while (0)
  FCA_TRY(mark(0), "event record");
  for (int k = 0; k < 2; ++k) {
    FCA_TRY(mark(1 + 2 * k), "event record");
    if (k < (int)P->launches.size()) FCA_TRY(launch_pass(P, gp, k, s), "attention launch");
    FCA_TRY(mark(2 + 2 * k), "event record");
  }
  FCA_TRY(mark(5), "event record");
  FCA_TRY(launch_merge(mp, s), "merge launch");
  FCA_TRY(mark(6), "event record");
#undef FCA_TRY
  return FCA_OK;
}

fca_status fca_time_launches(fca_plan plan, const void* q_dev, const void* const* k_caches,
                             const void* const* v_caches, int32_t n_caches, int32_t repeats, void* out_dev,
                             float* lse_dev, void* workspace_dev, size_t workspace_bytes, void* stream,
                             fca_profile* result) {
  if (!plan || !result) return fail(FCA_ERR_INVALID_ARG, "plan / result is NULL");
  if (!k_caches || (!plan->desc.v_aliases_k && !v_caches)) return fail(FCA_ERR_INVALID_ARG, "cache list is NULL");
  if (n_caches < 1 || repeats < 1) return fail(FCA_ERR_INVALID_ARG, "n_caches and repeats must be >= 1");
  const fca_plan_s* P = plan;
  fca_profile acc{};
  if (P->B == 0) {
    *result = acc;
    return FCA_OK;
  }
  const int n_launch = (int)P->launches.size();
  std::vector<GqaParams> gps(n_caches);
  MergeParams mp;
  for (int c = 0; c < n_caches; ++c) {
    fca_status st = decode_params(P, q_dev, k_caches[c], P->desc.v_aliases_k ? nullptr : v_caches[c], out_dev,
                                  lse_dev, workspace_dev, workspace_bytes, &gps[c], &mp);
    if (st != FCA_OK) return st;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  // events: begin/end of each attention launch's run, then of the merge's
  hipEvent_t ev[6] = {};
  hipError_t e = hipSuccess;
  const int n_ev = 2 * n_launch + 2;
  for (int j = 0; j < n_ev && e == hipSuccess; ++j) e = timing_event(&ev[j]);
  float t[3] = {0, 0, 0};
  if (e == hipSuccess) {
    // Each run issues one launch kind repeats x n_caches times back to back,
    // cycling the caches; the last attention launch is on the last cache, so
    // out / lse end up as the decode of that cache.
    for (int k = 0; k <= n_launch && e == hipSuccess; ++k) {
      e = hipEventRecord(ev[2 * k], s);
      for (int r = 0; r < repeats && e == hipSuccess; ++r)
        for (int c = 0; c < n_caches && e == hipSuccess; ++c)
          e = k < n_launch ? launch_pass(P, gps[c], k, s) : launch_merge(mp, s);
      if (e == hipSuccess) e = hipEventRecord(ev[2 * k + 1], s);
    }
  }
  if (e == hipSuccess) e = hipEventSynchronize(ev[n_ev - 1]);
  for (int k = 0; k <= n_launch && e == hipSuccess; ++k) e = hipEventElapsedTime(&t[k], ev[2 * k], ev[2 * k + 1]);
  for (int j = 0; j < n_ev; ++j)
    if (ev[j]) hipEventDestroy(ev[j]);
  if (e != hipSuccess) return hip_fail(e, "timed launches");
  const double n = (double)repeats * n_caches;
  for (int k = 0; k < n_launch; ++k) add_pass_time(P, k, t[k] / n, &acc);
  acc.merge_ms = t[n_launch] / n;
  acc.decode_ms = acc.attention_ms + acc.merge_ms;
  acc.calls = (int64_t)n;
  *result = acc;
  return FCA_OK;
}

fca_status fca_merge_states(int32_t n_states, const float* const* outs, const float* const* lses, int32_t batch,
                            int32_t num_heads, int32_t head_dim, void* out_dev, float* lse_dev, uint32_t flags,
                            void* stream) {
  if (n_states < 1 || n_states > kMaxStates)
    return fail(FCA_ERR_INVALID_ARG, "n_states %d outside [1, %d]", n_states, kMaxStates);
  if (batch < 0 || num_heads < 0) return fail(FCA_ERR_INVALID_ARG, "negative batch or num_heads");
  if ((int64_t)batch * num_heads >= ((int64_t)1 << 31)) return fail(FCA_ERR_INVALID_ARG, "batch * num_heads too large");
  if (head_dim != 128 && head_dim != 512) return fail(FCA_ERR_UNSUPPORTED, "head_dim %d is not built", head_dim);
  if (flags & ~FCA_MERGE_OUT_F32) return fail(FCA_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags);
  StatesParams sp;
  std::memset(&sp, 0, sizeof(sp));
  sp.n = n_states;
  sp.pairs = batch * num_heads;
  sp.D = head_dim;
  sp.out = out_dev;
  sp.lse = lse_dev;
  sp.out_f32 = (flags & FCA_MERGE_OUT_F32) ? 1 : 0;
  if (sp.pairs == 0) return FCA_OK;
  if (!outs || !lses || !out_dev) return fail(FCA_ERR_INVALID_ARG, "outs / lses / out is NULL");
  for (int j = 0; j < n_states; ++j) {
    if (!outs[j] || !lses[j]) return fail(FCA_ERR_INVALID_ARG, "state %d is NULL", j);
    sp.outs[j] = outs[j];
    sp.lses[j] = lses[j];
  }
  const hipError_t e = launch_merge_states(sp, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  return FCA_OK;
}

fca_status fca_kv_append(const fca_attn_desc* desc, const void* k_new_dev, const void* v_new_dev, void* k_cache_dev,
                         void* v_cache_dev, int32_t* block_tables_dev, int64_t bt_row_stride, int32_t max_blocks,
                         const int32_t* seq_lens_dev, const int32_t* cow_dst_dev, int32_t* status_dev, int32_t batch,
                         void* stream) {
  Kind kind;
  fca_status st = check_desc(desc, &kind);
  if (st != FCA_OK) return st;
  if (batch < 0 || batch > kMaxBatch) return fail(FCA_ERR_INVALID_ARG, "batch %d outside [0, %d]", batch, kMaxBatch);
  if (max_blocks < 1 || max_blocks > kMaxTableWidth)
    return fail(FCA_ERR_INVALID_ARG, "max_blocks %d outside [1, %d]", max_blocks, kMaxTableWidth);
  if (bt_row_stride < max_blocks) return fail(FCA_ERR_INVALID_ARG, "bt_row_stride < max_blocks");
  if (batch == 0) return FCA_OK;
  const bool alias = desc->v_aliases_k != 0;
  if (!k_new_dev || !k_cache_dev || !block_tables_dev || !seq_lens_dev || (!alias && (!v_new_dev || !v_cache_dev)))
    return fail(FCA_ERR_INVALID_ARG, "k_new / v_new / caches / block_tables / seq_lens is NULL");
  auto misaligned = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) != 0; };
  if (misaligned(k_new_dev) || misaligned(k_cache_dev) || (!alias && (misaligned(v_new_dev) || misaligned(v_cache_dev))))
    return fail(FCA_ERR_INVALID_ARG, "new rows and caches must be 16-byte aligned");
  AppendParams p;
  p.k_new = static_cast<const uint16_t*>(k_new_dev);
  p.v_new = alias ? nullptr : static_cast<const uint16_t*>(v_new_dev);
  p.k_cache = static_cast<uint16_t*>(k_cache_dev);
  p.v_cache = alias ? nullptr : static_cast<uint16_t*>(v_cache_dev);
  p.block_tables = block_tables_dev;
  p.bt_row_stride = bt_row_stride;
  p.seq_lens = seq_lens_dev;
  p.cow_dst = cow_dst_dev;
  p.status = status_dev;
  p.k_stride_block = desc->k_stride_block;
  p.k_stride_head = desc->k_stride_head;
  p.v_stride_block = alias ? 0 : desc->v_stride_block;
  p.v_stride_head = alias ? 0 : desc->v_stride_head;
  p.batch = batch;
  p.num_kv_heads = desc->num_kv_heads;
  p.max_blocks = max_blocks;
  p.num_blocks = desc->num_blocks;
  const hipError_t e = launch_append(p, kind == kMla, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "append launch");
  return FCA_OK;
}

fca_status fca_profile_enable(fca_plan plan, int32_t enable) {
  if (!plan) return fail(FCA_ERR_INVALID_ARG, "plan is NULL");
  plan->profiling = enable != 0;
  return FCA_OK;
}

fca_status fca_profile_read(fca_plan plan, fca_profile* out) {
  if (!plan || !out) return fail(FCA_ERR_INVALID_ARG, "plan / out is NULL");
  fca_profile acc{};
  hipError_t err = hipSuccess;
  // events per call: start, launch 1 begin/end, launch 2 begin/end, merge begin/end
  const int n_launch = (int)plan->launches.size();
  for (size_t c = 0; c + 7 <= plan->pending.size(); c += 7) {
    hipEvent_t* ev = plan->pending.data() + c;
    float t[4] = {0, 0, 0, 0};
    if (err == hipSuccess) err = hipEventSynchronize(ev[6]);
    if (err == hipSuccess) err = hipEventElapsedTime(&t[0], ev[1], ev[2]);
    if (err == hipSuccess) err = hipEventElapsedTime(&t[1], ev[3], ev[4]);
    if (err == hipSuccess) err = hipEventElapsedTime(&t[2], ev[5], ev[6]);
    if (err == hipSuccess) err = hipEventElapsedTime(&t[3], ev[0], ev[6]);
    for (int k = 0; k < n_launch && k < 2; ++k) add_pass_time(plan, k, t[k], &acc);
    acc.merge_ms += t[2];
    acc.decode_ms += t[3];
    acc.calls += 1;
  }
  plan->event_pool.insert(plan->event_pool.end(), plan->pending.begin(), plan->pending.end());
  plan->pending.clear();
  if (err != hipSuccess) return hip_fail(err, "profiling events");
  *out = acc;
  return FCA_OK;
}

fca_status fca_plan_export(fca_plan plan, fca_group_record* groups, int32_t* members, int32_t* requests) {
  if (!plan) return fail(FCA_ERR_INVALID_ARG, "plan is NULL");
  if (groups) std::copy(plan->groups.begin(), plan->groups.end(), groups);
  if (members) std::copy(plan->members.begin(), plan->members.end(), members);
  if (requests) std::copy(plan->req3.begin(), plan->req3.end(), requests);
  return FCA_OK;
}

fca_status fca_plan_export_folded(fca_plan plan, int32_t* folded) {
  if (!plan || !folded) return fail(FCA_ERR_INVALID_ARG, "plan / folded is NULL");
  std::copy(plan->folded.begin(), plan->folded.end(), folded);
  return FCA_OK;
}

fca_status fca_plan_export_schedule(fca_plan plan, fca_work_item* grouped, fca_work_item* suffix, int32_t* src_off,
                                    int32_t* src) {
  if (!plan) return fail(FCA_ERR_INVALID_ARG, "plan is NULL");
  const fca_plan_s* P = plan;
  if (grouped) std::memcpy(grouped, P->items_g.data(), P->items_g.size() * sizeof(WorkItem));
  if (suffix) std::memcpy(suffix, P->items_s.data(), P->items_s.size() * sizeof(WorkItem));
  if (src_off || src) {
    const int hq = P->desc.num_q_heads;
    int64_t n = 0;
    for (int i = 0; i < P->B; ++i)
      for (int h = 0; h < hq; ++h) {
        if (src_off) src_off[(int64_t)i * hq + h] = (int32_t)n;
        for_each_source(*P, i, h, [&](int64_t row) {
          if (src) src[n] = (int32_t)row;
          ++n;
        });
      }
    if (src_off) src_off[(int64_t)P->B * hq] = (int32_t)n;
  }
  return FCA_OK;
}

void fca_plan_destroy(fca_plan plan) { delete plan; }

}  // extern "C"
