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

constexpr size_t kAlign = kWsAlign;
size_t align_up(size_t x) { return ws_align_up(x); }

fca_status check_desc(const fca_attn_desc* d, Kind* kind) {
  if (!d) return fail(FCA_ERR_INVALID_ARG, "desc is NULL");
  if (d->reserved != 0) return fail(FCA_ERR_INVALID_ARG, "desc.reserved must be 0");
  if (d->num_q_heads <= 0 || d->num_kv_heads <= 0 || d->num_q_heads % d->num_kv_heads)
    return fail(FCA_ERR_INVALID_ARG, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                d->num_q_heads, d->num_kv_heads);
  if (d->num_blocks <= 0) return fail(FCA_ERR_INVALID_ARG, "num_blocks must be positive");
  if (!(d->scale > 0.f) || !std::isfinite(d->scale)) return fail(FCA_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (d->flags & ~(FCA_PLAN_DISABLE_CASCADE | FCA_PLAN_SEPARATE_PASSES | FCA_PLAN_OUT_F32 | FCA_PLAN_AUTO_FOLD |
                   FCA_PLAN_KEEP_GROUPS))
    return fail(FCA_ERR_INVALID_ARG, "unknown flag bits 0x%x", d->flags);
  const int r = d->num_q_heads / d->num_kv_heads;
  const bool rows = d->k_stride_token != 0;  // token rows, else tiles
  if (d->k_stride_token < 0 || d->v_stride_token < 0)
    return fail(FCA_ERR_INVALID_ARG, "token strides must not be negative");
  if (d->head_dim_qk == 128 && d->head_dim_v == 128 && d->block_size == 16 && !d->v_aliases_k) {
    if (r > 16) return fail(FCA_ERR_UNSUPPORTED, "GQA ratio %d > 16 is not built", r);
    if (rows != (d->v_stride_token != 0))
      return fail(FCA_ERR_INVALID_ARG, "k_stride_token and v_stride_token must both be 0 (tiles) or both positive");
    if (rows) {
      if (d->k_stride_token < 128 || d->v_stride_token < 128 || d->k_stride_head < 128 || d->v_stride_head < 128 ||
          d->k_stride_block < 128 || d->v_stride_block < 128)
        return fail(FCA_ERR_INVALID_ARG, "cache strides are shorter than a 128-dim row");
    } else if (d->k_stride_head < 128 * 16 || d->v_stride_head < 128 * 16 ||
               d->k_stride_block < (int64_t)d->num_kv_heads * d->k_stride_head ||
               d->v_stride_block < (int64_t)d->num_kv_heads * d->v_stride_head) {
      return fail(FCA_ERR_INVALID_ARG, "cache strides overlap tiles");
    }
    if ((d->k_stride_head | d->k_stride_block | d->v_stride_head | d->v_stride_block | d->k_stride_token |
         d->v_stride_token) % 8)
      return fail(FCA_ERR_INVALID_ARG, "cache strides must keep 16-byte alignment");
    *kind = kGqa;
    return FCA_OK;
  }
  if (d->head_dim_qk == 576 && d->head_dim_v == 512 && d->block_size == 64 && d->v_aliases_k) {
    if (rows) {
      if (d->k_stride_token < 576 || d->k_stride_token > (1 << 20))
        return fail(FCA_ERR_INVALID_ARG, "latent k_stride_token must lie in [576, 2^20]");
      if (d->k_stride_head < 0 || d->k_stride_block < 576)
        return fail(FCA_ERR_INVALID_ARG, "latent cache strides are shorter than a 576-dim row");
    } else if (d->k_stride_head < 576 * 64 || d->k_stride_block < (int64_t)d->num_kv_heads * d->k_stride_head) {
      return fail(FCA_ERR_INVALID_ARG, "cache strides overlap tiles");
    }
    if ((d->k_stride_head | d->k_stride_block | d->k_stride_token) % 8)
      return fail(FCA_ERR_INVALID_ARG, "cache strides must keep 16-byte alignment");
    *kind = kMla;
    return FCA_OK;
  }
  return fail(FCA_ERR_UNSUPPORTED, "unsupported shape: head_dim_qk=%d head_dim_v=%d block_size=%d v_aliases_k=%d",
              d->head_dim_qk, d->head_dim_v, d->block_size, d->v_aliases_k);
}

constexpr int kStateArrays = 10;  // per-request discovery state (DiscoveryPtrs)

// Caller-owned plan workspace: discovery read-back region, table copy and
// discovery state.  Its size depends only on (batch, max_blocks).
struct Layout {
  size_t header, lens, deepest, sfx_begin, records, readback_bytes;
  size_t bt, state;
  size_t total;
  int W4;  // row stride of the table copy: the width rounded up to 4 (16-byte rows)
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
  L.W4 = (W + 3) / 4 * 4;
  L.bt = off;
  off = align_up(off + b * (size_t)L.W4 * 4 + kLcpTail * 4);
  L.state = off;
  off = align_up(off + kStateArrays * b * 4);
  L.total = off;
  return L;
}

// Plan-owned device buffer holding the schedule.
struct SchedLayout {
  size_t items, heads, perm, req, grp, lanes, counter, upload;  // uploaded from the host: [0, upload)
  size_t src_span, src_row, total;                              // merge tables, built on the device
  int32_t src_stride;  // > 0: fixed-stride merge table (entries per (request, head))
  size_t src_rows;     // entries of src_row
};

// Merge-table stride for a plan: the bound on any (request, head)'s partial
// rows when it fits one wave's lanes and the padding stays modest (at most
// twice the rows, or 64 Ki entries), else 0 (packed tables).  Developer knob:
// FCA_TUNE_MERGE_PACKED=1 keeps packed tables.
int32_t merge_stride(int64_t pairs, int64_t rows, int64_t most) {
  const char* v = getenv("FCA_TUNE_MERGE_PACKED");
  if (v && atoi(v) == 1) return 0;
  if (most < 1 || most > 64) return 0;
  const int64_t entries = pairs * most;
  if (entries > std::max<int64_t>(2 * rows, rows + (1 << 16)) || entries > INT32_MAX) return 0;
  return (int32_t)most;
}


DiscoveryPtrs discovery_ptrs(char* ws, const Layout& L, int B) {
  DiscoveryPtrs p;
  p.header = reinterpret_cast<int32_t*>(ws + L.header);
  p.lens = reinterpret_cast<int32_t*>(ws + L.lens);
  p.deepest = reinterpret_cast<int32_t*>(ws + L.deepest);
  p.sfx_begin = reinterpret_cast<int32_t*>(ws + L.sfx_begin);
  p.records = reinterpret_cast<int32_t*>(ws + L.records);
  p.bt = reinterpret_cast<int32_t*>(ws + L.bt);
  int32_t* st = reinterpret_cast<int32_t*>(ws + L.state);
  int32_t** arr[] = {&p.nfull, &p.root, &p.depth_at, &p.node, &p.gdepth, &p.gparent, &p.active, &p.lcp0, &p.ngid,
                     &p.first};
  for (int a = 0; a < kStateArrays; ++a) *arr[a] = st + (size_t)a * B;
  return p;
}


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

struct fca_plan_s : PlanHost {
  char* ws;
  Layout L;
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
    hipError_t e = launch_discovery(block_tables_dev, bt_row_stride, seq_lens_dev, batch, max_blocks, L.W4,
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
    {
      const int32_t* hdr = rb.data();
      DiscoveryView dv;
      dv.header = hdr;
      dv.lens = hdr + (L.lens - L.header) / 4;
      dv.deepest = hdr + (L.deepest - L.header) / 4;
      dv.sfx_begin = hdr + (L.sfx_begin - L.header) / 4;
      dv.records = hdr + (L.records - L.header) / 4;
      std::string msg;
      st = build_plan(*P, dv, n_cu, &msg);
      if (st != FCA_OK) {
        delete P;
        return fail(st, "%s", msg.c_str());
      }
    }
    // Plan-owned device copy of the schedule, packed in the pinned staging
    // buffer and uploaded with one copy; the merge tables are then built on
    // the device from the uploaded metadata.
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
    S.req = place(P->req.size() * sizeof(ReqMeta));
    S.grp = place(P->grp.size() * sizeof(GroupMeta));
    S.lanes = place(P->lanes.size() * sizeof(LaneMeta));
    S.counter = place(4);  // zero in the upload: the merge-table kernel's row counter
    S.upload = off;
    const int64_t pairs = (int64_t)P->B * P->desc.num_q_heads;
    S.src_stride = merge_stride(pairs, P->info.num_partial_rows, P->max_pair_sources);
    S.src_rows = (size_t)std::max<int64_t>(P->info.num_partial_rows, pairs * S.src_stride);
    S.src_span = place((size_t)pairs * 8);
    S.src_row = place(S.src_rows * 4);
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
    e = stage_acquire(S.upload, &stage);
    if (e != hipSuccess) {
      delete P;
      return hip_fail(e, "schedule staging");
    }
    std::memset(stage, 0, S.upload);
    std::memcpy(stage + S.items, P->items.data(), P->items.size() * sizeof(WorkItem));
    BinHead* heads = reinterpret_cast<BinHead*>(stage + S.heads);
    for (size_t b = 0; b < n_heads; ++b) {
      heads[b].i_begin = P->bins[b];
      heads[b].i_end = P->bins[b + 1];
      heads[b].first = P->items[P->bins[b]];
    }
    std::memcpy(stage + S.perm, P->perm.data(), P->perm.size() * 4);
    std::memcpy(stage + S.req, P->req.data(), P->req.size() * sizeof(ReqMeta));
    std::memcpy(stage + S.grp, P->grp.data(), P->grp.size() * sizeof(GroupMeta));
    std::memcpy(stage + S.lanes, P->lanes.data(), P->lanes.size() * sizeof(LaneMeta));
    e = hipMemcpyAsync(P->sched, stage, S.upload, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = stage_in_use(s);
    if (e != hipSuccess) {
      delete P;
      return hip_fail(e, "schedule upload");
    }
    {
      TableParams tp;
      tp.req = reinterpret_cast<const ReqMeta*>(P->sched + S.req);
      tp.grp = reinterpret_cast<const GroupMeta*>(P->sched + S.grp);
      tp.lanes = reinterpret_cast<const LaneMeta*>(P->sched + S.lanes);
      tp.B = P->B;
      tp.Hq = P->desc.num_q_heads;
      tp.r = P->r;
      tp.item_cols = P->item_cols;
      tp.src_span = reinterpret_cast<int2*>(P->sched + S.src_span);
      tp.src_row = reinterpret_cast<int32_t*>(P->sched + S.src_row);
      tp.total = reinterpret_cast<int32_t*>(P->sched + S.counter);
      tp.stride = S.src_stride;
      tp.heads = reinterpret_cast<BinHead*>(P->sched + S.heads);
      tp.n_bins = (int32_t)n_heads;
      tp.bt = reinterpret_cast<const int32_t*>(P->ws + P->L.bt);
      tp.W4 = P->L.W4;
      tp.bs = P->desc.block_size;
      e = launch_plan_tables(tp, s);
      if (e != hipSuccess) {
        delete P;
        return hip_fail(e, "plan tables");
      }
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

// Device scratch of fca_decode_no_alloc: the partial (o, max, denominator)
// rows of one decode, for callers that cannot allocate.  One copy per
// device, held until the process ends; its device address is looked up once
// per device (the host-side name is not a device address).
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

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
  gp->W = P->L.W4;
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
  gp->k_stride_token = P->desc.k_stride_token;
  gp->v_stride_token = P->desc.v_aliases_k ? 0 : P->desc.v_stride_token;
  gp->part = part;
  gp->items = reinterpret_cast<const WorkItem*>(P->sched + S.items);
  gp->bins = nullptr;

  mp->src_span = reinterpret_cast<const int2*>(P->sched + S.src_span);
  mp->src_row = reinterpret_cast<const int32_t*>(P->sched + S.src_row);
  mp->src_stride = S.src_stride;
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
                         : launch_attention(gp, ln.n_bins, ln.passes, s);
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

// One decode: the plan's attention launches, then the merge.  Profiling
// events are recorded only when `profile` is set and the plan asks for them.
fca_status decode_impl(fca_plan plan, const void* q_dev, const void* k_cache_dev, const void* v_cache_dev,
                       void* out_dev, float* lse_dev, void* workspace_dev, size_t workspace_bytes, void* stream,
                       bool profile) {
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
  if (profile && P->profiling) {
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

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

fca_status scratch_for_device(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(FCA_ERR_UNSUPPORTED, "device %d: scratch kept for %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "scratch address");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return FCA_OK;
}

}  // namespace

extern "C" {

fca_status fca_decode(fca_plan plan, const void* q_dev, const void* k_cache_dev, const void* v_cache_dev,
                      void* out_dev, float* lse_dev, void* workspace_dev, size_t workspace_bytes, void* stream) {
  if (!plan) return fail(FCA_ERR_INVALID_ARG, "plan is NULL");
  return decode_impl(plan, q_dev, k_cache_dev, v_cache_dev, out_dev, lse_dev, workspace_dev, workspace_bytes, stream,
                     true);
}

fca_status fca_decode_no_alloc(fca_plan plan, const void* q_dev, const void* k_cache_dev, const void* v_cache_dev,
                               void* out_dev, float* lse_dev, void* stream) {
  if (!plan) return fail(FCA_ERR_INVALID_ARG, "plan is NULL");
  const fca_plan_s* P = plan;
  if (P->B == 0) return FCA_OK;
  if (P->info.decode_workspace_bytes > kScratchBytes)
    return fail(FCA_ERR_WORKSPACE, "decode needs %zu bytes of scratch, the static scratch holds %zu",
                P->info.decode_workspace_bytes, kScratchBytes);
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "current device");
  if (dev != P->dev) return fail(FCA_ERR_INVALID_ARG, "plan was made on device %d, device %d is current", P->dev, dev);
  void* ws = nullptr;
  const fca_status st = scratch_for_device(dev, &ws);
  if (st != FCA_OK) return st;
  return decode_impl(plan, q_dev, k_cache_dev, v_cache_dev, out_dev, lse_dev, ws, kScratchBytes, stream, false);
}

fca_status fca_decode_layers(fca_plan plan, int32_t n_layers, const void* const* q_dev, const void* const* k_caches_dev,
                             const void* const* v_caches_dev, void* const* out_dev, float* const* lse_dev,
                             void* workspace_dev, size_t workspace_bytes, void* stream) {
  if (!plan) return fail(FCA_ERR_INVALID_ARG, "plan is NULL");
  if (n_layers < 0) return fail(FCA_ERR_INVALID_ARG, "n_layers %d < 0", n_layers);
  const fca_plan_s* P = plan;
  if (P->B == 0 || n_layers == 0) return FCA_OK;
  if (!q_dev || !k_caches_dev || !out_dev || (!P->desc.v_aliases_k && !v_caches_dev))
    return fail(FCA_ERR_INVALID_ARG, "q / k_caches / v_caches / out array is NULL");
  try {
    // Every layer's arguments are checked before the first launch.
    std::vector<GqaParams> gps(n_layers);
    std::vector<MergeParams> mps(n_layers);
    for (int l = 0; l < n_layers; ++l) {
      fca_status st = decode_params(P, q_dev[l], k_caches_dev[l], P->desc.v_aliases_k ? nullptr : v_caches_dev[l],
                                    out_dev[l], lse_dev ? lse_dev[l] : nullptr, workspace_dev, workspace_bytes,
                                    &gps[l], &mps[l]);
      if (st != FCA_OK) {
        char buf[600];
        snprintf(buf, sizeof(buf), "layer %d: %s", l, g_last_error.c_str());
        return fail(st, "%s", buf);
      }
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int l = 0; l < n_layers; ++l) {
      for (int k = 0; k < (int)P->launches.size(); ++k) {
        const hipError_t e = launch_pass(P, gps[l], k, s);
        if (e != hipSuccess) return hip_fail(e, "attention launch");
      }
      const hipError_t e = launch_merge(mps[l], s);
      if (e != hipSuccess) return hip_fail(e, "merge launch");
    }
    return FCA_OK;
  } catch (const std::bad_alloc&) {
    return fail(FCA_ERR_HOST_ALLOC, "host allocation failed");
  }
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
    if (ev[j]) (void)hipEventDestroy(ev[j]);
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

fca_status fca_kv_append_layers(const fca_attn_desc* desc, int32_t n_layers, const void* const* k_new_dev,
                                const void* const* v_new_dev, void* const* k_caches_dev, void* const* v_caches_dev,
                                int32_t* block_tables_dev, int64_t bt_row_stride, int32_t max_blocks,
                                const int32_t* seq_lens_dev, const int32_t* cow_dst_dev, int32_t* status_dev,
                                int32_t batch, void* stream) {
  Kind kind;
  fca_status st = check_desc(desc, &kind);
  if (st != FCA_OK) return st;
  if (n_layers < 0) return fail(FCA_ERR_INVALID_ARG, "n_layers %d < 0", n_layers);
  if (batch < 0 || batch > kMaxBatch) return fail(FCA_ERR_INVALID_ARG, "batch %d outside [0, %d]", batch, kMaxBatch);
  if (max_blocks < 1 || max_blocks > kMaxTableWidth)
    return fail(FCA_ERR_INVALID_ARG, "max_blocks %d outside [1, %d]", max_blocks, kMaxTableWidth);
  if (bt_row_stride < max_blocks) return fail(FCA_ERR_INVALID_ARG, "bt_row_stride < max_blocks");
  if (batch == 0 || n_layers == 0) return FCA_OK;
  const bool alias = desc->v_aliases_k != 0;
  if (!k_new_dev || !k_caches_dev || !block_tables_dev || !seq_lens_dev || (!alias && (!v_new_dev || !v_caches_dev)))
    return fail(FCA_ERR_INVALID_ARG, "k_new / v_new / caches / block_tables / seq_lens is NULL");
  auto misaligned = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) != 0; };
  for (int l = 0; l < n_layers; ++l) {
    if (!k_new_dev[l] || !k_caches_dev[l] || (!alias && (!v_new_dev[l] || !v_caches_dev[l])))
      return fail(FCA_ERR_INVALID_ARG, "layer %d: k_new / v_new / cache is NULL", l);
    if (misaligned(k_new_dev[l]) || misaligned(k_caches_dev[l]) ||
        (!alias && (misaligned(v_new_dev[l]) || misaligned(v_caches_dev[l]))))
      return fail(FCA_ERR_INVALID_ARG, "layer %d: new rows and caches must be 16-byte aligned", l);
  }
  AppendParams p;
  std::memset(&p, 0, sizeof(p));
  p.block_tables = block_tables_dev;
  p.bt_row_stride = bt_row_stride;
  p.seq_lens = seq_lens_dev;
  p.cow_dst = cow_dst_dev;
  p.k_stride_block = desc->k_stride_block;
  p.k_stride_head = desc->k_stride_head;
  p.v_stride_block = alias ? 0 : desc->v_stride_block;
  p.v_stride_head = alias ? 0 : desc->v_stride_head;
  p.k_stride_token = desc->k_stride_token;
  p.v_stride_token = alias ? 0 : desc->v_stride_token;
  p.batch = batch;
  p.num_kv_heads = desc->num_kv_heads;
  p.max_blocks = max_blocks;
  p.num_blocks = desc->num_blocks;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // Every layer reads the table as the caller left it; the entries of copied
  // blocks are rewritten once, after the last layer.
  for (int l0 = 0; l0 < n_layers; l0 += kAppendLayers) {
    p.n_layers = std::min(kAppendLayers, n_layers - l0);
    for (int l = 0; l < p.n_layers; ++l) {
      p.k_new[l] = static_cast<const uint16_t*>(k_new_dev[l0 + l]);
      p.k_cache[l] = static_cast<uint16_t*>(k_caches_dev[l0 + l]);
      p.v_new[l] = alias ? nullptr : static_cast<const uint16_t*>(v_new_dev[l0 + l]);
      p.v_cache[l] = alias ? nullptr : static_cast<uint16_t*>(v_caches_dev[l0 + l]);
    }
    const hipError_t e = launch_append(p, kind == kMla, s);
    if (e != hipSuccess) return hip_fail(e, "append launch");
  }
  const hipError_t e = launch_append_commit(block_tables_dev, bt_row_stride, seq_lens_dev, cow_dst_dev, status_dev,
                                            batch, max_blocks, desc->block_size, desc->num_blocks, s);
  if (e != hipSuccess) return hip_fail(e, "append commit launch");
  return FCA_OK;
}

fca_status fca_kv_append(const fca_attn_desc* desc, const void* k_new_dev, const void* v_new_dev, void* k_cache_dev,
                         void* v_cache_dev, int32_t* block_tables_dev, int64_t bt_row_stride, int32_t max_blocks,
                         const int32_t* seq_lens_dev, const int32_t* cow_dst_dev, int32_t* status_dev, int32_t batch,
                         void* stream) {
  const void* kn[1] = {k_new_dev};
  const void* vn[1] = {v_new_dev};
  void* kc[1] = {k_cache_dev};
  void* vc[1] = {v_cache_dev};
  return fca_kv_append_layers(desc, 1, kn, vn, kc, vc, block_tables_dev, bt_row_stride, max_blocks, seq_lens_dev,
                              cow_dst_dev, status_dev, batch, stream);
}

fca_status fca_measure_read_bandwidth(const void* const* bufs_dev, int32_t n_bufs, size_t bytes, int32_t repeats,
                                      void* stream, double* gbps) {
  if (!bufs_dev || !gbps) return fail(FCA_ERR_INVALID_ARG, "buffers / gbps is NULL");
  if (n_bufs < 1 || repeats < 1) return fail(FCA_ERR_INVALID_ARG, "n_bufs and repeats must be >= 1");
  if (bytes < 16 || bytes % 16) return fail(FCA_ERR_INVALID_ARG, "bytes must be a positive multiple of 16");
  for (int b = 0; b < n_bufs; ++b)
    if (!bufs_dev[b] || reinterpret_cast<uintptr_t>(bufs_dev[b]) % 16)
      return fail(FCA_ERR_INVALID_ARG, "buffer %d is NULL or not 16-byte aligned", b);
  int dev = 0, n_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "compute-unit count");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t ev[2] = {nullptr, nullptr};
  for (int j = 0; j < 2 && e == hipSuccess; ++j) e = timing_event(&ev[j]);
  // Each launch shape: one untimed pass over every buffer, then the timed
  // ones; the faster shape is reported.
  float ms = 0.f;
  for (int shape = 0; shape < kReadShapes && e == hipSuccess; ++shape) {
    for (int b = 0; b < n_bufs && e == hipSuccess; ++b) e = launch_stream_read(bufs_dev[b], bytes, n_cu, shape, s);
    if (e == hipSuccess) e = hipEventRecord(ev[0], s);
    for (int r = 0; r < repeats && e == hipSuccess; ++r)
      for (int b = 0; b < n_bufs && e == hipSuccess; ++b) e = launch_stream_read(bufs_dev[b], bytes, n_cu, shape, s);
    if (e == hipSuccess) e = hipEventRecord(ev[1], s);
    if (e == hipSuccess) e = hipEventSynchronize(ev[1]);
    float t = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&t, ev[0], ev[1]);
    if (e == hipSuccess && t > 0.f && (ms == 0.f || t < ms)) ms = t;
  }
  for (int j = 0; j < 2; ++j)
    if (ev[j]) (void)hipEventDestroy(ev[j]);
  if (e != hipSuccess) return hip_fail(e, "read probe");
  *gbps = ms > 0.f ? (double)bytes * repeats * n_bufs / (ms * 1e-3) / 1e9 : 0.0;
  return FCA_OK;
}

fca_status fca_measure_mfma_rate(int32_t dtype, int32_t iters, void* stream, double* tflops) {
  if (!tflops) return fail(FCA_ERR_INVALID_ARG, "tflops is NULL");
  if (dtype != FCA_MFMA_BF16 && dtype != FCA_MFMA_F16) return fail(FCA_ERR_INVALID_ARG, "dtype must be FCA_MFMA_BF16 or FCA_MFMA_F16");
  if (iters < 1 || iters > (1 << 20)) return fail(FCA_ERR_INVALID_ARG, "iters must be in [1, 2^20]");
  int dev = 0, n_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "compute-unit count");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf16 = dtype == FCA_MFMA_BF16;
  hipEvent_t ev[2] = {nullptr, nullptr};
  for (int j = 0; j < 2 && e == hipSuccess; ++j) e = timing_event(&ev[j]);
  // One untimed launch, then the timed one.
  if (e == hipSuccess) e = launch_mfma_rate(bf16, iters, n_cu, s);
  if (e == hipSuccess) e = hipEventRecord(ev[0], s);
  if (e == hipSuccess) e = launch_mfma_rate(bf16, iters, n_cu, s);
  if (e == hipSuccess) e = hipEventRecord(ev[1], s);
  if (e == hipSuccess) e = hipEventSynchronize(ev[1]);
  float ms = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, ev[0], ev[1]);
  for (int j = 0; j < 2; ++j)
    if (ev[j]) (void)hipEventDestroy(ev[j]);
  if (e != hipSuccess) return hip_fail(e, "MFMA-rate probe");
  const double flops = (double)std::max(1, n_cu) * (kMfmaThreads / 64) * (double)iters * kMfmaPerIter * (2.0 * 16 * 16 * 32);
  *tflops = ms > 0.f ? flops / (ms * 1e-3) / 1e12 : 0.0;
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
  try {
    if (grouped) {
      const std::vector<WorkItem> v = pass_items(*P, true);
      std::memcpy(grouped, v.data(), v.size() * sizeof(WorkItem));
    }
    if (suffix) {
      const std::vector<WorkItem> v = pass_items(*P, false);
      std::memcpy(suffix, v.data(), v.size() * sizeof(WorkItem));
    }
    if ((src_off || src) && P->B > 0) {
      // the merge tables as the device built them, in (request, head) order
      const size_t pairs = (size_t)P->B * P->desc.num_q_heads;
      std::vector<int2> span(pairs);
      std::vector<int32_t> rows(P->SL.src_rows);
      hipError_t e = hipMemcpyAsync(span.data(), P->sched + P->SL.src_span, pairs * sizeof(int2), hipMemcpyDeviceToHost,
                                    P->stream);
      if (e == hipSuccess && !rows.empty())
        e = hipMemcpyAsync(rows.data(), P->sched + P->SL.src_row, rows.size() * 4, hipMemcpyDeviceToHost, P->stream);
      if (e == hipSuccess) e = hipStreamSynchronize(P->stream);
      if (e != hipSuccess) return hip_fail(e, "merge table read-back");
      int64_t n = 0;
      for (size_t q = 0; q < pairs; ++q) {
        if (span[q].x < 0 || span[q].y < 0 || (size_t)span[q].x + span[q].y > rows.size())
          return fail(FCA_ERR_HIP, "merge table entry %zu out of range", q);
        if (src_off) src_off[q] = (int32_t)n;
        if (src) std::memcpy(src + n, rows.data() + span[q].x, (size_t)span[q].y * 4);
        n += span[q].y;
      }
      if (src_off) src_off[pairs] = (int32_t)n;
    } else if (src_off) {
      src_off[0] = 0;
    }
    return FCA_OK;
  } catch (const std::bad_alloc&) {
    return fail(FCA_ERR_HOST_ALLOC, "host allocation failed");
  }
}

void fca_plan_destroy(fca_plan plan) { delete plan; }

}  // extern "C"
