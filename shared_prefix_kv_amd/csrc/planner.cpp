// Host planner: from the discovery read-back to the canonical grouping, the
// split schedule of both attention passes and the merge tables.  Plain C++
// (no HIP calls), so that it also builds and runs on its own on the CPU.
//
// The grouping is the prefix forest the discovery kernels found (ZoRRo
// Inference & Forest Cascade Attention page, "Core Mechanism", step 1);
// this file puts it in the canonical order (smallest member, depth), lays
// every group's members out contiguously, decides which groups pay for their
// partial rows (the activation heuristic), and cuts the work of the grouped
// and per-request passes (steps 2) into one run per persistent workgroup;
// the merge tables list, per (request, query head), the partial rows its
// exact log-sum-exp combination reads (step 3).

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <stdexcept>
#include <string>
#include <vector>

#include "plan_types.h"

namespace fca {
namespace {

fca_status pfail(std::string* err, fca_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  if (err) *err = buf;
  return st;
}

int env_int(const char* name, int dflt) {
  const char* s = getenv(name);
  if (!s || !*s) return dflt;
  const int v = atoi(s);
  return v > 0 ? v : dflt;
}

// Split-schedule targets (developer tuning knobs).
struct Tuning {
  int bins_per_cu;  // attention workgroups per compute unit; 0: chosen from the batch's bytes
  int wide_cost;    // cost of a stage of a two-column-group lane, in hundredths of another
};

// A GQA stage is one (block, head) K+V tile per wave.  In a lane of more
// than 32 query rows its two column-group waves each load every tile and
// take two 16-column product tiles, and a stage took 1.1-1.2x the time of a
// stage of a per-request lane (4 rows) on MI355X; the equal-work cut weighs
// it accordingly (long_rl attention launch 544 -> 519 us; 1.10-1.20 within
// 1 % of each other on forest_mixed).  Lanes of up to 32 rows keep weight
// 1: weighing them too made the Llama-3-8B batch slower.
constexpr int kWideStageCost = 115;

Tuning tuning() {
  Tuning t;
  t.bins_per_cu = env_int("FCA_TUNE_BINS_PER_CU", 0);
  t.wide_cost = env_int("FCA_TUNE_WIDE_COST", kWideStageCost);
  return t;
}

// Persistent workgroups per compute unit of a GQA launch.  Two per unit
// hide each other's stalls on small batches; on large ones a single
// workgroup per unit cuts every lane into half as many token pieces (half
// the partial rows and merge reads) and was as fast or faster on MI355X:
// equal at 3.2 GB of unique KV, 7 % faster at 4.6 GB, 3 % slower at 0.3 GB.
constexpr double kOneBinBytesPerCu = 4.0 * (1 << 20);

int bins_per_cu(const Tuning& t, double unique_bytes, int n_cu) {
  if (t.bins_per_cu > 0) return t.bins_per_cu;
  return unique_bytes >= kOneBinBytesPerCu * n_cu ? 1 : 2;
}

constexpr int kXcds = 8;  // accelerator dies per device; workgroup b is dispatched to die b mod 8
constexpr int kItemColsMla = 64;   // query rows of one latent-cache work item at most
constexpr int kItemWaves = kAttnWaves;  // waves per work item: heads x column groups x block stripes
constexpr int kWaveCols = 32;  // query rows one wave covers at most

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The read-back describes a forest over the batch: group ids in range, a
// parent one level up, nested block ranges inside the table, lengths and
// suffix starts consistent with them.  Anything else is reported instead of
// being followed (a parent cycle, an index past an array).
fca_status check_readback(const PlanHost& P, const DiscoveryView& d, std::string* err) {
  const int B = P.B, W = P.W, bs = P.desc.block_size;
  const int G = d.header[kHdrGroups];
  if (G < 0 || G > std::max(B - 1, 0))
    return pfail(err, FCA_ERR_HIP, "discovery produced %d groups for %d requests", G, B);
  for (int g = 0; g < G; ++g) {
    const int32_t* x = d.records + (size_t)g * kRecordInts;
    const int leader = x[0], depth = x[1], parent = x[2], b0 = x[3], b1 = x[4], cnt = x[5];
    if (leader < 0 || leader >= B || cnt < 2 || cnt > B || b0 < 0 || b1 <= b0 || b1 > W)
      return pfail(err, FCA_ERR_HIP, "inconsistent discovery output (group record %d)", g);
    if (parent < -1 || parent >= G)
      return pfail(err, FCA_ERR_HIP, "inconsistent discovery output (parent of group record %d)", g);
    if (parent < 0 ? depth != 0 : (depth != d.records[(size_t)parent * kRecordInts + 1] + 1 ||
                                   b0 != d.records[(size_t)parent * kRecordInts + 4]))
      return pfail(err, FCA_ERR_HIP, "inconsistent discovery output (nesting of group record %d)", g);
    if (parent < 0 && b0 != 0)
      return pfail(err, FCA_ERR_HIP, "inconsistent discovery output (root group record %d)", g);
  }
  for (int i = 0; i < B; ++i) {
    const int L = d.lens[i], g = d.deepest[i], sb = d.sfx_begin[i];
    if (L < 0 || (int64_t)L > (int64_t)W * bs || g < -1 || g >= G || sb < 0 || (int64_t)sb * bs > L)
      return pfail(err, FCA_ERR_HIP, "inconsistent discovery output (request %d)", i);
    if (sb != (g >= 0 ? d.records[(size_t)g * kRecordInts + 4] : 0))
      return pfail(err, FCA_ERR_HIP, "inconsistent discovery output (suffix of request %d)", i);
  }
  return FCA_OK;
}

// Values grouped by key in [0, n), each group in the order the values come
// (a counting sort; two flat arrays instead of one vector per key).
struct KeyLists {
  std::vector<int> at;   // [n + 1]: group k is val[at[k], at[k + 1])
  std::vector<int> val;
  // key(j) for j in [0, m): a key in [0, n), or -1 to leave value j out
  template <class Key>
  void build(int n, int m, Key key) {
    at.assign((size_t)n + 1, 0);
    for (int j = 0; j < m; ++j)
      if (key(j) >= 0) ++at[(size_t)key(j) + 1];
    for (int k = 0; k < n; ++k) at[(size_t)k + 1] += at[k];
    val.resize(at[n]);
    std::vector<int> fill(at.begin(), at.end() - 1);
    for (int j = 0; j < m; ++j)
      if (key(j) >= 0) val[fill[key(j)]++] = j;
  }
  int size(int k) const { return at[(size_t)k + 1] - at[k]; }
  const int* begin(int k) const { return val.data() + at[k]; }
  const int* end(int k) const { return val.data() + at[(size_t)k + 1]; }
};

}  // namespace

fca_status build_plan(PlanHost& plan, const DiscoveryView& disc, int n_cu_, std::string* err) {
  PlanHost* P = &plan;
  const int B = P->B;
  const int bs = P->desc.block_size;
  const int hkv = P->desc.num_kv_heads;
  const int hq = P->desc.num_q_heads;
  const int r = P->r;
  const int32_t* hdr = disc.header;
  const int32_t* lens = disc.lens;
  const int32_t* deep = disc.deepest;
  const int32_t* sfxb = disc.sfx_begin;
  const int32_t* rec = disc.records;
  const int G = hdr[kHdrGroups];
  {
    const fca_status st = check_readback(*P, disc, err);
    if (st != FCA_OK) return st;
  }

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
    if (gr.parent < 0) roots.push_back(c);
  }
  std::vector<int> deepest_c(B);
  for (int i = 0; i < B; ++i) deepest_c[i] = deep[i] >= 0 ? canon[deep[i]] : -1;
  KeyLists children, direct;  // child groups of each group; requests whose deepest group it is
  children.build(G, G, [&](int c) { return P->groups[c].parent; });
  direct.build(G, B, [&](int i) { return deepest_c[i]; });

  // Depth-first member order: every group is the contiguous range [r0, r1).
  P->perm.clear();
  P->perm.reserve(B);
  std::vector<int> r0(G), r1(G);
  {
    std::vector<std::pair<int, size_t>> stack;  // (group, next child)
    for (int root : roots) {
      stack.push_back({root, 0});
      r0[root] = (int)P->perm.size();
      P->perm.insert(P->perm.end(), direct.begin(root), direct.end(root));
      while (!stack.empty()) {
        auto& top = stack.back();
        const int c = top.first;
        if ((int)top.second < children.size(c)) {
          const int ch = children.begin(c)[top.second++];
          r0[ch] = (int)P->perm.size();
          P->perm.insert(P->perm.end(), direct.begin(ch), direct.end(ch));
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
  if ((int)P->perm.size() != B) return pfail(err, FCA_ERR_HIP, "inconsistent discovery output (member order)");
  std::vector<int> pos(B);
  for (int k = 0; k < B; ++k) pos[P->perm[k]] = k;

  P->members.clear();
  for (int c = 0; c < G; ++c) {
    if (r1[c] - r0[c] != count[c] || count[c] < 2)
      return pfail(err, FCA_ERR_HIP, "inconsistent discovery output (group %d: %d members, range %d)", c, count[c],
                  r1[c] - r0[c]);
    const size_t at = P->members.size();
    P->groups[c].member_begin = (int32_t)at;
    P->groups[c].member_count = count[c];
    P->members.insert(P->members.end(), P->perm.begin() + r0[c], P->perm.begin() + r1[c]);
    std::sort(P->members.begin() + at, P->members.end());
  }

  // Activation (GQA caches, unless FCA_PLAN_KEEP_GROUPS): a group is read
  // once for all members only if that saves more bytes than its partial
  // rows cost.
  // Reading a group of n members over T tokens once instead of n times
  // saves (n - 1) T t bytes (t: KV bytes per token); in exchange, each of
  // its token pieces writes n Hq partial rows that the merge reads back, and
  // a written byte costs about three read bytes here, so 4 (4 Dv + 8) bytes
  // per row.  The pieces are estimated as the group's bytes over one
  // workgroup's share of all unique bytes.  Leaves first: a group is folded
  // only when all its children are.
  const Tuning t = tuning();
  const double tok_bytes = (double)hkv * (P->desc.head_dim_qk + P->desc.head_dim_v) * 2;
  double unique_tok = 0;  // with every group read once
  for (int i = 0; i < B; ++i) unique_tok += lens[i] - bs * sfxb[i];
  for (int c = 0; c < G; ++c) unique_tok += (double)(P->groups[c].block_end - P->groups[c].block_begin) * bs;
  const int bpc = bins_per_cu(t, unique_tok * tok_bytes, n_cu_);

  P->folded.assign(G, 0);
  int n_folded = 0;
  std::vector<int> eff_deep(deepest_c);
  std::vector<int> eff_sb(sfxb, sfxb + B);
  if (!(P->desc.flags & FCA_PLAN_KEEP_GROUPS) && P->kind == kGqa && G > 0) {
    const double share = std::max(unique_tok * tok_bytes / ((double)n_cu_ * bpc), 1.0);
    const double row_cost = 4.0 * (4.0 * P->desc.head_dim_v + 8.0);
    for (int c = G - 1; c >= 0; --c) {  // children come after their parents
      bool leaves_folded = true;
      for (const int* ch = children.begin(c); ch != children.end(c); ++ch)
        leaves_folded = leaves_folded && P->folded[*ch];
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
    if (sfx_tokens[i] < 0) return pfail(err, FCA_ERR_HIP, "inconsistent discovery output (suffix of request %d)", i);
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
    int cost;  // of one stage in the cut (hundredths)
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
        const int C = col1 - col0 > kWaveCols ? 2 : 1;
        const int S = mla ? 1 : kItemWaves / (H * C);
        const int cost = !mla && C == 2 ? t.wide_cost : 100;
        lanes.push_back(Lane{request, member_off, ncols, tok0, tok_end, hb * H, H, col0, col1, S,
                             one_reader ? kItemStream : 0, ceil_div(nblk, S), 0, 0, cost});
      }
    *H_out = H;
    *chunks_out = chunks;
    return first;
  };
  // Cuts lanes [l0, l1) of `all` into one launch: its bins are appended to
  // P->bins / P->items.  An item's part_base holds its piece index until the
  // lane bases are known.
  std::vector<Lane> all;
  all.reserve((size_t)(G + B) * hkv * 2);
  std::vector<int> item_lane;
  P->items.clear();
  P->bins.assign(1, 0);
  P->launches.clear();
  auto cut = [&](size_t l0, size_t l1, PassSet passes) {
    int64_t W = 0, n_st = 0;  // cost and stages of the launch
    for (size_t k = l0; k < l1; ++k) {
      W += all[k].stages * all[k].cost;
      n_st += all[k].stages;
    }
    const int64_t nb = std::min<int64_t>(n_st, (int64_t)n_cu_ * bpc);
    if (nb == 0) return;
    // every bin boundary cuts at most one lane: items <= lanes + bins
    P->items.reserve(P->items.size() + (l1 - l0) + (size_t)nb);
    item_lane.reserve(P->items.capacity());
    P->bins.reserve(P->bins.size() + (size_t)nb);
    P->launches.push_back(Launch{(int)P->bins.size() - 1, (int)nb, passes});
    size_t li = l0;
    int64_t lpos = 0, pos = 0, rem = n_st;
    for (int64_t b = 0; b < nb; ++b) {
      // Bin b ends at cost (b + 1) W / nb, rounded up to whole stages; it
      // takes at least one stage and leaves at least one for each later bin.
      const int64_t end = (b + 1) * W / nb;
      const int64_t cap = rem - (nb - 1 - b);
      int64_t got = 0;
      while ((pos < end || got == 0) && got < cap) {
        Lane& L = all[li];
        const int64_t want = pos < end ? ceil_div(end - pos, (int64_t)L.cost) : 1;
        const int64_t take = std::min({L.stages - lpos, want, cap - got});
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
        pos += take * L.cost;
        got += take;
        rem -= take;
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
    // (bin, lane, stage range) of every piece, in placement order; emitted
    // bin by bin (stable) at the end
    struct Piece {
      int bin, lane;
      int64_t s0, s1;
    };
    std::vector<Piece> placed;
    placed.reserve((l1 - l0) * 4 + (size_t)nb);
    std::vector<int64_t> load(nb, 0);
    const int per_die = (nb + kXcds - 1) / kXcds;
    // The bins of each die, kept sorted by (load, bin).
    std::vector<std::vector<int>> die(kXcds);
    for (int b = 0; b < nb; ++b) die[b % kXcds].push_back(b);
    auto by_load = [&](int a, int b) { return load[a] != load[b] ? load[a] < load[b] : a < b; };
    // When every large unit has the same number of chunks C, the bins of
    // each die are grouped into tuples of C, the units are laid end to end
    // and the stream is cut into one equal run per tuple; chunk c of a piece
    // goes to bin c of its tuple.  Whole pieces of about T per unit instead
    // left bins of up to 1.5 T (the latent per-request pass: 30 stages
    // against a mean of 20.7, the launch ending at 40 us against 28).
    bool same_c = n_large > 0;
    for (size_t ui = 1; ui < n_large && same_c; ++ui)
      same_c = units[ui].l1 - units[ui].l0 == units[0].l1 - units[0].l0;
    const int Cu = same_c ? (int)(units[0].l1 - units[0].l0) : 0;
    std::vector<int> tuple_bin;  // bins of tuple k: [k C, k C + C)
    if (same_c)
      for (int j = 0;; ++j) {  // tuple j of every die in turn: consecutive tuples on different dies
        bool any = false;
        for (int x = 0; x < kXcds; ++x)
          if ((int)die[x].size() >= (j + 1) * Cu) {
            for (int c = 0; c < Cu; ++c) tuple_bin.push_back(die[x][j * Cu + c]);
            any = true;
          }
        if (!any) break;
      }
    const int64_t n_tuples = same_c ? (int64_t)(tuple_bin.size() / Cu) : 0;
    if (n_tuples > 0) {
      int64_t Wl = 0;  // stages of one chunk, summed over the large units
      for (size_t ui = 0; ui < n_large; ++ui) Wl += all[units[ui].l0].stages;
      const int64_t nt = std::min<int64_t>(n_tuples, Wl);
      size_t ui = 0;
      int64_t upos = 0, pos = 0;
      for (int64_t k = 0; k < nt; ++k) {
        const int64_t end = (k + 1) * Wl / nt;
        while (pos < end) {
          const Unit& u = units[ui];
          const int64_t n = all[u.l0].stages;
          const int64_t take = std::min(n - upos, end - pos);
          for (int c = 0; c < Cu; ++c) {
            const int b = tuple_bin[k * Cu + c];
            placed.push_back(Piece{b, (int)(u.l0 + c), upos, upos + take});
            load[b] += take;
          }
          pos += take;
          upos += take;
          if (upos == n) {
            ++ui;
            upos = 0;
          }
        }
      }
    }
    for (size_t ui = 0; ui < (n_tuples > 0 ? 0 : n_large); ++ui) {
      const Unit& u = units[ui];
      const int64_t n = all[u.l0].stages;
      const int64_t pieces = std::max<int64_t>(1, std::min<int64_t>(n, std::llround(n / T)));
      const int C = (int)(u.l1 - u.l0);
      for (int64_t p = 0; p < pieces; ++p) {
        const int64_t s0 = p * n / pieces, s1 = (p + 1) * n / pieces;
        for (int c0 = 0; c0 < C; c0 += per_die) {
          const int cn = std::min(per_die, C - c0);
          // The die whose cn least loaded bins carry the least work.
          int best_x = -1;
          int64_t best = INT64_MAX;
          for (int x = 0; x < kXcds && x < nb; ++x) {
            if ((int)die[x].size() < cn) continue;
            int64_t sum = 0;
            for (int j = 0; j < cn; ++j) sum += load[die[x][j]];
            if (sum < best) {
              best = sum;
              best_x = x;
            }
          }
          if (best_x < 0) best_x = 0;  // fewer bins per die than chunks: reuse the least loaded ones
          std::vector<int>& cand = die[best_x];
          const int take = std::min<int>(cn, (int)cand.size());
          for (int j = 0; j < cn; ++j) {
            const int b = cand[j % take];
            placed.push_back(Piece{b, (int)(u.l0 + c0 + j), s0, s1});
            load[b] += s1 - s0;
          }
          std::sort(cand.begin(), cand.end(), by_load);
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
          placed.push_back(Piece{fb, (int)k, s0, s0 + take});
          load[fb] += take;
          s0 += take;
        }
      }
    {  // stable counting sort by bin
      std::vector<int> at((size_t)nb + 1, 0);
      for (const Piece& e : placed) ++at[(size_t)e.bin + 1];
      for (int b = 0; b < nb; ++b) at[(size_t)b + 1] += at[b];
      std::vector<Piece> by_bin(placed.size());
      for (const Piece& e : placed) by_bin[at[e.bin]++] = e;
      placed.swap(by_bin);
    }
    const int first = (int)P->bins.size() - 1;
    int used = 0;
    P->items.reserve(P->items.size() + placed.size());
    item_lane.reserve(P->items.capacity());
    for (size_t q = 0; q < placed.size();) {
      const int b = placed[q].bin;
      for (; q < placed.size() && placed[q].bin == b; ++q) {
        const Piece& e = placed[q];
        Lane& L = all[e.lane];
        const int64_t stok = (int64_t)L.S * bs;
        WorkItem it{};
        it.request = L.request;
        it.tok_begin = (int)(L.tok0 + e.s0 * stok);
        it.tok_end = (int)std::min<int64_t>(L.tok0 + e.s1 * stok, L.tok_end);
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
        item_lane.push_back(e.lane);
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
  if (row > INT32_MAX) return pfail(err, FCA_ERR_UNSUPPORTED, "too many partial rows");
  int64_t n_grouped_items = 0;
  for (size_t k = 0; k < P->items.size(); ++k) {
    WorkItem& it = P->items[k];
    const Lane& L = all[item_lane[k]];
    it.part_base = (int32_t)(L.base + (int64_t)it.part_base * L.S * L.H * (L.col1 - L.col0));
    n_grouped_items += it.member_off >= 0;
  }
  P->lanes.clear();
  P->lanes.reserve(all.size());
  for (const Lane& L : all)
    P->lanes.push_back(LaneMeta{(int32_t)L.base, L.splits, L.kv0, L.H, L.col0, L.col1 - L.col0, 0, 0});

  // The most partial rows one (request, head) can merge: per request, the
  // most splits of any lane of each group on its path plus the most of any
  // lane of its suffix.
  {
    std::vector<int32_t> gmax(G, 0);
    for (int c = 0; c < G; ++c) {
      const GroupMeta& gm = P->grp[c];
      if (gm.lane0 < 0) continue;  // folded
      const int n = (hkv / gm.H) * gm.chunks;
      for (int k = 0; k < n; ++k) gmax[c] = std::max(gmax[c], P->lanes[gm.lane0 + k].splits);
    }
    int64_t most = 0;
    for (const ReqMeta& rq : P->req) {
      int64_t n = 0;
      for (int g = rq.deepest; g >= 0; g = P->grp[g].parent) n += gmax[g];
      if (rq.sfx_lane >= 0) {
        const int m = (hkv / rq.sfx_H) * rq.sfx_chunks;
        int32_t most_s = 0;
        for (int k = 0; k < m; ++k) most_s = std::max(most_s, P->lanes[rq.sfx_lane + k].splits);
        n += most_s;
      }
      most = std::max(most, n);
    }
    P->max_pair_sources = most;
  }

  // Merge sources: every partial row is read by exactly one (request, query
  // head), so there are as many sources as rows.  The table itself (per
  // (request, head) the rows of its path, for_each_source order) is built on
  // the device from req / grp / lanes.
  const int64_t sources = row;

  fca_plan_info& info = P->info;
  info.batch = B;
  info.num_groups = G;
  info.max_depth = max_depth;
  info.num_grouped_items = (int32_t)n_grouped_items;
  info.num_suffix_items = (int32_t)((int64_t)P->items.size() - n_grouped_items);
  info.num_merge_sources = (int32_t)std::min<int64_t>(sources, INT32_MAX);
  info.num_partial_rows = row;
  info.logical_tokens = logical;
  info.unique_tokens = unique;
  info.num_folded_groups = n_folded;
  const size_t dv = (size_t)P->desc.head_dim_v;
  info.decode_workspace_bytes = ws_align_up((size_t)row * dv * 4) + 2 * ws_align_up((size_t)row * 4) + kWsAlign;
  return FCA_OK;
}

}  // namespace fca
