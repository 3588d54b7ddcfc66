// Host-only driver of the planner (shared_prefix_kv_amd/csrc/planner.cpp)
// for CPU tests: reads one discovery read-back from a text file, runs
// build_plan, and prints the plan (canonical grouping, schedule, merge
// sources) as text.  Built with AddressSanitizer and UndefinedBehaviorSanitizer
// by tests/test_planner_cpu.py; no GPU and no HIP involved.
//
// Input (whitespace-separated integers):
//   B W block_size num_q_heads num_kv_heads head_dim_qk head_dim_v latent flags n_cu repeats
//   G
//   G records: leader depth parent begin end count
//   B lengths, B deepest group ids, B suffix starts
// Output: "status <code> <message>" and, on success, one line per part of
// the plan (see print_plan).  With repeats > 1 the planner runs that many
// times and "time_us <mean>" reports its average host time.

#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "plan_types.h"

using namespace fca;

namespace {

bool read_ints(FILE* f, int n, std::vector<int32_t>* out) {
  out->resize(n);
  for (int k = 0; k < n; ++k)
    if (fscanf(f, "%d", &(*out)[k]) != 1) return false;
  return true;
}

void print_items(const char* name, const std::vector<WorkItem>& v) {
  printf("%s %zu", name, v.size());
  for (const WorkItem& it : v)
    printf(" %d %d %d %d %d %d %d %d %d %d %d %d", it.request, it.tok_begin, it.tok_end, it.kv_head, it.member_off,
           it.ncols, it.col0, it.col1, it.part_base, it.kv_heads, it.stripes, it.flags);
  printf("\n");
}

void print_ints(const char* name, const std::vector<int32_t>& v) {
  printf("%s %zu", name, v.size());
  for (int32_t x : v) printf(" %d", x);
  printf("\n");
}

void print_plan(const PlanHost& P) {
  const fca_plan_info& in = P.info;
  printf("info %d %d %d %d %d %d %lld %lld %lld %zu %d\n", in.batch, in.num_groups, in.max_depth,
         in.num_grouped_items, in.num_suffix_items, in.num_merge_sources, (long long)in.num_partial_rows,
         (long long)in.logical_tokens, (long long)in.unique_tokens, in.decode_workspace_bytes, in.num_folded_groups);
  printf("groups %zu", P.groups.size());
  for (const fca_group_record& g : P.groups)
    printf(" %d %d %d %d %d %d", g.depth, g.parent, g.block_begin, g.block_end, g.member_begin, g.member_count);
  printf("\n");
  print_ints("members", P.members);
  print_ints("folded", P.folded);
  print_ints("requests", P.req3);
  print_items("grouped", pass_items(P, true));
  print_items("suffix", pass_items(P, false));
  // merge sources in the order of fca_plan_export_schedule
  const int hq = P.desc.num_q_heads;
  std::vector<int32_t> off, src;
  for (int i = 0; i < P.B; ++i)
    for (int h = 0; h < hq; ++h) {
      off.push_back((int32_t)src.size());
      for_each_source(P, i, h, [&](int64_t row) { src.push_back((int32_t)row); });
    }
  off.push_back((int32_t)src.size());
  print_ints("src_off", off);
  print_ints("src", src);
  printf("max_pair_sources %lld\n", (long long)P.max_pair_sources);
  // bins: items per persistent workgroup, and the launches
  print_ints("bins", P.bins);
  printf("launches %zu", P.launches.size());
  for (const Launch& l : P.launches) printf(" %d %d %d", l.bin0, l.n_bins, (int)l.passes);
  printf("\n");
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s input.txt\n", argv[0]);
    return 2;
  }
  FILE* f = fopen(argv[1], "r");
  if (!f) return 2;
  int B, W, bs, hq, hkv, dqk, dv, latent, flags, n_cu, repeats, G;
  if (fscanf(f, "%d %d %d %d %d %d %d %d %d %d %d %d", &B, &W, &bs, &hq, &hkv, &dqk, &dv, &latent, &flags, &n_cu,
             &repeats, &G) != 12)
    return 2;
  std::vector<int32_t> rec, lens, deep, sfx;
  if (G < 0 || B < 0 || !read_ints(f, G * 6, &rec) || !read_ints(f, B, &lens) || !read_ints(f, B, &deep) ||
      !read_ints(f, B, &sfx))
    return 2;
  fclose(f);
  std::vector<int32_t> header(kHdrWords, 0), records((size_t)std::max(B, 1) * kRecordInts, 0);
  header[kHdrGroups] = G;
  for (int g = 0; g < G; ++g)
    for (int k = 0; k < 6; ++k) records[(size_t)g * kRecordInts + k] = rec[(size_t)g * 6 + k];
  DiscoveryView d{header.data(), lens.data(), deep.data(), sfx.data(), records.data()};

  auto fresh = [&]() {
    PlanHost P;
    P.desc = fca_attn_desc{};
    P.desc.num_q_heads = hq;
    P.desc.num_kv_heads = hkv;
    P.desc.head_dim_qk = dqk;
    P.desc.head_dim_v = dv;
    P.desc.block_size = bs;
    P.desc.v_aliases_k = latent;
    P.desc.flags = (uint32_t)flags;
    P.kind = latent ? kMla : kGqa;
    P.B = B;
    P.W = W;
    P.r = hq / hkv;
    return P;
  };
  PlanHost P;
  std::string err;
  fca_status st = FCA_OK;
  const auto t0 = std::chrono::steady_clock::now();
  for (int rep = 0; rep < std::max(repeats, 1); ++rep) {
    P = fresh();
    try {
      st = build_plan(P, d, n_cu, &err);
    } catch (const std::exception& x) {
      printf("status -1 exception %s\n", x.what());
      return 0;
    }
    if (st != FCA_OK) break;
  }
  const double us = std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now() - t0).count() /
                    std::max(repeats, 1);
  printf("status %d %s\n", (int)st, st == FCA_OK ? "ok" : err.c_str());
  if (st == FCA_OK) {
    print_plan(P);
    printf("time_us %.1f\n", us);
  }
  return 0;
}
