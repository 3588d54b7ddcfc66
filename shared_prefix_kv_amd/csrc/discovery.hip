// Prefix-forest discovery over block IDs (gfx950).
//
// Groups are the requests whose block tables start with the same physical
// block IDs (ZoRRo Inference & Forest Cascade Attention page, "Core
// Mechanism", step 1: discover groups of requests sharing a KV-cache prefix;
// PagedAttention vs. RadixAttention page, "How PagedAttention Works", step 4:
// requests with the same prompt reference the same physical blocks).  Only
// full blocks take part; every node of the compressed trie of the rows that
// two or more requests pass through is a group.
//
// Kernels:
//   k_init_header  clears the counters and error flags.
//   k_prepare      copies the used table entries into the plan workspace,
//                  checks block IDs and lengths, initialises per-request state.
//   k_roots        one wave per request: the smallest request index with the
//                  same first block (the tree a request belongs to).
//   k_trees        one workgroup per tree.  Refinement rounds: members of a
//                  trie node are split by the block ID at the node's start;
//                  each part takes its smallest index as leader; each member's
//                  longest common prefix with the leader (wave-wide 64-entry
//                  compares with a ballot) gives the part's common prefix
//                  d* = min over members; a part with >= 2 members is a group
//                  covering [start, d*); members with more full blocks carry
//                  on from d*.  Work is O(sum of compared entries) plus an
//                  O(n^2) leader search per round inside LDS.
// Group IDs come from an atomic counter, so their numbering varies between
// runs; the host sorts groups into the canonical (smallest member, depth)
// order, which is unique.

#include <climits>

#include "fca_internal.h"

namespace fca {
namespace {

__global__ void k_init_header(int32_t* header) {
  int t = threadIdx.x;
  if (t < kHdrWords) header[t] = (t == kHdrBadReq) ? INT_MAX : 0;
}

__global__ __launch_bounds__(256) void k_prepare(const int32_t* __restrict__ bt_in, int64_t stride,
                                                 const int32_t* __restrict__ lens_in, int B, int W, int bs,
                                                 int num_blocks, DiscoveryPtrs p) {
  const int64_t total = (int64_t)B * W;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int i = (int)(idx / W);
    const int j = (int)(idx - (int64_t)i * W);
    const int L = lens_in[i];
    const bool badlen = L < 0 || (int64_t)L > (int64_t)W * bs;
    const int Lc = badlen ? 0 : L;
    const int nblk = (Lc + bs - 1) / bs;
    int id = -1;
    if (j < nblk) {
      id = bt_in[(int64_t)i * stride + j];
      if (id < 0 || id >= num_blocks) {
        atomicOr(&p.header[kHdrErr], kErrBadBlock);
        atomicMin(&p.header[kHdrBadReq], i);
      }
    }
    p.bt[idx] = id;
    if (j == 0) {
      if (badlen) {
        atomicOr(&p.header[kHdrErr], kErrBadLen);
        atomicMin(&p.header[kHdrBadReq], i);
      }
      p.lens[i] = Lc;
      p.nfull[i] = Lc / bs;
      p.deepest[i] = -1;
      p.sfx_begin[i] = 0;
      p.root[i] = -1;
      p.active[i] = 0;
    }
  }
}

__global__ __launch_bounds__(256) void k_roots(int B, int W, DiscoveryPtrs p) {
  const int i = (int)((blockIdx.x * (int64_t)blockDim.x + threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63;
  if (i >= B) return;
  if (p.nfull[i] == 0) return;  // root stays -1: nothing to share
  const int key = p.bt[(int64_t)i * W];
  int found = i;
  for (int k0 = 0; k0 <= i; k0 += 64) {
    const int k = k0 + lane;
    const bool hit = k <= i && p.nfull[k] > 0 && p.bt[(int64_t)k * W] == key;
    const unsigned long long mask = __ballot(hit);
    if (mask) {
      found = k0 + __ffsll((long long)mask) - 1;
      break;
    }
  }
  if (lane == 0) p.root[i] = found;
}

constexpr int kTreeThreads = 1024;

__global__ __launch_bounds__(kTreeThreads) void k_trees(int B, int W, DiscoveryPtrs p) {
  const int i = blockIdx.x;
  if (p.root[i] != i) return;  // not a tree root (uniform over the workgroup)

  __shared__ int mem[kMaxBatch];
  __shared__ int snode[kMaxBatch];
  __shared__ int skey[kMaxBatch];
  __shared__ int n_mem;
  __shared__ int any_active;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, nwaves = kTreeThreads / 64;
  if (tid == 0) n_mem = 0;
  __syncthreads();
  for (int k = tid; k < B; k += kTreeThreads)
    if (p.root[k] == i) mem[atomicAdd(&n_mem, 1)] = k;
  __syncthreads();
  const int nm = n_mem;
  if (nm < 2) return;  // a lone request: no group, suffix from block 0

  for (int x = tid; x < nm; x += kTreeThreads) {
    const int k = mem[x];
    p.depth_at[k] = 0;
    p.node[k] = i;
    p.gdepth[k] = 0;
    p.gparent[k] = -1;
    p.active[k] = 1;
  }
  __syncthreads();

  for (;;) {
    // Node and first block of every active member.
    for (int x = tid; x < nm; x += kTreeThreads) {
      const int k = mem[x];
      if (p.active[k]) {
        snode[x] = p.node[k];
        skey[x] = p.bt[(int64_t)k * W + p.depth_at[k]];
      } else {
        snode[x] = -1;
      }
    }
    __syncthreads();
    // Leader of each (node, first block) part: its smallest request index.
    for (int x = tid; x < nm; x += kTreeThreads) {
      const int nd = snode[x];
      if (nd < 0) continue;
      const int key = skey[x];
      int best = INT_MAX;
      for (int y = 0; y < nm; ++y)
        if (snode[y] == nd && skey[y] == key) best = min(best, mem[y]);
      p.newnode[mem[x]] = best;
    }
    __syncthreads();
    for (int x = tid; x < nm; x += kTreeThreads) {
      const int k = mem[x];
      if (!p.active[k]) continue;
      const int lead = p.newnode[k];
      p.node[k] = lead;
      if (lead == k) {
        p.ndstar[k] = INT_MAX;
        p.ncount[k] = 0;
      }
    }
    __syncthreads();
    // Longest common prefix with the leader, one wave per member.
    for (int x = wave; x < nm; x += nwaves) {
      const int k = mem[x];
      if (!p.active[k]) continue;
      const int lead = p.node[k];
      const int d0 = p.depth_at[k];
      int lcp;
      if (lead == k) {
        lcp = p.nfull[k];
      } else {
        const int cap = min(p.nfull[k], p.nfull[lead]);
        const int32_t* rk = p.bt + (int64_t)k * W;
        const int32_t* rl = p.bt + (int64_t)lead * W;
        lcp = cap;
        for (int j0 = d0; j0 < cap; j0 += 64) {
          const int j = j0 + lane;
          const bool diff = j < cap && rk[j] != rl[j];
          const unsigned long long mask = __ballot(diff);
          if (mask) {
            lcp = j0 + __ffsll((long long)mask) - 1;
            break;
          }
        }
      }
      if (lane == 0) {
        atomicMin(&p.ndstar[lead], lcp);
        atomicAdd(&p.ncount[lead], 1);
      }
    }
    __syncthreads();
    // Parts with two or more members become groups.
    for (int x = tid; x < nm; x += kTreeThreads) {
      const int k = mem[x];
      if (!p.active[k] || p.node[k] != k) continue;
      const int cnt = p.ncount[k];
      if (cnt >= 2) {
        const int gid = atomicAdd(&p.header[kHdrGroups], 1);
        int32_t* rec = p.records + (int64_t)gid * kRecordInts;
        rec[0] = k;
        rec[1] = p.gdepth[k];
        rec[2] = p.gparent[k];
        rec[3] = p.depth_at[k];
        rec[4] = p.ndstar[k];
        rec[5] = cnt;
        rec[6] = 0;
        rec[7] = 0;
        p.ngid[k] = gid;
      } else {
        p.ngid[k] = -1;
      }
    }
    __syncthreads();
    // Advance: finish lone members and members whose full blocks end here.
    for (int x = tid; x < nm; x += kTreeThreads) {
      const int k = mem[x];
      if (!p.active[k]) continue;
      const int lead = p.node[k];
      const int gid = p.ngid[lead];
      if (gid < 0) {
        p.sfx_begin[k] = p.depth_at[k];
        p.deepest[k] = p.gparent[k];
        p.active[k] = 0;
      } else {
        const int ds = p.ndstar[lead];
        p.gparent[k] = gid;
        p.gdepth[k] += 1;
        p.deepest[k] = gid;
        if (p.nfull[k] == ds) {
          p.sfx_begin[k] = ds;
          p.active[k] = 0;
        } else {
          p.depth_at[k] = ds;
        }
      }
    }
    if (tid == 0) any_active = 0;
    __syncthreads();
    for (int x = tid; x < nm; x += kTreeThreads)
      if (p.active[mem[x]]) any_active = 1;
    __syncthreads();
    if (!any_active) break;
  }
}

}  // namespace

// One thread per bin: the block IDs of the first four blocks of its first
// item (block IDs are validated by k_prepare).
__global__ __launch_bounds__(256) void k_bin_heads(BinHead* __restrict__ heads, int n_bins,
                                                   const int32_t* __restrict__ bt, int W, int bs) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= n_bins) return;
  BinHead& h = heads[b];
  const WorkItem& it = h.first;
  const int nblk = (it.tok_end - it.tok_begin + bs - 1) / bs;
  for (int j = 0; j < 4; ++j)
    h.id[j] = j < nblk ? bt[(int64_t)it.request * W + it.tok_begin / bs + j] : 0;
}

hipError_t launch_bin_heads(BinHead* heads, int n_bins, const int32_t* bt, int W, int bs, hipStream_t s) {
  if (n_bins <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_bin_heads, dim3((n_bins + 255) / 256), dim3(256), 0, s, heads, n_bins, bt, W, bs);
  return hipGetLastError();
}

hipError_t launch_discovery(const int32_t* bt_in, int64_t bt_stride, const int32_t* lens_in, int B, int W,
                            int block_size, int num_blocks, bool cascade, const DiscoveryPtrs& p, hipStream_t s) {
  hipLaunchKernelGGL(k_init_header, dim3(1), dim3(64), 0, s, p.header);
  if (B == 0) return hipGetLastError();
  const int64_t total = (int64_t)B * W;
  const int grid = (int)std::min<int64_t>((total + 255) / 256, 4096);
  hipLaunchKernelGGL(k_prepare, dim3(grid), dim3(256), 0, s, bt_in, bt_stride, lens_in, B, W, block_size,
                     num_blocks, p);
  if (cascade) {
    hipLaunchKernelGGL(k_roots, dim3((B + 3) / 4), dim3(256), 0, s, B, W, p);
    hipLaunchKernelGGL(k_trees, dim3(B), dim3(kTreeThreads), 0, s, B, W, p);
  }
  return hipGetLastError();
}

}  // namespace fca
