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
//   k_prepare      copies the used table entries into the plan workspace
//                  (rows padded to 16 bytes), checks block IDs and lengths,
//                  initialises per-request state.
//   k_roots        one wave per request: the smallest request index with the
//                  same first block (the tree a request belongs to).
//   k_lcp0         one wave per request: its common prefix with its tree's
//                  root (the leader of every tree's first round), for all
//                  trees at once across the device.
//   k_trees        one workgroup per tree, refinement rounds over the trie:
//                  every active member sits at a node (the request that
//                  leads it) and a depth; the members are sorted in LDS by
//                  (node, block ID at the depth, request), so each part -- the
//                  members of one node that continue with the same block -- is
//                  a contiguous run led by its smallest request; binary
//                  searches give every member its part's bounds.  For the
//                  members of parts with two or more requests, the longest
//                  common prefix with the leader's row is found by 16-lane
//                  groups comparing 256 entries per round trip (4 rows of 16
//                  bytes per lane in flight); the part's common prefix d* is
//                  the minimum.  Such a part is a group covering [depth, d*);
//                  members with more full blocks carry on from d*, the rest
//                  end there.  Parts of one request end.  Work per round:
//                  a sort of the active members (skipped when they form a
//                  single part, as in every tree's first round, whose common
//                  prefixes k_lcp0 has found) and the entries the common
//                  prefixes cover.
// Group IDs come from an atomic counter, so their numbering varies between
// runs; the host sorts groups into the canonical (smallest member, depth)
// order, which is unique.

#include <climits>
#include <cstdlib>

#include "fca_internal.h"

namespace fca {
namespace {

__global__ void k_init_header(int32_t* header) {
  int t = threadIdx.x;
  if (t < kHdrWords) header[t] = (t == kHdrBadReq) ? INT_MAX : 0;
}

__global__ __launch_bounds__(256) void k_prepare(const int32_t* __restrict__ bt_in, int64_t stride,
                                                 const int32_t* __restrict__ lens_in, int B, int W, int W4, int bs,
                                                 int num_blocks, DiscoveryPtrs p) {
  const int64_t total = (int64_t)B * W4;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int i = (int)(idx / W4);
    const int j = (int)(idx - (int64_t)i * W4);
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
      p.first[i] = Lc / bs > 0 ? id : -1;
      p.deepest[i] = -1;
      p.sfx_begin[i] = 0;
      p.root[i] = -1;
      p.active[i] = 0;
    }
  }
}

__global__ __launch_bounds__(256) void k_roots(int B, int W4, DiscoveryPtrs p) {
  const int i = (int)((blockIdx.x * (int64_t)blockDim.x + threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63;
  if (i >= B) return;
  const int key = p.first[i];
  if (key < 0) return;  // no full block: root stays -1, nothing to share
  int found = i;
  // first block IDs are contiguous: 64 candidates in 256 bytes per load
  for (int k0 = 0; k0 <= i; k0 += 64) {
    const int k = k0 + lane;
    const bool hit = k <= i && p.first[k] == key;
    const unsigned long long mask = __ballot(hit);
    if (mask) {
      found = k0 + __ffsll((long long)mask) - 1;
      break;
    }
  }
  if (lane == 0) p.root[i] = found;
}

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Entries 1 .. cap of request k's row against its root's (entry 0 is equal
// by the root's definition): 64 lanes x 4 loads x 4 entries per round trip.
__global__ __launch_bounds__(256) void k_lcp0(int B, int W4, DiscoveryPtrs p) {
  const int k = (int)((blockIdx.x * (int64_t)blockDim.x + threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63;
  if (k >= B) return;
  const int rt = p.root[k];
  if (rt < 0) return;
  const int cap = min(p.nfull[k], p.nfull[rt]);
  const int32_t* rk = p.bt + (int64_t)k * W4;
  const int32_t* rr = p.bt + (int64_t)rt * W4;
  int found = cap;
  if (rt != k) {
    for (int base = 0; base < cap; base += 1024) {
      i32x4 va[4], vb[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int pos = base + 4 * (64 * u + lane);
        if (pos < cap) {
          va[u] = *reinterpret_cast<const i32x4*>(rk + pos);
          vb[u] = *reinterpret_cast<const i32x4*>(rr + pos);
        }
      }
      int first = INT_MAX;
#pragma unroll
      for (int u = 3; u >= 0; --u) {
        const int pos = base + 4 * (64 * u + lane);
        if (pos < cap) {
#pragma unroll
          for (int e = 3; e >= 0; --e) {
            const int q = pos + e;
            if (q >= 1 && q < cap && va[u][e] != vb[u][e]) first = q;
          }
        }
      }
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) first = min(first, __shfl_xor(first, m));
      if (first != INT_MAX) {
        found = first;
        break;
      }
    }
  }
  if (lane == 0) p.lcp0[k] = found;
}

constexpr int kTreeThreads = 1024;
constexpr int kTreeWaves = kTreeThreads / 64;
constexpr int kHashBits = 11;  // part table of trees of up to kTreeThreads members
constexpr int kHashSlots = 1 << kHashBits;
constexpr int kPosBits = 10;   // member position in that table's leader field
static_assert(kHashSlots == 2 * kTreeThreads && (1 << kPosBits) == kTreeThreads, "part table");
constexpr int kIdxBits = 13;  // request index in a sort key (kMaxBatch = 8192)
static_assert((1 << kIdxBits) >= kMaxBatch, "request index field");
constexpr uint64_t kIdxMask = (1u << kIdxBits) - 1;

// Sort key of an active member: node (13 bits), block ID at its depth (31
// bits, validated non-negative), request (13 bits).  Ascending order puts the
// members of one part together, smallest request first.
__device__ __forceinline__ uint64_t part_key(int node, int block, int k) {
  return ((uint64_t)node << (31 + kIdxBits)) | ((uint64_t)(uint32_t)block << kIdxBits) | (uint64_t)k;
}

// First position in [0, n) whose key's part bits are >= those of `part`
// (keys sorted ascending).
__device__ __forceinline__ int lower_part(const uint64_t* key, int n, uint64_t part) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if ((key[mid] >> kIdxBits) < part)
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo;
}

// LCP_LANES lanes compare one member's row, each with LCP_LOADS 16-byte
// loads of both rows in flight: LCP_LANES * LCP_LOADS * 4 entries per round
// trip, 1024 / LCP_LANES members at once.
template <int LCP_LANES, int LCP_LOADS>
__global__ __launch_bounds__(kTreeThreads) void k_trees(int B, int W4, DiscoveryPtrs p) {
  constexpr int kLcpGroup = LCP_LANES;
  constexpr int kGroups = 64 / LCP_LANES;  // members per wave
  constexpr int kLcpSpan = LCP_LANES * LCP_LOADS * 4;
  static_assert(kLcpSpan <= kLcpTail, "loads past the compared range stay inside the workspace");
  const int i = blockIdx.x;
  if (p.root[i] != i) return;  // not a tree root (uniform over the workgroup)

  __shared__ uint64_t skey[kMaxBatch];  // active members; sorted keys during a round
  static_assert(kTreeThreads + kHashSlots + kHashSlots / 2 * 2 <= kMaxBatch, "part table inside skey");
  __shared__ int16_t sbeg[kMaxBatch];   // part start (position) of each sorted member
  __shared__ int16_t scnt[kMaxBatch];   // part size
  __shared__ int32_t sdiff[kMaxBatch];  // common prefix with the part's leader; d* at the leader
  __shared__ int n_act, n_next;
  __shared__ unsigned long long kmin, kmax;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  if (tid == 0) n_act = 0;
  __syncthreads();
  for (int k = tid; k < B; k += kTreeThreads)
    if (p.root[k] == i) skey[atomicAdd(&n_act, 1)] = (uint64_t)k;
  __syncthreads();
  int n = n_act;
  if (n < 2) return;  // a lone request: no group, suffix from block 0

  for (int x = tid; x < n; x += kTreeThreads) {
    const int k = (int)skey[x];
    p.depth_at[k] = 0;
    p.node[k] = i;
    p.gdepth[k] = 0;
    p.gparent[k] = -1;
    p.active[k] = 1;
  }
  __syncthreads();

  for (bool first_round = true;; first_round = false) {
    // Keys of the active members (skey holds their request indices).
    if (tid == 0) {
      kmin = ~0ull;
      kmax = 0ull;
      n_next = 0;
    }
    __syncthreads();
    {
      unsigned long long lo = ~0ull, hi = 0ull;
      for (int x = tid; x < n; x += kTreeThreads) {
        const int k = (int)(skey[x] & kIdxMask);
        const uint64_t key = part_key(p.node[k], p.bt[(int64_t)k * W4 + p.depth_at[k]], k);
        skey[x] = key;
        lo = min(lo, (unsigned long long)key);
        hi = max(hi, (unsigned long long)key);
      }
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        lo = min(lo, (unsigned long long)__shfl_xor((long long)lo, m));
        hi = max(hi, (unsigned long long)__shfl_xor((long long)hi, m));
      }
      if (lane == 0) {
        atomicMin(&kmin, lo);
        atomicMax(&kmax, hi);
      }
    }
    __syncthreads();
    const bool one_part = (kmin >> kIdxBits) == (kmax >> kIdxBits);
    // Up to kTreeThreads members: the parts are found through a hash table of
    // their (node, block) keys in LDS (the unused upper part of skey), one
    // member per thread, each part led by its smallest request; larger trees
    // sort their keys.
    const bool hashed = !one_part && n <= kTreeThreads;
    if (hashed) {
      unsigned long long* tkey = reinterpret_cast<unsigned long long*>(skey + kTreeThreads);
      unsigned int* tlead = reinterpret_cast<unsigned int*>(skey + kTreeThreads + kHashSlots);
      unsigned int* tcnt = tlead + kHashSlots;
      for (int i = tid; i < kHashSlots; i += kTreeThreads) {
        tkey[i] = ~0ull;
        tlead[i] = ~0u;
        tcnt[i] = 0u;
      }
      __syncthreads();
      int slot = 0;
      if (tid < n) {
        const unsigned long long part = skey[tid] >> kIdxBits;  // < 2^44: never the empty key
        int h = (int)((part * 0x9E3779B97F4A7C15ull) >> (64 - kHashBits));
        for (;;) {  // at most n of the kHashSlots = 2 kTreeThreads slots are taken
          const unsigned long long prev = atomicCAS(&tkey[h], ~0ull, part);
          if (prev == ~0ull || prev == part) break;
          h = (h + 1) & (kHashSlots - 1);
        }
        slot = h;
        atomicMin(&tlead[h], (unsigned)(((skey[tid] & kIdxMask) << kPosBits) | (uint64_t)tid));
        atomicAdd(&tcnt[h], 1u);
      }
      __syncthreads();
      if (tid < n) {
        sbeg[tid] = (int16_t)(tlead[slot] & ((1u << kPosBits) - 1));
        scnt[tid] = (int16_t)tcnt[slot];
      }
    } else if (!one_part) {
      // Bitonic sort of skey[0, N), padded with the largest key.
      int N = 1;
      while (N < n) N <<= 1;
      if (N <= kTreeThreads) {
        // One key per thread, in a register: partners within a wave
        // (stride < 64) are exchanged by shuffles, the others through LDS.
        uint64_t key = tid < n ? skey[tid] : ~0ull;
        __syncthreads();
        for (int size = 2; size <= N; size <<= 1)
          for (int stride = size >> 1; stride > 0; stride >>= 1) {
            uint64_t other;
            if (stride >= 64) {
              if (tid < N) skey[tid] = key;
              __syncthreads();
              other = tid < N ? skey[tid ^ stride] : key;
              __syncthreads();
            } else {
              other = (uint64_t)__shfl_xor((long long)key, stride);
            }
            // The lower index of a pair keeps the smaller key in an
            // ascending run (tid & size == 0), the larger in a descending one.
            const bool lower = (tid & stride) == 0;
            const bool up = (tid & size) == 0;
            key = (lower == up) ? (key < other ? key : other) : (key < other ? other : key);
          }
        if (tid < N) skey[tid] = key;
        __syncthreads();
      } else {
        for (int x = n + tid; x < N; x += kTreeThreads) skey[x] = ~0ull;
        __syncthreads();
        for (int size = 2; size <= N; size <<= 1)
          for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int t = tid; t < N / 2; t += kTreeThreads) {
              const int a = 2 * t - (t & (stride - 1));
              const int b = a + stride;
              const bool up = (a & size) == 0;
              const uint64_t ka = skey[a], kb = skey[b];
              if ((ka > kb) == up) {
                skey[a] = kb;
                skey[b] = ka;
              }
            }
            __syncthreads();
          }
      }
    }
    // Part bounds.  One part: its leader is the smallest key (the members are
    // not sorted then, so the leader is found by its key).
    for (int x = tid; x < n && !hashed; x += kTreeThreads) {
      int b0, cnt;
      if (one_part) {
        b0 = -1;
        cnt = n;
      } else {
        const uint64_t part = skey[x] >> kIdxBits;
        b0 = lower_part(skey, x + 1, part);
        cnt = lower_part(skey, n, part + 1) - b0;
      }
      sbeg[x] = (int16_t)b0;
      scnt[x] = (int16_t)cnt;
      if (one_part && skey[x] == kmin) n_next = x;  // the leader's position (unique key)
    }
    __syncthreads();
    const int lead_pos = n_next;  // valid when one_part
    __syncthreads();
    if (tid == 0) n_next = 0;
    for (int x = tid; x < n; x += kTreeThreads) {
      if (one_part) sbeg[x] = (int16_t)lead_pos;
      const int k = (int)(skey[x] & kIdxMask);
      const int lead = (int)(skey[one_part ? lead_pos : sbeg[x]] & kIdxMask);
      // first round: the leader is the root and k_lcp0 has the prefixes
      sdiff[x] = lead == k ? p.nfull[k] : first_round ? p.lcp0[k] : min(p.nfull[k], p.nfull[lead]);
    }
    __syncthreads();

    // Longest common prefix of every member of a part of two or more with the
    // part's leader, from its depth: groups of kLcpGroup lanes, kGroups
    // members per wave.
    if (!first_round) {
      const int g = lane / kLcpGroup, gl = lane % kLcpGroup;
      for (int x0 = kGroups * wave; x0 < n; x0 += kGroups * kTreeWaves) {
        const int x = x0 + g;
        bool busy = false;
        int k = 0, lead = 0, d0 = 0, cap = 0, a0 = 0;
        if (x < n && scnt[x] >= 2 && sbeg[x] != x) {
          k = (int)(skey[x] & kIdxMask);
          lead = (int)(skey[sbeg[x]] & kIdxMask);
          d0 = p.depth_at[k] + 1;  // the block at the depth is the part's key
          cap = sdiff[x];
          a0 = d0 & ~3;
          busy = d0 < cap;
        }
        const int32_t* rk = p.bt + (int64_t)k * W4;
        const int32_t* rl = p.bt + (int64_t)lead * W4;
        int found = INT_MAX;
        for (int base = a0; __ballot(busy) != 0; base += kLcpSpan) {
          if (busy) {
            // Unconditional loads from one address per row plus immediate
            // offsets (entries past cap are read but not compared; the
            // workspace keeps kLcpTail entries after the last row), which
            // leaves registers for LCP_LOADS loads of both rows in flight.
            i32x4 va[LCP_LOADS], vb[LCP_LOADS];
            const int32_t* rkb = rk + base + 4 * gl;
            const int32_t* rlb = rl + base + 4 * gl;
#pragma unroll
            for (int u = 0; u < LCP_LOADS; ++u) {
              va[u] = *reinterpret_cast<const i32x4*>(rkb + 4 * kLcpGroup * u);
              vb[u] = *reinterpret_cast<const i32x4*>(rlb + 4 * kLcpGroup * u);
            }
            int first = INT_MAX;
#pragma unroll
            for (int u = LCP_LOADS - 1; u >= 0; --u) {
              const int pos = base + 4 * (kLcpGroup * u + gl);
              if (pos < cap) {
#pragma unroll
                for (int e = 3; e >= 0; --e) {
                  const int q = pos + e;
                  if (q >= d0 && q < cap && va[u][e] != vb[u][e]) first = q;
                }
              }
            }
            found = min(found, first);
          }
          // minimum over the lanes of the group
#pragma unroll
          for (int m = kLcpGroup / 2; m >= 1; m >>= 1) found = min(found, __shfl_xor(found, m));
          if (busy && (found != INT_MAX || base + kLcpSpan >= cap)) {
            if (gl == 0 && found != INT_MAX) sdiff[x] = found;
            busy = false;
          }
        }
      }
    }
    __syncthreads();
    // Part common prefix d* = minimum over its members, kept at the leader.
    for (int x = tid; x < n; x += kTreeThreads)
      if (scnt[x] >= 2 && sbeg[x] != x) atomicMin(&sdiff[sbeg[x]], sdiff[x]);
    __syncthreads();
    // Parts with two or more members become groups.
    for (int x = tid; x < n; x += kTreeThreads) {
      if (sbeg[x] != x) continue;
      const int k = (int)(skey[x] & kIdxMask);
      const int cnt = scnt[x];
      if (cnt >= 2) {
        const int gid = atomicAdd(&p.header[kHdrGroups], 1);
        int32_t* rec = p.records + (int64_t)gid * kRecordInts;
        rec[0] = k;
        rec[1] = p.gdepth[k];
        rec[2] = p.gparent[k];
        rec[3] = p.depth_at[k];
        rec[4] = sdiff[x];
        rec[5] = cnt;
        rec[6] = 0;
        rec[7] = 0;
        p.ngid[k] = gid;
      } else {
        p.ngid[k] = -1;
      }
    }
    __syncthreads();
    // Advance: members of lone parts end at their depth; the others join
    // their group and end at d* or carry on from it.
    for (int x = tid; x < n; x += kTreeThreads) {
      const int k = (int)(skey[x] & kIdxMask);
      const int b0 = sbeg[x];
      const int lead = (int)(skey[b0] & kIdxMask);
      const int gid = p.ngid[lead];
      if (gid < 0) {
        p.sfx_begin[k] = p.depth_at[k];
        p.deepest[k] = p.gparent[k];
        p.active[k] = 0;
      } else {
        const int ds = sdiff[b0];
        p.gparent[k] = gid;
        p.gdepth[k] += 1;
        p.deepest[k] = gid;
        if (p.nfull[k] == ds) {
          p.sfx_begin[k] = ds;
          p.active[k] = 0;
        } else {
          p.depth_at[k] = ds;
          p.node[k] = lead;
        }
      }
    }
    __syncthreads();
    // The members still active, compacted for the next round (through sdiff,
    // whose values are no longer needed).
    for (int x = tid; x < n; x += kTreeThreads) {
      const int k = (int)(skey[x] & kIdxMask);
      if (p.active[k]) sdiff[atomicAdd(&n_next, 1)] = k;
    }
    __syncthreads();
    n = n_next;
    for (int x = tid; x < n; x += kTreeThreads) skey[x] = (uint64_t)sdiff[x];
    __syncthreads();
    if (n == 0) break;
  }
}

}  // namespace

hipError_t launch_discovery(const int32_t* bt_in, int64_t bt_stride, const int32_t* lens_in, int B, int W, int W4,
                            int block_size, int num_blocks, bool cascade, const DiscoveryPtrs& p, hipStream_t s) {
  hipLaunchKernelGGL(k_init_header, dim3(1), dim3(64), 0, s, p.header);
  if (B == 0) return hipGetLastError();
  const int64_t total = (int64_t)B * W4;
  const int grid = (int)std::min<int64_t>((total + 255) / 256, 4096);
  hipLaunchKernelGGL(k_prepare, dim3(grid), dim3(256), 0, s, bt_in, bt_stride, lens_in, B, W, W4, block_size,
                     num_blocks, p);
  if (cascade) {
    hipLaunchKernelGGL(k_roots, dim3((B + 3) / 4), dim3(256), 0, s, B, W4, p);
    hipLaunchKernelGGL(k_lcp0, dim3((B + 3) / 4), dim3(256), 0, s, B, W4, p);
    // Lanes per compared row x loads in flight per lane (developer tuning
    // knob FCA_TUNE_LCP = 44, 84 or 48): 4 lanes x 4 loads by default (most
    // members in flight; the common-prefix step of forest_mixed's second
    // round took 13-15 us with 4 or 8 loads, 84 against 116 VGPRs).
    static const int lcp = [] {
      const char* v = getenv("FCA_TUNE_LCP");
      const int x = v ? atoi(v) : 44;
      return (x == 48 || x == 84) ? x : 44;
    }();
    if (lcp == 44)
      hipLaunchKernelGGL((k_trees<4, 4>), dim3(B), dim3(kTreeThreads), 0, s, B, W4, p);
    else if (lcp == 84)
      hipLaunchKernelGGL((k_trees<8, 4>), dim3(B), dim3(kTreeThreads), 0, s, B, W4, p);
    else
      hipLaunchKernelGGL((k_trees<4, 8>), dim3(B), dim3(kTreeThreads), 0, s, B, W4, p);
  }
  return hipGetLastError();
}

}  // namespace fca
