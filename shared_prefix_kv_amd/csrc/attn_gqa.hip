// Grouped prefix pass and per-request suffix pass for GQA caches, gfx950.
//
// Both passes compute, for sets of query rows and runs of cached tokens, the
// partial softmax triples (o, max, denominator) that the merge combines
// ("Core Mechanism" of the ZoRRo Inference & Forest Cascade Attention page,
// step 2: one pass over each group's shared prefix blocks, read once per
// group, and one pass per request over its own suffix blocks).
//
// Work item = (token range, H consecutive KV heads, up to 16 * n_ct query
// rows) with H * n_ct <= 4.  Query rows ("columns") of a grouped item are
// members x (Hq/Hkv) rows that all read the same KV tiles, so QK^T and PV are
// real matrix products and run on bf16 MFMA.  A per-request item has
// Hq/Hkv <= 16 rows per head and takes up to 4 heads of one request.
//
// Persistent workgroups of 4 waves: the planner packs items into one bin per
// workgroup (longest first, least-loaded bin); a workgroup walks its bin as
// one stream of stages, so the copy of the next stage -- possibly the first
// stage of the next item -- is always in flight while the current one is
// computed.
//
// Stage = 4 (head, block) tiles of the current item: tile t is block
// (4/H)*s + t % (4/H) of head h0 + t / (4/H).  Wave t copies tile t straight
// from HBM into LDS with global_load_lds_dwordx4 (16 bytes per lane, 1 KiB
// contiguous per instruction: the K tile then the V tile, 4 KiB each), so
// every KV byte crosses the vector-memory front end once per workgroup.  Two
// 32 KiB stage slots alternate; one barrier per stage hands a landed stage to
// all waves and frees the other slot for the next copy.  Block IDs and item
// descriptors come in through scalar loads.
//
// Wave w < H * n_ct owns head h0 + w / n_ct and column tile w % n_ct and
// computes the 4/H blocks of its head in each stage; its columns' triples are
// written straight from registers when the item ends (no cross-wave fold).
//
// Math of one 16-token block of one wave, operands read from LDS:
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16: lane (g, c) reads d-chunk
//     4*ks + g of token c (the chunked key layout makes this 1 KiB contiguous);
//   * S^T lands with token 4*g + j in lane group g, register j, column c --
//     exactly the B operand (P^T) of v_mfma_f32_16x16x16_bf16 once rounded;
//   * O^T += V^T P^T: lane (g, c) reads tokens 4g..4g+3 at value dim
//     16*dt + c, 8 contiguous bytes of the transposed value tile;
//   * online softmax per column in the log2 domain; the column max is reduced
//     across the four lane groups with permlane swaps; accumulators are
//     rescaled only when some column's max grew (a wave-uniform test).
// Tokens at or past the end of the range are masked: their scores become
// -inf and their (possibly NaN) values are zeroed before PV.

#include <cmath>

#include "fca_internal.h"

namespace fca {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(4))) const int32_t cint32;

constexpr int kD = 128;                              // head dim (keys and values)
constexpr int kBS = 16;                              // tokens per cache block
constexpr int kWaves = 4;                            // waves per workgroup = tiles per stage
constexpr int kTileBytes = kBS * kD * 2;             // one (block, head) K or V tile: 4 KiB
constexpr int kSlotBytes = kWaves * 2 * kTileBytes;  // 32 KiB per stage

// x op x' where x' is the value of lane ^ 16 (resp. ^ 32).
__device__ __forceinline__ float xmax16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xmax32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xsum16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xsum32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// s_waitcnt until no vector-memory operation of this wave is outstanding
// (gfx9 encoding: vmcnt 0, expcnt and lgkmcnt at their no-wait maxima).
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8)); }

// Work item i read through the scalar path.
__device__ __forceinline__ WorkItem load_item(cint32* items, int i) {
  static_assert(sizeof(WorkItem) == 12 * 4, "work item layout");
  cint32* p = items + 12 * i;
  WorkItem w;
  w.request = p[0];
  w.tok_begin = p[1];
  w.tok_end = p[2];
  w.kv_head = p[3];
  w.member_off = p[4];
  w.ncols = p[5];
  w.col0 = p[6];
  w.col1 = p[7];
  w.part_base = p[8];
  w.kv_heads = p[9];
  w.pad1 = w.pad2 = 0;
  return w;
}

__device__ __forceinline__ int item_blocks(const WorkItem& it) { return (it.tok_end - it.tok_begin + kBS - 1) / kBS; }

// log2 of the blocks per stage of an item: 4 / kv_heads with kv_heads in {1, 2, 4}.
__device__ __forceinline__ int item_lg_bps(const WorkItem& it) { return it.kv_heads == 1 ? 2 : it.kv_heads == 2 ? 1 : 0; }

__device__ __forceinline__ int item_stages(const WorkItem& it) {
  const int lg = item_lg_bps(it);
  return (item_blocks(it) + (1 << lg) - 1) >> lg;
}

__device__ __forceinline__ void partial_kernel_body(const GqaParams& P) {
  __shared__ __attribute__((aligned(1024))) char lds[2 * kSlotBytes];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int c16 = lane & 15;
  const float NEG_INF = -INFINITY;
  const float sc = P.scale_log2;

  cint32* bin_off = (cint32*)(P.bin_off);
  cint32* items = (cint32*)(P.items);
  cint32* bt = (cint32*)(P.bt);
  cint32* perm = (cint32*)(P.perm);
  const int i_begin = bin_off[blockIdx.x];
  const int i_end = bin_off[blockIdx.x + 1];
  if (i_begin >= i_end) return;

  const char* kpool = static_cast<const char*>(P.k);
  const char* vpool = static_cast<const char*>(P.v);
  const __bf16* qbase = static_cast<const __bf16*>(P.q);

  // Q^T operand of this wave for an item: column tile w % n_ct of head
  // h0 + w / n_ct (d-chunk ks*32 + 8*g).  The Q of item k + 1 is loaded into
  // qn while item k is begun (right after its first stage copy is issued)
  // and taken into the MFMA operand when item k + 1 begins, after a stage
  // wait; one buffer suffices however short the items are.
  bf16x8 qn[4];
  auto load_q = [&](const WorkItem& it) {
    const int nct = (it.col1 - it.col0 + 15) >> 4;
    const int h = wave / nct;
    const int cb = it.col0 + 16 * (wave - h * nct);  // first column of this wave's tile
    const int col = cb + c16;
    int member = it.request;
    if (it.member_off >= 0 && cb < it.col1) {
      // The tile's columns belong to members (cb / r) .. (last / r); their
      // request indices come in through scalar loads, one select per member.
      const int last = min(cb + 15, it.col1 - 1);
      const int m0 = cb / P.r;
      const int mine = min(col, last) / P.r - m0;
      for (int k = 0; k <= last / P.r - m0; ++k) {
        const int pk = perm[it.member_off + m0 + k];
        member = mine == k ? pk : member;
      }
    }
    const bool use = h < it.kv_heads && col < it.col1;
    const int qh = (it.kv_head + h) * P.r + col % P.r;
    // Idle lanes read row 0 of the item (always in bounds) and are zeroed
    // when the operand is taken.
    const __bf16* qp =
        qbase + ((int64_t)(use ? member : it.request) * P.Hq + (use ? qh : it.kv_head * P.r)) * kD + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qn[ks] = *reinterpret_cast<const bf16x8*>(qp + 32 * ks);
  };

  // ---- copy cursor: item di, stage ds ----
  // The descriptor of item di + 1 and the block ID of this wave's next tile
  // are loaded one step ahead, so issuing a stage waits on nothing.
  int di = i_begin, ds = 0;
  WorkItem dit = load_item(items, di);
  WorkItem dnx = dit;
  if (di + 1 < i_end) dnx = load_item(items, di + 1);
  int dnst, dlg, dsub, dhead, dnblk;
  auto copy_item = [&]() {  // per-item constants of the copy cursor
    dnst = item_stages(dit);
    dlg = item_lg_bps(dit);
    dsub = wave & ((1 << dlg) - 1);
    dhead = dit.kv_head + (wave >> dlg);
    dnblk = item_blocks(dit);
  };
  copy_item();
  // Tiles past the item copy block 0, which always exists; the math never
  // reads them.
  auto tile_id = [&]() {
    const int b = (ds << dlg) + dsub;
    return b < dnblk ? bt[(int64_t)dit.request * P.W + dit.tok_begin / kBS + b] : 0;
  };
  int cur_id = tile_id();

  // Copy stage (di, ds) into a slot: this wave's tile is block
  // bps*ds + wave % bps of head h0 + wave / bps.
  auto issue = [&](int slot) {
    const char* ksrc =
        kpool + ((int64_t)cur_id * P.k_stride_block + (int64_t)dhead * P.k_stride_head) * 2 + lane * 16;
    const char* vsrc =
        vpool + ((int64_t)cur_id * P.v_stride_block + (int64_t)dhead * P.v_stride_head) * 2 + lane * 16;
    char* dst = lds + slot * kSlotBytes + wave * 2 * kTileBytes;
#pragma unroll
    for (int i = 0; i < kTileBytes / 1024; ++i)
      __builtin_amdgcn_global_load_lds(ksrc + i * 1024, (__attribute__((address_space(3))) void*)(dst + i * 1024), 16,
                                       0, 0);
#pragma unroll
    for (int i = 0; i < kTileBytes / 1024; ++i)
      __builtin_amdgcn_global_load_lds(vsrc + i * 1024,
                                       (__attribute__((address_space(3))) void*)(dst + kTileBytes + i * 1024), 16, 0,
                                       0);
    if (++ds == dnst) {  // on to the next item: its descriptor, its Q, the one after
      ds = 0;
      if (++di < i_end) {
        dit = dnx;
        copy_item();
        if (di + 1 < i_end) dnx = load_item(items, di + 1);
      }
    }
    if (di < i_end) cur_id = tile_id();
  };

  // ---- compute cursor: item ci, stage cs ----
  WorkItem cit = dit, cnx = dnx;
  int ci = i_begin, cs = 0, cnst = dnst;
  int hh = 0, ct = 0, lg = 0;
  bool active = false;
  bool q_pending = false;  // qn is free and the next item's Q is still to be loaded
  bf16x8 qb[4];
  f32x4 o[8];
  float mrow = NEG_INF, lsum = 0.f;

  auto begin_item = [&]() {
    const int nct = (cit.col1 - cit.col0 + 15) >> 4;
    lg = item_lg_bps(cit);
    hh = wave / nct;
    ct = wave - hh * nct;
    active = hh < cit.kv_heads;
    const bool use = active && cit.col0 + 16 * ct + c16 < cit.col1;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qb[ks] = use ? qn[ks] : bf16x8{};
    if (ci + 1 < i_end) {
      if (ci > i_begin) cnx = load_item(items, ci + 1);
      q_pending = true;
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    mrow = NEG_INF;
    lsum = 0.f;
  };

  // One 16-token block from LDS: S^T = K Q^T (16x16x32, K = head dim),
  // online softmax, O^T += V^T P^T (16x16x16, K = the block's tokens).  All
  // twelve LDS reads are issued first; V is consumed after the softmax.
  auto compute_block = [&](const char* kt, int t0) {
    const char* vt = kt + kTileBytes;
    bf16x8 ka[4];
    bf16x4 va[8];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) ka[ks] = *reinterpret_cast<const bf16x8*>(kt + ((4 * ks + g) * kBS + c16) * 16);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) va[dt] = *reinterpret_cast<const bf16x4*>(vt + ((16 * dt + c16) * kBS + 4 * g) * 2);
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[ks], qb[ks], s, 0, 0, 0);
    // Tokens at or past the end of the range: score -inf, value zeroed
    // (the tail of a block may hold NaN).
    const int nvalid = cit.tok_end - t0 - 4 * g;  // valid tokens of this lane's 4
    if (t0 + kBS > cit.tok_end) {
#pragma unroll
      for (int j = 0; j < 4; ++j) s[j] = j < nvalid ? s[j] : NEG_INF;
    }
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = xmax32(xmax16(mx));
    const float mnew = fmaxf(mrow, mx * sc);
    if (__builtin_amdgcn_ballot_w64(mnew > mrow)) {  // some column's max grew
      const float alpha = exp2f(mrow - mnew);           // 0 on the first block
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;
      mrow = mnew;
    }
    bf16x4 pb;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float p = exp2f(fmaf(s[j], sc, -mrow));
      pb[j] = (__bf16)p;
      lsum += p;
    }
    if (t0 + kBS > cit.tok_end) {
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      const u32x2 keep = {(nvalid > 0 ? 0xffffu : 0u) | (nvalid > 1 ? 0xffff0000u : 0u),
                          (nvalid > 2 ? 0xffffu : 0u) | (nvalid > 3 ? 0xffff0000u : 0u)};
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        u32x2 w = __builtin_bit_cast(u32x2, va[dt]);
        w &= keep;
        va[dt] = __builtin_bit_cast(bf16x4, w);
      }
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[dt], pb, o[dt], 0, 0, 0);
  };

  // Triple of this lane's column of the finished item, straight from
  // registers.  It is stored after the next stage barrier, beside the next
  // copy, so the stores never hold up a stage wait on their own.
  bool fin = false;
  int64_t fin_row = 0;
  float fin_l = 0.f;
  auto store_partial = [&]() {
    float* dst = P.part.o + fin_row * kD + 4 * g;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<f32x4*>(dst + 16 * dt) = o[dt];
    if (g == 0) {
      P.part.m[fin_row] = mrow;
      P.part.l[fin_row] = fin_l;
    }
  };

  load_q(dit);
  issue(0);
  for (int it = 0;; ++it) {
    // Stage `it` has landed for every wave, and every wave is done with
    // stage it - 1, whose slot the next copy reuses.
    wait_vm_all();
    __syncthreads();
    if (fin) {
      store_partial();
      fin = false;
    }
    if (cs == 0) begin_item();
    if (di < i_end) issue((it + 1) & 1);
    if (q_pending) {
      load_q(cnx);
      q_pending = false;
    }
    if (active) {
      const int bps = 1 << lg;
      const char* slot = lds + (it & 1) * kSlotBytes + hh * bps * 2 * kTileBytes;
      const int nblk = item_blocks(cit);
      for (int b = 0; b < bps; ++b) {
        const int blk = bps * cs + b;
        if (blk < nblk) compute_block(slot + b * 2 * kTileBytes, cit.tok_begin + blk * kBS);
      }
    }
    if (++cs == cnst) {
      // Row of head kv_head + hh, column col of the item's token split.
      fin_l = xsum32(xsum16(lsum));
      const int col = cit.col0 + 16 * ct + c16;
      fin = active && col < cit.col1;
      fin_row = (int64_t)cit.part_base + (int64_t)hh * (cit.col1 - cit.col0) + (col - cit.col0);
      if (++ci == i_end) break;
      cit = cnx;
      cnst = item_stages(cit);
      cs = 0;
    }
  }
  if (fin) store_partial();
}

}  // namespace

// Grouped prefix pass: members x Hq/Hkv query rows per item.
__global__ __launch_bounds__(256, 2) void fca_grouped_prefix_kernel(GqaParams P) { partial_kernel_body(P); }

// Per-request suffix pass: the Hq/Hkv rows of up to 4 KV heads of a request.
__global__ __launch_bounds__(256, 2) void fca_suffix_decode_kernel(GqaParams P) { partial_kernel_body(P); }

hipError_t launch_gqa_partial(int kind, const GqaParams& p, int n_bins, hipStream_t s) {
  if (n_bins <= 0) return hipSuccess;
  if (kind == 0)
    hipLaunchKernelGGL(fca_grouped_prefix_kernel, dim3(n_bins), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(fca_suffix_decode_kernel, dim3(n_bins), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace fca
