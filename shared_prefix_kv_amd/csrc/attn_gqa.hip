// Grouped prefix pass and per-request suffix pass for GQA caches, gfx950.
//
// Both passes compute, for sets of query rows and runs of cached tokens, the
// partial softmax triples (o, max, denominator) that the merge combines
// ("Core Mechanism" of the ZoRRo Inference & Forest Cascade Attention page,
// step 2: one pass over each group's shared prefix blocks, read once per
// group, and one pass per request over its own suffix blocks).
//
// Work item = (token range, H consecutive KV heads, up to 64 query rows).
// Query rows ("columns") of a grouped item are members x (Hq/Hkv) rows that
// all read the same KV tiles, so QK^T and PV are real matrix products and run
// on bf16 MFMA; a per-request item has the Hq/Hkv <= 16 rows of each head.
//
// Persistent workgroups of 4 independent waves, one per SIMD: the planner
// cuts each pass into one equal run of work per workgroup (its bin).  In an
// item, wave w takes head kv_head + w % H and block stripe w / H: blocks
// stripe, stripe + 4/H, ... of the range, for all of the item's columns.
// Each stripe writes its own partial triples (the merge folds them like
// token splits), so waves never wait for one another: no barrier anywhere.
//
// Each wave streams its (block, head) tiles through its own ring of P LDS
// slots with global_load_lds_dwordx4 (16 bytes per lane, 1 KiB contiguous per
// instruction: K tile then V tile, 4 KiB each), P - 1 tiles ahead of the
// math, and waits with explicit vmcnt counts.  Every tile copy is exactly 8
// instructions; any other vector-memory operation (Q copies, partial stores)
// only adds to the count of operations issued after a tile, so waiting for
// "8 x tiles issued after it" is always a lower bound and correct.  The Q
// rows of the next item the wave computes are copied into a per-wave LDS
// slot while the current item begins, so beginning an item never waits for
// memory issued after it.  Block IDs and item descriptors come in through
// scalar loads, a step ahead.
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
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(4))) const int32_t cint32;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kD = 128;                   // head dim (keys and values)
constexpr int kBS = 16;                   // tokens per cache block
constexpr int kWaves = 4;                 // waves per workgroup
constexpr int kTileBytes = kBS * kD * 2;  // one (block, head) K or V tile: 4 KiB
constexpr int kSlotBytes = 2 * kTileBytes;
constexpr int kTileOps = 2 * kTileBytes / 1024;  // vector-memory instructions per tile copy
constexpr int kQRowBytes = kD * 2;

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

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// in 6:4, lgkmcnt in 11:8; a field at its maximum does not wait).
constexpr int vm_wait_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }
constexpr int kLgkmWait0 = 15 | (7 << 4) | (3 << 14);

// Wait until at most 8 * n vector-memory operations of this wave are in
// flight, n >= 0 (n above 3 waits as for 3, which is longer, still correct).
__device__ __forceinline__ void wait_tiles_after(int n) {
  if (n >= 3)
    __builtin_amdgcn_s_waitcnt(vm_wait_imm(3 * kTileOps));
  else if (n == 2)
    __builtin_amdgcn_s_waitcnt(vm_wait_imm(2 * kTileOps));
  else if (n == 1)
    __builtin_amdgcn_s_waitcnt(vm_wait_imm(kTileOps));
  else
    __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
}

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

// This wave's share of an item: head kv_head + hh, blocks stripe,
// stripe + S, ... (S = 4 / kv_heads stripes, kv_heads in {1, 2, 4}).
struct Role {
  int lgh;     // log2 kv_heads
  int hh;      // head within the item
  int stripe;  // block stripe
  int nblk;    // blocks of the stripe
};

__device__ __forceinline__ Role role_of(const WorkItem& it, int wave) {
  Role r;
  r.lgh = it.kv_heads == 4 ? 2 : it.kv_heads == 2 ? 1 : 0;
  r.hh = wave & (it.kv_heads - 1);
  r.stripe = wave >> r.lgh;
  const int lgs = 2 - r.lgh;
  const int nb = (it.tok_end - it.tok_begin + kBS - 1) / kBS;
  r.nblk = nb > r.stripe ? ((nb - 1 - r.stripe) >> lgs) + 1 : 0;
  return r;
}

// Arguments the first tile copy needs, passed ahead of the parameter block
// so that they arrive preloaded in scalar registers.
struct CopyArgs {
  const BinHead* bins;
  const WorkItem* items;
  const char* k;
  const char* v;
  int64_t ksb, ksh, vsb, vsh;  // strides in elements: key block / head, value block / head
};

template <int NCT, int P>
__device__ __forceinline__ void stream_body(const CopyArgs& ca, const GqaParams& Pm) {
  constexpr int kQBytes = NCT * 16 * kQRowBytes;
  constexpr int kWaveBytes = P * kSlotBytes + kQBytes;
  __shared__ __attribute__((aligned(1024))) char lds[kWaves * kWaveBytes];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int c16 = lane & 15;
  const float NEG_INF = -INFINITY;
  const float sc = Pm.scale_log2;
  char* ring = lds + wave * kWaveBytes;
  char* qlds = ring + P * kSlotBytes;

  // The bin head: item range, first item, first block IDs (one line).
  cint32* head = (cint32*)(ca.bins + blockIdx.x);
  cint32* items = (cint32*)(ca.items);
  cint32* bt = (cint32*)(Pm.bt);
  cint32* perm = (cint32*)(Pm.perm);
  // Every bin holds at least one item (the planner never makes an empty
  // one), so nothing waits for the range before the first copy.
  typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
  const i32x8 h8 = *(__attribute__((address_space(4))) const i32x8*)head;  // one scalar load
  const int i_begin = h8[0];
  const int i_end = h8[1];

  const char* kpool = ca.k;
  const char* vpool = ca.v;
  const char* qbase = static_cast<const char*>(Pm.q);

  int n_iss = 0;  // tiles issued by this wave
  int n_cmp = 0;  // tiles computed

  // ---- copy cursor: item di, k-th block of this wave's stripe ----
  int di = i_begin, dk = 0;
  WorkItem dit = load_item(head + 8, 0);
  Role dr = role_of(dit, wave);
  // On to the next item with blocks for this wave.  Its descriptor load is
  // the one round trip of an item change on the copy side; P - 1 tiles are
  // in flight meanwhile.
  auto copy_next_item = [&]() {
    do {
      dk = 0;
      if (++di >= i_end) return;
      dit = load_item(items, di);
      dr = role_of(dit, wave);
    } while (dr.nblk == 0);
  };
  auto tile_id = [&]() {
    const int b = dr.stripe + (dk << (2 - dr.lgh));
    return bt[(int64_t)dit.request * Pm.W + dit.tok_begin / kBS + b];
  };
  // Block IDs of the first item's blocks 0..3, loaded with the rest of the
  // head; this wave's first tile is block `stripe`.
  const int id0 = h8[2], id1 = h8[3], id2 = h8[4], id3 = h8[5];
  int cur_id;
  if (dr.nblk > 0) {
    cur_id = dr.stripe == 0 ? id0 : dr.stripe == 1 ? id1 : dr.stripe == 2 ? id2 : id3;
  } else {
    copy_next_item();
    cur_id = di < i_end ? tile_id() : 0;
  }

  // Copy the next tile of the stream into ring slot n_iss % P.
  auto issue_next = [&]() {
    if (di >= i_end) return;
    const int head = dit.kv_head + dr.hh;
    const char* ksrc = kpool + ((int64_t)cur_id * ca.ksb + (int64_t)head * ca.ksh) * 2 + lane * 16;
    const char* vsrc = vpool + ((int64_t)cur_id * ca.vsb + (int64_t)head * ca.vsh) * 2 + lane * 16;
    char* dst = ring + (n_iss % P) * kSlotBytes;
#pragma unroll
    for (int i = 0; i < kTileBytes / 1024; ++i)
      __builtin_amdgcn_global_load_lds(ksrc + i * 1024, (lds_void*)(dst + i * 1024), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < kTileBytes / 1024; ++i)
      __builtin_amdgcn_global_load_lds(vsrc + i * 1024, (lds_void*)(dst + kTileBytes + i * 1024), 16, 0, 0);
    ++n_iss;
    if (++dk == dr.nblk) copy_next_item();
    if (di < i_end) cur_id = tile_id();
  };

  // Copy the Q rows of item `it` for this wave's head into the Q slot:
  // row n (n < 16 * NCT) is query row col0 + n of the item; rows past col1
  // repeat row col0 and are zeroed when read.
  auto issue_q = [&](const WorkItem& it, const Role& r) {
    const int head_q0 = (it.kv_head + r.hh) * Pm.r;  // first q head of the KV head
    // Request of every row: for a grouped item all scalar loads go out
    // before the first is used (one round trip).
    int req[NCT * 16];
#pragma unroll
    for (int n = 0; n < NCT * 16; ++n) {
      const int col = it.col0 + n < it.col1 ? it.col0 + n : it.col0;
      req[n] = it.member_off >= 0 ? perm[it.member_off + col / Pm.r] : it.request;
    }
#pragma unroll
    for (int i = 0; i < NCT * 4; ++i) {
      // Four rows per instruction, 16 lanes (256 bytes) per row.
      const int x = lane >> 4;
      const int rq = x == 0 ? req[4 * i] : x == 1 ? req[4 * i + 1] : x == 2 ? req[4 * i + 2] : req[4 * i + 3];
      int col = it.col0 + 4 * i + x;
      col = col < it.col1 ? col : it.col0;
      const int hq = head_q0 + (it.member_off >= 0 ? col % Pm.r : col);
      const char* src = qbase + ((int64_t)rq * Pm.Hq + hq) * kQRowBytes + c16 * 16;
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(qlds + i * 1024), 16, 0, 0);
    }
  };

  // ---- compute cursor ----
  // The first tile, the Q of the first item this wave computes, then the
  // next P - 2 tiles.
  int q_iss = 0;  // n_iss when the pending Q copy was issued
  const WorkItem qit = dit;
  const Role qr = dr;
  const bool have_q = di < i_end;
  issue_next();
  if (have_q) {
    issue_q(qit, qr);
    q_iss = n_iss;
  }
#pragma unroll
  for (int p = 1; p < P - 1; ++p) issue_next();

  f32x4 o[NCT][8];
  float mrow[NCT], lsum[NCT];
  bf16x8 qb[NCT][4];

  WorkItem cnx = load_item(head + 8, 0);
  for (int ci = i_begin; ci < i_end; ++ci) {
    const WorkItem cit = cnx;
    if (ci + 1 < i_end) cnx = load_item(items, ci + 1);
    const Role cr = role_of(cit, wave);
    const int ccols = cit.col1 - cit.col0;
    const int64_t row0 = (int64_t)cit.part_base + (int64_t)(cr.stripe << cr.lgh) * ccols + (int64_t)cr.hh * ccols;

#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      mrow[ct] = NEG_INF;
      lsum[ct] = 0.f;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[ct][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    if (cr.nblk > 0) {
      // Q of this item has landed once every tile issued before its copy
      // has; take it into registers, then start the copy of the next item's.
      wait_tiles_after(n_iss - q_iss);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const int col = 16 * ct + c16;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 v = *reinterpret_cast<const bf16x8*>(qlds + col * kQRowBytes + (32 * ks + 8 * g) * 2);
          qb[ct][ks] = col < ccols ? v : bf16x8{};
        }
      }
      __builtin_amdgcn_s_waitcnt(kLgkmWait0);  // Q slot read before it is overwritten
      for (int nj = ci + 1; nj < i_end; ++nj) {
        const WorkItem nit = nj == ci + 1 ? cnx : load_item(items, nj);
        const Role nr = role_of(nit, wave);
        if (nr.nblk > 0) {
          issue_q(nit, nr);
          q_iss = n_iss;
          break;
        }
      }

      for (int k = 0; k < cr.nblk; ++k) {
        issue_next();
        wait_tiles_after(n_iss - n_cmp - 1);
        const char* kt = ring + (n_cmp % P) * kSlotBytes;
        const char* vt = kt + kTileBytes;
        ++n_cmp;
        const int t0 = cit.tok_begin + (cr.stripe + (k << (2 - cr.lgh))) * kBS;

        // All twelve LDS reads first; V is consumed after the softmax.
        bf16x8 ka[4];
        bf16x4 va[8];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          ka[ks] = *reinterpret_cast<const bf16x8*>(kt + ((4 * ks + g) * kBS + c16) * 16);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
          va[dt] = *reinterpret_cast<const bf16x4*>(vt + ((16 * dt + c16) * kBS + 4 * g) * 2);
        f32x4 s[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          s[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
            s[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[ks], qb[ct][ks], s[ct], 0, 0, 0);
        }
        // Tokens at or past the end of the range: score -inf, value zeroed
        // (the tail of a block may hold NaN).
        const int nvalid = cit.tok_end - t0 - 4 * g;  // valid tokens of this lane's 4
        const bool partial = t0 + kBS > cit.tok_end;
        if (partial) {
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int j = 0; j < 4; ++j) s[ct][j] = j < nvalid ? s[ct][j] : NEG_INF;
        }
        bf16x4 pb[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          float mx = fmaxf(fmaxf(s[ct][0], s[ct][1]), fmaxf(s[ct][2], s[ct][3]));
          mx = xmax32(xmax16(mx));
          const float mnew = fmaxf(mrow[ct], mx * sc);
          if (__builtin_amdgcn_ballot_w64(mnew > mrow[ct])) {  // some column's max grew
            const float alpha = exp2f(mrow[ct] - mnew);        // 0 on the first block
            lsum[ct] *= alpha;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) o[ct][dt] *= alpha;
            mrow[ct] = mnew;
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float p = exp2f(fmaf(s[ct][j], sc, -mrow[ct]));
            pb[ct][j] = (__bf16)p;
            lsum[ct] += p;
          }
        }
        if (partial) {
          const u32x2 keep = {(nvalid > 0 ? 0xffffu : 0u) | (nvalid > 1 ? 0xffff0000u : 0u),
                              (nvalid > 2 ? 0xffffu : 0u) | (nvalid > 3 ? 0xffff0000u : 0u)};
#pragma unroll
          for (int dt = 0; dt < 8; ++dt)
            va[dt] = __builtin_bit_cast(bf16x4, __builtin_bit_cast(u32x2, va[dt]) & keep);
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int dt = 0; dt < 8; ++dt)
            o[ct][dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[dt], pb[ct], o[ct][dt], 0, 0, 0);
      }
    }

    // Triples of this wave's columns (empty if the stripe had no block):
    // row of (stripe, head, column).
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const float l = xsum32(xsum16(lsum[ct]));
      const int col = 16 * ct + c16;
      if (col < ccols) {
        const int64_t row = row0 + col;
        float* dst = Pm.part.o + row * kD + 4 * g;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<f32x4*>(dst + 16 * dt) = o[ct][dt];
        if (g == 0) {
          Pm.part.m[row] = mrow[ct];
          Pm.part.l[row] = l;
        }
      }
    }
  }
}

}  // namespace

// Both passes: the work items of the bin of each workgroup, up to 16 * NCT
// query rows per wave.  The bin heads and items come first among the
// arguments so that they can be preloaded into scalar registers.
template <int NCT, int P>
__global__ __launch_bounds__(256, 1) void fca_attention_kernel(const BinHead* __restrict__ bins,
                                                               const WorkItem* __restrict__ items, const char* k,
                                                               const char* v, int64_t ksb, int64_t ksh, int64_t vsb,
                                                               int64_t vsh, GqaParams p) {
  const CopyArgs ca{bins, items, k, v, ksb, ksh, vsb, vsh};
  stream_body<NCT, P>(ca, p);
}

hipError_t launch_attention(const GqaParams& p, int n_bins, int nct, hipStream_t s) {
  if (n_bins <= 0) return hipSuccess;
  const dim3 grid(n_bins), block(kWaves * 64);
#define KARGS                                                                                          \
  p.bins, p.items, static_cast<const char*>(p.k), static_cast<const char*>(p.v), p.k_stride_block, \
      p.k_stride_head, p.v_stride_block, p.v_stride_head, p
  switch (nct) {
    case 1:
      hipLaunchKernelGGL((fca_attention_kernel<1, 4>), grid, block, 0, s, KARGS);
      break;
    case 2:
      hipLaunchKernelGGL((fca_attention_kernel<2, 4>), grid, block, 0, s, KARGS);
      break;
    case 3:
      hipLaunchKernelGGL((fca_attention_kernel<3, 3>), grid, block, 0, s, KARGS);
      break;
    case 4:
      hipLaunchKernelGGL((fca_attention_kernel<4, 3>), grid, block, 0, s, KARGS);
      break;
    default:
      return hipErrorInvalidValue;
  }
#undef KARGS
  return hipGetLastError();
}

}  // namespace fca
