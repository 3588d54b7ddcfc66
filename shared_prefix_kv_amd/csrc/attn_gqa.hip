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
// Persistent workgroups of 4 independent waves, one or two workgroups per CU
// (the planner's choice: two on small batches, where they hide each other's
// stalls; one on large ones, which halves the token splits): the planner
// cuts the work items of both passes into one equal run of work per
// workgroup (its bin).  In an item the 4 waves are H
// heads x C column groups (up to 32 rows each; C = 2 only for items wider
// than 32 rows) x S = 4/(H C) block stripes; the wave of stripe t reads
// blocks t, t + S, ... of the range.  With the usual pool layout (the heads
// of a block side by side) the H heads of one block are one contiguous read
// per workgroup, which measured faster than S stripes over scattered blocks.
// Each (stripe, head) writes its own partial triples (the merge folds stripes
// like token splits), so waves never wait for one another: no barrier.
//
// Each wave streams its work through its own 2-slot LDS ring, one entry
// ahead of the math: per item, an entry with its Q rows, then one entry per
// (block, head) tile (K tile then V tile, 4 KiB each), all copied with
// global_load_lds_dwordx4 (16 bytes per lane, 1 KiB contiguous per
// instruction in the tile layout).  From a pool of token rows (one row of
// 128 dims per (block, head, slot)) each copy instruction moves 4 whole rows
// of keys or values, so LDS holds both token-major, with the 16-byte chunks
// of each row permuted by an XOR with the token index (keys: chunk ^ t,
// values: chunk ^ 2 (t % 8)) so that the operand reads hit distinct banks;
// values are read transposed (ds_read_b64_tr_b16).  Before using an entry the wave waits until at most the
// operations of the one entry issued after it are in flight (the count is
// known exactly; partial stores only add to it, which makes the wait longer,
// never wrong).  Block IDs and item descriptors come in through scalar loads
// a step ahead; the bin head carries the first ones.
//
// Math of one 16-token block of one wave, operands read from LDS:
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16: lane (g, c) reads d-chunk
//     4*ks + g of token c (the chunked key layout makes this 1 KiB contiguous);
//   * S^T lands with token 4*g + j in lane group g, register j, column c --
//     the tokens of lane group g in the P^T operand;
//   * O^T += V^T P^T with v_mfma_f32_16x16x32_bf16: lane (g, c) reads tokens
//     4g..4g+3 at value dim 16*dt + c, 8 contiguous bytes of the transposed
//     value tile, and feeds them twice, against the bf16 rounding of each
//     probability and against the bf16 rounding of its remainder (p - hi).
//     The 32-deep product thus applies p to about 16 bits at the issue cost
//     of the 16-deep one it replaces, so the probabilities add no error of
//     their own beyond that of fp32 accumulation;
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
constexpr int kWaves = kAttnWaves;        // waves per workgroup
constexpr int kRing = 2;                  // LDS slots per wave
constexpr int kTileBytes = kBS * kD * 2;  // one (block, head) K or V tile: 4 KiB
constexpr int kSlotBytes = 2 * kTileBytes;
constexpr int kTileOps = 2 * kTileBytes / 1024;  // vector-memory instructions per tile copy
constexpr int kQRowBytes = kD * 2;
constexpr int kWaveCols = 32;             // query rows one wave covers at most
constexpr int kCachePolicyNT = 2;         // cache-policy bits of a load: non-temporal

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

// Wait until at most n (0..8) vector-memory operations of this wave are in
// flight.
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(vm_wait_imm(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(vm_wait_imm(1)); break;
    case 2: __builtin_amdgcn_s_waitcnt(vm_wait_imm(2)); break;
    case 3: __builtin_amdgcn_s_waitcnt(vm_wait_imm(3)); break;
    case 4: __builtin_amdgcn_s_waitcnt(vm_wait_imm(4)); break;
    case 5: __builtin_amdgcn_s_waitcnt(vm_wait_imm(5)); break;
    case 6: __builtin_amdgcn_s_waitcnt(vm_wait_imm(6)); break;
    case 7: __builtin_amdgcn_s_waitcnt(vm_wait_imm(7)); break;
    default: __builtin_amdgcn_s_waitcnt(vm_wait_imm(8)); break;
  }
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
  w.stripes = 0;
  w.flags = p[11];
  return w;
}

// This wave's share of an item: head kv_head + hh, columns
// [col0 + c_lo, col0 + c_lo + ncol), blocks stripe, stripe + S, ... of the
// range.  Waves are numbered ((stripe * H) + hh) * C + column group.
struct Role {
  int hh;      // head within the item
  int stripe;  // block stripe
  int lgs;     // log2 of the stripe count S
  int lgh;     // log2 of the item's heads H
  int nblk;    // blocks of the stripe
  int c_lo;    // first column of the wave, relative to col0
  int ncol;    // columns of the wave (1..32)
};

__device__ __forceinline__ Role role_of(const WorkItem& it, int wave) {
  Role r;
  const int ccols = it.col1 - it.col0;
  const int lgc = ccols > kWaveCols ? 1 : 0;
  r.lgh = it.kv_heads == 8 ? 3 : it.kv_heads == 4 ? 2 : it.kv_heads == 2 ? 1 : 0;
  r.lgs = kAttnLgWaves - r.lgh - lgc;
  const int cg = wave & lgc;
  r.hh = (wave >> lgc) & (it.kv_heads - 1);
  r.stripe = wave >> (lgc + r.lgh);
  const int nb = (it.tok_end - it.tok_begin + kBS - 1) / kBS;
  r.nblk = nb > r.stripe ? ((nb - 1 - r.stripe) >> r.lgs) + 1 : 0;
  r.c_lo = cg * kWaveCols;
  r.ncol = min(kWaveCols, ccols - r.c_lo);
  return r;
}

// The 8 V^T operands of a block from a token-major value tile in LDS (16
// rows of 128 dims, 16-byte chunk c of token t at chunk c ^ 2 (t % 8) of its
// row): ds_read_b64_tr_b16, where lane (g, c16) addresses dims
// 4 (c16 % 4) .. + 3 of sub-tile dt (dims 16 dt .. 16 dt + 15) of token
// t = 4 g + c16 / 4 and receives dim c16 of tokens 4 g .. 4 g + 3 -- the
// operand the tile layout gives by a plain read.  Those 8 bytes sit at
// 256 t + 32 (dt ^ (t % 8)) + 8 (c16 % 4).  One block that waits for its own
// results.
__device__ __forceinline__ void read_vt_rows(const char* vt, int g, int c16, u32x2 (&r)[8]) {
  const int t = 4 * g + (c16 >> 2);
  const uint32_t a = (uint32_t)(uintptr_t)vt + t * 256 + (c16 & 3) * 8;
  uint32_t ad[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) ad[dt] = a + 32 * (dt ^ (t & 7));
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n"
      "ds_read_b64_tr_b16 %1, %9\n"
      "ds_read_b64_tr_b16 %2, %10\n"
      "ds_read_b64_tr_b16 %3, %11\n"
      "ds_read_b64_tr_b16 %4, %12\n"
      "ds_read_b64_tr_b16 %5, %13\n"
      "ds_read_b64_tr_b16 %6, %14\n"
      "ds_read_b64_tr_b16 %7, %15\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]), "v"(ad[7])
      : "memory");
}

// Arguments the first copies need, passed ahead of the parameter block so
// that they arrive preloaded in scalar registers.
struct CopyArgs {
  const BinHead* bins;
  const WorkItem* items;
  const char* k;
  const char* v;
  int64_t ksb, ksh, vsb, vsh;  // strides in elements: key block / head, value block / head
};

// ROWS: the pools hold token rows (Pm.k_stride_token, Pm.v_stride_token),
// else tiles.
template <bool ROWS>
__device__ __forceinline__ void stream_body(const CopyArgs& ca, const GqaParams& Pm) {
  constexpr int kWaveBytes = kRing * kSlotBytes;
  __shared__ __attribute__((aligned(1024))) char lds[kWaves * kWaveBytes];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int c16 = lane & 15;
  const float NEG_INF = -INFINITY;
  const float sc = Pm.scale_log2;
  char* ring = lds + wave * kWaveBytes;

  // The bin head: item range, first block IDs, first item (one line).
  cint32* head = (cint32*)(ca.bins + blockIdx.x);
  cint32* items = (cint32*)(ca.items);
  cint32* bt = (cint32*)(Pm.bt);
  cint32* perm = (cint32*)(Pm.perm);
  typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
  const i32x8 h8 = *(__attribute__((address_space(4))) const i32x8*)head;  // one scalar load
  // Every bin holds at least one item (the planner never makes an empty
  // one), so nothing waits for the range before the first copy.
  const int i_begin = h8[0];
  const int i_end = h8[1];
  const char* qbase = static_cast<const char*>(Pm.q);

  int n_iss = 0;     // ring entries issued by this wave
  int n_cmp = 0;     // ring entries consumed
  int last_ops = 0;  // vector-memory instructions of the last entry issued

  // ---- copy cursor: item di, entry dk of it (-1: its Q rows, k >= 0: tile k) ----
  int di = i_begin, dk = -1;
  WorkItem dit = load_item(head + 8, 0);
  Role dr = role_of(dit, wave);
  auto tile_id = [&](int k) {  // block ID of this wave's k-th tile of item di
    const int b = dr.stripe + (k << dr.lgs);
    return bt[(int64_t)dit.request * Pm.W + dit.tok_begin / kBS + b];
  };
  int cur_id = 0;  // block ID of the next tile to copy
  auto copy_next_item = [&]() {  // next item with blocks for this wave
    do {
      dk = -1;
      if (++di >= i_end) return;
      dit = load_item(items, di);
      dr = role_of(dit, wave);
    } while (dr.nblk == 0);
    cur_id = tile_id(0);
  };
  if (dr.nblk > 0) {
    // Block `stripe` of the first item comes with the bin head.
    const int id0 = h8[2], id1 = h8[3], id2 = h8[4], id3 = h8[5];
    cur_id = dr.stripe == 0 ? id0 : dr.stripe == 1 ? id1 : dr.stripe == 2 ? id2 : id3;
    if (dr.stripe > 3) cur_id = tile_id(0);
  } else {
    copy_next_item();
  }

  // Copy the next entry of the stream into ring slot n_iss % 2.
  auto issue_next = [&]() {
    if (di >= i_end) return;
    char* dst = ring + (n_iss & 1) * kSlotBytes;
    if (dk < 0) {
      // Q rows of this wave's columns: row n of the slot is query row
      // col0 + c_lo + n; four rows per instruction, 16 lanes (256 bytes) per
      // row; rows past the wave's columns repeat its first row (zeroed when
      // read).  For a grouped item all member loads go out at once.
      const int head_q0 = (dit.kv_head + dr.hh) * Pm.r;
      const int cbase = dit.col0 + dr.c_lo;
      const int nq = (dr.ncol + 3) >> 2;
      int req[kWaveCols];
#pragma unroll
      for (int n = 0; n < kWaveCols; ++n) {
        const int col = cbase + (n < dr.ncol ? n : 0);
        req[n] = dit.member_off >= 0 ? perm[dit.member_off + col / Pm.r] : dit.request;
      }
      const int x = lane >> 4;
#pragma unroll
      for (int i = 0; i < kWaveCols / 4; ++i) {
        if (i < nq) {
          const int rq = x == 0 ? req[4 * i] : x == 1 ? req[4 * i + 1] : x == 2 ? req[4 * i + 2] : req[4 * i + 3];
          const int n = 4 * i + x;
          const int col = cbase + (n < dr.ncol ? n : 0);
          const int hq = head_q0 + (dit.member_off >= 0 ? col % Pm.r : col);
          const char* src = qbase + ((int64_t)rq * Pm.Hq + hq) * kQRowBytes + c16 * 16;
          __builtin_amdgcn_global_load_lds(src, (lds_void*)(dst + i * 1024), 16, 0, 0);
        }
      }
      last_ops = nq;
      dk = 0;
    } else {
      const int hd = dit.kv_head + dr.hh;
      // Tiles: instruction i copies bytes [1024 i, 1024 i + 1024) of each
      // tile.  Token rows: instruction i copies rows 4 i .. 4 i + 3; lane l
      // fills LDS chunk l % 16 of row t = 4 i + l / 16 from the row's chunk
      // (l % 16) ^ t (keys) or (l % 16) ^ 2 (t % 8) (values).
      const char* kbase = ca.k + ((int64_t)cur_id * ca.ksb + (int64_t)hd * ca.ksh) * 2;
      const char* vbase = ca.v + ((int64_t)cur_id * ca.vsb + (int64_t)hd * ca.vsh) * 2;
      auto ksrc = [&](int i) -> const char* {
        if constexpr (ROWS) {
          const int t = 4 * i + (lane >> 4);
          return kbase + (int64_t)t * Pm.k_stride_token * 2 + ((lane & 15) ^ t) * 16;
        } else {
          return kbase + lane * 16 + i * 1024;
        }
      };
      auto vsrc = [&](int i) -> const char* {
        if constexpr (ROWS) {
          const int t = 4 * i + (lane >> 4);
          return vbase + (int64_t)t * Pm.v_stride_token * 2 + ((lane & 15) ^ (2 * (t & 7))) * 16;
        } else {
          return vbase + lane * 16 + i * 1024;
        }
      };
      // A tile that exactly one wave reads (the planner's kItemStream: a
      // suffix of a cascade plan, or a group whose query rows fit one wave)
      // streams through the caches with the non-temporal policy.  Other
      // tiles are loaded by two column-group waves of an item, by several
      // column chunks, or by several requests (shared blocks in suffixes of
      // plans without the cascade or with folded groups); their later loads
      // should find them in L2, which the non-temporal policy gives up.
      if (dit.flags & kItemStream) {
#pragma unroll
        for (int i = 0; i < kTileBytes / 1024; ++i)
          __builtin_amdgcn_global_load_lds(ksrc(i), (lds_void*)(dst + i * 1024), 16, 0, kCachePolicyNT);
#pragma unroll
        for (int i = 0; i < kTileBytes / 1024; ++i)
          __builtin_amdgcn_global_load_lds(vsrc(i), (lds_void*)(dst + kTileBytes + i * 1024), 16, 0,
                                           kCachePolicyNT);
      } else {
#pragma unroll
        for (int i = 0; i < kTileBytes / 1024; ++i)
          __builtin_amdgcn_global_load_lds(ksrc(i), (lds_void*)(dst + i * 1024), 16, 0, 0);
#pragma unroll
        for (int i = 0; i < kTileBytes / 1024; ++i)
          __builtin_amdgcn_global_load_lds(vsrc(i), (lds_void*)(dst + kTileBytes + i * 1024), 16, 0, 0);
      }
      last_ops = kTileOps;
      if (++dk == dr.nblk)
        copy_next_item();
      else
        cur_id = tile_id(dk);
    }
    ++n_iss;
  };

  // Wait for entry n_cmp: at most the one entry issued after it may still
  // be in flight.
  auto wait_entry = [&]() { wait_vm(n_iss - n_cmp > 1 ? last_ops : 0); };

  issue_next();

  WorkItem cnx = load_item(head + 8, 0);
  for (int ci = i_begin; ci < i_end; ++ci) {
    const WorkItem cit = cnx;
    if (ci + 1 < i_end) cnx = load_item(items, ci + 1);
    const Role cr = role_of(cit, wave);
    const int ccols = cit.col1 - cit.col0;
    // row of (stripe, head, column c_lo + n) of the item's piece
    const int64_t row0 =
        (int64_t)cit.part_base + (int64_t)((cr.stripe << cr.lgh) + cr.hh) * ccols + cr.c_lo;

    // The item's math: two 16-column tiles per wave; the second is skipped
    // (a wave-uniform test) when the wave has at most 16 columns.
    {
      constexpr int NCT = 2;
      const bool two = cr.ncol > 16;
      f32x4 o[NCT][8];
      float mrow[NCT], lsum[NCT];
      bf16x8 qb[NCT][4];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        mrow[ct] = NEG_INF;
        lsum[ct] = 0.f;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[ct][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      if (cr.nblk > 0) {
        // Q entry: into registers, then the slot is free again.
        issue_next();
        wait_entry();
        const char* qs = ring + (n_cmp & 1) * kSlotBytes;
        ++n_cmp;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const int col = 16 * ct + c16;
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const bf16x8 v = *reinterpret_cast<const bf16x8*>(qs + col * kQRowBytes + (32 * ks + 8 * g) * 2);
            qb[ct][ks] = col < cr.ncol ? v : bf16x8{};
          }
        }
        __builtin_amdgcn_s_waitcnt(kLgkmWait0);  // Q read before the slot is overwritten

        for (int k = 0; k < cr.nblk; ++k) {
          issue_next();
          wait_entry();
          const char* kt = ring + (n_cmp & 1) * kSlotBytes;
          const char* vt = kt + kTileBytes;
          ++n_cmp;
          const int t0 = cit.tok_begin + (cr.stripe + (k << cr.lgs)) * kBS;

          // All twelve LDS reads first; V is consumed after the softmax.
          bf16x8 ka[4];
          bf16x4 va[8];
          if constexpr (ROWS) {
            // chunk 4 ks + g of token c16, stored at chunk (4 ks + g) ^ c16
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
              ka[ks] = *reinterpret_cast<const bf16x8*>(kt + c16 * kQRowBytes + ((4 * ks + g) ^ c16) * 16);
          } else {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
              ka[ks] = *reinterpret_cast<const bf16x8*>(kt + ((4 * ks + g) * kBS + c16) * 16);
          }
          if constexpr (ROWS) {
            u32x2 vr[8];
            read_vt_rows(vt, g, c16, vr);
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) va[dt] = __builtin_bit_cast(bf16x4, vr[dt]);
          } else {
#pragma unroll
            for (int dt = 0; dt < 8; ++dt)
              va[dt] = *reinterpret_cast<const bf16x4*>(vt + ((16 * dt + c16) * kBS + 4 * g) * 2);
          }
          f32x4 s[NCT];
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) {
            s[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (ct == 0 || two) {
#pragma unroll
              for (int ks = 0; ks < 4; ++ks)
                s[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[ks], qb[ct][ks], s[ct], 0, 0, 0);
            }
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
          bf16x8 pb[NCT];  // [bf16(p) of tokens 4g..4g+3, bf16(p - bf16(p)) of the same]
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) {
            if (ct == 1 && !two) break;
            float mx = fmaxf(fmaxf(s[ct][0], s[ct][1]), fmaxf(s[ct][2], s[ct][3]));
            mx = xmax32(xmax16(mx));
            const float mnew = fmaxf(mrow[ct], mx * sc);
            if (__builtin_amdgcn_ballot_w64(mnew > mrow[ct])) {  // some column's max grew
              const float alpha = __builtin_amdgcn_exp2f(mrow[ct] - mnew);        // 0 on the first block
              lsum[ct] *= alpha;
#pragma unroll
              for (int dt = 0; dt < 8; ++dt) o[ct][dt] *= alpha;
              mrow[ct] = mnew;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float p = __builtin_amdgcn_exp2f(fmaf(s[ct][j], sc, -mrow[ct]));
              const __bf16 hi = (__bf16)p;
              pb[ct][j] = hi;
              pb[ct][4 + j] = (__bf16)(p - (float)hi);
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
          for (int ct = 0; ct < NCT; ++ct) {
            if (ct == 1 && !two) break;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
              const bf16x8 a = __builtin_shufflevector(va[dt], va[dt], 0, 1, 2, 3, 0, 1, 2, 3);
              o[ct][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[ct], o[ct][dt], 0, 0, 0);
            }
          }
        }
      }
      // Triples of this wave's columns (empty if the stripe had no block).
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const float l = xsum32(xsum16(lsum[ct]));
        const int col = 16 * ct + c16;
        if (col < cr.ncol) {
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
}

}  // namespace

// Both passes: the work items of the bin of each workgroup.  The bin heads,
// items, pools and strides come first among the arguments so that they can
// be preloaded into scalar registers.
__global__ __launch_bounds__(kWaves * 64, 2) void fca_attention_kernel(const BinHead* __restrict__ bins,
                                                                      const WorkItem* __restrict__ items,
                                                                      const char* k, const char* v, int64_t ksb,
                                                                      int64_t ksh, int64_t vsb, int64_t vsh,
                                                                      GqaParams p) {
  const CopyArgs ca{bins, items, k, v, ksb, ksh, vsb, vsh};
  stream_body<false>(ca, p);
}

// Plans that launch the two passes one after the other: the same body under
// one entry name per pass, so that kernel traces and counters tell the
// passes apart.
__global__ __launch_bounds__(kWaves * 64, 2) void fca_attention_grouped_kernel(const BinHead* __restrict__ bins,
                                                                              const WorkItem* __restrict__ items,
                                                                              const char* k, const char* v,
                                                                              int64_t ksb, int64_t ksh, int64_t vsb,
                                                                              int64_t vsh, GqaParams p) {
  const CopyArgs ca{bins, items, k, v, ksb, ksh, vsb, vsh};
  stream_body<false>(ca, p);
}
__global__ __launch_bounds__(kWaves * 64, 2) void fca_attention_suffix_kernel(const BinHead* __restrict__ bins,
                                                                             const WorkItem* __restrict__ items,
                                                                             const char* k, const char* v,
                                                                             int64_t ksb, int64_t ksh, int64_t vsb,
                                                                             int64_t vsh, GqaParams p) {
  const CopyArgs ca{bins, items, k, v, ksb, ksh, vsb, vsh};
  stream_body<false>(ca, p);
}

// The same for pools of token rows (every pass).
__global__ __launch_bounds__(kWaves * 64, 2) void fca_attention_rows_kernel(const BinHead* __restrict__ bins,
                                                                           const WorkItem* __restrict__ items,
                                                                           const char* k, const char* v,
                                                                           int64_t ksb, int64_t ksh, int64_t vsb,
                                                                           int64_t vsh, GqaParams p) {
  const CopyArgs ca{bins, items, k, v, ksb, ksh, vsb, vsh};
  stream_body<true>(ca, p);
}

hipError_t launch_attention(const GqaParams& p, int n_bins, PassSet passes, hipStream_t s) {
  if (n_bins <= 0) return hipSuccess;
  const auto kernel = p.k_stride_token != 0   ? fca_attention_rows_kernel
                      : passes == kGroupedPass ? fca_attention_grouped_kernel
                      : passes == kSuffixPass  ? fca_attention_suffix_kernel
                                               : fca_attention_kernel;
  hipLaunchKernelGGL(kernel, dim3(n_bins), dim3(kWaves * 64), 0, s, p.bins, p.items,
                     static_cast<const char*>(p.k), static_cast<const char*>(p.v), p.k_stride_block,
                     p.k_stride_head, p.v_stride_block, p.v_stride_head, p);
  return hipGetLastError();
}

}  // namespace fca
