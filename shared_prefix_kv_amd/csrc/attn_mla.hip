// Grouped prefix pass and per-request suffix pass for a latent (MLA-style)
// cache, gfx950: one 576-wide cache row per token, keys = the whole row,
// values = its first 512 columns (read once, as part of the key tile).
//
// Same method as the GQA kernel ("Core Mechanism" of the ZoRRo Inference &
// Forest Cascade Attention page, step 2), but every query row costs
// 2 x (576 + 512) flops per token and a request alone has Hq/Hkv = 128 query
// rows, so both passes are matrix products and the grouped pass is bound by
// the MFMA rate and by LDS, not by HBM.
//
// A workgroup of 8 waves (two per SIMD) owns an item of up to 64 query rows
// and walks its token range in 32-token stages (half a cache block, 36 KiB):
//   * a 4-slot LDS ring, filled two stages ahead by buffer_load_dwordx4 ... lds
//     issued by the value waves (which otherwise wait for the score waves at
//     the barrier; copies issued by the score waves stall their products),
//     one barrier per stage (s_barrier after the own copies and LDS writes
//     are done: no memory fence, which would wait for the copies still in
//     flight);
//   * score waves 0-3, 16 query rows each (the Q operand stays in registers
//     for the whole item): S^T = K Q^T with v_mfma_f32_16x16x32_bf16, online
//     softmax per row in the log2 domain with a lazy running max (raised
//     only when a score exceeds it by more than 2^8, so rescales are rare),
//     then P goes to LDS as one fp16 tile (11 significant bits; bf16 would
//     keep 8, which leaves errors above the tolerance on requests of a few
//     tokens whose value rows cancel) and the row's rescale factor beside it;
//   * value waves 4-7, one stage behind, each owning 128 of the 512 value
//     dims of all 64 rows: O^T += V^T P^T with v_mfma_f32_16x16x32_f16, the
//     V^T operand read from the key tile with ds_read_b64_tr_b16 (two 16-token
//     tiles per operand) and converted from bf16 to fp16 in registers (exact:
//     every bf16 value of magnitude below 65504 is an fp16 value, apart from
//     the fp16 subnormal range below 2^-14, where the conversion keeps an
//     absolute error under 2^-24), and the P^T operand as the score waves
//     wrote it.
// Splitting the value dims keeps every wave under 256 registers, so each
// SIMD runs a score wave and a value wave side by side, and the value tile
// is read from LDS once per workgroup instead of once per 16 rows.
// Tokens at or past the end of the range are masked (-inf scores, zeroed
// values: the tail of a block may hold NaN).

#include <cmath>

#include "fca_internal.h"

namespace fca {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(4))) const int32_t cint32;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kDq = 576;                         // key (and query) dims
constexpr int kDv = 512;                         // value dims: the first kDv key dims
constexpr int kBS = 64;                          // tokens per cache block
constexpr int kStage = 32;                       // tokens per pipeline stage
constexpr int kStageBytes = kStage * kDq * 2;    // 36 KiB
constexpr int kChunk = kStage * 16;              // one 8-dim chunk of a stage in LDS
constexpr int kSlots = 4;                        // LDS ring
constexpr int kKs = kDq / 32;                    // d-steps of the score product
constexpr int kQkWaves = 4;                      // score waves, 16 rows each
constexpr int kPvWaves = 4;                      // value waves
constexpr int kWaves = kQkWaves + kPvWaves;
constexpr int kPvDims = kDv / kPvWaves;          // value dims per value wave
constexpr int kPvTiles = kPvDims / 16;
constexpr int kDmaP = kStageBytes / 1024 / kPvWaves;  // 1 KiB copies per stage and value wave
static_assert(kPvWaves * kDmaP * 1024 == kStageBytes, "stage copy split");
constexpr float kTau = 8.f;                      // lazy-max threshold (log2 units)
constexpr int kBufferWord3 = 0x00020000;         // raw buffer resource, gfx9 family

constexpr int kOffP = kSlots * kStageBytes;      // P^T operands (fp16) [2][4 col tiles][64 lanes] x 16 B
constexpr int kPTile = kQkWaves * 64 * 16;
constexpr int kOffA = kOffP + 2 * kPTile;        // rescale factor of each row [2][64] fp32
constexpr int kLdsBytes = kOffA + 2 * 64 * 4;
static_assert(kLdsBytes <= 160 * 1024, "LDS");

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

// s_waitcnt until at most N vector-memory operations of this wave are
// outstanding (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// The 16 V^T operands of a value wave's stage: ds_read_b64_tr_b16 at
// kt + 1024 dt + 256 tt for dt < 8, tt < 2, in one block that waits for its
// own results (the compiler would otherwise wait for every LDS copy in
// flight before each transposing read, as it cannot tell them apart).
__device__ __forceinline__ void read_vt(const char* kt, u32x2 (&r)[8][2]) {
  const uint32_t a = (uint32_t)(uintptr_t)kt;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16 offset:0\n"
      "ds_read_b64_tr_b16 %1, %16 offset:256\n"
      "ds_read_b64_tr_b16 %2, %16 offset:1024\n"
      "ds_read_b64_tr_b16 %3, %16 offset:1280\n"
      "ds_read_b64_tr_b16 %4, %16 offset:2048\n"
      "ds_read_b64_tr_b16 %5, %16 offset:2304\n"
      "ds_read_b64_tr_b16 %6, %16 offset:3072\n"
      "ds_read_b64_tr_b16 %7, %16 offset:3328\n"
      "ds_read_b64_tr_b16 %8, %16 offset:4096\n"
      "ds_read_b64_tr_b16 %9, %16 offset:4352\n"
      "ds_read_b64_tr_b16 %10, %16 offset:5120\n"
      "ds_read_b64_tr_b16 %11, %16 offset:5376\n"
      "ds_read_b64_tr_b16 %12, %16 offset:6144\n"
      "ds_read_b64_tr_b16 %13, %16 offset:6400\n"
      "ds_read_b64_tr_b16 %14, %16 offset:7168\n"
      "ds_read_b64_tr_b16 %15, %16 offset:7424\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0][0]), "=&v"(r[0][1]), "=&v"(r[1][0]), "=&v"(r[1][1]), "=&v"(r[2][0]), "=&v"(r[2][1]),
        "=&v"(r[3][0]), "=&v"(r[3][1]), "=&v"(r[4][0]), "=&v"(r[4][1]), "=&v"(r[5][0]), "=&v"(r[5][1]),
        "=&v"(r[6][0]), "=&v"(r[6][1]), "=&v"(r[7][0]), "=&v"(r[7][1])
      : "v"(a)
      : "memory");
}
static_assert(2 * kChunk == 1024 && 16 * 16 == 256 && kPvTiles == 8, "read_vt offsets");

// Stage arrangement of a token-row pool (see Copier): 9 groups of 8 chunks,
// group G holding 128 bytes of each of the 32 tokens (4 KiB), the 16-byte
// chunk p of token t's row at position p ^ swz(t) with swz(t) = (t / 2) % 8,
// which spreads the 16 lanes of an operand read over all banks.
constexpr int kRowGroup = kStage * 128;  // bytes of one 8-chunk group
__device__ __forceinline__ int swz(int t) { return (t >> 1) & 7; }

// The 16 V^T operands from a token-row stage: ds_read_b64_tr_b16 at
// a[dt % 4] + 4096 (dt / 4) + 2048 tt.
__device__ __forceinline__ void read_vt_rows(const uint32_t (&a)[4], u32x2 (&r)[8][2]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16 offset:0\n"
      "ds_read_b64_tr_b16 %1, %16 offset:2048\n"
      "ds_read_b64_tr_b16 %2, %17 offset:0\n"
      "ds_read_b64_tr_b16 %3, %17 offset:2048\n"
      "ds_read_b64_tr_b16 %4, %18 offset:0\n"
      "ds_read_b64_tr_b16 %5, %18 offset:2048\n"
      "ds_read_b64_tr_b16 %6, %19 offset:0\n"
      "ds_read_b64_tr_b16 %7, %19 offset:2048\n"
      "ds_read_b64_tr_b16 %8, %16 offset:4096\n"
      "ds_read_b64_tr_b16 %9, %16 offset:6144\n"
      "ds_read_b64_tr_b16 %10, %17 offset:4096\n"
      "ds_read_b64_tr_b16 %11, %17 offset:6144\n"
      "ds_read_b64_tr_b16 %12, %18 offset:4096\n"
      "ds_read_b64_tr_b16 %13, %18 offset:6144\n"
      "ds_read_b64_tr_b16 %14, %19 offset:4096\n"
      "ds_read_b64_tr_b16 %15, %19 offset:6144\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0][0]), "=&v"(r[0][1]), "=&v"(r[1][0]), "=&v"(r[1][1]), "=&v"(r[2][0]), "=&v"(r[2][1]),
        "=&v"(r[3][0]), "=&v"(r[3][1]), "=&v"(r[4][0]), "=&v"(r[4][1]), "=&v"(r[5][0]), "=&v"(r[5][1]),
        "=&v"(r[6][0]), "=&v"(r[6][1]), "=&v"(r[7][0]), "=&v"(r[7][1])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
      : "memory");
}
static_assert(kRowGroup == 4096 && 16 * 128 == 2048 && kStageBytes == 9 * kRowGroup, "read_vt_rows offsets");

// Workgroup barrier for LDS hand-offs: this wave's LDS operations are done,
// then s_barrier.  The empty asm statements keep the compiler from moving
// memory accesses across it.  Copies into LDS are waited for separately.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((15 << 0) | (7 << 4) | (0 << 8) | (3 << 14));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

struct Item {
  int request, tok_begin, tok_end, kv_head, member_off, col0, col1, part_base;
};

__device__ __forceinline__ Item load_item(cint32* items, int i) {
  cint32* p = items + 12 * i;
  Item w;
  w.request = p[0];
  w.tok_begin = p[1];
  w.tok_end = p[2];
  w.kv_head = p[3];
  w.member_off = p[4];
  w.col0 = p[6];
  w.col1 = p[7];
  w.part_base = p[8];
  return w;
}

__device__ __forceinline__ int item_stages(const Item& it) { return (it.tok_end - it.tok_begin + kStage - 1) / kStage; }

// Copy cursor: the stages of the bin's items in order, two ahead of the
// score waves.  Each wave copies instructions [d0, d0 + N) of a stage:
// instruction i moves chunks 2i and 2i + 1 (32 tokens x 16 B each) of the
// stage into LDS bytes [1024 i, 1024 i + 1024) of the slot; each chunk is
// 512 contiguous bytes of the tile.  From token rows (ROWS) the stage is
// arranged by 8-chunk groups instead (kRowGroup): instruction i copies 128
// bytes of each of tokens 8 (i % 4) .. + 7 of group i / 4, 8 lanes per token
// reading one 128-byte segment of its row, lane l filling position l % 8
// from chunk (l % 8) ^ swz(t).
template <int N, bool ROWS>
struct Copier {
  cint32* items;
  int di, ds, dns, i_end;
  Item it;
  __device__ __forceinline__ void next() {
    if (++ds == dns) {
      ds = 0;
      if (++di < i_end) {
        it = load_item(items, di);
        dns = item_stages(it);
      }
    }
  }
  __device__ __forceinline__ void issue(const GqaParams& P, cint32* bt, char* slot, int d0, int lane) {
    const int t0 = it.tok_begin + ds * kStage;
    const int id = bt[(int64_t)it.request * P.W + t0 / kBS];
    const char* tile = static_cast<const char*>(P.k) +
                       ((int64_t)id * P.k_stride_block + (int64_t)it.kv_head * P.k_stride_head) * 2;
    if constexpr (ROWS) {
      // Raw buffer over the stage's 32 rows; the plan checks that
      // 64 * k_stride_token bytes stay far inside 32-bit offsets.
      const int rb = (int)P.k_stride_token * 2;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(tile + (int64_t)(t0 % kBS) * rb), (short)0, (kStage - 1) * rb + kDq * 2, kBufferWord3);
      // token t = 8 (i % 4) + l / 8: swz(t) = 4 (i % 2) + l / 16, so the lane
      // part of the offset depends on i only through i % 2.
      const int vrow = (lane >> 3) * rb;
      const int voff0 = vrow + 16 * ((lane & 7) ^ (lane >> 4));
      const int voff1 = vrow + 16 * ((lane & 7) ^ (4 + (lane >> 4)));
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int ii = d0 + i;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(slot + ii * 1024), 16, (ii & 1) ? voff1 : voff0,
                                                 8 * (ii & 3) * rb + 128 * (ii >> 2), 0, 0);
      }
    } else {
      // Raw buffer over the tile (MUBUF loads to LDS: counted by vmcnt alone).
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(tile), (short)0, kBS * kDq * 2, kBufferWord3);
      const int voff = (lane >> 5) * (kBS * 16) + (lane & 31) * 16;
      const int half = ((t0 / kStage) & 1) * kChunk;
#pragma unroll
      for (int i = 0; i < N; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(slot + (d0 + i) * 1024), 16, voff,
                                                 half + (d0 + i) * 2 * (kBS * 16), 0, 0);
    }
    next();
  }
};

}  // namespace

// ROWS: the pool holds token rows (P.k_stride_token), else tiles.
template <bool ROWS>
__device__ __forceinline__ void mla_body(GqaParams P) {
  __shared__ __attribute__((aligned(1024))) char lds[kLdsBytes];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int c16 = lane & 15;
  const float NEG_INF = -INFINITY;

  cint32* head = (cint32*)(P.bins + blockIdx.x);
  cint32* items = (cint32*)(P.items);
  const int i_begin = head[0];
  const int i_end = head[1];
  int N = 0;  // stages of the bin
  for (int i = i_begin; i < i_end; ++i) {
    cint32* p = items + 12 * i;
    N += (p[2] - p[1] + kStage - 1) / kStage;
  }
  if (N == 0) return;

  if (wave < kQkWaves) {
    // ---------------- score wave: rows 16 w .. 16 w + 15 of the item ----------------
    const int w = wave;

    const __bf16* qbase = static_cast<const __bf16*>(P.q);
    cint32* perm = (cint32*)(P.perm);
    const float sc = P.scale_log2;
    Item it = load_item(items, i_begin);
    int ci = i_begin, cs = 0, cns = item_stages(it);
    bf16x8 qb[kKs];
    float mrow = NEG_INF, lsum = 0.f;
    bool active = false;

    for (int t = 0; t <= N; ++t) {
      // Stage t has landed once the value waves that copy it pass the barrier.
      lds_barrier();
      if (t == N) break;

      const int ccols = it.col1 - it.col0;
      if (cs == 0) {
        // Q^T operand of the wave's 16 rows (d-chunk 32 ks + 8 g of row c16);
        // rows past the item read its first row.
        active = 16 * w < ccols;
        const int col = it.col0 + (16 * w + c16 < ccols ? 16 * w + c16 : 0);
        const int member = it.member_off >= 0 ? perm[it.member_off + col / P.r] : it.request;
        const int qh = it.kv_head * P.r + col % P.r;
        const __bf16* qp = qbase + ((int64_t)member * P.Hq + qh) * kDq + 8 * g;
#pragma unroll
        for (int ks = 0; ks < kKs; ++ks) qb[ks] = *reinterpret_cast<const bf16x8*>(qp + 32 * ks);
        wait_vm<0>();
        mrow = NEG_INF;
        lsum = 0.f;
      }
      const int buf = t & 1;
      if (active) {
        // S^T = K Q^T over 18 d-steps; the key operands are read from LDS
        // in 6 batches of 3 d-steps, one batch ahead of the products.
        // Key operand of d-step ks, tokens c16 and 16 + c16: chunk 4 ks + g.
        // Tiles: kt + 4 ks kChunk (+ 256).  Rows: group ks / 2, position
        // (4 (ks % 2) + g) ^ swz(c16): kr[ks % 2] + 4096 (ks / 2) (+ 2048).
        const char* stage = lds + (t % kSlots) * kStageBytes;
        const char* kt = stage + g * kChunk + c16 * 16;
        const char* kr0 = stage + c16 * 128 + ((g ^ swz(c16)) * 16);
        const char* kr1 = stage + c16 * 128 + (((4 + g) ^ swz(c16)) * 16);
        auto key = [&](int ks, int half) -> bf16x8 {
          if constexpr (ROWS)
            return *reinterpret_cast<const bf16x8*>(((ks & 1) ? kr1 : kr0) + (ks >> 1) * kRowGroup + half * 2048);
          else
            return *reinterpret_cast<const bf16x8*>(kt + 4 * ks * kChunk + half * 256);
        };
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0;
        constexpr int kB = 3;
        __builtin_amdgcn_s_setprio(1);  // the score products go first on the shared MFMA pipe
        bf16x8 ka[2][2 * kB];
#pragma unroll
        for (int i = 0; i < kB; ++i) {
          ka[0][2 * i] = key(i, 0);
          ka[0][2 * i + 1] = key(i, 1);
        }
#pragma unroll
        for (int b = 0; b < kKs / kB; ++b) {
          __builtin_amdgcn_sched_barrier(0);
          if (b + 1 < kKs / kB) {
#pragma unroll
            for (int i = 0; i < kB; ++i) {
              const int ks = (b + 1) * kB + i;
              ka[(b + 1) & 1][2 * i] = key(ks, 0);
              ka[(b + 1) & 1][2 * i + 1] = key(ks, 1);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < kB; ++i) {
            s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[b & 1][2 * i], qb[b * kB + i], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[b & 1][2 * i + 1], qb[b * kB + i], s1, 0, 0, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        const int nvalid = it.tok_end - (it.tok_begin + cs * kStage);
        if (nvalid < kStage) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            s0[j] = 4 * g + j < nvalid ? s0[j] : NEG_INF;
            s1[j] = 16 + 4 * g + j < nvalid ? s1[j] : NEG_INF;
          }
        }
        float mx = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])),
                         fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
        mx = xmax32(xmax16(mx)) * sc;
        float alpha = 1.f;
        if (__builtin_amdgcn_ballot_w64(mx > mrow + kTau)) {
          const float mnew = mx > mrow + kTau ? mx : mrow;
          alpha = __builtin_amdgcn_exp2f(mrow - mnew);
          lsum *= alpha;
          mrow = mnew;
        }
        f16x8 ph;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s0[j], sc, -mrow));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s1[j], sc, -mrow));
          lsum += p0 + p1;
          ph[j] = (_Float16)p0;
          ph[4 + j] = (_Float16)p1;
        }
        *reinterpret_cast<f16x8*>(lds + kOffP + buf * kPTile + (w * 64 + lane) * 16) = ph;
        if (g == 0) *reinterpret_cast<float*>(lds + kOffA + buf * 256 + (16 * w + c16) * 4) = alpha;
      }
      if (++cs == cns) {
        if (active) {
          const float l = xsum32(xsum16(lsum));
          if (g == 0 && 16 * w + c16 < ccols) {
            const int64_t row = (int64_t)it.part_base + 16 * w + c16;
            P.part.m[row] = mrow;
            P.part.l[row] = l;
          }
        }
        cs = 0;
        if (++ci < i_end) {
          it = load_item(items, ci);
          cns = item_stages(it);
        }
      }
    }
  } else {
    // ---------------- value wave: dims 128 v .. 128 v + 127 of all rows ----------------
    const int v = wave - kQkWaves;
    cint32* bt = (cint32*)(P.bt);
    Copier<kDmaP, ROWS> cp{items, i_begin, 0, 0, i_end, load_item(items, i_begin)};
    cp.dns = item_stages(cp.it);
    const int d0 = v * kDmaP;
    cp.issue(P, bt, lds, d0, lane);
    if (N > 1) cp.issue(P, bt, lds + kStageBytes, d0, lane);
    Item it = load_item(items, i_begin);
    int ci = i_begin, cs = 0, cns = item_stages(it);
    f32x4 o[4][kPvTiles];
    // ds_read_b64_tr_b16 source of lane (g, c16) in a 16 x 16 (token, dim)
    // tile: token 4 g + c16 / 4, dims 4 (c16 % 4) .. + 3; it receives dim
    // c16 of tokens 4 g .. 4 g + 3.
    const int tr_off = ((c16 & 3) >> 1) * kChunk + (4 * g + (c16 >> 2)) * 16 + (c16 & 1) * 8;
    // Token rows: chunk 16 v + 2 dt + (c16 % 4) / 2 of token t = 16 tt + 4 g +
    // c16 / 4 sits in group 2 v + dt / 4 at position (2 (dt % 4) + (c16 % 4) /
    // 2) ^ swz(t), and swz(t) does not depend on tt.
    uint32_t tr_rows[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      tr_rows[j] = (uint32_t)(2 * v * kRowGroup + (4 * g + (c16 >> 2)) * 128 +
                              (((2 * j + ((c16 & 3) >> 1)) ^ swz(4 * g + (c16 >> 2))) * 16) + (c16 & 1) * 8);

    for (int t = 0; t <= N; ++t) {
      if (t + 1 < N)
        wait_vm<kDmaP>();
      else
        wait_vm<0>();
      lds_barrier();
      if (t == 0) {
        if (2 < N) cp.issue(P, bt, lds + 2 * kStageBytes, d0, lane);
        continue;
      }

      // Stage t - 1.
      const int buf = (t - 1) & 1;
      const int ccols = it.col1 - it.col0;
      const int nct = (ccols + 15) >> 4;
      f16x8 ph[4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
        ph[ct] = *reinterpret_cast<const f16x8*>(lds + kOffP + buf * kPTile + (ct * 64 + lane) * 16);
      float al[4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) al[ct] = *reinterpret_cast<const float*>(lds + kOffA + buf * 256 + (16 * ct + c16) * 4);
      // The copy of stage t + 2 goes into the slot of stage t - 2, which
      // every wave finished before this barrier.  It is issued after the P
      // reads, which then reach LDS ahead of more of the score waves' key
      // reads (2 % faster than copying first).
      if (t + 2 < N) cp.issue(P, bt, lds + ((t + 2) % kSlots) * kStageBytes, d0, lane);
      u32x2 vr[kPvTiles][2];
      if constexpr (ROWS) {
        const uint32_t sb = (uint32_t)(uintptr_t)(lds + ((t - 1) % kSlots) * kStageBytes);
        const uint32_t a[4] = {sb + tr_rows[0], sb + tr_rows[1], sb + tr_rows[2], sb + tr_rows[3]};
        read_vt_rows(a, vr);
      } else {
        const char* kt = lds + ((t - 1) % kSlots) * kStageBytes + (2 * v * kPvTiles) * kChunk + tr_off;
        read_vt(kt, vr);
      }
      const int nvalid = it.tok_end - (it.tok_begin + cs * kStage);
      if (nvalid < kStage) {
        // Tokens past the range: zero their values (the operands are masked
        // here, before the products, so that the product sequence reads them
        // straight from the registers the transposing reads filled).
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int nv = nvalid - 16 * tt - 4 * g;
          const u32x2 keep = {(nv > 0 ? 0xffffu : 0u) | (nv > 1 ? 0xffff0000u : 0u),
                              (nv > 2 ? 0xffffu : 0u) | (nv > 3 ? 0xffff0000u : 0u)};
#pragma unroll
          for (int dt = 0; dt < kPvTiles; ++dt) vr[dt][tt] &= keep;
        }
      }
      // bf16 pair (low, high half of a word) -> fp16 pair: the bf16 bits are
      // the top half of the fp32 value, which converts exactly.
      auto to_f16 = [](const u32x2 (&w)[2]) {
        f16x8 a;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t x = w[i >> 1][i & 1];
          const auto h = __builtin_amdgcn_cvt_pkrtz(__uint_as_float(x << 16), __uint_as_float(x & 0xffff0000u));
          a[2 * i] = h[0];
          a[2 * i + 1] = h[1];
        }
        return a;
      };
      // The value products go first on the shared MFMA pipe (the score wave
      // of this SIMD is in its softmax or at the barrier by now).
      __builtin_amdgcn_s_setprio(2);
      // Each operand's conversion is interleaved with the products of the
      // previous one (one product, then three conversion instructions), so
      // the conversions run while the matrix pipe is busy (3 % faster than
      // converting right before each operand's products).
      auto products = [&](bool fresh) {
        f16x8 a = to_f16(vr[0]);
#pragma unroll
        for (int dt = 0; dt < kPvTiles; ++dt) {
          const f16x8 an = to_f16(vr[dt + 1 < kPvTiles ? dt + 1 : dt]);
#pragma unroll
          for (int ct = 0; ct < 4; ++ct)
            o[ct][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, ph[ct], fresh ? f32x4{0.f, 0.f, 0.f, 0.f} : o[ct][dt],
                                                               0, 0, 0);
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // three VALU
          }
          a = an;
        }
      };
      if (cs == 0) {
        // First stage of the item: fresh accumulators.
        products(true);
      } else {
        bool scale = false;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) scale |= ct < nct && al[ct] != 1.f;
        if (__builtin_amdgcn_ballot_w64(scale)) {
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) {
            const float f = ct < nct ? al[ct] : 1.f;
#pragma unroll
            for (int dt = 0; dt < kPvTiles; ++dt) o[ct][dt] *= f;
          }
        }
        products(false);
      }
      __builtin_amdgcn_s_setprio(0);
      if (++cs == cns) {
        // Partial rows hold the unnormalised sums (the merge divides).
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          if (16 * ct + c16 < ccols) {
            float* dst = P.part.o + ((int64_t)it.part_base + 16 * ct + c16) * kDv + v * kPvDims + 4 * g;
#pragma unroll
            for (int dt = 0; dt < kPvTiles; ++dt) *reinterpret_cast<f32x4*>(dst + 16 * dt) = o[ct][dt];
          }
        }
        cs = 0;
        if (++ci < i_end) {
          it = load_item(items, ci);
          cns = item_stages(it);
        }
      }
    }
  }
}

// One entry per pass, so that kernel traces tell the two launches of a decode
// apart; both run the same code.
__global__ __launch_bounds__(kWaves * 64, 1) void fca_mla_grouped_kernel(GqaParams P) { mla_body<false>(P); }
__global__ __launch_bounds__(kWaves * 64, 1) void fca_mla_suffix_kernel(GqaParams P) { mla_body<false>(P); }
__global__ __launch_bounds__(kWaves * 64, 1) void fca_mla_grouped_rows_kernel(GqaParams P) { mla_body<true>(P); }
__global__ __launch_bounds__(kWaves * 64, 1) void fca_mla_suffix_rows_kernel(GqaParams P) { mla_body<true>(P); }

hipError_t launch_mla(const GqaParams& p, int n_bins, bool grouped_pass, hipStream_t s) {
  if (n_bins <= 0) return hipSuccess;
  const bool rows = p.k_stride_token != 0;
  auto* kern = grouped_pass ? (rows ? fca_mla_grouped_rows_kernel : fca_mla_grouped_kernel)
                            : (rows ? fca_mla_suffix_rows_kernel : fca_mla_suffix_kernel);
  hipLaunchKernelGGL(kern, dim3(n_bins), dim3(kWaves * 64), 0, s, p);
  return hipGetLastError();
}

}  // namespace fca
