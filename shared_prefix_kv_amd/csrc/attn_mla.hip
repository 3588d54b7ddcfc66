// Grouped prefix pass and per-request suffix pass for a latent (MLA-style)
// cache, gfx950: one 576-wide cache row per token, keys = the whole row,
// values = its first 512 columns (read once, as part of the key tile).
//
// Same method as the GQA kernel ("Core Mechanism" of the ZoRRo Inference &
// Forest Cascade Attention page, step 2), but every query row now costs
// 2 x (576 + 512) flops per token and a request alone has Hq/Hkv = 128 query
// rows, so both passes are matrix products and the grouped pass is bound by
// the MFMA rate, not by HBM.  A workgroup of 4 waves (one per SIMD, up to
// 512 registers each) owns an item of up to 64 query rows (one 16-row tile
// per wave: the wave's Q operand and its 512-dim output stay in registers
// for the whole item) and one 64-token block at a time; the block's 72 KiB
// key tile is copied once into LDS (global_load_lds_dwordx4, a two-slot ring,
// one block ahead) and read by all four waves.
//
// Per 64-token block and wave:
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16: 4 token tiles x 18 d-steps,
//     the key A operand read straight from the chunked layout (1 KiB per
//     instruction), the Q B operand held in registers for the whole item;
//   * online softmax per query row in the log2 domain (4 lane groups reduced
//     with permlane swaps, lazy rescale on a wave-uniform test);
//   * O^T += V^T P^T with v_mfma_f32_16x16x16_bf16: the scores are already in
//     the P^T operand layout; the V^T operand (16 value dims x 4 tokens per
//     lane) is read from the same chunked key tile with ds_read_b64_tr_b16,
//     whose 16-lane transpose turns the token-major rows into dim-major
//     operands: lane (g, c) supplies the 8 bytes of token 4g + c/4, dims
//     4(c%4)..4(c%4)+3 of the tile and receives dim c of tokens 4g..4g+3.
// Tokens at or past the end of the range are masked (-inf scores, zeroed
// values: the tail of a block may hold NaN).

#include <cmath>

#include "fca_internal.h"

namespace fca {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(4))) const int32_t cint32;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kDq = 576;                   // key (and query) dims
constexpr int kDv = 512;                   // value dims: the first kDv key dims
constexpr int kBS = 64;                    // tokens per cache block
constexpr int kKs = kDq / 32;              // d-steps of the score product
constexpr int kDt = kDv / 16;              // 16-dim value tiles
constexpr int kTileBytes = kBS * kDq * 2;  // one (block, head) tile: 72 KiB
constexpr int kWaves = 4;
constexpr int kWaveCols = 16;              // query rows per wave
constexpr int kChunkStride = kBS * 16;     // bytes between 8-dim chunks of a tile

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

// s_waitcnt until no vector-memory operation of this wave is outstanding.
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8)); }

__device__ __forceinline__ WorkItem load_item(cint32* items, int i) {
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
  w.stripes = w.pad2 = 0;
  return w;
}

__device__ __forceinline__ int item_blocks(const WorkItem& it) { return (it.tok_end - it.tok_begin + kBS - 1) / kBS; }

}  // namespace

__global__ __launch_bounds__(kWaves * 64, 1) void fca_mla_kernel(GqaParams P) {
  __shared__ __attribute__((aligned(1024))) char lds[2 * kTileBytes];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int c16 = lane & 15;
  const float NEG_INF = -INFINITY;
  const float sc = P.scale_log2;

  cint32* head = (cint32*)(P.bins + blockIdx.x);
  cint32* items = (cint32*)(P.items);
  cint32* bt = (cint32*)(P.bt);
  cint32* perm = (cint32*)(P.perm);
  const int i_begin = head[0];
  const int i_end = head[1];
  const char* kpool = static_cast<const char*>(P.k);
  const __bf16* qbase = static_cast<const __bf16*>(P.q);

  // ---- copy cursor: item di, block db ----
  int di = i_begin, db = 0;
  WorkItem dit = load_item(items, di);
  int dnb = item_blocks(dit);
  // Copy block db of item di into a slot: 72 instructions of 1 KiB, 18 per
  // wave (wave w copies chunks 18w .. 18w + 17 of the 72 8-dim chunks).
  auto issue = [&](int slot) {
    const int id = bt[(int64_t)dit.request * P.W + dit.tok_begin / kBS + db];
    const char* src =
        kpool + ((int64_t)id * P.k_stride_block + (int64_t)dit.kv_head * P.k_stride_head) * 2 + lane * 16;
    char* dst = lds + slot * kTileBytes;
#pragma unroll
    for (int i = 0; i < kTileBytes / 1024 / kWaves; ++i) {
      const int off = (wave * (kTileBytes / 1024 / kWaves) + i) * 1024;
      __builtin_amdgcn_global_load_lds(src + off, (lds_void*)(dst + off), 16, 0, 0);
    }
    if (++db == dnb) {
      db = 0;
      if (++di < i_end) {
        dit = load_item(items, di);
        dnb = item_blocks(dit);
      }
    }
  };

  // ---- compute cursor ----
  WorkItem cit = load_item(items, i_begin);
  int ci = i_begin, cb = 0, cnb = item_blocks(cit);
  int c_lo = 0, ncol = 0;  // this wave's columns of the item, relative to col0
  bf16x8 qb[kKs];
  f32x4 o[kDt];
  float mrow = NEG_INF, lsum = 0.f;

  // Q^T operand of the wave's 16 columns (d-chunk 32 ks + 8 g of column
  // c16) and fresh accumulators.  Columns past the item read its first row
  // and are zeroed.
  auto begin_item = [&]() {
    const int ccols = cit.col1 - cit.col0;
    c_lo = wave * kWaveCols;
    ncol = min(kWaveCols, ccols - c_lo);
    const bool use = c16 < ncol;
    const int col = cit.col0 + (use ? c_lo + c16 : 0);
    const int member = cit.member_off >= 0 ? perm[cit.member_off + col / P.r] : cit.request;
    const int qh = cit.kv_head * P.r + col % P.r;
    const __bf16* qp = qbase + ((int64_t)member * P.Hq + qh) * kDq + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + 32 * ks);
      qb[ks] = use ? v : bf16x8{};
    }
    mrow = NEG_INF;
    lsum = 0.f;
#pragma unroll
    for (int dt = 0; dt < kDt; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  };

  auto compute_block = [&](const char* kt, int t0) {
    // Scores of the 4 token tiles.
    f32x4 s[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) s[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt + (4 * ks + g) * kChunkStride + (16 * tt + c16) * 16);
        s[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[ks], s[tt], 0, 0, 0);
      }
    }
    const bool partial = t0 + kBS > cit.tok_end;
    if (partial) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int nvalid = cit.tok_end - t0 - 16 * tt - 4 * g;
#pragma unroll
        for (int j = 0; j < 4; ++j) s[tt][j] = j < nvalid ? s[tt][j] : NEG_INF;
      }
    }
    float mx = NEG_INF;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) mx = fmaxf(mx, fmaxf(fmaxf(s[tt][0], s[tt][1]), fmaxf(s[tt][2], s[tt][3])));
    mx = xmax32(xmax16(mx));
    const float mnew = fmaxf(mrow, mx * sc);
    if (__builtin_amdgcn_ballot_w64(mnew > mrow)) {  // some column's max grew
      const float alpha = exp2f(mrow - mnew);
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < kDt; ++dt) o[dt] *= alpha;
      mrow = mnew;
    }
    bf16x4 pb[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p = exp2f(fmaf(s[tt][j], sc, -mrow));
        pb[tt][j] = (__bf16)p;
        lsum += p;
      }
    // Values: the V^T operand of (value tile dt, token tile tt) through the
    // transposing LDS read; tokens past the range are zeroed.
    const int tr_off = ((c16 & 3) / 2) * kChunkStride + (4 * g + c16 / 4) * 16 + (c16 & 1) * 8;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      u32x2 keep = {0xffffffffu, 0xffffffffu};
      if (partial) {
        const int nvalid = cit.tok_end - t0 - 16 * tt - 4 * g;
        keep = u32x2{(nvalid > 0 ? 0xffffu : 0u) | (nvalid > 1 ? 0xffff0000u : 0u),
                     (nvalid > 2 ? 0xffffu : 0u) | (nvalid > 3 ? 0xffff0000u : 0u)};
      }
#pragma unroll
      for (int dt = 0; dt < kDt; ++dt) {
        const char* src = kt + 2 * dt * kChunkStride + 16 * tt * 16 + tr_off;
        const i16x4 raw = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)src);
        const bf16x4 a = __builtin_bit_cast(bf16x4, __builtin_bit_cast(u32x2, raw) & keep);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pb[tt], o[dt], 0, 0, 0);
      }
    }
  };

  auto finish_item = [&]() {
    const float l = xsum32(xsum16(lsum));
    if (c16 < ncol) {
      const int64_t row = (int64_t)cit.part_base + c_lo + c16;
      float* dst = P.part.o + row * kDv + 4 * g;
#pragma unroll
      for (int dt = 0; dt < kDt; ++dt) *reinterpret_cast<f32x4*>(dst + 16 * dt) = o[dt];
      if (g == 0) {
        P.part.m[row] = mrow;
        P.part.l[row] = l;
      }
    }
  };

  issue(0);
  for (int it = 0;; ++it) {
    // Block `it` has landed for every wave, and every wave is done with
    // block it - 1, whose slot the next copy reuses.
    wait_vm_all();
    __syncthreads();
    if (cb == 0) begin_item();
    if (di < i_end) issue((it + 1) & 1);
    if (ncol > 0) compute_block(lds + (it & 1) * kTileBytes, cit.tok_begin + cb * kBS);
    if (++cb == cnb) {
      if (ncol > 0) finish_item();
      if (++ci == i_end) break;
      cit = load_item(items, ci);
      cnb = item_blocks(cit);
      cb = 0;
    }
  }
}

hipError_t launch_mla(const GqaParams& p, int n_bins, hipStream_t s) {
  if (n_bins <= 0) return hipSuccess;
  hipLaunchKernelGGL(fca_mla_kernel, dim3(n_bins), dim3(kWaves * 64), 0, s, p);
  return hipGetLastError();
}

}  // namespace fca
