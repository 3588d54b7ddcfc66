// Grouped prefix pass and per-request suffix pass for GQA caches, gfx950.
//
// Both passes compute, for a set of query rows and a run of cached tokens,
// the partial softmax triple (o, max, denominator) that the merge combines
// ("Core Mechanism" of the ZoRRo Inference & Forest Cascade Attention page,
// step 2: one pass over each group's shared prefix blocks, read once per
// group, and one pass per request over its own suffix blocks).
//
// Work item = (token range, KV head, column range).  Columns are the query
// rows: grouped items cover members x (Hq/Hkv) rows that all read the same
// KV tiles, so QK^T and PV are real matrix products and run on bf16 MFMA
// (v_mfma_f32_16x16x32_bf16).  A per-request item has Hq/Hkv <= 16 rows and
// uses the same code with one 16-column tile.
//
// Data flow of one 32-token step (two 16-token blocks) of one wave:
//   * keys of the step are the A operand of S^T = K Q^T: lane (g, c) loads
//     the 16-byte d-chunk 4*ks + g of token c of block mt; in the chunked key
//     layout those are 1 KiB contiguous per instruction.
//   * S^T lands with token 4*g + j of block mt in lane group g, register j,
//     column c: exactly the P^T operand of the PV product once rounded to
//     bf16 (token order inside a 32-token step is free as long as V uses it).
//   * values of the step are the A operand of O^T = V^T P^T: lane (g, c)
//     loads tokens 4g..4g+3 of block mt at value dim 16*dt + c, 8 bytes that
//     are contiguous in the transposed value layout (512 B per instruction).
//   * online softmax per column in the log2 domain; the row max is reduced
//     across the four lane groups that share a column.
// The four waves of a workgroup take interleaved 32-token steps of the item
// and fold their triples through LDS before one partial row per column is
// written.  Tokens at or past the end of the range are masked: their scores
// become -inf and their (possibly NaN) value entries are zeroed before PV.

#include <cmath>

#include "fca_internal.h"

namespace fca {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;   // head dim (keys and values)
constexpr int kBS = 16;   // tokens per cache block
constexpr int kWaves = 4;
constexpr int kLdsPad = 4;  // floats of padding per LDS row

__device__ __forceinline__ float wave_xor_max(float x, int mask) { return fmaxf(x, __shfl_xor(x, mask)); }
__device__ __forceinline__ float wave_xor_sum(float x, int mask) { return x + __shfl_xor(x, mask); }

// K/V registers of one 32-token step of one wave.
struct StepRegs {
  bf16x8 ka[2][4];
  bf16x4 va[2][8];
};

template <int NCT>
__device__ __forceinline__ void run_item(const GqaParams& P, const WorkItem& it, float* lds_o, float* lds_m,
                                         float* lds_l) {
  constexpr int NC = 16 * NCT;  // columns per wave pass
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int c16 = lane & 15;

  const int ntok = it.tok_end - it.tok_begin;
  const int ntiles = (ntok + kTileTokens - 1) / kTileTokens;
  // steps of this wave: tiles wave, wave + 4, ...
  const int nsteps = ntiles > wave ? (ntiles - wave + kWaves - 1) / kWaves : 0;
  const int32_t* btrow = P.bt + (int64_t)it.request * P.W + it.tok_begin / kBS;
  const int nblk_item = (ntok + kBS - 1) / kBS;
  const __bf16* kbase = static_cast<const __bf16*>(P.k) + (int64_t)it.kv_head * P.k_stride_head;
  const __bf16* vbase = static_cast<const __bf16*>(P.v) + (int64_t)it.kv_head * P.v_stride_head;
  const __bf16* qbase = static_cast<const __bf16*>(P.q);
  const float NEG_INF = -INFINITY;

  // Block IDs of 32 consecutive steps of this wave, two per step: lane l
  // holds the ID of block 2*(wave + 4*(k0 + l/2)) + l%2 of the item.  Slots
  // past the item read as block 0, which always exists; every token they
  // stand for is masked.
  auto load_ids = [&](int k0) -> int {
    const int b = 2 * (wave + kWaves * (k0 + (lane >> 1))) + (lane & 1);
    return b < nblk_item ? btrow[b] : 0;
  };

  for (int mc0 = it.col0; mc0 < it.col1; mc0 += NC) {
    // Q^T operand: column 16*c + c16 of this pass, d-chunk ks*32 + 8*g.
    bf16x8 qb[NCT][4];
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      const int col = mc0 + 16 * c + c16;
      if (col < it.col1) {
        const int member = it.member_off >= 0 ? P.perm[it.member_off + col / P.r] : it.request;
        const int qh = it.kv_head * P.r + col % P.r;
        const __bf16* qp = qbase + ((int64_t)member * P.Hq + qh) * kD + 8 * g;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qb[c][ks] = *reinterpret_cast<const bf16x8*>(qp + 32 * ks);
      } else {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qb[c][ks] = bf16x8{};
      }
    }

    f32x4 o[8][NCT];
    float mrow[NCT], lsum[NCT];
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      mrow[c] = NEG_INF;
      lsum[c] = 0.f;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[dt][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // Issue the loads of wave-local step k into R (both blocks always: a
    // step whose second block lies past the range reads block 0 and masks
    // all of its tokens).
    auto load_step = [&](int k, StepRegs& R, int idv) {
      const int id0 = __builtin_amdgcn_readlane(idv, 2 * (k & 31));
      const int id1 = __builtin_amdgcn_readlane(idv, 2 * (k & 31) + 1);
      const __bf16* k0 = kbase + (int64_t)id0 * P.k_stride_block;
      const __bf16* k1 = kbase + (int64_t)id1 * P.k_stride_block;
      const __bf16* v0 = vbase + (int64_t)id0 * P.v_stride_block;
      const __bf16* v1 = vbase + (int64_t)id1 * P.v_stride_block;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int off = ((4 * ks + g) * kBS + c16) * 8;
        R.ka[0][ks] = *reinterpret_cast<const bf16x8*>(k0 + off);
        R.ka[1][ks] = *reinterpret_cast<const bf16x8*>(k1 + off);
      }
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const int off = (16 * dt + c16) * kBS + 4 * g;
        R.va[0][dt] = *reinterpret_cast<const bf16x4*>(v0 + off);
        R.va[1][dt] = *reinterpret_cast<const bf16x4*>(v1 + off);
      }
    };

    // Scores, online softmax and PV of wave-local step k held in R.
    auto compute_step = [&](int k, StepRegs& R) {
      const int t0 = it.tok_begin + (wave + kWaves * k) * kTileTokens;
      // S^T = K Q^T for the two blocks of the step.
      f32x4 s[2][NCT];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int c = 0; c < NCT; ++c) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(R.ka[mt][ks], qb[c][ks], acc, 0, 0, 0);
          s[mt][c] = acc;
        }

      // Token validity (only the last step of a range can be partial).
      const bool partial = t0 + kTileTokens > it.tok_end;
      bool valid[2][4];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) valid[mt][j] = !partial || (t0 + 16 * mt + 4 * g + j < it.tok_end);
      if (partial) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int dt = 0; dt < 8; ++dt)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (!valid[mt][j]) R.va[mt][dt][j] = (__bf16)0.f;
      }

      // Online softmax per column, P^T operand in bf16.
      bf16x8 pb[NCT];
#pragma unroll
      for (int c = 0; c < NCT; ++c) {
        float sv[2][4];
        float mx = NEG_INF;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float x = valid[mt][j] ? s[mt][c][j] * P.scale_log2 : NEG_INF;
            sv[mt][j] = x;
            mx = fmaxf(mx, x);
          }
        mx = wave_xor_max(mx, 16);
        mx = wave_xor_max(mx, 32);
        const float mnew = fmaxf(mrow[c], mx);
        const float muse = (mnew == NEG_INF) ? 0.f : mnew;
        const float alpha = exp2f(mrow[c] - muse);
        mrow[c] = mnew;
        float ps = 0.f;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float p = exp2f(sv[mt][j] - muse);
            pb[c][4 * mt + j] = (__bf16)p;
            ps += p;
          }
        lsum[c] = lsum[c] * alpha + ps;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[dt][c] *= alpha;
      }

      // O^T += V^T P^T.
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const bf16x8 a = {R.va[0][dt][0], R.va[0][dt][1], R.va[0][dt][2], R.va[0][dt][3],
                          R.va[1][dt][0], R.va[1][dt][1], R.va[1][dt][2], R.va[1][dt][3]};
#pragma unroll
        for (int c = 0; c < NCT; ++c) o[dt][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[c], o[dt][c], 0, 0, 0);
      }
    };

    // Two register sets in ping-pong: the loads of step k+1 are in flight
    // while step k is computed.  The prefetch is issued unconditionally (the
    // last step re-reads its own addresses, which hit the caches) so that
    // every wait before a step's math is the same static count.  Block IDs
    // are refreshed once per 32 steps, outside the inner loop.
    StepRegs A, B;
    for (int kc = 0; kc < nsteps; kc += 32) {
      const int kend = min(nsteps, kc + 32);
      const int idv = load_ids(kc);
      int k = kc;
      load_step(k, A, idv);
      while (k + 1 < kend) {
        load_step(k + 1, B, idv);
        __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the math
        compute_step(k, A);
        load_step(min(k + 2, kend - 1), A, idv);
        __builtin_amdgcn_sched_barrier(0);
        compute_step(k + 1, B);
        k += 2;
      }
      if (k < kend) compute_step(k, A);
    }

    // Fold the four waves' triples through LDS.
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      lsum[c] = wave_xor_sum(lsum[c], 16);
      lsum[c] = wave_xor_sum(lsum[c], 32);
      const int col = 16 * c + c16;
      float* row = lds_o + (wave * NC + col) * (kD + kLdsPad);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<f32x4*>(row + 16 * dt + 4 * g) = o[dt][c];
      if (g == 0) {
        lds_m[wave * NC + col] = mrow[c];
        lds_l[wave * NC + col] = lsum[c];
      }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < NC * (kD / 4); idx += kWaves * 64) {
      const int col = idx / (kD / 4);
      const int d4 = idx % (kD / 4);
      const int n = mc0 + col;
      if (n >= it.col1) continue;
      float M = NEG_INF;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) M = fmaxf(M, lds_m[w * NC + col]);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      float L = 0.f;
      if (M != NEG_INF) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const float sc = exp2f(lds_m[w * NC + col] - M);
          L += sc * lds_l[w * NC + col];
          acc += sc * *reinterpret_cast<const f32x4*>(lds_o + (w * NC + col) * (kD + kLdsPad) + 4 * d4);
        }
      }
      const int64_t prow = (int64_t)it.part_base + n;
      *reinterpret_cast<f32x4*>(P.part.o + prow * kD + 4 * d4) = acc;
      if (d4 == 0) {
        P.part.m[prow] = M;
        P.part.l[prow] = L;
      }
    }
    __syncthreads();
  }
}

template <int NCT>
__device__ __forceinline__ void partial_kernel_body(const GqaParams& P) {
  __shared__ float lds_o[kWaves * 16 * NCT * (kD + kLdsPad)];
  __shared__ float lds_m[kWaves * 16 * NCT];
  __shared__ float lds_l[kWaves * 16 * NCT];
  const WorkItem it = P.items[blockIdx.x];
  run_item<NCT>(P, it, lds_o, lds_m, lds_l);
}

}  // namespace

// Grouped prefix pass: 32 query rows (members x Hq/Hkv) per wave pass.
__global__ __launch_bounds__(256) void fca_grouped_prefix_kernel(GqaParams P) { partial_kernel_body<2>(P); }

// Per-request suffix pass: the Hq/Hkv rows of one request.
__global__ __launch_bounds__(256, 2) void fca_suffix_decode_kernel(GqaParams P) { partial_kernel_body<1>(P); }

hipError_t launch_gqa_partial(int kind, const GqaParams& p, int n_items, hipStream_t s) {
  if (n_items <= 0) return hipSuccess;
  if (kind == 0)
    hipLaunchKernelGGL(fca_grouped_prefix_kernel, dim3(n_items), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(fca_suffix_decode_kernel, dim3(n_items), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace fca
