// Exact log-sum-exp merge of partial attention triples, gfx950.
//
// For request i and query head h the partial rows on i's path are: every
// token split of every group that contains i (walked from the deepest group
// up through its parents) and every split of i's own suffix.  Each row p
// holds o_p = sum_t 2^(s_t - m_p) v_t (unnormalised), m_p (log2 domain) and
// l_p = sum_t 2^(s_t - m_p).  With M = max_p m_p over rows with l_p > 0:
//
//   out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p
//   lse = (M + log2 sum_p 2^(m_p - M) l_p) * ln 2
//
// which is the weighting of the partial results in "Core Mechanism", step 3
// of the ZoRRo Inference & Forest Cascade Attention page, folding the
// split-K pieces and the depth levels in one pass.  Rows are taken 64 at a
// time (one per lane); the running maximum is updated per batch of rows and
// the accumulators rescaled when it grows.  The order of rows is fixed, so
// results are bit-reproducible.  A request with no tokens gets zeros and
// -inf.

#include <cmath>

#include "fca_internal.h"

namespace fca {
namespace {


__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

__device__ __forceinline__ float lane_f(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

// x + x' where x' is the value of lane ^ 32.
__device__ __forceinline__ float xsum32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Row values acc[0..N) * inv at element offset `at` of `out`, bf16 or float32.
template <int N>
__device__ __forceinline__ void store_row(void* out, int32_t out_f32, int64_t at, const float* acc, float inv) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  if (out_f32) {
    float* dst = static_cast<float*>(out) + at;
#pragma unroll
    for (int v = 0; v < N; v += 4)
      *reinterpret_cast<float4*>(dst + v) = float4{acc[v] * inv, acc[v + 1] * inv, acc[v + 2] * inv, acc[v + 3] * inv};
  } else {
    __bf16* dst = static_cast<__bf16*>(out) + at;
#pragma unroll
    for (int v = 0; v < N; v += 4) {
      const bf16x4 ob = {(__bf16)(acc[v] * inv), (__bf16)(acc[v + 1] * inv), (__bf16)(acc[v + 2] * inv),
                         (__bf16)(acc[v + 3] * inv)};
      *reinterpret_cast<bf16x4*>(dst + v) = ob;
    }
  }
}

// One wave per (request, head).  Lane j reads the j-th partial row index of
// the pair from the plan's source table, so that all (m, l) loads are issued
// at once after two dependent loads; the value rows
// are then accumulated two at a time (lanes 0-31 take even sources, lanes
// 32-63 odd ones, each lane DV/32 value dims), 2U rows in flight per wave,
// and the two halves are added at the end.  U keeps the kernel at eight
// waves per SIMD, which measured faster on MI355X than more rows per round
// trip: 8 rows of 128 dims (16 rows: 76 VGPRs, 6 waves, 2-6 % slower), 2
// rows of 512 dims (8 rows: 114 VGPRs, 4 waves, 7 % slower).
template <int DV>
__device__ __forceinline__ void merge_body(const MergeParams& P) {
  constexpr int VPL = DV / 32;         // floats per lane
  constexpr int U = DV <= 128 ? 4 : 1;  // row pairs per batch of loads
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;
  const int hl = lane & 31;
  const int64_t pair = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (pair >= (int64_t)P.B * P.Hq) return;
  // Fixed-stride tables: the row indices come straight from the pair's
  // slot (valid ones first, -1 after), one memory round trip fewer.
  const bool strided = P.src_stride > 0;
  int off0, n_src, row_first = -1;
  if (strided) {
    off0 = (int)(pair * P.src_stride);
    row_first = lane < P.src_stride ? P.src_row[off0 + lane] : -1;
    n_src = __popcll(__ballot(row_first >= 0));
  } else {
    const int2 span = P.src_span[pair];
    off0 = span.x;
    n_src = span.y;
  }

  float M = -INFINITY, L = 0.f;
  float acc[VPL];
#pragma unroll
  for (int v = 0; v < VPL; ++v) acc[v] = 0.f;
  // Value rows of sources s .. s + 2U - 1 (even ones in the lower half
  // wave, odd ones in the upper); slots past the sources are not loaded
  // and get weight 0.
  float x[U][VPL];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int v = 0; v < VPL; ++v) x[u][v] = 0.f;

  for (int base = 0; base < n_src; base += 64) {
    const int j = base + lane;
    // (strided: n_src <= 64, one batch, already loaded)
    const int row = strided ? row_first : j < n_src ? P.src_row[off0 + j] : -1;
    const int cnt = min(64, n_src - base);
    auto load_rows = [&](int s) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int se = s + 2 * u;
        if (se >= cnt) continue;  // wave-uniform
        const int re = __builtin_amdgcn_readlane(row, se);
        // a missing odd source: the upper half loads the even row (weight 0)
        const int ro = se + 1 < cnt ? __builtin_amdgcn_readlane(row, se + 1) : re;
        const float* src = P.part.o + (int64_t)(half ? ro : re) * DV + hl * VPL;
#pragma unroll
        for (int v = 0; v < VPL; v += 4) {
          const float4 t = *reinterpret_cast<const float4*>(src + v);
          x[u][v] = t.x;
          x[u][v + 1] = t.y;
          x[u][v + 2] = t.z;
          x[u][v + 3] = t.w;
        }
      }
    };
    // The first batch goes out with the (m, l) loads: one memory round
    // trip instead of two before the first accumulation.
    load_rows(0);
    float m = -INFINITY, l = 0.f;
    if (row >= 0) {
      l = P.part.l[row];
      m = P.part.m[row];
      if (!(l > 0.f)) {
        l = 0.f;
        m = -INFINITY;
      }
    }
    const float Mn = fmaxf(M, wave_max(m));
    const float muse = Mn == -INFINITY ? 0.f : Mn;
    const float sc = exp2f(M - muse);
    L *= sc;
#pragma unroll
    for (int v = 0; v < VPL; ++v) acc[v] *= sc;
    const float w = l > 0.f ? exp2f(m - muse) : 0.f;
    L += wave_sum(w * l);
    M = Mn;
    for (int s = 0; s < cnt; s += 2 * U) {
      if (s > 0) load_rows(s);
      float ws[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int se = s + 2 * u;  // even source; odd one is se + 1 (wave-uniform indices)
        const float we = se < cnt ? lane_f(w, se) : 0.f;
        const float wo = se + 1 < cnt ? lane_f(w, se + 1) : 0.f;
        ws[u] = half ? wo : we;
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int v = 0; v < VPL; ++v) acc[v] += ws[u] > 0.f ? ws[u] * x[u][v] : 0.f;  // NaN-safe for w = 0
    }
  }

#pragma unroll
  for (int v = 0; v < VPL; ++v) acc[v] = xsum32(acc[v]);
  const float inv = L > 0.f ? 1.f / L : 0.f;
  if (half == 0) store_row<VPL>(P.out, P.out_f32, pair * DV + hl * VPL, acc, inv);
  if (P.lse && lane == 0) P.lse[pair] = L > 0.f ? (M + log2f(L)) * 0.69314718055994531f : -INFINITY;
}

// Attention states: one wave per (request, head); lane j < n holds lse_j,
// then every lane accumulates its D / 64 dims over the states in order
// (fixed order: bit-reproducible).
template <int D>
__device__ __forceinline__ void states_body(const StatesParams& P) {
  constexpr int VPL = D / 64;  // floats per lane
  constexpr float kLog2e = 1.4426950408889634f;
  const int lane = threadIdx.x & 63;
  const int64_t pair = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (pair >= P.pairs) return;
  float x = -INFINITY;
#pragma unroll
  for (int j = 0; j < kMaxStates; ++j)
    if (j < P.n && lane == j) x = P.lses[j][pair];
  // a state with no keys (lse = -inf, or NaN from an empty decode) weighs nothing
  if (!(x > -INFINITY)) x = -INFINITY;
  const float M = wave_max(x);
  const float w = (x == -INFINITY) ? 0.f : exp2f((x - M) * kLog2e);
  const float L = wave_sum(w);
  float acc[VPL];
#pragma unroll
  for (int v = 0; v < VPL; ++v) acc[v] = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxStates; ++j) {
    if (j >= P.n) break;
    const float wj = lane_f(w, j);
    if (wj > 0.f) {  // wave-uniform; skipping also keeps NaN rows of empty states out
      const float* src = P.outs[j] + pair * D + lane * VPL;
#pragma unroll
      for (int v = 0; v < VPL; v += 2) {
        const float2 t = *reinterpret_cast<const float2*>(src + v);
        acc[v] = fmaf(wj, t.x, acc[v]);
        acc[v + 1] = fmaf(wj, t.y, acc[v + 1]);
      }
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  if constexpr (VPL % 4 == 0) {
    store_row<VPL>(P.out, P.out_f32, pair * D + lane * VPL, acc, inv);
  } else {
    if (P.out_f32) {
      float* dst = static_cast<float*>(P.out) + pair * D + lane * VPL;
#pragma unroll
      for (int v = 0; v < VPL; ++v) dst[v] = acc[v] * inv;
    } else {
      __bf16* dst = static_cast<__bf16*>(P.out) + pair * D + lane * VPL;
#pragma unroll
      for (int v = 0; v < VPL; ++v) dst[v] = (__bf16)(acc[v] * inv);
    }
  }
  if (P.lse && lane == 0) P.lse[pair] = L > 0.f ? M + logf(L) : -INFINITY;
}

}  // namespace

__global__ __launch_bounds__(256) void fca_merge_states_d128(StatesParams P) { states_body<128>(P); }
__global__ __launch_bounds__(256) void fca_merge_states_d512(StatesParams P) { states_body<512>(P); }

hipError_t launch_merge_states(const StatesParams& p, hipStream_t s) {
  if (p.pairs == 0) return hipSuccess;
  const dim3 grid((unsigned)((p.pairs + 3) / 4));
  if (p.D == 128) {
    hipLaunchKernelGGL(fca_merge_states_d128, grid, dim3(256), 0, s, p);
  } else if (p.D == 512) {
    hipLaunchKernelGGL(fca_merge_states_d512, grid, dim3(256), 0, s, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void fca_merge_kernel_d128(MergeParams P) { merge_body<128>(P); }
__global__ __launch_bounds__(256) void fca_merge_kernel_d512(MergeParams P) { merge_body<512>(P); }

hipError_t launch_merge(const MergeParams& p, hipStream_t s) {
  const int64_t pairs = (int64_t)p.B * p.Hq;
  if (pairs == 0) return hipSuccess;
  const dim3 grid((unsigned)((pairs + 3) / 4));
  if (p.Dv == 128) {
    hipLaunchKernelGGL(fca_merge_kernel_d128, grid, dim3(256), 0, s, p);
  } else if (p.Dv == 512) {
    hipLaunchKernelGGL(fca_merge_kernel_d512, grid, dim3(256), 0, s, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fca
