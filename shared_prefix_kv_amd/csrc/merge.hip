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

// One wave per (request, head); lane j resolves the j-th partial row of the
// request's path so that all (m, l) loads are issued at once, then the value
// rows are accumulated with the broadcast weights.  Each lane owns DV/64
// value dims.
template <int DV>
__device__ __forceinline__ void merge_body(const MergeParams& P) {
  constexpr int VPL = DV / 64;  // floats per lane
  const int lane = threadIdx.x & 63;
  const int64_t pair = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (pair >= (int64_t)P.B * P.Hq) return;
  const int i = (int)(pair / P.Hq);
  const int h = (int)(pair % P.Hq);
  const int kvh = h / P.r;
  const int rr = h % P.r;
  const ReqMeta rq = P.req[i];

  int n_src = rq.sfx_splits;
  for (int g = rq.deepest; g >= 0; g = P.grp[g].parent) n_src += P.grp[g].splits;

  float M = -INFINITY, L = 0.f;
  float acc[VPL];
#pragma unroll
  for (int v = 0; v < VPL; ++v) acc[v] = 0.f;

  for (int base = 0; base < n_src; base += 64) {
    // Row of source j: splits of the deepest group first, then its
    // ancestors, then the suffix splits.
    const int j = base + lane;
    int64_t row = -1;
    if (j < n_src) {
      int rem = j;
      for (int g = rq.deepest; g >= 0;) {
        const GroupMeta gm = P.grp[g];
        if (rem < gm.splits) {
          row = (int64_t)gm.unit + ((int64_t)rem * P.Hkv + kvh) * gm.ncols + (int64_t)(rq.pos - gm.r0) * P.r + rr;
          break;
        }
        rem -= gm.splits;
        g = gm.parent;
      }
      if (row < 0) row = (int64_t)rq.sfx_unit + (int64_t)rem * P.Hq + h;
    }
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
    const int cnt = min(64, n_src - base);
    const int row_lo = (int)(row & 0xffffffff), row_hi = (int)(row >> 32);
    for (int s = 0; s < cnt; ++s) {
      const float ws = __shfl(w, s);
      const int64_t rs = ((int64_t)__shfl(row_hi, s) << 32) | (uint32_t)__shfl(row_lo, s);
      if (ws > 0.f) {
        const float* src = P.part.o + rs * DV + lane * VPL;
#pragma unroll
        for (int v = 0; v < VPL; v += 2) {
          const float2 x = *reinterpret_cast<const float2*>(src + v);
          acc[v] += ws * x.x;
          acc[v + 1] += ws * x.y;
        }
      }
    }
  }

  const float inv = L > 0.f ? 1.f / L : 0.f;
  __bf16* dst = static_cast<__bf16*>(P.out) + pair * DV + lane * VPL;
#pragma unroll
  for (int v = 0; v < VPL; v += 2) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 ob = {(__bf16)(acc[v] * inv), (__bf16)(acc[v + 1] * inv)};
    *reinterpret_cast<bf16x2*>(dst + v) = ob;
  }
  if (P.lse && lane == 0) P.lse[pair] = L > 0.f ? (M + log2f(L)) * 0.69314718055994531f : -INFINITY;
}

}  // namespace

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
