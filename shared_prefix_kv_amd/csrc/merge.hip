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
// split-K pieces and the depth levels in one pass.  The running maximum is
// updated as rows arrive (accumulators rescaled on a new maximum); the order
// of rows is fixed, so results are bit-reproducible.  A request with no
// tokens gets zeros and -inf.
//
// One half-wave (32 lanes x 4 floats) per (request, head) and 128 value dims.

#include <cmath>

#include "fca_internal.h"

namespace fca {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

template <int DV>
__device__ __forceinline__ void merge_body(const MergeParams& P) {
  constexpr int LANES = DV / 4;  // lanes per (request, head)
  constexpr int PER_WG = 256 / LANES;
  const int64_t pair = (int64_t)blockIdx.x * PER_WG + threadIdx.x / LANES;
  if (pair >= (int64_t)P.B * P.Hq) return;
  const int sub = threadIdx.x % LANES;
  const int i = (int)(pair / P.Hq);
  const int h = (int)(pair % P.Hq);
  const int kvh = h / P.r;
  const int rr = h % P.r;

  float M = -INFINITY, L = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  auto add = [&](int64_t row) {
    const float l = P.part.l[row];
    if (!(l > 0.f)) return;
    const float m = P.part.m[row];
    if (m > M) {
      const float sc = exp2f(M - m);
      acc *= sc;
      L *= sc;
      M = m;
    }
    const float w = exp2f(m - M);
    L += w * l;
    acc += w * *reinterpret_cast<const f32x4*>(P.part.o + row * DV + 4 * sub);
  };

  const ReqMeta rq = P.req[i];
  for (int g = rq.deepest; g >= 0;) {
    const GroupMeta gm = P.grp[g];
    const int k = rq.pos - gm.r0;
    for (int s = 0; s < gm.splits; ++s)
      add((int64_t)gm.unit + ((int64_t)s * P.Hkv + kvh) * gm.ncols + (int64_t)k * P.r + rr);
    g = gm.parent;
  }
  for (int s = 0; s < rq.sfx_splits; ++s) add((int64_t)rq.sfx_unit + (int64_t)s * P.Hq + h);

  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  if (L > 0.f) o = acc * (1.f / L);
  bf16x4 ob = {(__bf16)o[0], (__bf16)o[1], (__bf16)o[2], (__bf16)o[3]};
  *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(P.out) + pair * DV + 4 * sub) = ob;
  if (P.lse && sub == 0) P.lse[pair] = L > 0.f ? (M + log2f(L)) * 0.69314718055994531f : -INFINITY;
}

}  // namespace

__global__ __launch_bounds__(256) void fca_merge_kernel_d128(MergeParams P) { merge_body<128>(P); }
__global__ __launch_bounds__(256) void fca_merge_kernel_d512(MergeParams P) { merge_body<512>(P); }

hipError_t launch_merge(const MergeParams& p, hipStream_t s) {
  const int64_t pairs = (int64_t)p.B * p.Hq;
  if (pairs == 0) return hipSuccess;
  if (p.Dv == 128) {
    hipLaunchKernelGGL(fca_merge_kernel_d128, dim3((unsigned)((pairs + 7) / 8)), dim3(256), 0, s, p);
  } else if (p.Dv == 512) {
    hipLaunchKernelGGL(fca_merge_kernel_d512, dim3((unsigned)((pairs + 1) / 2)), dim3(256), 0, s, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fca
