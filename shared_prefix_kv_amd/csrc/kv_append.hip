// Decode-token append into the paged KV cache, with copy-on-write, gfx950.
//
// A paged cache grows one token at a time inside fixed-size blocks listed by
// each request's block table, and requests that start from the same prompt
// reference the same physical blocks; when one of them writes into a shared
// block it first gets its own copy, so the others keep reading the old
// contents (PagedAttention vs. RadixAttention page, "How PagedAttention
// Works", steps 3 and 4).  This is the step that runs before the attention
// path each decode step: it writes the new token's key and value at position
// L = seq_len of its request, into block table[i][L / block_size], slot
// L % block_size, after copying that block to cow_dst[i] and pointing the
// table entry at the copy when cow_dst[i] >= 0.
//
// The copy takes only the request's own tokens of the shared block, slots
// 0 .. t-1 with t = L % block_size: the slots after t may hold tokens of a
// longer sharer (which may be appending in place at that very moment), and
// none of them belongs to this request.  Slots after t of the target keep
// what they held.
//
// One workgroup per request.  Blocks hold every KV head, so the copy moves
// num_kv_heads key and value tiles in 16-byte pieces: a key piece is 8 dims
// of one token, so slot t's pieces come from the new token and later ones are
// skipped; a value piece is 8 tokens of one dim, and the one holding slot t
// is merged from the source (slots before t), the new value (slot t) and the
// target (slots after t).  Each target byte is written once.  Without a copy
// only the new token's bytes are written.  Requests whose length or block
// IDs are out of range are skipped and set a bit of *status.

#include "fca_internal.h"

namespace fca {
namespace {

constexpr int kAppendThreads = 256;

__device__ __forceinline__ void raise_status(int32_t* status, int bit) {
  if (status) atomicOr(status, bit);
}

template <int DQK, int DV, int BS, bool ALIAS>
__device__ __forceinline__ void append_body(const AppendParams& p) {
  static_assert(DQK % 8 == 0 && DV % 8 == 0 && BS % 8 == 0, "16-byte pieces");
  constexpr int kKPieces = DQK / 8 * BS;            // key tile of one head: [DQK/8][BS][8]
  constexpr int kVPieces = ALIAS ? 0 : DV * BS / 8;  // value tile of one head: [DV][BS]
  const int i = blockIdx.x;
  const int tid = threadIdx.x;
  const int L = p.seq_lens[i];
  if (L < 0 || L >= p.max_blocks * BS) {
    if (tid == 0) raise_status(p.status, FCA_APPEND_BAD_LEN);
    return;
  }
  const int j = L / BS, t = L % BS;
  int32_t* entry = p.block_tables + (int64_t)i * p.bt_row_stride + j;
  const int cur = *entry;
  const int dst = p.cow_dst ? p.cow_dst[i] : -1;
  // Every wave has read the table entry before thread 0 may replace it.
  __syncthreads();
  if (cur < 0 || cur >= p.num_blocks) {
    if (tid == 0) raise_status(p.status, FCA_APPEND_BAD_BLOCK);
    return;
  }
  if (dst >= p.num_blocks) {
    if (tid == 0) raise_status(p.status, FCA_APPEND_BAD_COW);
    return;
  }
  const uint16_t* kn = p.k_new + (int64_t)i * p.num_kv_heads * DQK;
  const uint16_t* vn = ALIAS ? nullptr : p.v_new + (int64_t)i * p.num_kv_heads * DV;

  if (dst >= 0 && dst != cur) {
    const int per_head = kKPieces + kVPieces;
    const int total = p.num_kv_heads * per_head;
    for (int c = tid; c < total; c += kAppendThreads) {
      const int h = c / per_head;
      const int r = c - h * per_head;
      if (r < kKPieces) {
        const int dc = r / BS, tok = r - dc * BS;
        if (tok > t) continue;
        const int64_t off = (int64_t)h * p.k_stride_head + (int64_t)r * 8;
        uint4 piece;
        if (tok == t)
          piece = *reinterpret_cast<const uint4*>(kn + h * DQK + dc * 8);
        else
          piece = *reinterpret_cast<const uint4*>(p.k_cache + (int64_t)cur * p.k_stride_block + off);
        *reinterpret_cast<uint4*>(p.k_cache + (int64_t)dst * p.k_stride_block + off) = piece;
      } else if (!ALIAS) {
        const int rv = r - kKPieces;
        const int d = rv / (BS / 8), tok0 = (rv - d * (BS / 8)) * 8;
        if (tok0 > t) continue;
        const int64_t off = (int64_t)h * p.v_stride_head + (int64_t)rv * 8;
        uint16_t* to = p.v_cache + (int64_t)dst * p.v_stride_block + off;
        uint4 piece = *reinterpret_cast<const uint4*>(p.v_cache + (int64_t)cur * p.v_stride_block + off);
        if (t < tok0 + 8) {
          const uint4 old = *reinterpret_cast<const uint4*>(to);
          uint16_t e[8], o[8];
          __builtin_memcpy(e, &piece, 16);
          __builtin_memcpy(o, &old, 16);
#pragma unroll
          for (int x = 0; x < 8; ++x)
            if (tok0 + x > t) e[x] = o[x];
          e[t - tok0] = vn[h * DV + d];
          __builtin_memcpy(&piece, e, 16);
        }
        *reinterpret_cast<uint4*>(to) = piece;
      }
    }
    if (tid == 0) *entry = dst;
    return;
  }

  // Write in place: one key piece per (head, 8 dims), one value element per
  // (head, dim).
  for (int c = tid; c < p.num_kv_heads * (DQK / 8); c += kAppendThreads) {
    const int h = c / (DQK / 8), dc = c - h * (DQK / 8);
    const uint4 piece = *reinterpret_cast<const uint4*>(kn + h * DQK + dc * 8);
    *reinterpret_cast<uint4*>(p.k_cache + (int64_t)cur * p.k_stride_block + (int64_t)h * p.k_stride_head +
                              ((int64_t)dc * BS + t) * 8) = piece;
  }
  if (!ALIAS) {
    for (int c = tid; c < p.num_kv_heads * DV; c += kAppendThreads) {
      const int h = c / DV, d = c - h * DV;
      p.v_cache[(int64_t)cur * p.v_stride_block + (int64_t)h * p.v_stride_head + (int64_t)d * BS + t] =
          vn[h * DV + d];
    }
  }
}

}  // namespace

__global__ __launch_bounds__(kAppendThreads) void fca_kv_append_gqa_kernel(AppendParams p) {
  append_body<128, 128, 16, false>(p);
}
__global__ __launch_bounds__(kAppendThreads) void fca_kv_append_mla_kernel(AppendParams p) {
  append_body<576, 512, 64, true>(p);
}

hipError_t launch_append(const AppendParams& p, bool latent, hipStream_t s) {
  if (p.batch == 0) return hipSuccess;
  const dim3 grid((unsigned)p.batch);
  if (latent)
    hipLaunchKernelGGL(fca_kv_append_mla_kernel, grid, dim3(kAppendThreads), 0, s, p);
  else
    hipLaunchKernelGGL(fca_kv_append_gqa_kernel, grid, dim3(kAppendThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace fca
