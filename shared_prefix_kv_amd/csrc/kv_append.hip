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
// Several layers share one block table (each layer has its own pool, the
// same block IDs): the copy of every layer reads the table entry as it was,
// and one commit launch afterwards points the entry at the copy.  A layer
// that read the entry after another layer had already rewritten it would
// find source and target equal and skip its copy.
//
// One workgroup per (request, layer).  Blocks hold every KV head, so the copy moves
// num_kv_heads key and value tiles in 16-byte pieces: a key piece is 8 dims
// of one token, so slot t's pieces come from the new token and later ones are
// skipped; a value piece is 8 tokens of one dim, and the one holding slot t
// is merged from the source (slots before t), the new value (slot t) and the
// target (slots after t).  In a pool of token rows every piece is 8 dims of
// one token, keys and values alike, so slot t's pieces come from the new
// token and later slots are skipped.  Each target byte is written once.
// Without a copy only the new token's bytes are written.  Requests whose length or block
// IDs are out of range are skipped; the commit launch sets a bit of *status
// for them.

#include "fca_internal.h"

namespace fca {
namespace {

constexpr int kAppendThreads = 256;

__device__ __forceinline__ void raise_status(int32_t* status, int bit) {
  if (status) atomicOr(status, bit);
}

// What request i does this step: the block of its new slot (cur), the copy
// target (dst, -1 for none or when it is cur), the slot t; false when the
// request is skipped (bit set in *why).
__device__ __forceinline__ bool append_target(const int32_t* bt, int64_t stride, const int32_t* seq_lens,
                                              const int32_t* cow_dst, int i, int max_blocks, int bs,
                                              int num_blocks, int* cur, int* dst, int* t, int* why) {
  const int L = seq_lens[i];
  *why = 0;
  if (L < 0 || L >= max_blocks * bs) {
    *why = FCA_APPEND_BAD_LEN;
    return false;
  }
  const int j = L / bs;
  *t = L % bs;
  *cur = bt[(int64_t)i * stride + j];
  const int c = cow_dst ? cow_dst[i] : -1;
  if (*cur < 0 || *cur >= num_blocks) {
    *why = FCA_APPEND_BAD_BLOCK;
    return false;
  }
  if (c >= num_blocks) {
    *why = FCA_APPEND_BAD_COW;
    return false;
  }
  *dst = (c >= 0 && c != *cur) ? c : -1;
  return true;
}

// One pool of token rows: slots tok0 .. tok0 + n_tok - 1 of every head of
// block blk, in 16-byte pieces (8 dims of one token) taken from block cur,
// except slot t, which takes the new row (fresh: [num_kv_heads][D]).
template <int D>
__device__ __forceinline__ void rows_copy(const uint16_t* fresh, uint16_t* cache, int64_t sb, int64_t sh, int64_t st,
                                          int num_kv_heads, int cur, int blk, int tok0, int n_tok, int t, int tid) {
  constexpr int kRow = D / 8;  // pieces per row
  const int per_head = kRow * n_tok;
  for (int c = tid; c < num_kv_heads * per_head; c += kAppendThreads) {
    const int h = c / per_head;
    const int r = c - h * per_head;
    const int tok = tok0 + r / kRow, dc = r % kRow;
    const int64_t off = (int64_t)h * sh + (int64_t)tok * st + dc * 8;
    const uint4 piece = tok == t ? *reinterpret_cast<const uint4*>(fresh + h * D + dc * 8)
                                 : *reinterpret_cast<const uint4*>(cache + (int64_t)cur * sb + off);
    *reinterpret_cast<uint4*>(cache + (int64_t)blk * sb + off) = piece;
  }
}

template <int DQK, int DV, int BS, bool ALIAS>
__device__ __forceinline__ void append_body(const AppendParams& p) {
  static_assert(DQK % 8 == 0 && DV % 8 == 0 && BS % 8 == 0, "16-byte pieces");
  constexpr int kKPieces = DQK / 8 * BS;            // key tile of one head: [DQK/8][BS][8]
  constexpr int kVPieces = ALIAS ? 0 : DV * BS / 8;  // value tile of one head: [DV][BS]
  const int i = blockIdx.x;
  const int layer = blockIdx.y;
  const int tid = threadIdx.x;
  int cur, dst, t, why;
  if (!append_target(p.block_tables, p.bt_row_stride, p.seq_lens, p.cow_dst, i, p.max_blocks, BS, p.num_blocks, &cur,
                     &dst, &t, &why))
    return;
  const uint16_t* kn = p.k_new[layer] + (int64_t)i * p.num_kv_heads * DQK;
  const uint16_t* vn = ALIAS ? nullptr : p.v_new[layer] + (int64_t)i * p.num_kv_heads * DV;
  uint16_t* kc = p.k_cache[layer];
  uint16_t* vc = ALIAS ? nullptr : p.v_cache[layer];

  if (p.k_stride_token != 0) {
    // Token rows: key (h, tok, d) at h * k_stride_head + tok * k_stride_token + d.
    // Slots 0 .. t of the copy target, or slot t alone in place.
    const int blk = dst >= 0 ? dst : cur;
    const int tok0 = dst >= 0 ? 0 : t;
    const int n_tok = t + 1 - tok0;
    rows_copy<DQK>(kn, kc, p.k_stride_block, p.k_stride_head, p.k_stride_token, p.num_kv_heads, cur, blk, tok0, n_tok,
                   t, tid);
    if constexpr (!ALIAS)
      rows_copy<DV>(vn, vc, p.v_stride_block, p.v_stride_head, p.v_stride_token, p.num_kv_heads, cur, blk, tok0,
                    n_tok, t, tid);
    return;
  }

  if (dst >= 0) {
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
          piece = *reinterpret_cast<const uint4*>(kc + (int64_t)cur * p.k_stride_block + off);
        *reinterpret_cast<uint4*>(kc + (int64_t)dst * p.k_stride_block + off) = piece;
      } else if (!ALIAS) {
        const int rv = r - kKPieces;
        const int d = rv / (BS / 8), tok0 = (rv - d * (BS / 8)) * 8;
        if (tok0 > t) continue;
        const int64_t off = (int64_t)h * p.v_stride_head + (int64_t)rv * 8;
        uint16_t* to = vc + (int64_t)dst * p.v_stride_block + off;
        uint4 piece = *reinterpret_cast<const uint4*>(vc + (int64_t)cur * p.v_stride_block + off);
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
    return;
  }

  // Write in place: one key piece per (head, 8 dims), one value element per
  // (head, dim).
  for (int c = tid; c < p.num_kv_heads * (DQK / 8); c += kAppendThreads) {
    const int h = c / (DQK / 8), dc = c - h * (DQK / 8);
    const uint4 piece = *reinterpret_cast<const uint4*>(kn + h * DQK + dc * 8);
    *reinterpret_cast<uint4*>(kc + (int64_t)cur * p.k_stride_block + (int64_t)h * p.k_stride_head +
                              ((int64_t)dc * BS + t) * 8) = piece;
  }
  if (!ALIAS) {
    for (int c = tid; c < p.num_kv_heads * DV; c += kAppendThreads) {
      const int h = c / DV, d = c - h * DV;
      vc[(int64_t)cur * p.v_stride_block + (int64_t)h * p.v_stride_head + (int64_t)d * BS + t] = vn[h * DV + d];
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

// One thread per request, after every layer's copy.
__global__ __launch_bounds__(256) void fca_kv_append_commit_kernel(int32_t* block_tables, int64_t stride,
                                                                   const int32_t* seq_lens, const int32_t* cow_dst,
                                                                   int32_t* status, int batch, int max_blocks,
                                                                   int bs, int num_blocks) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= batch) return;
  int cur, dst, t, why;
  if (!append_target(block_tables, stride, seq_lens, cow_dst, i, max_blocks, bs, num_blocks, &cur, &dst, &t, &why)) {
    raise_status(status, why);
    return;
  }
  if (dst >= 0) block_tables[(int64_t)i * stride + seq_lens[i] / bs] = dst;
}

hipError_t launch_append(const AppendParams& p, bool latent, hipStream_t s) {
  if (p.batch == 0 || p.n_layers == 0) return hipSuccess;
  const dim3 grid((unsigned)p.batch, (unsigned)p.n_layers);
  if (latent)
    hipLaunchKernelGGL(fca_kv_append_mla_kernel, grid, dim3(kAppendThreads), 0, s, p);
  else
    hipLaunchKernelGGL(fca_kv_append_gqa_kernel, grid, dim3(kAppendThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_append_commit(int32_t* block_tables, int64_t bt_row_stride, const int32_t* seq_lens,
                                const int32_t* cow_dst, int32_t* status, int batch, int max_blocks, int block_size,
                                int num_blocks, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  hipLaunchKernelGGL(fca_kv_append_commit_kernel, dim3((batch + 255) / 256), dim3(256), 0, s, block_tables,
                     bt_row_stride, seq_lens, cow_dst, status, batch, max_blocks, block_size, num_blocks);
  return hipGetLastError();
}

}  // namespace fca
