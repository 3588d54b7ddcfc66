"""Byte and token accounting of a decode batch (test infrastructure only).

* KV bytes per cached token and layer: ``2 * Hkv * D * bytes`` for separate
  keys and values (one key row and one value row per KV head).  The
  PagedAttention vs. RadixAttention page ("Why memory becomes the limiting
  factor") quotes ~128 KiB per token for a 32-layer model with 8 KV heads of
  dimension 128 in a 2-byte format; 32 * 2 * 8 * 128 * 2 = 131072 B matches
  it, which pins this formula (the page's own formula did not survive
  extraction).  A latent cache whose values alias the keys stores one
  ``Dqk``-wide row per head.
* Logical KV bytes: what a per-request kernel reads, sum_i L_i tokens.
* Unique KV bytes: what must be read at least once when every group's
  prefix range is read once per group ("each shared prefix block is read once
  per group instead of once per request", ZoRRo Inference & Forest Cascade
  Attention page, "Core Mechanism") -- every group's range once plus every
  request's suffix tokens.
"""

from __future__ import annotations


def kv_bytes_per_token(num_kv_heads, head_dim_qk, head_dim_v, elem_bytes=2, v_aliases_k=False, layers=1):
    if v_aliases_k:
        return layers * num_kv_heads * head_dim_qk * elem_bytes
    return layers * num_kv_heads * (head_dim_qk + head_dim_v) * elem_bytes


def logical_tokens(seq_lens):
    return int(sum(int(x) for x in seq_lens))


def unique_tokens(grouping, block_size):
    """Tokens read once per group plus once per request suffix."""
    shared = sum((g["block_end"] - g["block_begin"]) * block_size for g in grouping["groups"])
    own = sum(r[1] for r in grouping["requests"])
    return int(shared + own)
