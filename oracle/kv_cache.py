"""Appending a decode token to a paged KV cache, with copy-on-write (test
infrastructure only).

A paged cache keeps each request's tokens in fixed-size blocks listed in its
block table; requests forked from one prompt reference the same physical
blocks (PagedAttention vs. RadixAttention page, "How PagedAttention Works",
steps 1-4).  Before a decode step writes a request's new key and value, a
block it shares with other requests must be copied so that the others still
see the old contents (the same page, copy-on-write of shared blocks).  This
module states that step on host arrays in the documented cache layout:

    key   (blk, h, t, d) at k[blk, h, d // 8, t, d % 8]
    value (blk, h, t, d) at v[blk, h, d, t]

For request i with L = seq_lens[i] cached tokens the new token is token L:
block table entry j = L // block_size, slot t = L % block_size.  If
cow_dst[i] >= 0 (and differs from table[i, j]), the request's tokens in block
table[i, j] (slots 0 .. t-1, every head, keys and values) are first copied
to block cow_dst[i] and the table entry is set to it; the token is then
written at slot t of the (possibly new) block.  Slots after t of the copy are
left as they were: the pages say the shared block is copied when a request
diverges, and the slots after t hold no token of this request (they may
hold other sharers' tokens), so only the request's own tokens are copied.
The lengths are not changed here (the caller's next plan uses L + 1).
"""

from __future__ import annotations

import numpy as np


def append(k_pool, v_pool, tables, seq_lens, k_new, v_new, block_size, cow_dst=None):
    """Returns (k_pool, v_pool, tables) after the append (copies; inputs are
    not modified).  k_new [B, Hkv, Dqk], v_new [B, Hkv, Dv] (v_pool and v_new
    None for a latent cache, whose values are the first key dims)."""
    k = k_pool.copy()
    v = None if v_pool is None else v_pool.copy()
    bt = tables.copy()
    for i, L in enumerate(seq_lens):
        j, t = int(L) // block_size, int(L) % block_size
        if cow_dst is not None and cow_dst[i] >= 0 and int(cow_dst[i]) != int(bt[i, j]):
            src, dst = int(bt[i, j]), int(cow_dst[i])
            k[dst, :, :, :t, :] = k[src, :, :, :t, :]
            if v is not None:
                v[dst, :, :, :t] = v[src, :, :, :t]
            bt[i, j] = dst
        blk = int(bt[i, j])
        dq = k_new.shape[2]
        for d in range(dq):
            k[blk, :, d // 8, t, d % 8] = k_new[i, :, d]
        if v is not None:
            v[blk, :, :, t] = v_new[i]
    return k, v, bt
