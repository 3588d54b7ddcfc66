"""fp64 reference attention over a paged KV cache (test infrastructure only).

Forest Cascade Attention is stated to be mathematically equivalent to
standard attention (ZoRRo Inference & Forest Cascade Attention page,
"Overview" and "Performance Characteristics"), so this module is that
standard attention written out plainly, per request, with no cascade:

    s_t  = scale * <q_h, K_t[kvh]>          for every cached token t < L
    m    = max_t s_t,  w_t = exp(s_t - m),  l = sum_t w_t
    o_h  = sum_t w_t V_t[kvh] / l,          lse_h = m + ln l

with kvh = h // (Hq / Hkv).  A request with L = 0 yields o = 0 and
lse = -inf.  Keys and values are gathered through the request's block table:
token t lives in physical block ``table[t // block_size]`` at slot
``t % block_size`` (PagedAttention vs. RadixAttention page, "How
PagedAttention Works", steps 1-2).

``partial`` / ``merge`` restate the split form used by the merge step: a token
subset P gives the triple (o_P, m_P, l_P); triples combine as

    M = max_P m_P,  w_P = l_P exp(m_P - M),
    o = sum_P w_P o_P / sum_P w_P,  lse = M + ln sum_P w_P,

with empty subsets (m = -inf, l = 0) carrying no weight (the exact weighting
of partial results in "Core Mechanism", step 3; the online-softmax merge of
partial attention on the "Move the Query, Not the Cache" page, Metodologia).
"""

from __future__ import annotations

import numpy as np


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def gather_kv(k_pool, v_pool, table_row, L, block_size, head_dim_v, v_aliases_k):
    """Keys [L, Hkv, Dqk] and values [L, Hkv, Dv] of one request, float64.

    k_pool: [num_blocks, Hkv, Dqk/8, block_size, 8] bf16 bits; element
            (blk, h, t, d) sits at [blk, h, d // 8, t, d % 8].
    v_pool: [num_blocks, Hkv, Dv, block_size] bf16 bits; element
            (blk, h, t, d) sits at [blk, h, d, t].  Ignored when the values
            are the first Dv key columns (v_aliases_k).
    """
    nblk = -(-L // block_size)
    blocks = np.asarray(table_row[:nblk], dtype=np.int64)
    nb, hkv, dchunks, bs, eight = k_pool.shape
    kb = k_pool[blocks]  # [nblk, Hkv, Dqk/8, bs, 8]
    K = kb.transpose(0, 3, 1, 2, 4).reshape(nblk * bs, hkv, dchunks * eight)[:L]
    K = widen_bf16(K)
    if v_aliases_k:
        V = K[:, :, :head_dim_v]
    else:
        vb = v_pool[blocks]  # [nblk, Hkv, Dv, bs]
        V = widen_bf16(vb.transpose(0, 3, 1, 2).reshape(nblk * bs, hkv, vb.shape[2])[:L])
    return K, V


def attend_one(q, K, V, scale, num_kv_heads):
    """Standard softmax attention of one request's query heads.

    q: [Hq, Dqk] float64;  K: [L, Hkv, Dqk];  V: [L, Hkv, Dv].
    Returns o [Hq, Dv], lse [Hq] (float64).

    The query heads that read one KV head (h // r == kvh) are one matrix
    product against that head's keys; every row is still its own softmax.
    """
    hq = q.shape[0]
    r = hq // num_kv_heads
    L = K.shape[0]
    dv = V.shape[2]
    o = np.zeros((hq, dv))
    lse = np.full(hq, -np.inf)
    if L == 0:
        return o, lse
    for kvh in range(num_kv_heads):
        rows = slice(kvh * r, (kvh + 1) * r)
        Kh = np.ascontiguousarray(K[:, kvh, :])  # [L, Dqk]
        Vh = np.ascontiguousarray(V[:, kvh, :])  # [L, Dv]
        s = scale * (q[rows] @ Kh.T)  # [r, L]
        m = s.max(axis=1)
        w = np.exp(s - m[:, None])
        l = w.sum(axis=1)
        o[rows] = (w @ Vh) / l[:, None]
        lse[rows] = m + np.log(l)
    return o, lse


def attend(q_bits, k_pool, v_pool, block_tables, seq_lens, shape, requests=None):
    """Reference decode attention for a batch (or the listed requests).

    Returns (out [B, Hq, Dv], lse [B, Hq]) in float64; rows of requests not
    listed stay zero / -inf.
    """
    B = len(seq_lens)
    out = np.zeros((B, shape.num_q_heads, shape.head_dim_v))
    lse = np.full((B, shape.num_q_heads), -np.inf)
    idx = range(B) if requests is None else requests
    for i in idx:
        L = int(seq_lens[i])
        K, V = gather_kv(
            k_pool, v_pool, block_tables[i], L, shape.block_size, shape.head_dim_v, shape.v_aliases_k
        )
        q = widen_bf16(q_bits[i])
        out[i], lse[i] = attend_one(q, K, V, shape.scale, shape.num_kv_heads)
    return out, lse


def partial(q_rows, K, V, scale):
    """(o, m, l) of query rows [n, D] over keys K [T, D], values V [T, Dv].

    o is normalised by its own l.  An empty token set gives o = 0, m = -inf,
    l = 0.
    """
    n = q_rows.shape[0]
    if K.shape[0] == 0:
        return np.zeros((n, V.shape[1])), np.full(n, -np.inf), np.zeros(n)
    s = scale * (q_rows @ K.T)  # [n, T]
    m = s.max(axis=1)
    w = np.exp(s - m[:, None])
    l = w.sum(axis=1)
    o = (w @ V) / l[:, None]
    return o, m, l


def merge(parts):
    """Exact log-sum-exp combination of (o, m, l) triples -> (o, lse)."""
    ms = np.stack([p[1] for p in parts])  # [P, n]
    M = ms.max(axis=0)
    n = ms.shape[1]
    dv = parts[0][0].shape[1]
    num = np.zeros((n, dv))
    den = np.zeros(n)
    for o, m, l in parts:
        live = l > 0
        w = np.zeros(n)
        w[live] = l[live] * np.exp(m[live] - M[live])
        num += w[:, None] * o
        den += w
    out = np.zeros((n, dv))
    lse = np.full(n, -np.inf)
    ok = den > 0
    out[ok] = num[ok] / den[ok, None]
    lse[ok] = M[ok] + np.log(den[ok])
    return out, lse


def merge_states(outs, lses):
    """Combine attention states over disjoint key sets -> (out, lse).

    States are [n, Dv] outputs and [n] lses.  A state (o, lse) is the triple
    (o, m = lse, l = 1), or the empty triple (o = 0, l = 0) when lse = -inf,
    whatever its o holds, so this is ``merge`` over those triples (the
    online-softmax merge of partial attention routed to the holder of the
    keys, "Move the Query, Not the Cache" page, Metodologia).
    """
    parts = []
    for o, lse in zip(outs, lses):
        lse = np.asarray(lse, dtype=np.float64)
        live = np.isfinite(lse)
        o = np.where(live[:, None], np.asarray(o, dtype=np.float64), 0.0)  # no keys: output undefined
        parts.append((o, np.where(live, lse, -np.inf), live.astype(np.float64)))
    return merge(parts)

