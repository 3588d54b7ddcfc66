"""Seeded K/V pool and query values, in the cache layout the library reads.

Layouts (bf16, stored here as uint16 bit patterns):

* keys   ``k[num_blocks, Hkv, Dqk/8, block_size, 8]`` -- inside one
  (block, head) tile, the head dimension is cut into 16-byte chunks of 8
  values; each chunk holds that slice for every token of the block.
* values ``v[num_blocks, Hkv, Dv, block_size]`` -- one (block, head) tile is
  stored transposed, a row of ``block_size`` tokens per value dimension.
* latent caches whose values alias the keys (values are the first ``Dv``
  columns of the key row) have no separate ``v``.
* queries ``q[B, Hq, Dqk]``.

Values are N(0, 1) draws rounded to bf16 (round to nearest, ties to even).
For correctness runs, pool blocks no request uses and the cache slots past a
request's last token are set to NaN, so any read of them shows in the output.
"""

from __future__ import annotations

import numpy as np

BF16_NAN = np.uint16(0x7FC0)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (NaN stays NaN)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded = rounded.copy()
        rounded[nan] = BF16_NAN
    return rounded


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def k_pool_shape(shape, num_blocks):
    return (num_blocks, shape.num_kv_heads, shape.head_dim_qk // 8, shape.block_size, 8)


def v_pool_shape(shape, num_blocks):
    return (num_blocks, shape.num_kv_heads, shape.head_dim_v, shape.block_size)


def _poison_numpy(batch, k, v):
    bs = batch.shape.block_size
    unused = ~batch.used_blocks
    k[unused] = BF16_NAN
    if v is not None:
        v[unused] = BF16_NAN
    for i in range(batch.batch):
        L = int(batch.seq_lens[i])
        tail = L % bs
        if L == 0 or tail == 0:
            continue
        blk = int(batch.block_tables[i, L // bs])
        k[blk, :, :, tail:, :] = BF16_NAN
        if v is not None:
            v[blk, :, :, tail:] = BF16_NAN


def fill_values_numpy(batch, poison: bool = True):
    """Draw K/V pool then queries from ``batch.rng`` (CPU, small batches)."""
    sh = batch.shape
    rng = batch.rng
    k = f32_to_bf16_bits(rng.standard_normal(k_pool_shape(sh, batch.num_blocks), dtype=np.float32))
    v = None
    if not sh.v_aliases_k:
        v = f32_to_bf16_bits(rng.standard_normal(v_pool_shape(sh, batch.num_blocks), dtype=np.float32))
    q = f32_to_bf16_bits(rng.standard_normal((batch.batch, sh.num_q_heads, sh.head_dim_qk), dtype=np.float32))
    if poison:
        _poison_numpy(batch, k, v)
    return dict(q=q, k=k, v=v)


def fill_values_torch(batch, device, seed: int, poison: bool = True):
    """Draw K/V pool then queries on ``device`` with torch (large batches).

    Returns bf16 torch tensors in the same layouts as ``fill_values_numpy``.
    The stream of numbers differs from the numpy one; each run reads back
    whatever it compares against.
    """
    import torch

    sh = batch.shape
    g = torch.Generator(device=device)
    g.manual_seed(seed)

    def randn_bf16(shape):
        out = torch.empty(shape, dtype=torch.bfloat16, device=device)
        flat = out.view(-1)
        step = 1 << 26
        for s in range(0, flat.numel(), step):
            n = min(step, flat.numel() - s)
            flat[s : s + n] = torch.randn(n, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
        return out

    k = randn_bf16(k_pool_shape(sh, batch.num_blocks))
    v = None if sh.v_aliases_k else randn_bf16(v_pool_shape(sh, batch.num_blocks))
    q = randn_bf16((batch.batch, sh.num_q_heads, sh.head_dim_qk))
    if poison:
        nan = float("nan")
        unused = torch.from_numpy(np.nonzero(~batch.used_blocks)[0]).to(device)
        if unused.numel():
            k.index_fill_(0, unused, nan)
            if v is not None:
                v.index_fill_(0, unused, nan)
        bs = sh.block_size
        for i in range(batch.batch):
            L = int(batch.seq_lens[i])
            tail = L % bs
            if L == 0 or tail == 0:
                continue
            blk = int(batch.block_tables[i, L // bs])
            k[blk, :, :, tail:, :] = nan
            if v is not None:
                v[blk, :, :, tail:] = nan
    return dict(q=q, k=k, v=v)
