"""Shared test helpers: tolerance, device upload, sampled oracle runs."""

from __future__ import annotations

import numpy as np

from oracle import attention as A

# Tolerance on bf16 outputs vs the fp64 oracle: |out - ref| <= ATOL + RTOL*|ref|
# element-wise (max-abs 2e-3 and relative 1e-2 read as an allclose pair).
ATOL = 2e-3
RTOL = 1e-2
# log-sum-exp: fp32 scores and a denominator summed from bf16-rounded weights.
LSE_ATOL = 1e-3


def bf16_tensor_to_f64(t) -> np.ndarray:
    import torch

    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def to_device_bf16(bits: np.ndarray, device="cuda"):
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def to_bits(t) -> np.ndarray:
    import torch

    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def error_report(out, ref):
    err = np.abs(out - ref)
    rowmax = np.abs(ref).max(axis=-1, keepdims=True)
    with np.errstate(invalid="ignore", divide="ignore"):
        rowrel = np.where(rowmax > 0, err.max(axis=-1, keepdims=True) / rowmax, 0.0)
    return dict(max_abs=float(err.max()) if err.size else 0.0, row_rel=float(rowrel.max()) if rowrel.size else 0.0)


def assert_close(out, ref, what=""):
    assert np.isfinite(out).all(), f"{what}: non-finite output"
    err = np.abs(out - ref)
    bound = ATOL + RTOL * np.abs(ref)
    bad = err > bound
    if bad.any():
        idx = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())} elements out of tolerance; worst at {idx}: "
            f"out={out[idx]!r} ref={ref[idx]!r}; {error_report(out, ref)}"
        )
    return error_report(out, ref)


def assert_lse_close(lse, ref, what=""):
    both_inf = np.isneginf(lse) & np.isneginf(ref)
    with np.errstate(invalid="ignore"):
        diff = np.where(both_inf, 0.0, np.abs(lse - ref))
    assert (diff <= LSE_ATOL).all(), f"{what}: lse max diff {np.nanmax(diff)}"


def oracle_requests_from_device(batch, vals, requests):
    """Oracle output for the listed requests, reading their blocks back from
    the device pool into a compact pool (blocks relabelled 0..n-1)."""
    import torch

    sh = batch.shape
    bs = sh.block_size
    outs, lses = [], []
    q_bits = to_bits(vals["q"])
    for i in requests:
        L = int(batch.seq_lens[i])
        nblk = -(-L // bs)
        blocks = torch.from_numpy(batch.block_tables[i, :nblk].astype(np.int64)).to(vals["k"].device)
        k = to_bits(vals["k"].index_select(0, blocks))
        v = None if sh.v_aliases_k else to_bits(vals["v"].index_select(0, blocks))
        table = np.arange(nblk, dtype=np.int32)
        K, V = A.gather_kv(k, v, table, L, bs, sh.head_dim_v, sh.v_aliases_k)
        o, l = A.attend_one(A.widen_bf16(q_bits[i]), K, V, sh.scale, sh.num_kv_heads)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)
