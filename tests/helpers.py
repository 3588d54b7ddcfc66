"""Shared test helpers: tolerance, device upload, oracle runs over whole batches."""

from __future__ import annotations

import numpy as np

from oracle import attention as A

# Tolerance vs the fp64 oracle (max-abs 2e-3, relative 1e-2):
#  * every output: the row-relative error max_(i,h) ||out - ref||_inf /
#    ||ref||_inf <= ROW_RTOL (rows whose reference is all zero are held to the
#    absolute bound alone);
#  * bf16 outputs: element-wise |out - ref| <= ATOL + RTOL*|ref| (rounding the
#    output to bf16 alone moves an element by up to 2^-9 |ref|, so a plain
#    2e-3 absolute bound cannot hold where |ref| exceeds about 1);
#  * float32 outputs (FCA_PLAN_OUT_F32): max |out - ref| <= ATOL.
ATOL = 2e-3
RTOL = 1e-2
ROW_RTOL = 1e-2
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


def _check_rows(out, ref, what):
    err = np.abs(out - ref).max(axis=-1)
    rowmax = np.abs(ref).max(axis=-1)
    live = rowmax > 0
    with np.errstate(invalid="ignore", divide="ignore"):
        rel = np.where(live, err / np.where(live, rowmax, 1.0), 0.0)
    if (rel > ROW_RTOL).any():
        idx = np.unravel_index(np.argmax(rel), rel.shape)
        raise AssertionError(
            f"{what}: row-relative error {rel[idx]:.3g} > {ROW_RTOL} at row {idx} "
            f"(max |err| {err[idx]:.3g}, max |ref| {rowmax[idx]:.3g}); {error_report(out, ref)}"
        )
    dead = ~live
    if dead.any() and (err[dead] > ATOL).any():
        raise AssertionError(f"{what}: rows with an all-zero reference are off by more than {ATOL}")


def assert_close(out, ref, what=""):
    """bf16 outputs: element-wise bound and row-relative bound."""
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
    _check_rows(out, ref, what)
    return error_report(out, ref)


def assert_close_f32(out, ref, what=""):
    """float32 outputs: max-abs bound and row-relative bound."""
    assert np.isfinite(out).all(), f"{what}: non-finite output"
    err = np.abs(out - ref)
    if err.size and err.max() > ATOL:
        idx = np.unravel_index(np.argmax(err), err.shape)
        raise AssertionError(f"{what}: max |err| {err[idx]:.3g} > {ATOL} at {idx}; {error_report(out, ref)}")
    _check_rows(out, ref, what)
    return error_report(out, ref)


def assert_lse_close(lse, ref, what=""):
    both_inf = np.isneginf(lse) & np.isneginf(ref)
    with np.errstate(invalid="ignore"):
        diff = np.where(both_inf, 0.0, np.abs(lse - ref))
    assert (diff <= LSE_ATOL).all(), f"{what}: lse max diff {np.nanmax(diff)}"


def host_values(vals):
    """Host copies (uint16 bf16 bits) of device q / k / v, taken before any
    decode runs, so that the oracle sees the inputs and not whatever a
    kernel might leave in device memory."""
    return {k: (to_bits(v) if v is not None else None) for k, v in vals.items()}


def oracle_all(batch, host, requests=None, threads=None, say=None):
    """fp64 oracle attention of every request (or the listed ones) of a batch
    from host copies of its inputs; requests run on a pool of threads (one
    BLAS thread each).  Returns (out [B, Hq, Dv], lse [B, Hq])."""
    import os
    import time
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    sh = batch.shape
    reqs = list(range(batch.batch)) if requests is None else list(requests)
    out = np.zeros((batch.batch, sh.num_q_heads, sh.head_dim_v))
    lse = np.full((batch.batch, sh.num_q_heads), -np.inf)
    n_threads = threads or min(16, len(os.sched_getaffinity(0)))
    t0 = time.perf_counter()
    done = [0]

    def one(i):
        o, l = A.attend(host["q"], host["k"], host["v"], batch.block_tables, batch.seq_lens, sh, requests=[i])
        out[i], lse[i] = o[i], l[i]
        done[0] += 1
        if say is not None and done[0] % 64 == 0:
            say(f"oracle: {done[0]} of {len(reqs)} requests, {time.perf_counter() - t0:.1f} s")

    with threadpool_limits(limits=1):
        with ThreadPoolExecutor(n_threads) as ex:
            list(ex.map(one, reqs))
    if say is not None:
        say(f"oracle: {len(reqs)} requests in {time.perf_counter() - t0:.1f} s on {n_threads} threads")
    return out, lse
