#!/usr/bin/env python3
"""Forest Cascade Attention decode benchmark (one MI355X).

One step = one ``fca_decode`` of a whole batch (grouped prefix pass,
per-request suffix pass, log-sum-exp merge) for one attention layer.  The
batch is a seeded synthetic shared-prefix rollout batch (default: the
long-context RL rollout, the largest of the five workloads: 256 requests =
16 prompts x 16 samples, prefix 16384, suffix U{1..4096}, GQA 32/8, head dim
128, 16-token blocks).  Steps cycle
through ``--layers`` independent KV pools that share one plan, as the layers
of a model do, so each step reads KV that is not resident in L2 / MALL.

Printed (one JSON line on stdout): logical-KV tokens/s (the value), unique-KV
GB/s and its share of the 8 TB/s HBM peak, per-pass times measured with HIP
events on the kernels' stream, the roofline of the dominant kernel, the
non-cascade baseline (same kernels, every request read whole), the CPU
oracle timed on a bounded sample, the streaming-read rate a plain kernel
reaches on the device, and a short record of each of the other workloads
(cascade vs non-cascade).  Progress goes to stderr.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
RIDGE_FLOP_PER_BYTE = 312.0  # 2.5 PFLOP/s bf16 over 8 TB/s
COPY_BYTES = 1 << 30
MFMA_BF16_PEAK_TFLOPS = 2500.0
# kernel entry of each pass when the two passes are launched one after the
# other (the latent-cache plans always; GQA plans with separate passes)
PASS_KERNELS = {
    "gqa": ("fca_attention_grouped_kernel", "fca_attention_suffix_kernel"),
    "mla": ("fca_mla_grouped_kernel", "fca_mla_suffix_kernel"),
}


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="long_rl")
    ap.add_argument(
        "--others",
        default="tiny,llama3_8b,forest_mixed,mla",
        help="workloads given a short cascade / non-cascade record beside the headline one ('' for none)",
    )
    ap.add_argument("--layers", type=int, default=8, help="independent KV pools cycled by the steps")
    ap.add_argument("--cpu-seconds", type=float, default=24.0, help="budget of the CPU oracle sample (split between the all-threads and one-thread runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-noncascade", action="store_true")
    ap.add_argument("--profile-only", action="store_true", help="few steps, no baselines (for rocprofv3)")
    ap.add_argument(
        "--no-cascade",
        action="store_true",
        help="time the non-cascade plan as the main one (to profile the baseline's launches)",
    )
    ap.add_argument(
        "--separate-passes",
        action="store_true",
        help="time the plan that launches the grouped and the per-request pass one after the other as the main "
        "one (to profile each pass's launch)",
    )
    ap.add_argument(
        "--group-sweep",
        action="store_true",
        help="also time cascade vs non-cascade over group sizes 1..64 (64 requests, Llama-3 layer shape)",
    )
    ap.add_argument(
        "--copy-calibration",
        action="store_true",
        help="also run a plain elementwise copy of known size (scale of the HBM byte counters)",
    )
    return ap.parse_args()


def pass_bytes(batch, plan, sched):
    """Algorithmic bytes per launch.

    Attention (both passes): every unique KV token row once (a group's prefix
    range once for the group, each request's suffix once) plus each
    request's Q row once.  Grouped / suffix alone: their share of that.
    Merge: the partial triples it reads plus the output (and lse) it writes.
    Partial-triple writes of the attention kernel are not counted: they
    follow from the token splits, not from the method.
    """
    sh = batch.shape
    bs = sh.block_size
    tok_bytes = (sh.num_kv_heads * sh.head_dim_qk * 2) if sh.v_aliases_k else sh.num_kv_heads * (sh.head_dim_qk + sh.head_dim_v) * 2
    ex = plan.export()
    prefix_tokens = sum((g["block_end"] - g["block_begin"]) * bs for g in ex["groups"])
    suffix_tokens = sum(r[1] for r in ex["requests"])
    q_bytes = batch.batch * sh.num_q_heads * sh.head_dim_qk * 2
    row_bytes = sh.head_dim_v * 4 + 8
    rows = plan.info.num_partial_rows
    merge = rows * row_bytes + batch.batch * sh.num_q_heads * (sh.head_dim_v * 2 + 4)
    flops_g = sum(
        (g["block_end"] - g["block_begin"]) * bs * len(g["members"]) * sh.num_q_heads * 2 * (sh.head_dim_qk + sh.head_dim_v)
        for g in ex["groups"]
    )
    return dict(
        attention=(prefix_tokens + suffix_tokens) * tok_bytes + q_bytes,
        grouped=prefix_tokens * tok_bytes + q_bytes,
        suffix=suffix_tokens * tok_bytes + q_bytes,
        merge=merge,
        prefix_tokens=prefix_tokens,
        suffix_tokens=suffix_tokens,
        tok_bytes=tok_bytes,
        grouped_flops=flops_g,
        suffix_flops=suffix_tokens * sh.num_q_heads * 2 * (sh.head_dim_qk + sh.head_dim_v),
    )


def time_steps(plan, q, pools, out, lse, steps, torch, fca):
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for s in range(steps):
        k, v = pools[s % len(pools)]
        fca.fca_decode(q[s % len(q)], k, v, plan, out=out, lse=lse)
    stop.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1000.0 / steps
    return start.elapsed_time(stop) / steps, wall


def warm(plan, q, pools, out, lse, steps, torch, fca, min_s=0.2):
    """At least `steps` untimed decodes and at least `min_s` seconds of them,
    so that every timed loop starts with the GPU at its working clocks."""
    t0 = time.perf_counter()
    n = 0
    while n < steps or time.perf_counter() - t0 < min_s:
        k, v = pools[n % len(pools)]
        fca.fca_decode(q[n % len(q)], k, v, plan, out=out, lse=lse)
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def cpu_baseline(batch, vals, budget_s, threads, cache=None):
    """The fp64 oracle on a bounded sample of the same batch: its requests in
    order, again from the first once all are done, until the budget is spent,
    with `threads` BLAS threads.  Only the oracle's own work is timed (the
    read-back of each request's blocks is not); `cache` keeps the read-back
    blocks between calls."""
    from threadpoolctl import threadpool_limits

    from oracle import attention as A
    import torch

    def to_bits(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    sh = batch.shape
    bs = sh.block_size
    q_bits = to_bits(vals["q"])
    cache = {} if cache is None else cache
    tokens = 0
    done = 0
    elapsed = 0.0
    with threadpool_limits(limits=threads):
        while elapsed < budget_s:
            i = done % batch.batch
            L = int(batch.seq_lens[i])
            nblk = -(-L // bs)
            if i not in cache:
                blocks = torch.from_numpy(batch.block_tables[i, :nblk].astype(np.int64)).to(vals["k"].device)
                k = to_bits(vals["k"].index_select(0, blocks))
                v = None if sh.v_aliases_k else to_bits(vals["v"].index_select(0, blocks))
                cache[i] = (k, v)
            k, v = cache[i]
            table = np.arange(nblk, dtype=np.int32)
            t0 = time.perf_counter()
            K, V = A.gather_kv(k, v, table, L, bs, sh.head_dim_v, sh.v_aliases_k)
            A.attend_one(A.widen_bf16(q_bits[i]), K, V, sh.scale, sh.num_kv_heads)
            elapsed += time.perf_counter() - t0
            tokens += L
            done += 1
    passes = done / batch.batch
    return dict(
        value=tokens / elapsed,
        unit="logical KV tokens/s",
        cores=threads,
        kind="oracle",
        sample=f"{done} request decodes ({passes:.2f} passes over the {batch.batch} requests of the batch, "
        f"{tokens} logical tokens), fp64 numpy oracle, {threads} BLAS thread(s), {elapsed:.1f} s",
    )


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def read_peak(torch, fca):
    """HBM read rate of a plain streaming kernel (fca_measure_read_bandwidth):
    two 2 GiB buffers, each far larger than the 256 MB last-level cache, read
    alternately 4 times each."""
    bufs = [torch.ones((1 << 31) // 2, dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    torch.cuda.synchronize()
    gbps = fca.measure_read_bandwidth(bufs, repeats=4)
    del bufs
    torch.cuda.empty_cache()
    return gbps


def token_row_pools(pools):
    """The same pools as token rows, [blocks][slots][kv heads][dims] (the
    descriptor's default row strides), rearranged on the device."""
    out = []
    for k, v in pools:
        nb, H, c, bs, e = k.shape
        kr = k.permute(0, 3, 1, 2, 4).reshape(nb, bs, H, c * e).contiguous()
        vr = v.permute(0, 3, 1, 2).contiguous() if v is not None else None
        out.append((kr, vr))
    return out


def pass_traffic(name, pb, latent, main, sep=None):
    """Each pass's own launch and the merge, measured by counters, from the
    committed rocprofv3 summaries of the same sources (None where there are
    none): the passes from `sep` or else from the summary of the workload's
    plan with one launch per pass (latent-cache plans always launch them so:
    their timed plan's summary `main`), the merge from `main`.  Per launch:
    HBM bytes (FETCH_SIZE + WRITE_SIZE, calibrated), the median duration, and
    the algorithmic bytes over that duration against the 8 TB/s peak."""
    from shared_prefix_kv_amd.profiling import load_traffic

    if sep is None:
        sep = main if latent else load_traffic(name + ".separate_passes")
    names = dict(zip(("grouped", "suffix"), PASS_KERNELS["mla" if latent else "gqa"]), merge="fca_merge_kernel")
    src = {"grouped": sep, "suffix": sep, "merge": main}
    pt = {}
    for pname, kname in names.items():
        d = src[pname]
        t = d["traffic"].get(kname) if d else None
        us = d.get("launch_us", {}).get(kname) if d else None
        if t and us and pb[pname] > 0:
            moved = t["fetch_bytes"] + t["write_bytes"]
            rate = pb[pname] / (us * 1e-6) / 1e9
            pt[pname] = {
                "kernel": kname,
                "launch_us_profiled": round(us, 2),
                "traffic": int(moved),
                "algorithmic_bytes": int(pb[pname]),
                "traffic_over_algorithmic": round(moved / pb[pname], 4),
                "algorithmic_GBps": round(rate, 1),
                "algorithmic_frac_of_hbm_peak": round(rate / HBM_PEAK_GBPS, 4),
            }
    if "suffix" in pt and "merge" in pt:
        us = pt["suffix"]["launch_us_profiled"] + pt["merge"]["launch_us_profiled"]
        rate = (pb["suffix"] + pb["merge"]) / (us * 1e-6) / 1e9
        pt["suffix_plus_merge"] = {"algorithmic_GBps": round(rate, 1), "algorithmic_frac_of_hbm_peak": round(rate / HBM_PEAK_GBPS, 4)}
    return pt or None


def short_record(name, torch, fca, steps, warmup, layers=4):
    """Cascade vs non-cascade on another workload: decode time per step, the
    logical-KV rate, unique-KV GB/s, the byte ratio R and the speedup."""
    from shared_prefix_kv_amd.profiling import load_traffic
    from workloads import CONFIGS, build_batch
    from workloads.values import fill_values_torch

    cfg = CONFIGS[name]
    batch = build_batch(cfg)
    sh = batch.shape
    pools, qs = [], []
    for layer in range(layers):
        v = fill_values_torch(batch, "cuda", seed=cfg.seed * 1000 + layer, poison=False)
        pools.append((v["k"], v["v"]))
        qs.append(v["q"])
    bt = torch.from_numpy(batch.block_tables).cuda()
    sl = torch.from_numpy(batch.seq_lens).cuda()
    out = torch.empty((batch.batch, sh.num_q_heads, sh.head_dim_v), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((batch.batch, sh.num_q_heads), dtype=torch.float32, device="cuda")
    res = {}
    latent = None
    desc = fca.desc_from_shape(sh, batch.num_blocks)
    fca.fca_plan(bt, sl, desc)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    create = []
    for _ in range(5):
        create.append(fca.fca_plan(bt, sl, desc).create_ms)
    torch.cuda.synchronize()
    plan_ms = (time.perf_counter() - t0) * 1000 / 5
    plans = {
        "fca": fca.fca_plan(bt, sl, desc),
        "non_cascade": fca.fca_plan(bt, sl, fca.desc_from_shape(sh, batch.num_blocks, cascade=False)),
    }
    # The two plans' samples alternate (three each, medians), so that both
    # see the same clocks.
    samples = {key: [] for key in plans}
    for plan in plans.values():
        plan.decode_workspace(out.device)
    for _ in range(3):
        for key, plan in plans.items():
            warm(plan, qs, pools, out, lse, warmup, torch, fca, min_s=0.1)
            samples[key].append(time_steps(plan, qs, pools, out, lse, steps, torch, fca)[0])
    for key, plan in plans.items():
        res[key] = (float(np.median(samples[key])), plan.info)
        if key == "fca":
            pb_fca = pass_bytes(batch, plan, None)
        if key == "fca" and sh.v_aliases_k:
            # Latent cache: the two passes are separate launches; time each.
            t = plan.time_launches(qs[0], pools, 10, out, lse)
            pb = pb_fca
            launch = {k[:-3]: round(v, 5) for k, v in t.items() if k.endswith("_ms") and v > 0}
            g_tf = pb["grouped_flops"] / (t["grouped_ms"] / 1000.0) / 1e12 if t["grouped_ms"] > 0 else 0.0
            latent = {
                "per_launch_ms": launch,
                "grouped_mfma_TFLOPs": round(g_tf, 1),
                "grouped_mfma_frac_of_peak": round(g_tf / MFMA_BF16_PEAK_TFLOPS, 4),
                "suffix_GBps": round(pb["suffix"] / (t["suffix_ms"] / 1000.0) / 1e9, 1) if t["suffix_ms"] > 0 else None,
            }
    del plans
    # The same plan over pools of token rows.
    rpools = token_row_pools(pools)
    plan = fca.fca_plan(bt, sl, fca.desc_from_shape(sh, batch.num_blocks, token_rows=True))
    plan.decode_workspace(out.device)
    warm(plan, qs, rpools, out, lse, warmup, torch, fca)
    ms_rows, _ = time_steps(plan, qs, rpools, out, lse, steps, torch, fca)
    del plan, rpools
    ms, info = res["fca"]
    ms_nc, _ = res["non_cascade"]
    tok_bytes = sh.kv_bytes_per_token()
    rec = {
        "workload": f"{cfg.name}: {cfg.description}",
        "fca_us_per_step": round(ms * 1000, 2),
        "non_cascade_us_per_step": round(ms_nc * 1000, 2),
        "token_rows_us_per_step": round(ms_rows * 1000, 2),
        "logical_kv_tokens_per_s": round(int(info.logical_tokens) / (ms / 1000.0), 1),
        "unique_kv_GBps": round(int(info.unique_tokens) * tok_bytes / (ms / 1000.0) / 1e9, 1),
        "byte_ratio_R": round(int(info.logical_tokens) / max(int(info.unique_tokens), 1), 3),
        "speedup_vs_non_cascade": round(ms_nc / ms, 3),
        "plan_ms": round(plan_ms, 3),
        "plan_ms_per_layer_of_32": round(plan_ms / 32, 4),
        "plan_create_call_ms": round(float(np.median(create)), 3),
        "folded_groups": int(info.num_folded_groups),
    }
    if latent:
        rec["latent"] = latent
    pt = pass_traffic(name, pb_fca, sh.v_aliases_k, load_traffic(name))
    if pt:
        rec["pass_traffic"] = pt
    del pools, qs
    torch.cuda.empty_cache()
    return rec


def kv_append_leg(batch, pool, torch, fca):
    sh = batch.shape
    B = batch.batch
    k, v = pool
    desc = fca.desc_from_shape(sh, batch.num_blocks)
    bt = torch.from_numpy(batch.block_tables).cuda()
    pos = torch.from_numpy(np.maximum(batch.seq_lens - 1, 0).astype(np.int32)).cuda()
    kn = torch.randn((B, sh.num_kv_heads, sh.head_dim_qk), device="cuda").to(torch.bfloat16)
    vn = None if sh.v_aliases_k else torch.randn((B, sh.num_kv_heads, sh.head_dim_v), device="cuda").to(torch.bfloat16)
    free = np.nonzero(~batch.used_blocks)[0].astype(np.int32)
    res = {}
    legs = [("in_place_us", None)]
    if len(free) >= 2 * B:
        legs.append(("copy_on_write_us", (torch.from_numpy(free[:B]).cuda(), torch.from_numpy(free[B : 2 * B]).cuda())))
    per_graph, reps = 20, 10
    for name, cows in legs:
        def call(j):
            fca.kv_append(kn, vn, k, v, bt, pos, desc, cow_dst=None if cows is None else cows[j % 2])

        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call(0)
            call(1)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for j in range(per_graph):
                call(j)
        for _ in range(3):
            g.replay()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        res[name] = round(e0.elapsed_time(e1) * 1000 / (reps * per_graph), 2)
        del g
    return res


def group_sweep(torch, fca, steps, warmup):
    """Cascade vs non-cascade over the group size: 64 requests of the
    Llama-3-8B layer shape, prefix 4096, suffix U{256..1024}, as 64 / s
    prompts x s samples for s = 1 .. 64.  Two KV pools are cycled."""
    from workloads import build_batch
    from workloads.forest import GQA_LLAMA, Config, Node
    from workloads.values import fill_values_torch

    rows = []
    for s in (1, 2, 4, 8, 16, 32, 64):
        if s == 1:  # no sharing: 64 unshared requests of the same lengths
            cfg = Config(name="sweep_s1", shape=GQA_LLAMA, trees=[], singletons=64,
                         singleton_len=(4096 + 256, 4096 + 1024), seed=101)
        else:
            cfg = Config(
                name=f"sweep_s{s}",
                shape=GQA_LLAMA,
                trees=[Node(4096, samples=s, suffix=(256, 1024)) for _ in range(64 // s)],
                seed=100 + s,
            )
        batch = build_batch(cfg)
        sh = batch.shape
        pools, qs = [], []
        for layer in range(2):
            v = fill_values_torch(batch, "cuda", seed=cfg.seed * 1000 + layer, poison=False)
            pools.append((v["k"], v["v"]))
            qs.append(v["q"])
        bt = torch.from_numpy(batch.block_tables).cuda()
        sl = torch.from_numpy(batch.seq_lens).cuda()
        out = torch.empty((batch.batch, sh.num_q_heads, sh.head_dim_v), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((batch.batch, sh.num_q_heads), dtype=torch.float32, device="cuda")
        res = {}
        for cascade in (True, False):
            plan = fca.fca_plan(bt, sl, fca.desc_from_shape(sh, batch.num_blocks, cascade=cascade))
            plan.decode_workspace(out.device)
            warm(plan, qs, pools, out, lse, warmup, torch, fca)
            ms, _ = time_steps(plan, qs, pools, out, lse, steps, torch, fca)
            res[cascade] = (ms, plan.info)
        ms_c, info = res[True]
        ms_n, _ = res[False]
        row = {
            "samples_per_prompt": s,
            "groups": int(info.num_groups),
            "byte_ratio_R": round(int(info.logical_tokens) / max(int(info.unique_tokens), 1), 3),
            "cascade_us": round(ms_c * 1000, 2),
            "non_cascade_us": round(ms_n * 1000, 2),
            "speedup": round(ms_n / ms_c, 3),
        }
        log("group sweep:", row)
        rows.append(row)
        del pools, qs
        torch.cuda.empty_cache()
    return rows


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(
            "bench.py measures one GPU: this decode path runs on a single MI355X and "
            "has no multi-GPU mode (--gpus must be 1).",
            file=sys.stderr,
        )
        sys.exit(2)

    import torch

    import shared_prefix_kv_amd as fca
    from workloads import CONFIGS, build_batch
    from workloads.values import fill_values_torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    fca.lib()
    cfg = CONFIGS[args.config]
    batch = build_batch(cfg)
    sh = batch.shape
    log(f"config {cfg.name}: B={batch.batch} pool={batch.num_blocks} blocks, layers={args.layers}")

    pools = []
    qs = []
    for layer in range(args.layers):
        vals = fill_values_torch(batch, "cuda", seed=cfg.seed * 1000 + layer, poison=False)
        pools.append((vals["k"], vals["v"]))
        qs.append(vals["q"])
        if layer == 0:
            vals0 = vals
    torch.cuda.synchronize()
    log("pools ready")

    bt = torch.from_numpy(batch.block_tables).cuda()
    sl = torch.from_numpy(batch.seq_lens).cuda()
    desc = fca.desc_from_shape(sh, batch.num_blocks, cascade=not args.no_cascade, separate_passes=args.separate_passes)
    t0 = time.perf_counter()
    plan = fca.fca_plan(bt, sl, desc)
    torch.cuda.synchronize()
    plan_ms_first = (time.perf_counter() - t0) * 1000
    t0 = time.perf_counter()
    create = []
    for _ in range(5):
        plan = fca.fca_plan(bt, sl, desc)
        create.append(plan.create_ms)
    torch.cuda.synchronize()
    plan_ms = (time.perf_counter() - t0) * 1000 / 5
    info = plan.info
    # The same batch with the grouped and per-request passes launched one
    # after the other, for per-pass kernel times.
    plan_sep = fca.fca_plan(
        bt, sl, fca.desc_from_shape(sh, batch.num_blocks, separate_passes=True, cascade=not args.no_cascade)
    )
    sched = plan.export_schedule()
    pb = pass_bytes(batch, plan, sched)
    log(f"plan: {info.num_groups} groups, {info.num_grouped_items} grouped + {info.num_suffix_items} suffix items, {plan_ms:.2f} ms")

    out = torch.empty((batch.batch, sh.num_q_heads, sh.head_dim_v), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((batch.batch, sh.num_q_heads), dtype=torch.float32, device="cuda")
    plan.decode_workspace(out.device)

    plan_sep.decode_workspace(out.device)
    steps, warmup = args.steps, args.warmup
    if args.profile_only:
        # Only the launch-timing loops: the kernel trace then holds the timed
        # plan's launches only, the ones the roofline figures come from.
        steps, warmup = min(steps, 32), min(warmup, 2)
        ms = wall_ms = float("nan")
    else:
        warm(plan, qs, pools, out, lse, warmup, torch, fca)
        ms, wall_ms = time_steps(plan, qs, pools, out, lse, steps, torch, fca)
        log(f"fca decode: {ms * 1000:.1f} us/step (events), {wall_ms * 1000:.1f} us/step (wall)")

    if args.copy_calibration:
        # A plain bf16 copy (read + write COPY_BYTES each) whose FETCH_SIZE /
        # WRITE_SIZE give the scale of those counters on this chip.
        src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        log(f"calibration copy: {COPY_BYTES} bytes read and written per launch")
        del src, dst

    # Kernel times: each launch kind of a decode issued back to back between
    # two HIP events on the kernels' stream (fca_time_launches), cycling over
    # the KV pools like the timed loop (separate loops, so the events do not
    # touch `value`).  Latent caches launch the grouped and the per-request
    # pass one after the other in every plan, so the timed plan gives each
    # pass's time; otherwise the separate-pass plan does.
    reps = max(1, steps // len(pools))

    def launch_times(pl):
        warm(pl, qs, pools, out, lse, warmup, torch, fca)
        return pl.time_launches(qs[0], pools, reps, out, lse)

    per = launch_times(plan)
    two_launches = per["grouped_ms"] > 0 or per["suffix_ms"] > 0
    per = {k: per[f"{k}_ms"] for k in ("attention", "grouped", "suffix", "merge", "decode")}
    if two_launches:
        pass
    elif args.profile_only:
        # only the timed plan's launches, so that counter runs see one kind
        per["grouped"] = per["suffix"] = float("nan")
    else:
        per_sep = launch_times(plan_sep)
        per["grouped"], per["suffix"] = per_sep["grouped_ms"], per_sep["suffix_ms"]
    log("per launch (ms):", {k: round(v, 4) for k, v in per.items()})
    if args.profile_only:
        ms = per["decode"]

    logical = int(info.logical_tokens)
    unique_bytes = int(info.unique_tokens) * pb["tok_bytes"]
    value = logical / (ms / 1000.0)
    unique_gbps = unique_bytes / (ms / 1000.0) / 1e9

    merge_kernel = "fca_merge_kernel_d128" if sh.head_dim_v == 128 else "fca_merge_kernel_d512"
    # Launches of one decode: (kernel, launch, algorithmic bytes, flops).  The
    # roofline is taken on the longest one.
    launches = [(merge_kernel, "merge", pb["merge"], 0)]
    if two_launches:
        # the latent-cache kernel, one entry name per pass
        g_name, s_name = PASS_KERNELS["mla" if sh.v_aliases_k else "gqa"]
        launches += [
            (g_name, "grouped", pb["grouped"], pb["grouped_flops"]),
            (s_name, "suffix", pb["suffix"], pb["suffix_flops"]),
        ]
    else:
        launches.append(("fca_attention_kernel", "attention", pb["attention"], pb["grouped_flops"] + pb["suffix_flops"]))
    dom_name, dom_pass, dom_bytes, dom_flops = max(launches, key=lambda x: per[x[1]])
    if dom_flops / dom_bytes > RIDGE_FLOP_PER_BYTE:
        # The latent cache: every query row costs 2 (Dqk + Dv) flops per
        # token, above the ridge, so the bound is the bf16 MFMA rate.
        achieved = dom_flops / (per[dom_pass] / 1000.0) / 1e12
        roofline = {
            "kernel": dom_name,
            "launch": dom_pass,
            "bound": "mfma",
            "achieved": round(achieved, 1),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": None,
            "flops_per_launch": int(dom_flops),
            "bytes_per_launch": int(dom_bytes),
            "avg_launch_ms": round(per[dom_pass], 5),
        }
    else:
        achieved = dom_bytes / (per[dom_pass] / 1000.0) / 1e9
        roofline = {
            "kernel": dom_name,
            "launch": dom_pass,
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": None,
            "bytes_per_launch": int(dom_bytes),
            "avg_launch_ms": round(per[dom_pass], 5),
        }
    # HBM bytes per launch measured with FETCH_SIZE / WRITE_SIZE (calibrated
    # against a copy of known size) in the committed profile summary, used
    # only while the library sources are the ones it was taken with.
    from shared_prefix_kv_amd.profiling import load_traffic

    variant = ".non_cascade" if args.no_cascade else ".separate_passes" if args.separate_passes else ""
    tr = load_traffic(cfg.name + variant)
    if tr and dom_name == tr["kernel"] and dom_name in tr["traffic"]:
        t = tr["traffic"][dom_name]
        roofline["traffic"] = int(t["fetch_bytes"] + t["write_bytes"])
        roofline["traffic_detail"] = {
            "fetch_bytes": int(t["fetch_bytes"]),
            "write_bytes": int(t["write_bytes"]),
            "counter_scale": {"fetch": round(tr["fetch_factor"], 4), "write": round(tr["write_factor"], 4)},
        }
        u = tr.get("util", {}).get(dom_name)
        if u:
            # matrix-core and LDS use of the same kernel (derived rocprofv3 counters)
            roofline["counters"] = {
                "mfma_busy_pct": round(u.get("MfmaUtil", float("nan")), 1),
                "lds_active_pct": round(u.get("LdsUtil", float("nan")), 1),
                "lds_bank_conflict_pct": round(u.get("LDSBankConflict", float("nan")), 1),
                "bf16_mfma_TFLOPs_counted": round(u.get("bf16_TFLOPs", float("nan")), 1),
            }
    def gbps(nbytes, ms_):
        return round(nbytes / (ms_ / 1000.0) / 1e9, 1) if ms_ > 0 else None  # None for nan / 0

    sfx_merge_gbps = gbps(pb["suffix"] + pb["merge"], per["suffix"] + per["merge"])
    grouped_tflops = pb["grouped_flops"] / (per["grouped"] / 1000.0) / 1e12 if per["grouped"] > 0 else 0.0

    result = {
        "metric": "decode attn: unique-KV HBM GB/s (% of peak) + logical KV tokens/s",
        "value": round(value, 1),
        "unit": "logical KV tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: {cfg.description}",
            "batch": batch.batch,
            "logical_kv_tokens": logical,
            "unique_kv_tokens": int(info.unique_tokens),
            "groups": int(info.num_groups),
            "kv_pools_cycled": args.layers,
            "folded_groups": int(info.num_folded_groups),
        },
        "unique_kv_GBps": round(unique_gbps, 1),
        "unique_kv_frac_of_hbm_peak": round(unique_gbps / HBM_PEAK_GBPS, 4),
        "wall_ms_per_step": round(wall_ms, 5),
        "per_launch_ms": {k: (round(v, 5) if v == v else None) for k, v in per.items()},
        "pass_GBps": {
            "attention": gbps(pb["attention"], per["attention"]),
            "grouped": gbps(pb["grouped"], per["grouped"]),
            "suffix": gbps(pb["suffix"], per["suffix"]),
            "merge": gbps(pb["merge"], per["merge"]),
            "suffix_plus_merge": sfx_merge_gbps,
        },
        "grouped_mfma_TFLOPs": round(grouped_tflops, 1),
        "grouped_mfma_frac_of_peak": round(grouped_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "plan_ms": round(plan_ms, 3),
        "plan_ms_per_layer_of_32": round(plan_ms / 32, 4),
        "plan_create_call_ms": round(float(np.median(create)), 3),
        "plan_ms_first_call": round(plan_ms_first, 3),
        "roofline": roofline,
    }

    if not args.no_cascade:
        pt = pass_traffic(cfg.name, pb, sh.v_aliases_k, tr, sep=tr if two_launches else None)
        if pt:
            result["pass_traffic"] = pt

    if not args.profile_only:
        warm(plan_sep, qs, pools, out, lse, warmup, torch, fca)
        ms_sep, _ = time_steps(plan_sep, qs, pools, out, lse, steps, torch, fca)
        log(f"fca decode, separate pass launches: {ms_sep * 1000:.1f} us/step")
        result["separate_passes_ms_per_step"] = round(ms_sep, 5)

    if not args.profile_only and not sh.v_aliases_k:
        # Every discovered group kept (FCA_PLAN_KEEP_GROUPS): the timed plan
        # above runs the library's default activation heuristic, which reads
        # groups that cannot pay for their partial rows per request.
        plan_kg = fca.fca_plan(bt, sl, fca.desc_from_shape(sh, batch.num_blocks, auto_fold=False))
        plan_kg.decode_workspace(out.device)
        warm(plan_kg, qs, pools, out, lse, warmup, torch, fca)
        ms_kg, _ = time_steps(plan_kg, qs, pools, out, lse, steps, torch, fca)
        n_f = int(info.num_folded_groups)
        log(f"fca decode keeping every group: {ms_kg * 1000:.1f} us/step (default plan: {n_f} of {info.num_groups} groups folded)")
        result["activation"] = {
            "folded_groups": n_f,
            "groups": int(info.num_groups),
            "keep_groups_ms_per_step": round(ms_kg, 5),
        }
        del plan_kg

    if not args.profile_only:
        # The same batch over pools of token rows ([blocks][slots][kv heads]
        # [dims]), which the kernels gather into the tile arrangement.
        rpools = token_row_pools(pools)
        plan_r = fca.fca_plan(bt, sl, fca.desc_from_shape(sh, batch.num_blocks, token_rows=True,
                                                          cascade=not args.no_cascade))
        plan_r.decode_workspace(out.device)
        warm(plan_r, qs, rpools, out, lse, warmup, torch, fca)
        ms_r, _ = time_steps(plan_r, qs, rpools, out, lse, steps, torch, fca)
        log(f"fca decode from token-row pools: {ms_r * 1000:.1f} us/step")
        result["token_rows"] = {
            "layout": "[blocks][slots][kv_heads][dims]",
            "ms_per_step": round(ms_r, 5),
            "value": round(logical / (ms_r / 1000.0), 1),
            "time_over_tiles": round(ms_r / ms, 4),
        }
        del plan_r, rpools
        torch.cuda.empty_cache()

    if not args.no_noncascade and not args.profile_only:
        desc_nc = fca.desc_from_shape(sh, batch.num_blocks, cascade=False)
        plan_nc = fca.fca_plan(bt, sl, desc_nc)
        plan_nc.decode_workspace(out.device)
        # Non-cascade and cascade samples alternate (three each, medians).
        # The cascade samples then run right after the long non-cascade
        # launches and are slower than the headline steps (the chip is
        # warmer), so both ratios are given: against the headline step, and
        # against the adjacent samples.
        nc_s, fca_s = [], []
        for _ in range(3):
            warm(plan_nc, qs, pools, out, lse, warmup, torch, fca, min_s=0.1)
            nc_s.append(time_steps(plan_nc, qs, pools, out, lse, steps, torch, fca)[0])
            warm(plan, qs, pools, out, lse, warmup, torch, fca, min_s=0.1)
            fca_s.append(time_steps(plan, qs, pools, out, lse, steps, torch, fca)[0])
        ms_nc, ms_fca_adj = float(np.median(nc_s)), float(np.median(fca_s))
        log(f"non-cascade: {ms_nc * 1000:.1f} us/step (cascade between its samples: {ms_fca_adj * 1000:.1f} us/step)")
        result["non_cascade"] = {
            "ms_per_step": round(ms_nc, 5),
            "value": round(logical / (ms_nc / 1000.0), 1),
            "speedup_fca": round(ms_nc / ms, 3),
            "fca_adjacent_ms_per_step": round(ms_fca_adj, 5),
            "speedup_fca_adjacent": round(ms_nc / ms_fca_adj, 3),
            "byte_ratio_R": round(logical / max(int(info.unique_tokens), 1), 3),
        }
        # HBM bytes the non-cascade attention launch moves (committed counter
        # summary of the same sources), against the logical KV bytes it reads:
        # below 1 where the last-level cache serves repeated prefix blocks.
        trn = load_traffic(cfg.name + ".non_cascade")
        if trn and "fca_attention_kernel" in trn["traffic"]:
            t = trn["traffic"]["fca_attention_kernel"]
            logical_bytes = logical * pb["tok_bytes"] + batch.batch * sh.num_q_heads * sh.head_dim_qk * 2
            result["non_cascade"]["traffic"] = int(t["fetch_bytes"] + t["write_bytes"])
            result["non_cascade"]["traffic_over_logical_bytes"] = round(
                (t["fetch_bytes"] + t["write_bytes"]) / logical_bytes, 4
            )
            result["non_cascade"]["attention_launch_us_profiled"] = round(trn["avg_launch_us"], 2)
        del plan_nc

    if not args.profile_only:
        # The same steps from a HIP graph: one capture of one decode per KV
        # pool (one plan shared by the layers), replayed; shows the launch
        # overhead a graph removes.
        ws = plan.decode_workspace(out.device)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for li, (k, v) in enumerate(pools):
                fca.fca_decode(qs[li], k, v, plan, out=out, lse=lse)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for li, (k, v) in enumerate(pools):
                fca.fca_decode(qs[li], k, v, plan, out=out, lse=lse)
        torch.cuda.synchronize()
        reps = max(1, steps // len(pools))
        t_w = time.perf_counter()
        while time.perf_counter() - t_w < 0.2:
            graph.replay()
            torch.cuda.synchronize()
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)

        def graph_ms():
            g0.record()
            for _ in range(reps):
                graph.replay()
            g1.record()
            torch.cuda.synchronize()
            return g0.elapsed_time(g1) / (reps * len(pools))

        # Replays and eager steps alternate, so that both see the same clocks
        # (this leg runs after the long non-cascade one); medians of three.
        pairs = [(graph_ms(), time_steps(plan, qs, pools, out, lse, reps * len(pools), torch, fca)[0]) for _ in range(3)]
        ms_graph = float(np.median([p[0] for p in pairs]))
        ms_eager_adj = float(np.median([p[1] for p in pairs]))
        log(f"fca decode from a HIP graph ({len(pools)} layers per replay): {ms_graph * 1000:.1f} us/step "
            f"(eager steps between the replays: {ms_eager_adj * 1000:.1f} us/step)")
        result["graph_ms_per_step"] = round(ms_graph, 5)
        result["graph_eager_adjacent_ms_per_step"] = round(ms_eager_adj, 5)
        del graph, ws

    if not args.profile_only:
        # The route-the-query merge (fca_merge_states) of two float32 states
        # of this batch's shape: bytes = both states and lses read, the bf16
        # output and the lse written.
        Bq, Hq_, Dv = batch.batch, sh.num_q_heads, sh.head_dim_v
        st_o = [torch.randn((Bq, Hq_, Dv), device="cuda") for _ in range(2)]
        st_l = [torch.randn((Bq, Hq_), device="cuda") for _ in range(2)]
        mo = torch.empty((Bq, Hq_, Dv), dtype=torch.bfloat16, device="cuda")
        ml = torch.empty((Bq, Hq_), dtype=torch.float32, device="cuda")
        # 20 launches captured in a HIP graph, so that the timing is the
        # device's and not the Python call rate
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fca.merge_states(st_o, st_l, out=mo, lse=ml)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        per_graph = 20
        mg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(mg):
            for _ in range(per_graph):
                fca.merge_states(st_o, st_l, out=mo, lse=ml)
        for _ in range(3):
            mg.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        reps = 10
        e0.record()
        for _ in range(reps):
            mg.replay()
        e1.record()
        torch.cuda.synchronize()
        ms_m = e0.elapsed_time(e1) / (reps * per_graph)
        del mg
        mbytes = 2 * Bq * Hq_ * (Dv * 4 + 4) + Bq * Hq_ * (Dv * 2 + 4)
        result["merge_states"] = {"states": 2, "us": round(ms_m * 1000, 2), "GBps": gbps(mbytes, ms_m), "bytes": mbytes}
        log(f"merge of two float32 states: {ms_m * 1000:.1f} us ({gbps(mbytes, ms_m)} GB/s)")
        del st_o, st_l, mo, ml

    if not args.profile_only:
        # The step before the path: one new token per request appended to the
        # last KV pool (over each request's last cached token, so the pools
        # keep their shape), in place and with a copy-on-write of every
        # request's last block (targets alternating between two sets of
        # unused blocks, so every call copies).  20 calls per HIP graph.
        result["kv_append"] = kv_append_leg(batch, pools[-1], torch, fca)
        log(f"kv append ({batch.batch} requests): {result['kv_append']}")

    if args.group_sweep and not args.profile_only:
        result["group_sweep"] = group_sweep(torch, fca, steps, warmup)

    if not args.profile_only:
        rp = read_peak(torch, fca)
        result["read_peak_GBps"] = round(rp, 1)
        result["roofline"]["measured_read_peak_GBps"] = round(rp, 1)
        result["roofline"]["frac_of_measured_read_peak"] = (
            round(roofline["achieved"] / rp, 4) if roofline["unit"] == "GB/s" and rp > 0 else None
        )
        log(f"streaming read, plain kernel: {rp:.0f} GB/s")
        # Matrix-core counterpart: a loop of independent 16x16x32 products.
        mf = {d: round(fca.measure_mfma_rate(d, iters=4000), 1) for d in ("bf16", "f16")}
        result["mfma_peak_TFLOPs"] = mf
        if roofline["unit"] == "TFLOP/s":
            result["roofline"]["measured_mfma_peak_TFLOPs"] = mf["bf16"]
            result["roofline"]["frac_of_measured_mfma_peak"] = round(roofline["achieved"] / mf["bf16"], 4)
        log(f"dense MFMA loop, plain kernel: {mf} TFLOP/s")

    if not args.no_cpu_baseline and not args.profile_only:
        ncpu = len(os.sched_getaffinity(0))
        log(f"cpu baseline (oracle), {ncpu} threads then 1 ...")
        blocks = {}
        result["cpu_baseline"] = cpu_baseline(batch, vals0, args.cpu_seconds / 2, ncpu, blocks)
        result["cpu_baseline_1_thread"] = cpu_baseline(batch, vals0, args.cpu_seconds / 2, 1, blocks)
        for k in ("cpu_baseline", "cpu_baseline_1_thread"):
            result[k]["cpu_model"] = cpu_model()
        del blocks

    others = [o for o in args.others.split(",") if o and o != cfg.name] if not args.profile_only else []
    if others:
        del pools, qs, vals0, vals
        torch.cuda.empty_cache()
        result["other_workloads"] = {}
        for name in others:
            rec = short_record(name, torch, fca, max(steps // 2, 8), warmup)
            if "latent" in rec and "mfma_peak_TFLOPs" in result:
                peak = result["mfma_peak_TFLOPs"]["bf16"]
                rec["latent"]["grouped_frac_of_measured_mfma_peak"] = round(rec["latent"]["grouped_mfma_TFLOPs"] / peak, 4)
            log(f"{name}: {rec}")
            result["other_workloads"][name] = rec

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
