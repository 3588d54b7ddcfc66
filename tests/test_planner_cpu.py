"""The host planner on the CPU, built with AddressSanitizer and
UndefinedBehaviorSanitizer (tests/native/planner_harness.cpp linked with
shared_prefix_kv_amd/csrc/planner.cpp; no GPU, no HIP).

The planner's input is the discovery read-back: group records (leader,
depth, parent, block range, member count) in whatever order the device
emitted them, and per request its length, deepest group and suffix start.
Here that read-back is written from the oracle's grouping (with the records
shuffled), so each test checks the planner's index arithmetic -- canonical
order, depth-first member order, the activation heuristic, the split
schedule, the merge tables -- against the oracle and the exact-coverage
rules, on the five workloads, fuzzed forests, a deep chain and 8192
requests, and feeds it malformed read-backs that it must reject.
"""

from __future__ import annotations

import math
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle.grouping import group
from tests.forests import random_forest
from tests.schedule_check import check_schedule_data
from workloads import CONFIGS, build_batch
from workloads.forest import AttnShape

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HARNESS = os.path.join(ROOT, "tests", "native", "planner_harness.cpp")
PLANNER = os.path.join(ROOT, "shared_prefix_kv_amd", "csrc", "planner.cpp")
INCLUDES = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "shared_prefix_kv_amd", "csrc")]

DISABLE_CASCADE, SEPARATE_PASSES, KEEP_GROUPS = 1, 2, 16
N_CU = 256
ERR_HIP = 5


def _build(tmp, name, flags):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = os.path.join(tmp, name)
    cmd = [cxx, "-std=c++17", "-Wall", "-Wextra", "-Wno-unused-parameter", *flags, *INCLUDES, HARNESS, PLANNER, "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return exe


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    """Sanitized build: every out-of-bounds access, leak or undefined
    operation ends the run with a report."""
    tmp = str(tmp_path_factory.mktemp("planner"))
    return _build(tmp, "planner_asan", ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                                        "-fno-sanitize-recover=undefined"])


@pytest.fixture(scope="module")
def harness_fast(tmp_path_factory):
    """Optimised build without sanitizers (the library's host flags), for the
    planner's host time."""
    tmp = str(tmp_path_factory.mktemp("planner_fast"))
    return _build(tmp, "planner_o3", ["-O3"])


def readback_from_oracle(tables, lens, bs, cascade=True, seed=0):
    """Discovery read-back of a batch: the oracle's groups as device records
    (leader = smallest member), shuffled into an arbitrary record order."""
    exp = group(tables, lens, bs, cascade=cascade)
    G = len(exp["groups"])
    slot = np.random.default_rng(seed).permutation(G) if G else np.zeros(0, int)
    rec = np.zeros((G, 6), np.int64)
    for c, g in enumerate(exp["groups"]):
        rec[slot[c]] = (min(g["members"]), g["depth"], slot[g["parent"]] if g["parent"] >= 0 else -1,
                        g["block_begin"], g["block_end"], len(g["members"]))
    deep = np.array([slot[d] if d >= 0 else -1 for _, _, d in exp["requests"]], np.int64)
    sfx = np.array([sb for sb, _, _ in exp["requests"]], np.int64)
    return exp, rec, deep, sfx


def run_harness(exe, shape, W, flags, rec, lens, deep, sfx, tmp_path, repeats=1, tag="case"):
    path = tmp_path / f"{tag}.txt"
    B = len(lens)
    head = [B, W, shape.block_size, shape.num_q_heads, shape.num_kv_heads, shape.head_dim_qk, shape.head_dim_v,
            int(shape.v_aliases_k), flags, N_CU, repeats, len(rec)]
    with open(path, "w") as fh:
        fh.write(" ".join(map(str, head)) + "\n")
        for row in rec:
            fh.write(" ".join(map(str, row)) + "\n")
        for arr in (lens, deep, sfx):
            fh.write(" ".join(str(int(x)) for x in arr) + "\n")
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([exe, str(path)], capture_output=True, text=True, env=env, timeout=600)
    assert res.returncode == 0, f"{tag}: harness exited {res.returncode}\n{res.stderr[-4000:]}"
    assert "ERROR: AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr, res.stderr[-4000:]
    return parse(res.stdout, shape)


def parse(text, shape):
    out = {}
    for line in text.splitlines():
        key, _, rest = line.partition(" ")
        if key == "status":
            code, _, msg = rest.partition(" ")
            out["status"], out["message"] = int(code), msg
        elif key == "time_us":
            out["time_us"] = float(rest)
        else:
            out[key] = [int(x) for x in rest.split()]
    if out.get("status") != 0:
        return out
    names = ["request", "tok_begin", "tok_end", "kv_head", "member_off", "ncols", "col0", "col1", "part_base",
             "kv_heads", "stripes", "flags"]
    for k in ("grouped", "suffix"):
        v = out[k]
        n = v[0]
        out[k] = [dict(zip(names, v[1 + 12 * j : 13 + 12 * j])) for j in range(n)]
    g = out["groups"]
    members = out["members"][1:]
    groups = []
    for j in range(g[0]):
        depth, parent, b0, b1, mb, mc = g[1 + 6 * j : 7 + 6 * j]
        groups.append(dict(depth=depth, parent=parent, block_begin=b0, block_end=b1,
                           members=tuple(members[mb : mb + mc])))
    req = out["requests"][1:]
    B = len(req) // 3
    hq = shape.num_q_heads
    off, src = out["src_off"][1:], out["src"][1:]
    sources = [[src[off[i * hq + h] : off[i * hq + h + 1]] for h in range(hq)] for i in range(B)]
    info = dict(zip(["batch", "num_groups", "max_depth", "num_grouped_items", "num_suffix_items",
                     "num_merge_sources", "num_partial_rows", "logical_tokens", "unique_tokens",
                     "decode_workspace_bytes", "num_folded_groups"], out["info"]))
    out["export"] = dict(groups=groups, requests=[tuple(req[3 * i : 3 * i + 3]) for i in range(B)],
                         folded=out["folded"][1:])
    out["schedule"] = dict(grouped=out["grouped"], suffix=out["suffix"], sources=sources)
    out["info"] = info
    return out


def with_block_ids(groups, tables):
    return [dict(g, block_ids=tuple(int(x) for x in tables[g["members"][0]][g["block_begin"] : g["block_end"]]))
            for g in groups]


def check_plan(res, shape, tables, lens, exp, keep_groups, cascade):
    assert res["status"] == 0, res.get("message")
    ex, info = res["export"], res["info"]
    bs = shape.block_size
    assert with_block_ids(ex["groups"], tables) == exp["groups"]
    if keep_groups or not cascade:
        assert ex["requests"] == exp["requests"]
        assert sum(ex["folded"]) == 0
    assert info["logical_tokens"] == int(np.sum(lens, dtype=np.int64))
    kept = [g for g, f in zip(ex["groups"], ex["folded"]) if not f]
    assert info["unique_tokens"] == sum((g["block_end"] - g["block_begin"]) * bs for g in kept) + sum(
        r[1] for r in ex["requests"])
    assert info["num_merge_sources"] == sum(len(v) for row in res["schedule"]["sources"] for v in row)
    # the bound the fixed-stride merge table is sized by covers every (request, head)
    assert res["max_pair_sources"][0] >= max((len(v) for row in res["schedule"]["sources"] for v in row), default=0)
    assert info["decode_workspace_bytes"] >= info["num_partial_rows"] * (shape.head_dim_v * 4 + 8)
    bins, launches = res["bins"][1:], res["launches"][1:]
    assert bins[0] == 0 and all(a < b for a, b in zip(bins, bins[1:]))  # no empty bin
    assert bins[-1] == info["num_grouped_items"] + info["num_suffix_items"]
    assert sum(launches[1::3]) == len(bins) - 1
    check_schedule_data(shape, lens, info["num_partial_rows"], ex, res["schedule"])


MODES = {
    "keep_groups": KEEP_GROUPS,
    "default": 0,
    "separate_passes": KEEP_GROUPS | SEPARATE_PASSES,
    "non_cascade": DISABLE_CASCADE,
}


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("name", ["tiny", "llama3_8b", "long_rl", "forest_mixed", "mla"])
def test_planner_on_workloads(harness, tmp_path, name, mode):
    b = build_batch(CONFIGS[name])
    flags = MODES[mode]
    cascade = not flags & DISABLE_CASCADE
    exp, rec, deep, sfx = readback_from_oracle(b.block_tables, b.seq_lens, b.shape.block_size, cascade=cascade,
                                               seed=hash(name) % 1000)
    res = run_harness(harness, b.shape, b.max_blocks, flags, rec, b.seq_lens, deep, sfx, tmp_path, tag=name)
    check_plan(res, b.shape, b.block_tables, b.seq_lens, exp, keep_groups=bool(flags & KEEP_GROUPS), cascade=cascade)
    if name == "tiny" and mode == "default":
        assert res["export"]["folded"] == [1]  # the one group cannot pay: the cascade is bypassed


def test_planner_fuzz_forests(harness, tmp_path):
    rng = np.random.default_rng(4321)
    shapes = [AttnShape(8, 2, 128, 128, 16, 0.1), AttnShape(16, 1, 128, 128, 16, 0.1),
              AttnShape(12, 4, 128, 128, 16, 0.1), AttnShape(32, 1, 576, 512, 64, 0.05, v_aliases_k=True)]
    n = 0
    for B in [1, 2, 3, 7, 19, 64, 150]:
        for width in [1, 4, 40]:
            for alphabet in [1, 3, 40]:
                shape = shapes[n % len(shapes)]
                tables, lens = random_forest(rng, B, width, shape.block_size, alphabet)
                flags = [KEEP_GROUPS, 0, KEEP_GROUPS | SEPARATE_PASSES][n % 3]
                exp, rec, deep, sfx = readback_from_oracle(tables, lens, shape.block_size, seed=n)
                res = run_harness(harness, shape, width, flags, rec, lens, deep, sfx, tmp_path, tag=f"fuzz{n}")
                check_plan(res, shape, tables, lens, exp, keep_groups=bool(flags & KEEP_GROUPS), cascade=True)
                n += 1


def test_planner_deep_chain_and_8192_requests(harness, tmp_path):
    # caterpillar: request i shares i + 1 blocks with request i + 1, plus duplicates
    shape = AttnShape(4, 4, 128, 128, 16, 0.1)
    B, W = 40, 48
    t = np.arange(B * W, dtype=np.int32).reshape(B, W) + 1000
    for i in range(1, B):
        t[i, :i] = t[i - 1, :i]
    tables = np.concatenate([t, t[:5]])
    lens = np.full(len(tables), W * 16, np.int32)
    exp, rec, deep, sfx = readback_from_oracle(tables, lens, 16, seed=1)
    res = run_harness(harness, shape, W, KEEP_GROUPS, rec, lens, deep, sfx, tmp_path, tag="chain")
    check_plan(res, shape, tables, lens, exp, keep_groups=True, cascade=True)
    assert res["info"]["max_depth"] > 10
    # 8192 requests: 256 prompts of 64 blocks x 32 samples with 1-40 own blocks
    shape = AttnShape(32, 8, 128, 128, 16, 1 / math.sqrt(128))
    rng = np.random.default_rng(8)
    P, S, W = 256, 32, 104
    B = P * S
    tables = np.zeros((B, W), np.int32)
    lens = np.zeros(B, np.int32)
    nxt = 0
    for p_ in range(P):
        prefix = np.arange(nxt, nxt + 64)
        nxt += 64
        for s_ in range(S):
            i = p_ * S + s_
            own = int(rng.integers(1, 41))
            tables[i, :64] = prefix
            tables[i, 64 : 64 + own] = np.arange(nxt, nxt + own)
            nxt += own
            lens[i] = 64 * 16 + own * 16 - int(rng.integers(0, 16))
    perm = rng.permutation(B)
    tables, lens = tables[perm], lens[perm]
    exp, rec, deep, sfx = readback_from_oracle(tables, lens, 16, seed=2)
    for flags in (KEEP_GROUPS, 0):
        res = run_harness(harness, shape, W, flags, rec, lens, deep, sfx, tmp_path, tag=f"b8192_{flags}")
        check_plan(res, shape, tables, lens, exp, keep_groups=bool(flags & KEEP_GROUPS), cascade=True)


def test_planner_rejects_bad_readbacks(harness, tmp_path):
    """A read-back that is not a forest over the batch is an error, never an
    out-of-range access or a loop."""
    b = build_batch(CONFIGS["forest_mixed"])
    sh = b.shape
    exp, rec, deep, sfx = readback_from_oracle(b.block_tables, b.seq_lens, sh.block_size, seed=3)
    root = int(np.argmax(rec[:, 1] == 0))
    child = int(np.argmax(rec[:, 1] == 1))

    def bad(tag, rec_=None, lens_=None, deep_=None, sfx_=None):
        res = run_harness(harness, sh, b.max_blocks, KEEP_GROUPS, rec if rec_ is None else rec_,
                          b.seq_lens if lens_ is None else lens_, deep if deep_ is None else deep_,
                          sfx if sfx_ is None else sfx_, tmp_path, tag=tag)
        assert res["status"] == ERR_HIP, (tag, res.get("message"))

    r = rec.copy(); r[child, 2] = len(rec)  # parent past the records
    bad("parent_range", r)
    r = rec.copy(); r[root, 2] = child; r[root, 1] = 2  # a parent cycle
    bad("cycle", r)
    r = rec.copy(); r[child, 5] = 1  # a group of one
    bad("count", r)
    r = rec.copy(); r[child, 4] = b.max_blocks + 1  # range past the table
    bad("range", r)
    r = rec.copy(); r[child, 0] = len(b.seq_lens)  # leader past the batch
    bad("leader", r)
    r = rec.copy(); r[child, 5] += 1  # more members than the requests that end in it
    bad("members", r)
    d = deep.copy(); d[0] = len(rec)  # deepest group past the records
    bad("deepest", deep_=d)
    s = sfx.copy(); s[0] += 1  # suffix start not at its deepest group's end
    bad("suffix", sfx_=s)
    ln = b.seq_lens.copy(); ln[1] = -5
    bad("length", lens_=ln)


def test_planner_host_time(harness_fast, tmp_path):
    """Host time of the planner (optimised build, no sanitizers) for each
    workload, reported; the plan is made once per decode step for all
    layers."""
    for name in ["tiny", "llama3_8b", "long_rl", "forest_mixed", "mla"]:
        b = build_batch(CONFIGS[name])
        exp, rec, deep, sfx = readback_from_oracle(b.block_tables, b.seq_lens, b.shape.block_size)
        res = run_harness(harness_fast, b.shape, b.max_blocks, 0, rec, b.seq_lens, deep, sfx, tmp_path,
                          repeats=20, tag=f"time_{name}")
        assert res["status"] == 0
        print(f"[planner] {name}: {res['time_us']:.0f} us per plan (host), "
              f"{res['info']['num_grouped_items'] + res['info']['num_suffix_items']} items, "
              f"{res['info']['num_merge_sources']} merge sources")
