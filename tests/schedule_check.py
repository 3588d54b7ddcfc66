"""Exact-coverage check of a decode schedule (pure Python, no GPU): used on
plans exported from the library on the GPU and on plans the host planner
builds on the CPU."""

from __future__ import annotations

import numpy as np


def check_schedule_data(sh, seq_lens, nrows, ex, sc):
    """The schedule of a plan covers the work exactly: every (group or
    suffix, KV head, query row, token) is computed by one work item, every
    partial row is written once, and query head h of request i merges
    exactly the rows of its path's units for its own KV head and column,
    deepest group first, suffix last, each row read by one (request, head).

    ``ex``: the canonical export (groups, requests, folded); ``sc``: the
    schedule export (grouped / suffix items, per-request-head sources)."""
    r = sh.num_q_heads // sh.num_kv_heads
    hkv = sh.num_kv_heads
    bs = sh.block_size
    written = np.zeros(nrows, dtype=np.int64)
    row_info = {}  # row -> (unit key, kv head, column, tok_begin, tok_end, stripe, stripes)

    def record(it, key):
        # The item's waves are kv_heads heads x C column groups (2 above 32
        # rows) x S block stripes; stripe t of head h writes row
        # part_base + (t * kv_heads + h - kv_head) * w + n - col0.
        assert it["tok_begin"] < it["tok_end"]
        assert 0 <= it["col0"] < it["col1"] <= it["ncols"] and it["col1"] - it["col0"] <= 64
        assert it["kv_heads"] in (1, 2, 4, 8) and it["kv_head"] % it["kv_heads"] == 0
        w = it["col1"] - it["col0"]
        S = it["stripes"]
        assert S >= 1 and S & (S - 1) == 0 and it["kv_heads"] * S <= 8
        for t in range(S):
            for h in range(it["kv_head"], it["kv_head"] + it["kv_heads"]):
                for c in range(it["col0"], it["col1"]):
                    row = it["part_base"] + (t * it["kv_heads"] + h - it["kv_head"]) * w + (c - it["col0"])
                    assert 0 <= row < nrows
                    written[row] += 1
                    row_info[row] = (key, h, c, it["tok_begin"], it["tok_end"], t, S)

    # grouped items: unit key (member_off, ncols); the group is the one whose
    # member list holds the item's request and whose range and width match.
    spans_g = {}
    first_req = {}
    for it in sc["grouped"]:
        assert it["member_off"] >= 0
        key = ("g", it["member_off"], it["ncols"])
        first_req.setdefault(key, it["request"])
        assert first_req[key] == it["request"]
        record(it, key)
        for h in range(it["kv_head"], it["kv_head"] + it["kv_heads"]):
            for c in range(it["col0"], it["col1"]):
                spans_g.setdefault(key, {}).setdefault((h, c), []).append((it["tok_begin"], it["tok_end"]))
    kept = [k for k in range(len(ex["groups"])) if not ex["folded"][k]]
    group_key = {}
    for key, arr in spans_g.items():
        assert len(arr) == hkv * key[2]
        lo = min(s0 for v in arr.values() for s0, _ in v)
        hi = max(s1 for v in arr.values() for _, s1 in v)
        for v in arr.values():  # each (head, column) tiles the whole range once
            v = sorted(v)
            assert v[0][0] == lo and v[-1][1] == hi
            assert all(x1 == y0 for (_, x1), (y0, _) in zip(v, v[1:]))
        match = [k for k in kept
                 if (ex["groups"][k]["block_begin"] * bs, ex["groups"][k]["block_end"] * bs,
                     len(ex["groups"][k]["members"]) * r) == (lo, hi, key[2])
                 and first_req[key] in ex["groups"][k]["members"]]
        assert len(match) == 1
        group_key[match[0]] = key
    assert len(group_key) == len(kept)  # folded groups have no grouped work

    # suffix items: each request's suffix tokens once per (head, column)
    spans_s = {}
    for it in sc["suffix"]:
        assert it["member_off"] == -1 and 0 <= it["col0"] < it["col1"] <= r and it["ncols"] == r
        key = ("s", it["request"])
        record(it, key)
        for h in range(it["kv_head"], it["kv_head"] + it["kv_heads"]):
            for c in range(it["col0"], it["col1"]):
                spans_s.setdefault((it["request"], h, c), []).append((it["tok_begin"], it["tok_end"]))
    for i, (sb, st, _) in enumerate(ex["requests"]):
        for h, c in ((h, c) for h in range(hkv) for c in range(r)):
            v = sorted(spans_s.get((i, h, c), []))
            assert sum(e - s0 for s0, e in v) == st
            if st:
                assert v[0][0] == sb * bs and v[-1][1] == int(seq_lens[i])
                assert all(x1 == y0 for (_, x1), (y0, _) in zip(v, v[1:]))
    assert (written == 1).all()

    # merge sources
    seen = np.zeros(nrows, dtype=np.int64)
    for i, (sb, st, deepest) in enumerate(ex["requests"]):
        path = []
        g = deepest
        while g >= 0:
            path.append(group_key[g])
            g = ex["groups"][g]["parent"]
        if st:
            path.append(("s", i))
        for h in range(sh.num_q_heads):
            rows = sc["sources"][i][h]
            per_unit = {}
            for row in rows:
                seen[row] += 1
                key, kvh, col, t0, t1, t, S = row_info[row]
                assert kvh == h // r and col % r == h % r
                per_unit.setdefault(key, []).append((col, t0, t1, t, S))
            assert list(per_unit) == path  # deepest group first, suffix last
            for key, v in per_unit.items():
                assert len({x[0] for x in v}) == 1  # one column per unit
                pieces = {}
                for _, t0, t1, t, S in v:
                    pieces.setdefault((t0, t1, S), set()).add(t)
                assert all(len(ts) == S for (_, _, S), ts in pieces.items())  # every stripe of every piece
                spans = sorted((t0, t1) for t0, t1, _ in pieces)
                assert all(x1 == y0 for (_, x1), (y0, _) in zip(spans, spans[1:]))
    assert (seen == 1).all()
