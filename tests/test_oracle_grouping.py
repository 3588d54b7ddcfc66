"""Pins of the oracle's prefix grouping: construction truth of every seeded
forest, a brute-force set definition on random tiny forests, invariances and
the worked examples of the PagedAttention vs. RadixAttention page.  CPU only."""

import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import accounting
from oracle.grouping import group
from workloads import CONFIGS, build_batch
from workloads.forest import CONFIG_ORDER


@pytest.mark.parametrize("name", CONFIG_ORDER)
def test_matches_construction(name):
    b = build_batch(CONFIGS[name])
    got = group(b.block_tables, b.seq_lens, b.shape.block_size)
    assert got == b.truth
    expected_groups = {"tiny": 1, "llama3_8b": 8, "long_rl": 16, "forest_mixed": 33, "mla": 4}[name]
    assert len(got["groups"]) == expected_groups


def brute_force_groups(tables, lens, bs):
    """S(i, l) = {k : nfull_k >= l, row_k[:l] == row_i[:l]}; groups are the
    distinct S with |S| >= 2, block range [min l - 1, max l)."""
    B = len(lens)
    nfull = [int(lens[i]) // bs for i in range(B)]
    sets = {}
    for i in range(B):
        for l in range(1, nfull[i] + 1):
            S = frozenset(
                k for k in range(B) if nfull[k] >= l and list(tables[k][:l]) == list(tables[i][:l])
            )
            if len(S) >= 2:
                lo, hi = sets.get(S, (l, l))
                sets[S] = (min(lo, l), max(hi, l))
    raw = [(S, lo - 1, hi) for S, (lo, hi) in sets.items()]

    def depth(S):
        return sum(1 for T, _, _ in raw if S < T)

    raw.sort(key=lambda x: (min(x[0]), depth(x[0])))
    out = []
    for S, b0, b1 in raw:
        supers = [j for j, (T, _, _) in enumerate(raw) if S < T]
        parent = min(supers, key=lambda j: len(raw[j][0])) if supers else -1
        first = min(S)
        out.append(
            dict(
                depth=depth(S),
                parent=parent,
                block_begin=b0,
                block_end=b1,
                members=tuple(sorted(S)),
                block_ids=tuple(int(x) for x in tables[first][b0:b1]),
            )
        )
    reqs = []
    for i in range(B):
        mine = [g for g in range(len(out)) if i in out[g]["members"]]
        if not mine:
            reqs.append((0, int(lens[i]), -1))
        else:
            d = max(mine, key=lambda g: out[g]["depth"])
            reqs.append((out[d]["block_end"], int(lens[i]) - bs * out[d]["block_end"], d))
    return dict(groups=out, requests=reqs)


@st.composite
def tiny_forest(draw):
    """Rows drawn from a tiny alphabet so that prefixes collide often, plus
    duplicates, short rows, garbage padding and reused IDs off the prefix."""
    bs = draw(st.sampled_from([1, 2, 4]))
    B = draw(st.integers(0, 9))
    width = draw(st.integers(1, 6))
    alphabet = draw(st.integers(1, 4))
    rows, lens = [], []
    for _ in range(B):
        if rows and draw(st.booleans()):
            base = list(rows[draw(st.integers(0, len(rows) - 1))])
            cut = draw(st.integers(0, width))
            tail = draw(st.lists(st.integers(0, alphabet), min_size=width - cut, max_size=width - cut))
            row = base[:cut] + tail
        else:
            row = draw(st.lists(st.integers(0, alphabet), min_size=width, max_size=width))
        rows.append(row)
        lens.append(draw(st.integers(0, width * bs)))
    tables = np.array(rows, dtype=np.int32).reshape(B, width)
    # garbage past each request's last block
    for i in range(B):
        nb = -(-lens[i] // bs)
        tables[i, nb:] = draw(st.integers(-5, 5))
    return tables, np.array(lens, dtype=np.int32), bs


@settings(max_examples=300, deadline=None)
@given(tiny_forest())
def test_brute_force_sets(f):
    tables, lens, bs = f
    assert group(tables, lens, bs) == brute_force_groups(tables, lens, bs)


@settings(max_examples=100, deadline=None)
@given(tiny_forest(), st.randoms(use_true_random=False))
def test_relabel_and_permutation(f, rnd):
    tables, lens, bs = f
    B = len(lens)
    base = group(tables, lens, bs)
    # relabel block IDs with a bijection
    ids = sorted(set(int(x) for x in tables.flatten()))
    new = list(range(100, 100 + len(ids)))
    rnd.shuffle(new)
    mp = dict(zip(ids, new))
    t2 = np.vectorize(lambda x: mp[int(x)])(tables).astype(np.int32) if B else tables
    g2 = group(t2, lens, bs)
    assert [(g["depth"], g["parent"], g["block_begin"], g["block_end"], g["members"]) for g in g2["groups"]] == [
        (g["depth"], g["parent"], g["block_begin"], g["block_end"], g["members"]) for g in base["groups"]
    ]
    assert all(tuple(mp[x] for x in a["block_ids"]) == b["block_ids"] for a, b in zip(base["groups"], g2["groups"]))
    assert g2["requests"] == base["requests"]
    # permuting requests permutes member sets and request rows
    p = list(range(B))
    rnd.shuffle(p)
    g3 = group(tables[p], lens[p], bs)
    inv = {old: new for new, old in enumerate(p)}
    sets_base = sorted(tuple(sorted(inv[m] for m in g["members"])) for g in base["groups"])
    sets_perm = sorted(g["members"] for g in g3["groups"])
    assert sets_base == sets_perm
    for new_i, old_i in enumerate(p):
        assert g3["requests"][new_i][:2] == base["requests"][old_i][:2]


def test_edge_cases():
    assert group(np.zeros((0, 3), np.int32), np.zeros(0, np.int32), 4) == dict(groups=[], requests=[])
    # identical rows and lengths: one group over the common full blocks
    t = np.array([[1, 2, 3], [1, 2, 3], [1, 2, 3]], np.int32)
    g = group(t, np.array([10, 10, 10]), 4)
    assert len(g["groups"]) == 1 and g["groups"][0]["block_end"] == 2
    assert g["requests"] == [(2, 2, 0)] * 3
    # only partial blocks: nothing shared
    g = group(t, np.array([3, 3, 0]), 4)
    assert g["groups"] == [] and g["requests"] == [(0, 3, -1), (0, 3, -1), (0, 0, -1)]
    # the same ID off the prefix is not sharing
    t = np.array([[5, 6], [6, 5]], np.int32)
    assert group(t, np.array([8, 8]), 4)["groups"] == []
    # cascade disabled: no groups, everything is suffix
    t = np.array([[1, 2], [1, 2]], np.int32)
    g = group(t, np.array([8, 7]), 4, cascade=False)
    assert g["groups"] == [] and g["requests"] == [(0, 8, -1), (0, 7, -1)]
    # nested three levels deep
    t = np.array([[1, 2, 3, 4], [1, 2, 3, 9], [1, 2, 8, 8], [1, 7, 7, 7]], np.int32)
    g = group(t, np.array([16, 16, 16, 16]), 4)
    assert [(x["depth"], x["block_begin"], x["block_end"], x["members"]) for x in g["groups"]] == [
        (0, 0, 1, (0, 1, 2, 3)),
        (1, 1, 2, (0, 1, 2)),
        (2, 2, 3, (0, 1)),
    ]
    assert [x["parent"] for x in g["groups"]] == [-1, 0, 1]


def test_golden_three_requests(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "radix_three_requests.json")))
    got = group(np.array(g["block_tables"], np.int32), np.array(g["seq_lens"]), g["block_size"])
    exp = g["expected"]
    assert [dict(x, members=list(x["members"]), block_ids=list(x["block_ids"])) for x in got["groups"]] == exp["groups"]
    assert [list(r) for r in got["requests"]] == exp["requests"]


def test_golden_1900_of_2000(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "radix_1900_of_2000.json")))
    bs = g["block_size"]
    a, b = g["cached_tokens"], g["prompt_tokens"]
    na, nb = -(-a // bs), -(-b // bs)
    shared = list(range(1000, 1000 + a // bs))
    row_a = shared + [1 + 5000]  # the cached request's partial block
    row_b = shared + list(range(6000, 6000 + nb - len(shared)))  # copy on divergence
    t = np.full((2, nb), -1, np.int32)
    t[0, :na] = row_a
    t[1, :nb] = row_b
    got = group(t, np.array([a, b]), bs)
    exp = g["expected"]
    assert len(got["groups"]) == 1
    assert got["groups"][0]["block_end"] - got["groups"][0]["block_begin"] == exp["shared_blocks"]
    assert [r[0] * bs for r in got["requests"]] == [exp["suffix_begin_token"]] * 2
    assert [r[1] for r in got["requests"]] == exp["suffix_tokens"]


def test_golden_bytes_per_token(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "kv_bytes_per_token.json")))
    got = accounting.kv_bytes_per_token(g["kv_heads"], g["head_dim"], g["head_dim"], g["elem_bytes"], layers=g["layers"])
    assert got == g["bytes_per_token"] == 128 * 1024


@pytest.mark.parametrize("name", CONFIG_ORDER)
def test_unique_and_logical_tokens(name):
    b = build_batch(CONFIGS[name])
    cfg = CONFIGS[name]
    bs = cfg.shape.block_size
    g = group(b.block_tables, b.seq_lens, bs)
    # every group's tokens once plus every request's own tokens
    exp_shared = 0

    def walk(n):
        nonlocal exp_shared
        exp_shared += n.prefix_tokens
        for c in n.children:
            walk(c)

    for t in cfg.trees:
        walk(t)
    assert accounting.unique_tokens(g, bs) == exp_shared + sum(r[1] for r in b.truth["requests"])
    assert accounting.logical_tokens(b.seq_lens) == int(b.seq_lens.sum())
