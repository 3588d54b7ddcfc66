"""Pins of the fp64 attention oracle against brute force, closed forms and
invariants.  CPU only."""

import json
import math
import os

import numpy as np
import pytest

from oracle import attention as A
from workloads.values import f32_to_bf16_bits


class Shape:
    def __init__(self, hq, hkv, dqk, dv, bs, scale, alias=False):
        self.num_q_heads, self.num_kv_heads = hq, hkv
        self.head_dim_qk, self.head_dim_v = dqk, dv
        self.block_size, self.scale, self.v_aliases_k = bs, scale, alias


def rand_bits(rng, shape, sigma=1.0):
    return f32_to_bf16_bits((sigma * rng.standard_normal(shape)).astype(np.float32))


def make_paged(rng, shape, lens, extra_blocks=3, sigma=1.0):
    """Random pool + tables with distinct blocks per request."""
    bs = shape.block_size
    need = sum(-(-L // bs) for L in lens)
    nb = need + extra_blocks
    perm = rng.permutation(nb)
    maxb = max([-(-L // bs) for L in lens] + [1])
    tables = np.full((len(lens), maxb), -7, dtype=np.int32)
    c = 0
    for i, L in enumerate(lens):
        n = -(-L // bs)
        tables[i, :n] = perm[c : c + n]
        c += n
    k = rand_bits(rng, (nb, shape.num_kv_heads, shape.head_dim_qk // 8, bs, 8), sigma)
    v = None if shape.v_aliases_k else rand_bits(rng, (nb, shape.num_kv_heads, shape.head_dim_v, bs), sigma)
    q = rand_bits(rng, (len(lens), shape.num_q_heads, shape.head_dim_qk), sigma)
    return q, k, v, tables


def brute_force(q_bits, k_pool, v_pool, table, L, shape):
    """Pure-Python loops: exp without max subtraction, math.fsum sums."""
    bs = shape.block_size
    r = shape.num_q_heads // shape.num_kv_heads
    w16 = lambda b: float(A.widen_bf16(np.uint16(b)))
    out, lse = [], []
    for h in range(shape.num_q_heads):
        kvh = h // r
        scores = []
        vals = []
        for t in range(L):
            blk, off = int(table[t // bs]), t % bs
            krow = [w16(k_pool[blk, kvh, d // 8, off, d % 8]) for d in range(shape.head_dim_qk)]
            if shape.v_aliases_k:
                vrow = krow[: shape.head_dim_v]
            else:
                vrow = [w16(v_pool[blk, kvh, d, off]) for d in range(shape.head_dim_v)]
            qrow = [w16(q_bits[h, d]) for d in range(shape.head_dim_qk)]
            scores.append(shape.scale * math.fsum(a * b for a, b in zip(qrow, krow)))
            vals.append(vrow)
        e = [math.exp(s) for s in scores]
        den = math.fsum(e)
        out.append([math.fsum(e[t] * vals[t][d] for t in range(L)) / den for d in range(shape.head_dim_v)])
        lse.append(math.log(den))
    return np.array(out), np.array(lse)


@pytest.mark.parametrize(
    "shape,lens",
    [
        (Shape(4, 2, 16, 16, 4, 0.25), [1, 5, 17, 40]),
        (Shape(2, 1, 24, 16, 8, 1 / math.sqrt(24), alias=True), [3, 8, 33]),
        (Shape(6, 3, 8, 16, 2, 0.3), [2, 7]),
    ],
)
def test_brute_force_tiny(shape, lens):
    rng = np.random.default_rng(11)
    q, k, v, tables = make_paged(rng, shape, lens, sigma=0.5)
    out, lse = A.attend(q, k, v, tables, np.array(lens), shape)
    for i, L in enumerate(lens):
        bo, bl = brute_force(q[i], k, v, tables[i], L, shape)
        np.testing.assert_allclose(out[i], bo, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[i], bl, rtol=1e-12, atol=1e-13)


def test_layout_pin_coded_values():
    """Keys: (blk, h, t, d) at [blk, h, d//8, t, d%8]; values at [blk, h, d, t]."""
    nb, hkv, dqk, dv, bs = 5, 2, 16, 8, 4
    code = np.arange(nb * hkv * dqk * bs, dtype=np.uint16).reshape(nb, hkv, dqk // 8, bs, 8)
    vcode = (np.arange(nb * hkv * dv * bs) + 20000).astype(np.uint16).reshape(nb, hkv, dv, bs)
    table = np.array([3, 0, 4], dtype=np.int32)
    L = 10
    K, V = A.gather_kv(code, vcode, table, L, bs, dv, False)
    # Undo the widening of the raw codes to compare integers.
    Kb = (K.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    Vb = (V.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    for t in range(L):
        blk, off = table[t // bs], t % bs
        for h in range(hkv):
            for d in range(dqk):
                assert Kb[t, h, d] == code[blk, h, d // 8, off, d % 8]
            for d in range(dv):
                assert Vb[t, h, d] == vcode[blk, h, d, off]
    Ka, Va = A.gather_kv(code, None, table, L, bs, dv, True)
    np.testing.assert_array_equal(Va, Ka[:, :, :dv])


def test_golden_60_tokens_block_count(golden_dir):
    """Only ceil(60 / bs) table entries are read; tail slots are excluded."""
    g = json.load(open(os.path.join(golden_dir, "paged_60_tokens.json")))
    L = g["tokens"]
    for case in g["cases"]:
        bs = case["block_size"]
        nblocks = case["blocks"]
        shape = Shape(2, 1, 8, 8, bs, 0.5)
        rng = np.random.default_rng(bs)
        k = rand_bits(rng, (nblocks, 1, 1, bs, 8))
        v = rand_bits(rng, (nblocks, 1, 8, bs))
        tail = case["tokens_in_last_block"]
        k[nblocks - 1, :, :, tail:, :] = 0x7FC0  # NaN past the last token
        v[nblocks - 1, :, :, tail:] = 0x7FC0
        # entries past the used blocks point outside the pool
        table = np.array(list(range(nblocks)) + [10**6, -1], dtype=np.int32)
        K, V = A.gather_kv(k, v, table, L, bs, 8, False)
        assert K.shape[0] == L and V.shape[0] == L
        assert case["full_blocks"] == L // bs
        q = rand_bits(rng, (1, 2, 8))
        out, lse = A.attend(q, k, v, table[None], np.array([L]), shape)
        assert np.isfinite(out).all() and np.isfinite(lse).all()


def _one(shape, q, K, V):
    return A.attend_one(q, K, V, shape.scale, shape.num_kv_heads)


def test_closed_forms():
    rng = np.random.default_rng(3)
    D, L = 16, 9
    sh = Shape(2, 1, D, D, 4, 0.7)
    V = rng.standard_normal((L, 1, D))
    q = rng.standard_normal((2, D))
    # identical keys -> uniform weights -> mean of V
    K = np.repeat(rng.standard_normal((1, 1, D)), L, axis=0)
    o, _ = _one(sh, q, K, V)
    np.testing.assert_allclose(o[0], V[:, 0].mean(0), rtol=1e-12, atol=1e-14)
    # q = 0 -> mean of V, lse = ln L
    K = rng.standard_normal((L, 1, D))
    o, lse = _one(sh, np.zeros((2, D)), K, V)
    np.testing.assert_allclose(o[1], V[:, 0].mean(0), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, math.log(L), rtol=1e-14)
    # constant value rows -> that constant
    c = rng.standard_normal(D)
    o, _ = _one(sh, q, K, np.broadcast_to(c, (L, 1, D)).copy())
    np.testing.assert_allclose(o, np.stack([c, c]), rtol=1e-12)
    # L = 1 -> v_0, lse = s_0
    o, lse = _one(sh, q, K[:1], V[:1])
    np.testing.assert_allclose(o[0], V[0, 0], rtol=1e-14)
    np.testing.assert_allclose(lse[0], sh.scale * K[0, 0] @ q[0], rtol=1e-13)
    # L = 2 with q = a e0, k0 = e0, k1 = -e0: o = sig(2 a s) v0 + sig(-2 a s) v1
    a = 1.3
    qq = np.zeros((2, D))
    qq[:, 0] = a
    K2 = np.zeros((2, 1, D))
    K2[0, 0, 0], K2[1, 0, 0] = 1.0, -1.0
    o, lse = _one(sh, qq, K2, V[:2])
    sig = 1.0 / (1.0 + math.exp(-2 * a * sh.scale))
    np.testing.assert_allclose(o[0], sig * V[0, 0] + (1 - sig) * V[1, 0], rtol=1e-13)
    np.testing.assert_allclose(lse[0], math.log(math.exp(a * sh.scale) + math.exp(-a * sh.scale)), rtol=1e-13)
    # one-hot values, scores scale * t -> o_t = softmax weights
    Lh = 6
    Kt = np.zeros((Lh, 1, D))
    Kt[:, 0, 1] = np.arange(Lh)
    q1 = np.zeros((2, D))
    q1[:, 1] = 1.0
    Vh = np.zeros((Lh, 1, D))
    Vh[np.arange(Lh), 0, np.arange(Lh)] = 1.0
    o, lse = _one(sh, q1, Kt, Vh)
    w = np.exp(sh.scale * np.arange(Lh))
    np.testing.assert_allclose(o[0, :Lh], w / w.sum(), rtol=1e-13)
    np.testing.assert_allclose(o[0, Lh:], 0.0)
    np.testing.assert_allclose(lse[0], math.log(w.sum()), rtol=1e-13)
    # L = 0 -> zeros, -inf
    o, lse = _one(sh, q, K[:0], V[:0])
    assert (o == 0).all() and np.isneginf(lse).all()


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_split_merge_equals_full(seed):
    """Any partition of the tokens (empty parts allowed), merged, is full attention."""
    rng = np.random.default_rng(seed)
    L, D, Dv, n = int(rng.integers(1, 200)), 16, 12, 3
    q = rng.standard_normal((n, D))
    K = 2.0 * rng.standard_normal((L, D))
    V = rng.standard_normal((L, Dv))
    full, full_lse = A.merge([A.partial(q, K, V, 0.4)])
    # direct definition
    s = 0.4 * q @ K.T
    w = np.exp(s - s.max(1, keepdims=True))
    np.testing.assert_allclose(full, (w @ V) / w.sum(1, keepdims=True), rtol=1e-12)
    parts = int(rng.integers(1, 8))
    label = rng.integers(0, parts + 1, size=L)  # part `parts` may be empty or not
    pieces = [A.partial(q, K[label == p], V[label == p], 0.4) for p in range(parts + 2)]  # last is empty
    out, lse = A.merge(pieces)
    np.testing.assert_allclose(out, full, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, full_lse, rtol=1e-12)
    # prefix/suffix split at a block boundary = cascade with one member
    cut = int(rng.integers(0, L + 1))
    out2, _ = A.merge([A.partial(q, K[:cut], V[:cut], 0.4), A.partial(q, K[cut:], V[cut:], 0.4)])
    np.testing.assert_allclose(out2, full, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("seed", [0, 1])
def test_merge_states_of_split_is_full(seed):
    """States (normalised output, natural lse) of disjoint key sets, merged,
    are attention over their union, checked against the direct definition;
    a state without keys (lse = -inf, its output arbitrary) weighs nothing."""
    rng = np.random.default_rng(10 + seed)
    L, D, Dv, n = int(rng.integers(2, 150)), 8, 6, 4
    q = rng.standard_normal((n, D))
    K = 3.0 * rng.standard_normal((L, D))
    V = rng.standard_normal((L, Dv))
    s = 0.5 * q @ K.T
    w = np.exp(s - s.max(1, keepdims=True))
    ref = (w @ V) / w.sum(1, keepdims=True)
    ref_lse = s.max(1) + np.log(w.sum(1))
    cuts = np.sort(rng.integers(0, L + 1, size=2))
    outs, lses = [], []
    for a, b in [(0, cuts[0]), (cuts[0], cuts[1]), (cuts[1], L)]:
        if a == b:
            outs.append(np.full((n, Dv), 7.0))  # no keys: must not leak in
            lses.append(np.full(n, -np.inf))
            continue
        sa = 0.5 * q @ K[a:b].T
        wa = np.exp(sa - sa.max(1, keepdims=True))
        outs.append((wa @ V[a:b]) / wa.sum(1, keepdims=True))
        lses.append(sa.max(1) + np.log(wa.sum(1)))
    outs.append(np.full((n, Dv), 3.0))
    lses.append(np.full(n, -np.inf))
    out, lse = A.merge_states(outs, lses)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12)
    # one state is itself; only empty states give zeros and -inf
    o1, l1 = A.merge_states([ref], [ref_lse])
    np.testing.assert_allclose(o1, ref, rtol=1e-14)
    np.testing.assert_allclose(l1, ref_lse, rtol=1e-14)
    o0, l0 = A.merge_states([outs[-1]], [lses[-1]])
    assert (o0 == 0).all() and np.isneginf(l0).all()


def test_all_empty_merge():
    e = A.partial(np.ones((2, 4)), np.zeros((0, 4)), np.zeros((0, 3)), 1.0)
    out, lse = A.merge([e, e])
    assert (out == 0).all() and np.isneginf(lse).all()


def test_invariants_paged():
    rng = np.random.default_rng(5)
    sh = Shape(8, 2, 16, 16, 4, 0.25)
    lens = [13, 16, 1, 30, 0]
    q, k, v, tables = make_paged(rng, sh, lens)
    out, lse = A.attend(q, k, v, tables, np.array(lens), sh)
    # block order within a table: permute full blocks, keep a partial last block last
    t2 = tables.copy()
    for i, L in enumerate(lens):
        nfull = L // sh.block_size
        t2[i, :nfull] = t2[i, rng.permutation(nfull)]
    o2, l2 = A.attend(q, k, v, t2, np.array(lens), sh)
    np.testing.assert_allclose(o2, out, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l2, lse, rtol=1e-12)
    # physical relabelling (data moves with its label)
    pi = rng.permutation(k.shape[0])
    k3 = np.empty_like(k)
    v3 = np.empty_like(v)
    k3[pi] = k
    v3[pi] = v
    t3 = np.where(tables >= 0, pi[np.clip(tables, 0, None)], tables).astype(np.int32)
    o3, _ = A.attend(q, k3, v3, t3, np.array(lens), sh)
    np.testing.assert_allclose(o3, out, rtol=1e-12, atol=1e-14)
    # request permutation -> permuted rows
    p = rng.permutation(len(lens))
    o4, _ = A.attend(q[p], k, v, tables[p], np.array(lens)[p], sh)
    np.testing.assert_allclose(o4, out[p], rtol=1e-12, atol=1e-14)
    # empty request
    assert (out[4] == 0).all() and np.isneginf(lse[4]).all()


def test_gqa_equals_replicated_mha():
    """Query head h reads KV head h // (Hq/Hkv): replicating KV heads gives MHA."""
    rng = np.random.default_rng(8)
    g = Shape(6, 2, 16, 8, 4, 0.3)
    m = Shape(6, 6, 16, 8, 4, 0.3)
    lens = [9, 21]
    q, k, v, tables = make_paged(rng, g, lens)
    rep = np.arange(6) // 3
    out_g, lse_g = A.attend(q, k, v, tables, np.array(lens), g)
    out_m, lse_m = A.attend(q, k[:, rep], v[:, rep], tables, np.array(lens), m)
    np.testing.assert_allclose(out_g, out_m, rtol=1e-13)
    np.testing.assert_allclose(lse_g, lse_m, rtol=1e-13)
    # the other plausible mapping (h % Hkv) differs on this input
    rep_bad = np.arange(6) % 2
    out_b, _ = A.attend(q, k[:, rep_bad], v[:, rep_bad], tables, np.array(lens), m)
    assert np.abs(out_b - out_g).max() > 1e-3


def test_planted_mistakes_are_caught(monkeypatch):
    """Plausible slips in the oracle fail at least one pin."""
    rng = np.random.default_rng(21)
    sh = Shape(4, 2, 16, 16, 4, 0.25)
    lens = [5, 17]
    q, k, v, tables = make_paged(rng, sh, lens, sigma=0.5)
    good = A.attend_one

    def no_scale(qh, K, V, scale, hkv):
        return good(qh, K, V, 1.0, hkv)

    def wrong_head(qh, K, V, scale, hkv):
        # query head h reads KV head h % Hkv instead of h // (Hq / Hkv)
        o = np.zeros((qh.shape[0], V.shape[2]))
        l = np.zeros(qh.shape[0])
        for h in range(qh.shape[0]):
            s = scale * (K[:, h % hkv, :] @ qh[h])
            w = np.exp(s - s.max())
            o[h] = (w @ V[:, h % hkv, :]) / w.sum()
            l[h] = s.max() + np.log(w.sum())
        return o, l

    def sign_flip(qh, K, V, scale, hkv):
        return good(-qh, K, V, scale, hkv)

    def drop_last_token(qh, K, V, scale, hkv):
        return good(qh, K[:-1], V[:-1], scale, hkv)

    for mutant in (no_scale, wrong_head, sign_flip, drop_last_token):
        monkeypatch.setattr(A, "attend_one", mutant)
        caught = False
        for i, L in enumerate(lens):
            out, lse = A.attend(q, k, v, tables, np.array(lens), sh)
            bo, bl = brute_force(q[i], k, v, tables[i], L, sh)
            if not (np.allclose(out[i], bo, rtol=1e-9) and np.allclose(lse[i], bl, rtol=1e-9)):
                caught = True
        monkeypatch.setattr(A, "attend_one", good)
        assert caught, mutant.__name__
