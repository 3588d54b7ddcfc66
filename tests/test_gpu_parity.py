"""GPU parity: plans (bit-exact) and decode outputs (tolerance) of libfca
against the CPU oracle, through the C ABI.  Needs an MI355X."""

from __future__ import annotations

import math
import sys

import numpy as np
import pytest

from oracle import attention as A
from oracle.grouping import group
from tests.forests import random_forest
from tests.schedule_check import check_schedule_data
from tests.helpers import (
    assert_close,
    assert_close_f32,
    assert_lse_close,
    bf16_tensor_to_f64,
    host_values,
    oracle_all,
    to_device_bf16,
)
from workloads import CONFIGS, build_batch, fill_values_numpy
from workloads.forest import AttnShape, Config, Node
from workloads.values import BF16_NAN, fill_values_torch, f32_to_bf16_bits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import shared_prefix_kv_amd as fca  # noqa: E402

GQA_CONFIGS = ["tiny", "llama3_8b", "long_rl", "forest_mixed"]
PLAN_CONFIGS = GQA_CONFIGS + ["mla"]


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fca.lib()


def dev_tables(batch):
    return (
        torch.from_numpy(batch.block_tables).cuda(),
        torch.from_numpy(batch.seq_lens).cuda(),
    )


def plan_for(batch, cascade=True, auto_fold=False):
    """Plan of a batch; by default every discovered group is kept, so that
    the export is the discovery itself."""
    bt, sl = dev_tables(batch)
    desc = fca.desc_from_shape(batch.shape, batch.num_blocks, cascade=cascade, auto_fold=auto_fold)
    return fca.fca_plan(bt, sl, desc)


def with_block_ids(exported, tables):
    groups = []
    for g in exported["groups"]:
        first = g["members"][0]
        groups.append(dict(g, block_ids=tuple(int(x) for x in tables[first][g["block_begin"] : g["block_end"]])))
    return dict(groups=groups, requests=exported["requests"])


# ---------------------------------------------------------------- plans ----


@pytest.mark.parametrize("name", PLAN_CONFIGS)
def test_plan_matches_oracle(name):
    b = build_batch(CONFIGS[name])
    say("plan", name, "B", b.batch)
    p = plan_for(b)
    got = with_block_ids(p.export(), b.block_tables)
    assert got == group(b.block_tables, b.seq_lens, b.shape.block_size)
    assert p.info.unique_tokens == sum((g["block_end"] - g["block_begin"]) * b.shape.block_size for g in got["groups"]) + sum(r[1] for r in got["requests"])
    pn = plan_for(b, cascade=False)
    assert with_block_ids(pn.export(), b.block_tables) == group(b.block_tables, b.seq_lens, b.shape.block_size, cascade=False)


def test_plan_fuzz_forests():
    rng = np.random.default_rng(1234)
    shape = AttnShape(8, 2, 128, 128, 16, 0.1)
    cases = 0
    for B in [1, 2, 3, 5, 8, 17, 40, 100, 300]:
        for width in [1, 3, 8, 70]:
            for alphabet in [1, 2, 3, 50]:
                tables, lens = random_forest(rng, B, width, 16, alphabet)
                desc = fca.desc_from_shape(shape, 64, auto_fold=False)
                p = fca.fca_plan(torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda(), desc)
                got = with_block_ids(p.export(), tables)
                exp = group(tables, lens, 16)
                assert got == exp, (B, width, alphabet)
                cases += 1
    say("fuzz plans", cases)


def test_plan_deep_chain_and_duplicates():
    # caterpillar: request i shares i+1 blocks with request i+1
    B, W = 40, 48
    t = np.arange(B * W, dtype=np.int32).reshape(B, W) + 1000
    for i in range(1, B):
        t[i, :i] = t[i - 1, :i]
    lens = np.full(B, W * 16, np.int32)
    tables = np.concatenate([t, t[:5]])  # plus exact duplicates
    lens = np.concatenate([lens, lens[:5]])
    desc = fca.desc_from_shape(AttnShape(4, 4, 128, 128, 16, 0.1), 10**6, auto_fold=False)
    p = fca.fca_plan(torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda(), desc)
    assert with_block_ids(p.export(), tables) == group(tables, lens, 16)
    assert p.info.max_depth > 10


def test_plan_copies_tables_and_bad_tables():
    b = build_batch(CONFIGS["tiny"])
    bt, sl = dev_tables(b)
    desc = fca.desc_from_shape(b.shape, b.num_blocks)
    p = fca.fca_plan(bt, sl, desc)
    before = with_block_ids(p.export(), b.block_tables)
    bt.fill_(0)
    sl.fill_(0)
    torch.cuda.synchronize()
    assert with_block_ids(p.export(), b.block_tables) == before
    # block ID outside the pool in a used slot
    bad = b.block_tables.copy()
    bad[3, 1] = b.num_blocks
    with pytest.raises(fca.FcaError) as e:
        fca.fca_plan(torch.from_numpy(bad).cuda(), torch.from_numpy(b.seq_lens).cuda(), desc)
    assert e.value.status == 4 and "request 3" in str(e.value)
    bad[3, 1] = -1
    with pytest.raises(fca.FcaError):
        fca.fca_plan(torch.from_numpy(bad).cuda(), torch.from_numpy(b.seq_lens).cuda(), desc)
    # seq_len longer than the table can hold
    lens = b.seq_lens.copy()
    lens[5] = b.max_blocks * 16 + 1
    with pytest.raises(fca.FcaError) as e:
        fca.fca_plan(torch.from_numpy(b.block_tables).cuda(), torch.from_numpy(lens).cuda(), desc)
    assert e.value.status == 4
    # an out-of-pool ID past the last used block is fine (padding)
    ok = b.block_tables.copy()
    ok[0, -1] = 10**9
    if b.seq_lens[0] <= (b.max_blocks - 1) * 16:
        fca.fca_plan(torch.from_numpy(ok).cuda(), torch.from_numpy(b.seq_lens).cuda(), desc)


@pytest.mark.parametrize("name", PLAN_CONFIGS)
def test_schedule_covers_each_token_once(name):
    """Every (group or suffix, KV head, query row, token) is computed by
    exactly one work item, every partial row is written once, and query head
    h of request i merges exactly the rows of its path's units for its own KV
    head and column, each row read by one (request, head)."""
    b = build_batch(CONFIGS[name])
    check_schedule(b, plan_for(b))


def check_schedule(b, p):
    check_schedule_data(b.shape, b.seq_lens, p.info.num_partial_rows, p.export(), p.export_schedule())


# --------------------------------------------------------------- decode ----


def run_decode(batch, vals, cascade=True, lse=True, separate=False, out_f32=False, auto_fold=True):
    bt, sl = dev_tables(batch)
    desc = fca.desc_from_shape(batch.shape, batch.num_blocks, cascade=cascade, separate_passes=separate, out_f32=out_f32,
                               auto_fold=auto_fold)
    p = fca.fca_plan(bt, sl, desc)
    dt = torch.float32 if out_f32 else torch.bfloat16
    out = torch.empty((batch.batch, batch.shape.num_q_heads, batch.shape.head_dim_v), dtype=dt, device="cuda")
    l = torch.empty((batch.batch, batch.shape.num_q_heads), dtype=torch.float32, device="cuda") if lse else None
    fca.fca_decode(vals["q"], vals["k"], vals["v"], p, out=out, lse=l)
    torch.cuda.synchronize()
    return p, out, l


# (cascade, activation heuristic): every group kept, the library's default
# (groups that cannot pay are read per request), no cascade
MODES = ((True, False), (True, True), (False, True))


def upload(vals_np):
    return {k: (to_device_bf16(v) if v is not None else None) for k, v in vals_np.items()}


@pytest.mark.parametrize("cascade,fold", MODES)
def test_decode_tiny_full(cascade, fold):
    b = build_batch(CONFIGS["tiny"])
    vn = fill_values_numpy(b, poison=True)
    say("decode tiny cascade", cascade, "fold", fold)
    ref, ref_lse = A.attend(vn["q"], vn["k"], vn["v"], b.block_tables, b.seq_lens, b.shape)
    _, out, lse = run_decode(b, upload(vn), cascade=cascade, auto_fold=fold)
    rep = assert_close(bf16_tensor_to_f64(out), ref, f"tiny cascade={cascade}")
    assert_lse_close(lse.cpu().numpy(), ref_lse, "tiny")
    say("tiny", rep)


def test_decode_llama3_8b_full():
    b = build_batch(CONFIGS["llama3_8b"])
    vn = fill_values_numpy(b, poison=True)
    say("decode llama3_8b (all 64 requests vs oracle)")
    ref, ref_lse = A.attend(vn["q"], vn["k"], vn["v"], b.block_tables, b.seq_lens, b.shape)
    vals = upload(vn)
    p, out, lse = run_decode(b, vals)
    rep = assert_close(bf16_tensor_to_f64(out), ref, "llama3_8b")
    assert_lse_close(lse.cpu().numpy(), ref_lse, "llama3_8b")
    say("llama3_8b cascade", rep, "groups", p.info.num_groups)
    _, out_nc, _ = run_decode(b, vals, cascade=False)
    rep2 = assert_close(bf16_tensor_to_f64(out_nc), ref, "llama3_8b non-cascade")
    say("llama3_8b non-cascade", rep2)
    # bitwise determinism of one plan
    _, out2, lse2 = run_decode(b, vals)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    # the passes launched one after the other (their own token splits)
    _, out3, lse3 = run_decode(b, vals, separate=True)
    rep3 = assert_close(bf16_tensor_to_f64(out3), ref, "llama3_8b separate passes")
    assert_lse_close(lse3.cpu().numpy(), ref_lse, "llama3_8b separate passes")
    say("llama3_8b separate passes", rep3)


@pytest.mark.parametrize("name", ["long_rl", "forest_mixed", "mla"])
def test_decode_full_size_every_request(name):
    """Every request of the full-size workload against the oracle, with the
    cascade, without it (the non-cascade baseline the speedups are quoted
    against) and with float32 output (held to max |err| <= 2e-3).  The
    oracle reads host copies of the inputs taken before any decode, and the
    device inputs are checked unchanged afterwards."""
    b = build_batch(CONFIGS[name])
    say("decode", name, "full size: every request vs the oracle, B", b.batch)
    vals = fill_values_torch(b, "cuda", seed=CONFIGS[name].seed, poison=True)
    host = host_values(vals)
    keep = {k: v.clone() for k, v in vals.items() if v is not None}
    ref, ref_lse = oracle_all(b, host, say=say)
    for cascade in (True, False):
        p, out, lse = run_decode(b, vals, cascade=cascade)
        rep = assert_close(bf16_tensor_to_f64(out), ref, f"{name} cascade={cascade}")
        assert_lse_close(lse.cpu().numpy(), ref_lse, f"{name} cascade={cascade}")
        say(name, "cascade" if cascade else "non-cascade", rep, "groups", p.info.num_groups,
            "items", p.info.num_grouped_items, p.info.num_suffix_items)
        del out, lse
    p, out, lse = run_decode(b, vals, out_f32=True)
    rep = assert_close_f32(out.cpu().numpy().astype(np.float64), ref, f"{name} float32 output")
    assert_lse_close(lse.cpu().numpy(), ref_lse, f"{name} float32 output")
    say(name, "float32 output", rep)
    for k, v in keep.items():
        assert torch.equal(vals[k].view(torch.int16), v.view(torch.int16)), f"{name}: decode changed input {k}"
    del vals, keep, out, lse
    torch.cuda.empty_cache()


def small_case(shape, tables, lens, num_blocks, seed=0):
    rng = np.random.default_rng(seed)
    k = f32_to_bf16_bits(rng.standard_normal((num_blocks, shape.num_kv_heads, shape.head_dim_qk // 8, shape.block_size, 8), dtype=np.float32))
    v = f32_to_bf16_bits(rng.standard_normal((num_blocks, shape.num_kv_heads, shape.head_dim_v, shape.block_size), dtype=np.float32))
    q = f32_to_bf16_bits(rng.standard_normal((len(lens), shape.num_q_heads, shape.head_dim_qk), dtype=np.float32))
    bs = shape.block_size
    used = np.zeros(num_blocks, bool)
    for i, L in enumerate(lens):
        nb = -(-int(L) // bs)
        used[tables[i, :nb]] = True
        if L % bs:
            blk = tables[i, L // bs]
            k[blk, :, :, L % bs :, :] = BF16_NAN
            v[blk, :, :, L % bs :] = BF16_NAN
    k[~used] = BF16_NAN
    v[~used] = BF16_NAN
    return dict(q=q, k=k, v=v)


class _B:
    def __init__(self, shape, tables, lens, num_blocks):
        self.shape, self.block_tables, self.seq_lens, self.num_blocks = shape, tables, lens, num_blocks
        self.batch = len(lens)


@pytest.mark.parametrize("hq,hkv", [(8, 8), (8, 4), (16, 2), (16, 1), (12, 4)])
def test_decode_edge_lengths_and_ratios(hq, hkv):
    """Lengths 0, 1, block and tile boundaries, nested sharing, duplicates."""
    shape = AttnShape(hq, hkv, 128, 128, 16, 1 / math.sqrt(128))
    lens = np.array([0, 1, 15, 16, 17, 31, 32, 33, 47, 48, 200, 513, 513, 530, 700, 64], np.int32)
    W = 48
    B = len(lens)
    nb = 4096
    rng = np.random.default_rng(hq * 100 + hkv)
    perm = rng.permutation(nb)
    tables = perm[: B * W].reshape(B, W).astype(np.int32)
    # requests 10..15 share 12 blocks; 11..13 share 32 blocks; 11 and 12 identical
    tables[11:16, :12] = tables[10, :12]
    tables[12:14, :32] = tables[11, :32]
    tables[12] = tables[11]
    tables[15, :4] = tables[10, :4]
    case = small_case(shape, tables, lens, nb, seed=hq + hkv)
    ref, ref_lse = A.attend(case["q"], case["k"], case["v"], tables, lens, shape)
    b = _B(shape, tables, lens, nb)
    vals = upload(case)
    for cascade, fold in MODES:
        p, out, lse = run_decode(b, vals, cascade=cascade, auto_fold=fold)
        assert_close(bf16_tensor_to_f64(out), ref, f"edge hq={hq} hkv={hkv} cascade={cascade} fold={fold}")
        assert_lse_close(lse.cpu().numpy(), ref_lse, "edge")
        o = bf16_tensor_to_f64(out)
        assert (o[0] == 0).all() and np.isneginf(lse[0].cpu().numpy()).all()
    say("edge", hq, hkv, "groups", p.info.num_groups)


@pytest.mark.parametrize("kind", ["gqa", "mla"])
def test_decode_short_requests_precision(kind):
    """Requests of 2 to 9 tokens: the output is a weighted mean of a few
    value rows, so rounding the probabilities alone to bf16 (8 bits) would
    leave errors above the tolerance wherever the rows cancel.  The GQA
    kernel applies each probability to about 16 bits (two bf16 operands);
    the latent kernel rounds it to fp16 (11 bits) and multiplies fp16 copies
    of the value rows (exact below 65504).  Both must stay within the
    tolerance on every element."""
    if kind == "gqa":
        shape = AttnShape(32, 8, 128, 128, 16, 1 / math.sqrt(128))
    else:
        shape = AttnShape(16, 1, 576, 512, 64, 1 / math.sqrt(576), v_aliases_k=True)
    B, W, nb = 96, 1, 128
    rng = np.random.default_rng(77)
    lens = rng.integers(2, 10, size=B).astype(np.int32)
    tables = rng.permutation(nb)[:B].reshape(B, W).astype(np.int32)
    tables[1::4] = tables[0::4]  # pairs that share their only (partial) block
    lens[1::4] = lens[0::4]
    case = small_case(shape, tables, lens, nb, seed=78)
    ref, ref_lse = A.attend(case["q"], case["k"], case["v"], tables, lens, shape)
    vals = upload(case)
    for cascade, fold in MODES:
        say("short requests", kind, "cascade", cascade, "fold", fold)
        _, out, lse = run_decode(_B(shape, tables, lens, nb), vals, cascade=cascade, auto_fold=fold)
        rep = assert_close(bf16_tensor_to_f64(out), ref, f"short requests {kind} cascade={cascade} fold={fold}")
        assert_lse_close(lse.cpu().numpy(), ref_lse, "short requests")
        say("short", kind, rep)


def test_decode_empty_batch_and_all_empty():
    shape = AttnShape(8, 2, 128, 128, 16, 0.1)
    desc = fca.desc_from_shape(shape, 8)
    p = fca.fca_plan(torch.zeros((0, 4), dtype=torch.int32, device="cuda"), torch.zeros(0, dtype=torch.int32, device="cuda"), desc)
    assert p.info.batch == 0
    q = torch.zeros((0, 8, 128), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((8, 2, 16, 16, 8), dtype=torch.bfloat16, device="cuda")
    out = fca.fca_decode(q, kv, kv, p)
    assert out.shape == (0, 8, 128)
    # all requests empty
    p = fca.fca_plan(torch.zeros((3, 4), dtype=torch.int32, device="cuda"), torch.zeros(3, dtype=torch.int32, device="cuda"), desc)
    q = torch.ones((3, 8, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((3, 8), dtype=torch.float32, device="cuda")
    out = fca.fca_decode(q, kv, kv, p, lse=lse)
    torch.cuda.synchronize()
    assert (out.float() == 0).all() and torch.isneginf(lse).all()


def test_plan_and_decode_largest_batch():
    """The largest batch the library takes (8192 requests), all in one tree:
    a 3-block root shared by every request, 64 branches of 2 more blocks,
    128 samples per branch with a suffix of 1 to 16 tokens.  Discovery sorts
    all 8192 members in one workgroup's LDS; the grouping must equal the
    oracle's and every request's decode must match the oracle."""
    shape = AttnShape(4, 1, 128, 128, 16, 1 / math.sqrt(128))
    B, branches, W = 8192, 64, 6
    per = B // branches
    rng = np.random.default_rng(8192)
    sfx = rng.integers(1, 17, size=B).astype(np.int32)
    n_used = 3 + 2 * branches + B
    nb = n_used + 64
    ids = rng.permutation(nb).astype(np.int32)
    tables = rng.integers(0, nb, size=(B, W)).astype(np.int32)  # entries past a request's blocks: arbitrary
    for i in range(B):
        br = i // per
        tables[i, :3] = ids[:3]
        tables[i, 3:5] = ids[3 + 2 * br : 5 + 2 * br]
        tables[i, 5] = ids[3 + 2 * branches + i]
    order = rng.permutation(B)  # members of a branch are not contiguous in the batch
    tables, lens = tables[order], (5 * 16 + sfx)[order].astype(np.int32)
    say("largest batch: B", B, "blocks", nb)
    bt, sl = torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda()
    p = fca.fca_plan(bt, sl, fca.desc_from_shape(shape, nb, auto_fold=False))
    exp = group(tables, lens, 16)
    assert with_block_ids(p.export(), tables) == exp
    assert p.info.num_groups == 1 + branches
    say("largest batch: groups", p.info.num_groups, "equal to the oracle's")
    case = small_case(shape, tables, lens, nb, seed=8193)
    ref, ref_lse = A.attend(case["q"], case["k"], case["v"], tables, lens, shape)
    b = _B(shape, tables, lens, nb)
    vals = upload(case)
    for cascade, fold in MODES:
        _, out, lse = run_decode(b, vals, cascade=cascade, auto_fold=fold)
        rep = assert_close(bf16_tensor_to_f64(out), ref, f"largest batch cascade={cascade} fold={fold}")
        assert_lse_close(lse.cpu().numpy(), ref_lse, "largest batch")
        say("largest batch", "cascade" if cascade else "non-cascade", "fold" if fold else "keep", rep)
        del out, lse


@pytest.mark.parametrize("token_rows", [False, True], ids=["tiles", "rows"])
@pytest.mark.parametrize("name", ["tiny", "llama3_8b"])
def test_decode_one_workgroup_per_unit(name, token_rows, monkeypatch):
    """The plan shape of large batches (one attention workgroup per compute
    unit, so every lane is cut into half as many token pieces) forced on
    small batches (FCA_TUNE_BINS_PER_CU=1), in both cache layouts, with
    every group kept and with the default decision, against the oracle."""
    monkeypatch.setenv("FCA_TUNE_BINS_PER_CU", "1")
    b = build_batch(CONFIGS[name])
    vn = fill_values_numpy(b, poison=True)
    sh = b.shape
    say("one workgroup per unit", name, "rows" if token_rows else "tiles")
    ref, ref_lse = A.attend(vn["q"], vn["k"], vn["v"], b.block_tables, b.seq_lens, sh)
    k, v = vn["k"], vn["v"]
    if token_rows:  # [blocks][slots][kv heads][dims]
        k = np.ascontiguousarray(k.transpose(0, 3, 1, 2, 4)).reshape(b.num_blocks, 16, sh.num_kv_heads, 128)
        v = np.ascontiguousarray(v.transpose(0, 3, 1, 2))
    kd, vd, qd = to_device_bf16(k), to_device_bf16(v), to_device_bf16(vn["q"])
    bt, sl = dev_tables(b)
    for fold in (False, True):
        p = fca.fca_plan(bt, sl, fca.desc_from_shape(sh, b.num_blocks, auto_fold=fold, token_rows=token_rows))
        check_schedule(b, p)
        out = torch.empty((b.batch, sh.num_q_heads, sh.head_dim_v), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((b.batch, sh.num_q_heads), dtype=torch.float32, device="cuda")
        fca.fca_decode(qd, kd, vd, p, out=out, lse=lse)
        torch.cuda.synchronize()
        rep = assert_close(bf16_tensor_to_f64(out), ref, f"{name} one workgroup per unit fold={fold}")
        assert_lse_close(lse.cpu().numpy(), ref_lse, name)
        say(name, "fold", fold, rep, "groups", p.info.num_groups)


def test_decode_strided_pool():
    """Pools that are slices of a larger buffer (head/block strides)."""
    b = build_batch(CONFIGS["tiny"])
    vn = fill_values_numpy(b, poison=True)
    sh = b.shape
    ref, _ = A.attend(vn["q"], vn["k"], vn["v"], b.block_tables, b.seq_lens, sh)
    # embed each pool in a buffer with 3 extra heads per block
    nb = b.num_blocks
    kbig = np.full((nb, sh.num_kv_heads + 3, 16, 16, 8), BF16_NAN, np.uint16)
    vbig = np.full((nb, sh.num_kv_heads + 3, 128, 16), BF16_NAN, np.uint16)
    kbig[:, 1 : 1 + sh.num_kv_heads] = vn["k"]
    vbig[:, 2 : 2 + sh.num_kv_heads] = vn["v"]
    kd, vd = to_device_bf16(kbig), to_device_bf16(vbig)
    ksh = 128 * 16
    desc = fca.make_desc(
        sh.num_q_heads, sh.num_kv_heads, 128, 128, 16, nb, sh.scale,
        k_strides=((sh.num_kv_heads + 3) * ksh, ksh), v_strides=((sh.num_kv_heads + 3) * ksh, ksh),
    )
    bt, sl = dev_tables(b)
    p = fca.fca_plan(bt, sl, desc)
    out = fca.fca_decode(to_device_bf16(vn["q"]), kd[:, 1:], vd[:, 2:], p)
    torch.cuda.synchronize()
    assert_close(bf16_tensor_to_f64(out), ref, "strided pool")


# ------------------------------------------------------------- latent cache ----

MLA = AttnShape(128, 1, 576, 512, 64, 1 / math.sqrt(576), v_aliases_k=True)


@pytest.mark.parametrize("hq,hkv", [(128, 1), (16, 1), (64, 2)])
def test_decode_mla_small(hq, hkv):
    """Latent cache (576-wide keys, values = first 512 dims, 64-token
    blocks): two prompts of 4 blocks with 3 samples each plus an unshared
    request, suffixes from 1 token to several blocks, against the oracle."""
    shape = AttnShape(hq, hkv, 576, 512, 64, MLA.scale, v_aliases_k=True)
    cfg = Config(
        name=f"mla_small_{hq}_{hkv}",
        shape=shape,
        trees=[Node(256, samples=3, suffix=(1, 150)), Node(192, samples=3, suffix=(60, 200))],
        singletons=1,
        singleton_len=(1, 130),
        seed=40 + hq + hkv,
    )
    b = build_batch(cfg)
    vn = fill_values_numpy(b, poison=True)
    ref, ref_lse = A.attend(vn["q"], vn["k"], vn["v"], b.block_tables, b.seq_lens, shape)
    vals = upload(vn)
    for cascade in (True, False):
        p, out, lse = run_decode(b, vals, cascade=cascade, auto_fold=False)
        rep = assert_close(bf16_tensor_to_f64(out), ref, f"mla small hq={hq} hkv={hkv} cascade={cascade}")
        assert_lse_close(lse.cpu().numpy(), ref_lse, "mla small")
        say("mla small", hq, hkv, "cascade", cascade, rep, "groups", p.info.num_groups)


def test_decode_hip_graph_replay():
    """The decode step (both launches) captured once into a HIP graph and
    replayed: each replay, with new query values copied into the captured
    buffer and eager decodes of the same plan in between, equals the eager
    result bit for bit (the plan is built once and reused, as by the layers
    of a model)."""
    b = build_batch(CONFIGS["tiny"])
    vn = fill_values_numpy(b, poison=True)
    vals = upload(vn)
    bt, sl = dev_tables(b)
    p = fca.fca_plan(bt, sl, fca.desc_from_shape(b.shape, b.num_blocks, auto_fold=False))
    sh = b.shape
    q_static = vals["q"].clone()
    out_g = torch.empty((b.batch, sh.num_q_heads, sh.head_dim_v), dtype=torch.bfloat16, device="cuda")
    lse_g = torch.empty((b.batch, sh.num_q_heads), dtype=torch.float32, device="cuda")
    out_e = torch.empty_like(out_g)
    lse_e = torch.empty_like(lse_g)
    ws = p.decode_workspace(q_static.device)
    # warm up on the capture stream, then capture
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        p.decode(q_static, vals["k"], vals["v"], out=out_g, lse=lse_g, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        p.decode(q_static, vals["k"], vals["v"], out=out_g, lse=lse_g, workspace=ws)
    torch.cuda.synchronize()
    gen = torch.Generator(device="cuda").manual_seed(7)
    for rep in range(4):
        q_new = torch.randn(q_static.shape, generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
        q_static.copy_(q_new)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ws_e = torch.empty_like(ws)
        p.decode(q_new, vals["k"], vals["v"], out=out_e, lse=lse_e, workspace=ws_e)
        torch.cuda.synchronize()
        assert torch.equal(out_g.view(torch.int16), out_e.view(torch.int16)), f"replay {rep}: output differs from eager"
        assert torch.equal(lse_g, lse_e), f"replay {rep}: lse differs from eager"
    # and the replayed output is the attention of the last queries (oracle)
    ref, _ = A.attend(to_bits_np(q_static), vn["k"], vn["v"], b.block_tables, b.seq_lens, sh)
    assert_close(bf16_tensor_to_f64(out_g), ref, "graph replay")
    say("graph replay: 4 replays equal to eager")


@pytest.mark.parametrize("name", ["tiny", "llama3_8b"])
def test_decode_layers_graph_replay_every_layer(name):
    """One plan, four layers (their own KV pools and queries) decoded by one
    fca_decode_layers call captured in a HIP graph: three replays with new
    queries copied into the captured buffers, eager calls between them; each
    replay equals the eager call bit for bit, and every layer of the last
    replay matches the oracle."""
    b = build_batch(CONFIGS[name])
    sh = b.shape
    n_layers = 4
    say("decode layers", name, "layers", n_layers)
    layers = [fill_values_torch(b, "cuda", seed=1000 + l, poison=True) for l in range(n_layers)]
    hosts = [host_values(v) for v in layers]
    caches = [(v["k"], v["v"]) for v in layers]
    bt, sl = dev_tables(b)
    p = fca.fca_plan(bt, sl, fca.desc_from_shape(sh, b.num_blocks))
    shape_out = (b.batch, sh.num_q_heads, sh.head_dim_v)
    q_static = [v["q"].clone() for v in layers]
    outs_g = [torch.empty(shape_out, dtype=torch.bfloat16, device="cuda") for _ in range(n_layers)]
    lses_g = [torch.empty((b.batch, sh.num_q_heads), dtype=torch.float32, device="cuda") for _ in range(n_layers)]
    outs_e = [torch.empty_like(o) for o in outs_g]
    lses_e = [torch.empty_like(l) for l in lses_g]
    ws = p.decode_workspace(q_static[0].device)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        p.decode_layers(q_static, caches, outs_g, lses_g, workspace=ws, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        p.decode_layers(q_static, caches, outs_g, lses_g, workspace=ws)
    torch.cuda.synchronize()
    gen = torch.Generator(device="cuda").manual_seed(11)
    for rep in range(3):
        q_new = [torch.randn(q.shape, generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
                 for q in q_static]
        for qs_, qn in zip(q_static, q_new):
            qs_.copy_(qn)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ws_e = torch.empty_like(ws)
        p.decode_layers(q_new, caches, outs_e, lses_e, workspace=ws_e)
        torch.cuda.synchronize()
        for l in range(n_layers):
            assert torch.equal(outs_g[l].view(torch.int16), outs_e[l].view(torch.int16)), f"replay {rep} layer {l}"
            assert torch.equal(lses_g[l], lses_e[l]), f"replay {rep} layer {l}: lse"
    for l in range(n_layers):
        host = dict(hosts[l], q=to_bits_np(q_static[l]))
        ref, ref_lse = oracle_all(b, host)
        rep = assert_close(bf16_tensor_to_f64(outs_g[l]), ref, f"{name} layer {l}")
        assert_lse_close(lses_g[l].cpu().numpy(), ref_lse, f"{name} layer {l}")
        say("decode layers", name, "layer", l, rep)
    del graph, layers, caches


def to_bits_np(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def mla_small_config(seed=52):
    return Config(
        name="mla_small_timing",
        shape=MLA,
        trees=[Node(256, samples=3, suffix=(1, 150)), Node(192, samples=2, suffix=(60, 200))],
        singletons=1,
        singleton_len=(1, 130),
        seed=seed,
    )


@pytest.mark.parametrize("kind", ["gqa", "mla"])
def test_time_launches_and_profile(kind):
    """The measurement entry points: fca_time_launches leaves out / lse equal
    to a plain decode of the last cache it cycled over, bit for bit, and
    returns positive per-launch times (per pass on the latent cache, whose
    plans launch the passes separately); fca_profile_enable / read sum the
    launch times of profiled decodes."""
    b = build_batch(CONFIGS["tiny"] if kind == "gqa" else mla_small_config())
    caches = []
    for _ in range(2):
        vn = fill_values_numpy(b, poison=True)  # the batch's rng moves on: new values each time
        caches.append(upload(vn))
    q = caches[0]["q"]
    sh = b.shape
    bt, sl = dev_tables(b)
    p = fca.fca_plan(bt, sl, fca.desc_from_shape(sh, b.num_blocks))
    out_t = torch.empty((b.batch, sh.num_q_heads, sh.head_dim_v), dtype=torch.bfloat16, device="cuda")
    lse_t = torch.empty((b.batch, sh.num_q_heads), dtype=torch.float32, device="cuda")
    say("time launches", kind)
    t = p.time_launches(q, [(c["k"], c["v"]) for c in caches], 3, out_t, lse_t)
    torch.cuda.synchronize()
    assert t["calls"] == 6
    assert t["attention_ms"] > 0 and t["merge_ms"] > 0
    assert t["decode_ms"] == pytest.approx(t["attention_ms"] + t["merge_ms"])
    if kind == "mla":
        assert t["grouped_ms"] > 0 and t["suffix_ms"] > 0
        assert t["attention_ms"] == pytest.approx(t["grouped_ms"] + t["suffix_ms"])
    else:
        assert t["grouped_ms"] == 0 and t["suffix_ms"] == 0
    out_d = torch.empty_like(out_t)
    lse_d = torch.empty_like(lse_t)
    ws = torch.empty_like(p.decode_workspace(q.device))
    p.decode(q, caches[1]["k"], caches[1]["v"], out=out_d, lse=lse_d, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out_t.view(torch.int16), out_d.view(torch.int16))
    assert torch.equal(lse_t, lse_d)
    with pytest.raises(fca.FcaError):
        p.time_launches(q, [], 1, out_t, lse_t)
    with pytest.raises(fca.FcaError):
        p.time_launches(q, [(caches[0]["k"], caches[0]["v"])], 0, out_t, lse_t)

    p.profile(True)
    for c in caches:
        p.decode(q, c["k"], c["v"], out=out_d, lse=lse_d)
    pr = p.read_profile()
    p.profile(False)
    assert pr["calls"] == 2
    assert pr["attention_ms"] > 0 and pr["merge_ms"] > 0 and pr["decode_ms"] >= pr["attention_ms"]
    if kind == "mla":
        assert pr["grouped_ms"] > 0 and pr["suffix_ms"] > 0
    assert torch.equal(out_d.view(torch.int16), out_t.view(torch.int16))
    say("time launches", kind, {k: round(v, 4) for k, v in t.items()})


def test_plan_schedule_memory_reuse():
    """Plans created and destroyed in turn (their schedules recycled through
    the library's stream-ordered pool) decode correctly, and a plan kept
    alive meanwhile still decodes bit for bit as it did at first."""
    import gc

    keep_b = build_batch(CONFIGS["tiny"])
    keep_vn = fill_values_numpy(keep_b, poison=True)
    keep_vals = upload(keep_vn)
    keep_p, keep_out, keep_lse = run_decode(keep_b, keep_vals)
    first = keep_out.clone()
    rng = np.random.default_rng(5)
    shape = AttnShape(8, 2, 128, 128, 16, 1 / math.sqrt(128))
    W, bs, nb = 16, 16, 512
    for it in range(6):
        B = int(rng.integers(2, 12))
        tables = rng.permutation(nb)[: B * W].reshape(B, W).astype(np.int32)
        lens = rng.integers(0, W * bs + 1, size=B).astype(np.int32)
        for i in range(1, B):
            # share whole blocks that are full in both rows (no poisoned tails shared)
            base = int(rng.integers(0, i))
            cut = int(rng.integers(0, min(lens[i], lens[base]) // bs + 1))
            tables[i, :cut] = tables[base, :cut]
        case = small_case(shape, tables, lens, nb, seed=it)
        ref, _ = A.attend(case["q"], case["k"], case["v"], tables, lens, shape)
        p, out, _ = run_decode(_B(shape, tables, lens, nb), upload(case))
        assert_close(bf16_tensor_to_f64(out), ref, f"reuse round {it}")
        del p, out
        gc.collect()
    out2 = torch.empty_like(keep_out)
    fca.fca_decode(keep_vals["q"], keep_vals["k"], keep_vals["v"], keep_p, out=out2)
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), first.view(torch.int16))


# ------------------------------------------------- route-the-query merge ----


def split_tables(b, frac):
    """Each request's blocks cut in two at a block boundary: (tables, lens)
    of the first part and of the rest (empty parts allowed)."""
    bs = b.shape.block_size
    lens = b.seq_lens.astype(np.int64)
    nb = -(-lens // bs)
    na = np.minimum((nb * frac).astype(np.int64), lens // bs)
    ta = b.block_tables.copy()
    tb = np.zeros_like(b.block_tables)
    for i in range(b.batch):
        rest = b.block_tables[i, na[i] : nb[i]]
        tb[i, : len(rest)] = rest
    la = (na * bs).astype(np.int32)
    lb = (lens - na * bs).astype(np.int32)
    return (ta, la), (tb, lb)


@pytest.mark.parametrize("name,frac", [("tiny", 0.5), ("tiny", 0.0), ("llama3_8b", 0.7)])
def test_route_the_query_split_merge(name, frac):
    """The cache of every request cut in two (as if half of it lived on
    another GPU): each part decoded to a float32 state with its lse, the two
    states combined by fca_merge_states, against the oracle's attention over
    the whole cache (and the float32 decode of the whole cache)."""
    b = build_batch(CONFIGS[name])
    sh = b.shape
    if name == "tiny":
        vn = fill_values_numpy(b, poison=True)
        vals = upload(vn)
        ref, ref_lse = A.attend(vn["q"], vn["k"], vn["v"], b.block_tables, b.seq_lens, sh)
        pick = list(range(b.batch))
    else:
        vals = fill_values_torch(b, "cuda", seed=CONFIGS[name].seed, poison=True)
        ref, ref_lse = oracle_all(b, host_values(vals))
        pick = list(range(b.batch))
    states = []
    for tables, lens in split_tables(b, frac):
        bt = torch.from_numpy(tables).cuda()
        sl = torch.from_numpy(lens).cuda()
        p = fca.fca_plan(bt, sl, fca.desc_from_shape(sh, b.num_blocks, out_f32=True))
        o = torch.empty((b.batch, sh.num_q_heads, sh.head_dim_v), dtype=torch.float32, device="cuda")
        l = torch.empty((b.batch, sh.num_q_heads), dtype=torch.float32, device="cuda")
        fca.fca_decode(vals["q"], vals["k"], vals["v"], p, out=o, lse=l)
        states.append((o, l))
    lse = torch.empty((b.batch, sh.num_q_heads), dtype=torch.float32, device="cuda")
    out = fca.merge_states([s[0] for s in states], [s[1] for s in states], lse=lse)
    torch.cuda.synchronize()
    rep = assert_close(bf16_tensor_to_f64(out[pick]), ref, f"{name} split {frac}")
    assert_lse_close(lse[pick].cpu().numpy(), ref_lse, f"{name} split {frac}")
    # float32 state of the whole cache, merged with nothing, is the whole decode
    p = fca.fca_plan(torch.from_numpy(b.block_tables).cuda(), torch.from_numpy(b.seq_lens).cuda(),
                     fca.desc_from_shape(sh, b.num_blocks, out_f32=True))
    of = torch.empty_like(states[0][0])
    lf = torch.empty_like(states[0][1])
    fca.fca_decode(vals["q"], vals["k"], vals["v"], p, out=of, lse=lf)
    out1 = fca.merge_states([of], [lf], out_f32=True)
    torch.cuda.synchronize()
    assert torch.equal(out1, of)
    assert (out.float() - of).abs().max().item() < 8e-3
    say("route-the-query", name, frac, rep)


@pytest.mark.parametrize("D", [128, 512])
def test_merge_states_against_oracle(D):
    """Random states (including states without keys, whose outputs hold
    garbage, and pairs where every state is empty) merged on the device
    against the oracle's merge_states, in bf16 and float32 output, with the
    output aliasing the first state."""
    rng = np.random.default_rng(D)
    B, H, n = 7, 5, 5
    outs = [rng.standard_normal((B, H, D)).astype(np.float32) for _ in range(n)]
    lses = [(3.0 * rng.standard_normal((B, H))).astype(np.float32) for _ in range(n)]
    for j in range(n):
        dead = rng.random((B, H)) < 0.3
        lses[j][dead] = -np.inf
        outs[j][dead] = np.nan  # an empty state's output must not leak in
    lses[0][2, 3] = lses[1][2, 3] = lses[2][2, 3] = lses[3][2, 3] = lses[4][2, 3] = -np.inf
    ref, ref_lse = A.merge_states([o.reshape(B * H, D) for o in outs], [l.reshape(B * H) for l in lses])
    ref, ref_lse = ref.reshape(B, H, D), ref_lse.reshape(B, H)
    d_outs = [torch.from_numpy(o).cuda() for o in outs]
    d_lses = [torch.from_numpy(l).cuda() for l in lses]
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    out = fca.merge_states(d_outs, d_lses, lse=lse)
    torch.cuda.synchronize()
    assert_close(bf16_tensor_to_f64(out), ref, f"merge states D={D}")
    assert_lse_close(lse.cpu().numpy(), ref_lse, f"merge states D={D}")
    assert (bf16_tensor_to_f64(out)[2, 3] == 0).all() and np.isneginf(lse[2, 3].item())
    # float32, written over the first state
    out32 = fca.merge_states(d_outs, d_lses, out=d_outs[0], out_f32=True)
    torch.cuda.synchronize()
    o32 = out32.cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(o32, ref, rtol=1e-5, atol=1e-6)


# ------------------------------------------------------ activation (fold) ----


def fold_case():
    """64 requests of the Llama-3-8B layer shape: 16 pairs sharing one block,
    8 pairs sharing 48 blocks, and a root shared by 16 requests over 2
    blocks whose children are 8 pairs sharing 40 more blocks each."""
    shape = AttnShape(32, 8, 128, 128, 16, 1 / math.sqrt(128))
    rng = np.random.default_rng(77)
    W, bs = 112, 16
    B = 64
    nb = B * W + 64
    perm = rng.permutation(nb)
    tables = perm[: B * W].reshape(B, W).astype(np.int32)
    lens = np.zeros(B, np.int32)
    for k in range(16):  # pairs over one shared block
        i = 2 * k
        tables[i + 1, :1] = tables[i, :1]
        lens[i], lens[i + 1] = rng.integers(40, 120, size=2) * bs // 2
    for k in range(8):  # pairs over 48 shared blocks
        i = 32 + 2 * k
        tables[i + 1, :48] = tables[i, :48]
        lens[i], lens[i + 1] = (48 + rng.integers(2, 40, size=2)) * bs - 3
    for k in range(8):  # root of 16 over 2 blocks, then pairs over 40 more
        i = 48 + 2 * k
        tables[i, :2] = tables[48, :2]
        tables[i + 1, :42] = tables[i, :42]
        lens[i], lens[i + 1] = (42 + rng.integers(2, 30, size=2)) * bs - 5
    return shape, tables, lens, nb


@pytest.mark.parametrize("case", ["fold", "tiny", "llama3_8b"])
def test_auto_fold_plan_schedule_and_decode(case):
    """FCA_PLAN_AUTO_FOLD: discovered groups are those of the oracle; groups
    that cannot pay for their partial rows are folded into their members'
    suffixes (leaves first), the schedule still covers every token once,
    and the decode matches the oracle."""
    if case == "fold":
        shape, tables, lens, nb = fold_case()
        b = _B(shape, tables, lens, nb)
        vn = small_case(shape, tables, lens, nb, seed=3)
    else:
        b = build_batch(CONFIGS[case])
        shape, tables, lens, nb = b.shape, b.block_tables, b.seq_lens, b.num_blocks
        vn = fill_values_numpy(b, poison=True) if case == "tiny" else None
    bt, sl = dev_tables(b)
    p = fca.fca_plan(bt, sl, fca.desc_from_shape(shape, nb, auto_fold=True))
    ex = p.export()
    ref_plan = group(tables, lens, shape.block_size)
    assert with_block_ids(ex, tables)["groups"] == ref_plan["groups"]
    folded = ex["folded"]
    assert p.info.num_folded_groups == sum(folded)
    # leaves first: a kept group's parent is kept
    for k, g in enumerate(ex["groups"]):
        if not folded[k] and g["parent"] >= 0:
            assert not folded[g["parent"]]
    # a request's range as read: its suffix starts where its nearest kept group ends
    for i, (sb, st, deep) in enumerate(ex["requests"]):
        ref_sb, _, ref_deep = ref_plan["requests"][i]
        d = ref_deep
        while d >= 0 and folded[d]:
            d = ex["groups"][d]["parent"]
        assert deep == d
        assert sb == (ex["groups"][d]["block_end"] if d >= 0 else 0)
        assert st == lens[i] - sb * shape.block_size
    if case == "fold":
        # the one-block pairs fold, the 48-block pairs stay, the 2-block root
        # stays because its children (40 more blocks each) stay
        by_len = {(g["block_begin"], g["block_end"]): folded[k] for k, g in enumerate(ex["groups"])}
        assert by_len[(0, 1)] == 1 and by_len[(0, 48)] == 0 and by_len[(0, 2)] == 0 and by_len[(2, 42)] == 0
    if case == "tiny":
        assert folded == [1]
        # every group folded: the schedule is the non-cascade one (bypass)
        nc = fca.fca_plan(bt, sl, fca.desc_from_shape(shape, nb, cascade=False)).export_schedule()
        assert p.export_schedule() == nc
    if case == "llama3_8b":
        assert sum(folded) == 0
    check_schedule(b, p)
    if vn is not None:
        ref, ref_lse = A.attend(vn["q"], vn["k"], vn["v"], tables, lens, shape)
        vals = upload(vn)
        out = torch.empty((len(lens), shape.num_q_heads, shape.head_dim_v), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((len(lens), shape.num_q_heads), dtype=torch.float32, device="cuda")
        fca.fca_decode(vals["q"], vals["k"], vals["v"], p, out=out, lse=lse)
        torch.cuda.synchronize()
        rep = assert_close(bf16_tensor_to_f64(out), ref, f"auto fold {case}")
        assert_lse_close(lse.cpu().numpy(), ref_lse, f"auto fold {case}")
        say("auto fold", case, "folded", sum(folded), "of", len(folded), rep)


@pytest.mark.parametrize("case", ["tiny", "llama3_8b", "long_rl", "fold"])
def test_streaming_flags_mark_single_reader_tiles(case):
    """Work items carry kItemStream (non-temporal tile loads) exactly when
    each of their tiles has one reader: a suffix of a cascade plan of a
    request in no folded group, or a group whose query rows fit one wave
    (32).  Plans without the cascade mark nothing (shared prefixes sit in
    every member's suffix)."""
    if case == "fold":
        shape, tables, lens, nb = fold_case()
    else:
        b = build_batch(CONFIGS[case])
        shape, tables, lens, nb = b.shape, b.block_tables, b.seq_lens, b.num_blocks
    bt, sl = torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda()
    for cascade, fold in ((True, False), (True, True), (False, False)):
        p = fca.fca_plan(bt, sl, fca.desc_from_shape(shape, nb, cascade=cascade, auto_fold=fold))
        ex, sc = p.export(), p.export_schedule()
        folded = ex["folded"]
        n_flagged = 0
        for it in sc["grouped"] + sc["suffix"]:
            if it["member_off"] >= 0:
                want = it["ncols"] <= 32
            else:
                in_folded = any(f and it["request"] in g["members"] for f, g in zip(folded, ex["groups"]))
                want = cascade and not in_folded
            assert bool(it["flags"] & 1) == want, (case, cascade, fold, it)
            n_flagged += bool(it["flags"] & 1)
        say("stream flags", case, "cascade", cascade, "fold", fold, "flagged", n_flagged, "of", len(sc["grouped"]) + len(sc["suffix"]))
        if not cascade:
            assert n_flagged == 0
