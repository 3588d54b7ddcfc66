"""GPU parity of the decode-token append with copy-on-write (fca_kv_append)
against the oracle: pools and block tables bit-exact after every step, and
the attention path reading the appended cache against oracle attention.
Needs an MI355X."""

from __future__ import annotations

import math
import sys

import numpy as np
import pytest

from oracle import attention as A
from oracle import kv_cache as KV
from tests.helpers import assert_close, assert_lse_close, bf16_tensor_to_f64, to_bits, to_device_bf16
from workloads.forest import AttnShape
from workloads.values import BF16_NAN, f32_to_bf16_bits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import shared_prefix_kv_amd as fca  # noqa: E402

GQA = AttnShape(32, 8, 128, 128, 16, 1 / math.sqrt(128))
MLA = AttnShape(16, 1, 576, 512, 64, 1 / math.sqrt(576), v_aliases_k=True)


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fca.lib()


def fills(tables, lens, bs):
    """Tokens each request holds in each block it references."""
    held = {}
    for i, L in enumerate(lens):
        for j in range(-(-int(L) // bs)):
            held.setdefault(int(tables[i, j]), []).append((i, min(bs, int(L) - j * bs)))
    return held


def choose_step(tables, lens, bs, free):
    """Host side of one decode step of a paged cache: a fresh block where a
    request's last block is full, and a copy-on-write target for every
    request whose next slot is already held by another request (of the
    requests sharing a partly filled block, only the lowest-numbered of those
    with the most tokens writes in place)."""
    tables = tables.copy()
    cow = np.full(len(lens), -1, np.int32)
    held = fills(tables, lens, bs)
    for i, L in enumerate(lens):
        L = int(L)
        if L % bs == 0:
            tables[i, L // bs] = free.pop()
            continue
        blk = int(tables[i, L // bs])
        top = max(f for _, f in held[blk])
        owner = min(r for r, f in held[blk] if f == top)
        if owner != i or top != L % bs:
            cow[i] = free.pop()
    return tables, cow


def forked_case(shape, seed):
    """Two prompts of 2 blocks + 5 tokens.  Prompt A: four forks at its full
    length (one appends in place, three copy), one fork a token earlier, one
    request that shares only its first block (full: the next token starts a
    block).  Prompt B: two forks and a longer request that filled B's third
    block itself (both forks copy).  Plus an empty request and an unshared
    one."""
    bs = shape.block_size
    P = 2 * bs + 5
    W = 8
    nb = 64
    rng = np.random.default_rng(seed)
    free = [int(x) for x in rng.permutation(nb)]
    a = [free.pop() for _ in range(3)]
    b = [free.pop() for _ in range(4)]
    tables = np.full((12, W), -1, np.int32)
    lens = np.zeros(12, np.int32)
    for i in range(4):
        tables[i, :3], lens[i] = a, P
    tables[4, :3], lens[4] = a, P - 1
    tables[5, :1], lens[5] = a[:1], bs
    tables[6, :2], lens[6] = b[:2], 2 * bs
    tables[7, :3], lens[7] = b[:3], P
    tables[8, :3], lens[8] = b[:3], P
    tables[9, :4], lens[9] = b, 3 * bs + 2
    lens[10] = 0
    tables[11, :2], lens[11] = [free.pop(), free.pop()], bs + 3
    tables[tables < 0] = 0  # unused entries: any valid ID
    k = f32_to_bf16_bits(rng.standard_normal((nb, shape.num_kv_heads, shape.head_dim_qk // 8, bs, 8), dtype=np.float32))
    v = None
    if not shape.v_aliases_k:
        v = f32_to_bf16_bits(rng.standard_normal((nb, shape.num_kv_heads, shape.head_dim_v, bs), dtype=np.float32))
    # poison every slot no request holds
    held = fills(tables, lens, bs)
    for blk in range(nb):
        top = max((f for _, f in held.get(blk, [])), default=0)
        k[blk, :, :, top:, :] = BF16_NAN
        if v is not None:
            v[blk, :, :, top:] = BF16_NAN
    return tables, lens, k, v, free


def new_rows(rng, shape, B):
    kn = f32_to_bf16_bits(rng.standard_normal((B, shape.num_kv_heads, shape.head_dim_qk), dtype=np.float32))
    vn = None
    if not shape.v_aliases_k:
        vn = f32_to_bf16_bits(rng.standard_normal((B, shape.num_kv_heads, shape.head_dim_v), dtype=np.float32))
    return kn, vn


@pytest.mark.parametrize("shape", [GQA, MLA], ids=["gqa", "mla"])
def test_append_cow_steps_bitexact_then_decode(shape):
    """Three decode steps: each appends through fca_kv_append and through
    the oracle; pools and tables agree bit for bit, and the attention path
    over the grown cache (with the forks now owning their blocks) agrees
    with oracle attention."""
    bs = shape.block_size
    tables, lens, k, v, free = forked_case(shape, seed=11 + shape.head_dim_qk)
    B = len(lens)
    rng = np.random.default_rng(5)
    kd = to_device_bf16(k)
    vd = to_device_bf16(v) if v is not None else None
    desc = fca.desc_from_shape(shape, k.shape[0])
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for step in range(3):
        tables, cow = choose_step(tables, lens, bs, free)
        kn, vn = new_rows(rng, shape, B)
        say("append", "mla" if shape.v_aliases_k else "gqa", "step", step, "cow", cow.tolist())
        bt = torch.from_numpy(tables).cuda()
        fca.kv_append(
            to_device_bf16(kn),
            to_device_bf16(vn) if vn is not None else None,
            kd,
            vd,
            bt,
            torch.from_numpy(lens).cuda(),
            desc,
            cow_dst=torch.from_numpy(cow).cuda(),
            status=status,
        )
        torch.cuda.synchronize()
        k, v, tables = KV.append(k, v, tables, lens, kn, vn, bs, cow)
        assert int(status.item()) == 0
        assert (bt.cpu().numpy() == tables).all(), f"step {step}: block tables differ"
        assert (to_bits(kd) == k).all(), f"step {step}: key pool differs"
        if v is not None:
            assert (to_bits(vd) == v).all(), f"step {step}: value pool differs"
        lens = lens + 1
        # the grown cache through the attention path
        q = f32_to_bf16_bits(rng.standard_normal((B, shape.num_q_heads, shape.head_dim_qk), dtype=np.float32))
        ref, ref_lse = A.attend(q, k, v, tables, lens, shape)
        p = fca.fca_plan(bt, torch.from_numpy(lens).cuda(), desc)
        out = torch.empty((B, shape.num_q_heads, shape.head_dim_v), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((B, shape.num_q_heads), dtype=torch.float32, device="cuda")
        fca.fca_decode(to_device_bf16(q), kd, vd, p, out=out, lse=lse)
        torch.cuda.synchronize()
        rep = assert_close(bf16_tensor_to_f64(out), ref, f"decode after append step {step}")
        assert_lse_close(lse.cpu().numpy(), ref_lse, "decode after append")
        say("step", step, rep, "groups", p.info.num_groups)
    # after the first step every fork owns its last block: no copies remain
    _, cow = choose_step(tables, lens, bs, list(range(k.shape[0])))
    assert (cow < 0).all()


def test_append_skips_bad_requests_and_flags_them():
    """A length past the table, a block ID outside the pool and a cow target
    outside the pool each skip their request and set their status bit; the
    other requests are appended as the oracle does."""
    shape = GQA
    bs, W, nb = shape.block_size, 4, 32
    rng = np.random.default_rng(9)
    k = f32_to_bf16_bits(rng.standard_normal((nb, 8, 16, bs, 8), dtype=np.float32))
    v = f32_to_bf16_bits(rng.standard_normal((nb, 8, 128, bs), dtype=np.float32))
    tables = rng.permutation(5 * W).reshape(5, W).astype(np.int32)  # blocks 20.. unused
    lens = np.array([W * bs, 20, 7, 33, 0], np.int32)
    tables[1, 1] = nb  # request 1's next slot would be in block table[1][1]
    cow = np.array([-1, -1, nb, 25, -1], np.int32)
    kn, vn = new_rows(rng, shape, 5)
    kd, vd = to_device_bf16(k), to_device_bf16(v)
    bt = torch.from_numpy(tables).cuda()
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    say("append bad requests")
    fca.kv_append(
        to_device_bf16(kn), to_device_bf16(vn), kd, vd, bt, torch.from_numpy(lens).cuda(),
        fca.desc_from_shape(shape, nb), cow_dst=torch.from_numpy(cow).cuda(), status=status,
    )
    torch.cuda.synchronize()
    assert int(status.item()) == fca.FCA_APPEND_BAD_LEN | fca.FCA_APPEND_BAD_BLOCK | fca.FCA_APPEND_BAD_COW
    good = [3, 4]
    k2, v2, t2 = KV.append(k, v, tables[good], lens[good], kn[good], vn[good], bs, cow[good])
    exp_t = tables.copy()
    exp_t[good] = t2
    assert (bt.cpu().numpy() == exp_t).all()
    assert (to_bits(kd) == k2).all() and (to_bits(vd) == v2).all()


def test_append_graph_replays_match_eager_and_edge_targets():
    """Appends captured in a HIP graph (four replays, eager work and
    synchronisation between them) leave the same pools and tables as eager
    calls; a copy target equal to the request's own block, and a request
    whose new token starts a block, are written in place."""
    shape = GQA
    bs, W, nb = shape.block_size, 6, 96
    rng = np.random.default_rng(21)
    k = f32_to_bf16_bits(rng.standard_normal((nb, 8, 16, bs, 8), dtype=np.float32))
    v = f32_to_bf16_bits(rng.standard_normal((nb, 8, 128, bs), dtype=np.float32))
    B = 8
    tables = rng.permutation(B * W).reshape(B, W).astype(np.int32)  # blocks 48.. unused
    lens = np.array([5, 16, 37, 0, 50, 9, 31, 80], np.int32)
    cow = np.array([60, -1, 61, -1, tables[4, 50 // bs], 62, -1, 63], np.int32)  # request 4: own block
    desc = fca.desc_from_shape(shape, nb)
    kn_all = [new_rows(rng, shape, B) for _ in range(4)]

    def run(graph):
        kd, vd = to_device_bf16(k), to_device_bf16(v)
        bt = torch.from_numpy(tables).cuda()
        knd = to_device_bf16(kn_all[0][0])
        vnd = to_device_bf16(kn_all[0][1])
        sl = torch.from_numpy(lens).cuda()
        cw = torch.from_numpy(cow).cuda()
        snaps = []
        if graph:
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(side):
                with torch.cuda.graph(g, stream=side):
                    fca.kv_append(knd, vnd, kd, vd, bt, sl, desc, cow_dst=cw, stream=side)
            torch.cuda.current_stream().wait_stream(side)
        for r in range(4):
            knd.copy_(to_device_bf16(kn_all[r][0]))
            vnd.copy_(to_device_bf16(kn_all[r][1]))
            if graph:
                g.replay()
            else:
                fca.kv_append(knd, vnd, kd, vd, bt, sl, desc, cow_dst=cw)
            torch.cuda.synchronize()
            snaps.append((to_bits(kd), to_bits(vd), bt.cpu().numpy().copy()))
            sl.add_(1)  # eager work between replays: the next token
        return snaps

    say("append graph vs eager")
    eager, graphed = run(False), run(True)
    kk, vv, tt = k, v, tables
    ln = lens.copy()
    for r in range(4):
        kk, vv, tt = KV.append(kk, vv, tt, ln, kn_all[r][0], kn_all[r][1], bs, cow)
        ln = ln + 1
        for snap in (eager[r], graphed[r]):
            assert (snap[0] == kk).all() and (snap[1] == vv).all() and (snap[2] == tt).all(), f"replay {r}"
    assert tt[4, 50 // bs] == tables[4, 50 // bs]


@pytest.mark.parametrize("shape", [GQA, MLA], ids=["gqa", "mla"])
def test_append_layers_share_one_table(shape):
    """Three layers with their own pools and one block table (as the layers
    of a model share the plan): fca_kv_append_layers over three decode steps
    leaves every layer's pools and the table as the oracle's append of each
    layer from the same table, and the decode of every layer over the grown
    caches matches oracle attention.  Appending layer by layer with
    fca_kv_append would rewrite the table after the first layer and leave
    the later layers' copies without the request's earlier tokens."""
    bs = shape.block_size
    n_layers = 3
    tables, lens, k0, v0, free = forked_case(shape, seed=31 + shape.head_dim_qk)
    B = len(lens)
    rng = np.random.default_rng(17)
    nan_k = k0 == BF16_NAN
    nan_v = None if v0 is None else v0 == BF16_NAN
    ks, vs = [k0], [v0]
    for _ in range(1, n_layers):  # same poisoned slots, new values
        k = f32_to_bf16_bits(rng.standard_normal(k0.shape, dtype=np.float32))
        k[nan_k] = BF16_NAN
        ks.append(k)
        if v0 is None:
            vs.append(None)
        else:
            v = f32_to_bf16_bits(rng.standard_normal(v0.shape, dtype=np.float32))
            v[nan_v] = BF16_NAN
            vs.append(v)
    kd = [to_device_bf16(k) for k in ks]
    vd = [to_device_bf16(v) if v is not None else None for v in vs]
    desc = fca.desc_from_shape(shape, k0.shape[0])
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for step in range(3):
        tables, cow = choose_step(tables, lens, bs, free)
        rows = [new_rows(rng, shape, B) for _ in range(n_layers)]
        say("append layers", "mla" if shape.v_aliases_k else "gqa", "step", step, "cow", cow.tolist())
        bt = torch.from_numpy(tables).cuda()
        fca.kv_append_layers(
            [to_device_bf16(r[0]) for r in rows],
            [to_device_bf16(r[1]) if r[1] is not None else None for r in rows],
            list(zip(kd, vd)),
            bt,
            torch.from_numpy(lens).cuda(),
            desc,
            cow_dst=torch.from_numpy(cow).cuda(),
            status=status,
        )
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        new_tables = None
        for l in range(n_layers):
            ks[l], vs[l], t_l = KV.append(ks[l], vs[l], tables, lens, rows[l][0], rows[l][1], bs, cow)
            new_tables = t_l if new_tables is None else new_tables
            assert (t_l == new_tables).all()
            assert (to_bits(kd[l]) == ks[l]).all(), f"step {step} layer {l}: key pool differs"
            if vs[l] is not None:
                assert (to_bits(vd[l]) == vs[l]).all(), f"step {step} layer {l}: value pool differs"
        tables = new_tables
        assert (bt.cpu().numpy() == tables).all(), f"step {step}: block tables differ"
        lens = lens + 1
        p = fca.fca_plan(bt, torch.from_numpy(lens).cuda(), desc)
        qs = [f32_to_bf16_bits(rng.standard_normal((B, shape.num_q_heads, shape.head_dim_qk), dtype=np.float32))
              for _ in range(n_layers)]
        outs = [torch.empty((B, shape.num_q_heads, shape.head_dim_v), dtype=torch.bfloat16, device="cuda")
                for _ in range(n_layers)]
        p.decode_layers([to_device_bf16(q) for q in qs], list(zip(kd, vd)), outs)
        torch.cuda.synchronize()
        for l in range(n_layers):
            ref, _ = A.attend(qs[l], ks[l], vs[l], tables, lens, shape)
            assert_close(bf16_tensor_to_f64(outs[l]), ref, f"step {step} layer {l}")
        say("append layers step", step, "ok")
