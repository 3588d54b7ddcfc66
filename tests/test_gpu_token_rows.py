"""GPU parity for pools of token rows (k_stride_token > 0): the same batches
as the tile-layout tests, their pools rearranged on the host into
[blocks][slots][heads][dims], [blocks][heads][slots][dims] or a padded
variant, decoded through the C ABI and compared with the oracle, which reads
the tile-layout copy.  Appends into a row pool are compared bit for bit with
the oracle's append.  Needs an MI355X."""

from __future__ import annotations

import math
import sys

import numpy as np
import pytest

from oracle import attention as A
from oracle import kv_cache as KV
from tests.helpers import assert_close, assert_lse_close, bf16_tensor_to_f64, to_bits, to_device_bf16
from tests.test_gpu_kv_append import choose_step, forked_case, new_rows
from workloads import CONFIGS, build_batch, fill_values_numpy
from workloads.forest import AttnShape, Config, Node
from workloads.values import BF16_NAN, f32_to_bf16_bits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import shared_prefix_kv_amd as fca  # noqa: E402


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fca.lib()


# ------------------------------------------------- layout conversions ----
# Tile pools are what the oracle reads: keys [nb][H][D/8][bs][8], values
# [nb][H][D][bs].  "Logical" is [nb][H][bs][D].


def logical_k(k):
    nb, H, c, bs, e = k.shape
    return np.ascontiguousarray(k.transpose(0, 1, 3, 2, 4)).reshape(nb, H, bs, c * e)


def logical_v(v):
    return np.ascontiguousarray(v.transpose(0, 1, 3, 2))


def tiles_k(x):
    nb, H, bs, D = x.shape
    return np.ascontiguousarray(x.reshape(nb, H, bs, D // 8, 8).transpose(0, 1, 3, 2, 4))


def tiles_v(x):
    return np.ascontiguousarray(x.transpose(0, 1, 3, 2))


# order: "bthd" = [blocks][slots][heads][dims], "bhtd" = [blocks][heads][slots][dims];
# pad: extra (NaN) dims after each row.
LAYOUTS = {"bthd": ("bthd", 0), "bhtd": ("bhtd", 0), "bthd_padded": ("bthd", 64)}


def to_rows(x, order, pad):
    """Row pool of logical x, and its (block, head, token) strides."""
    nb, H, bs, D = x.shape
    Dp = D + pad
    if order == "bthd":
        buf = np.full((nb, bs, H, Dp), BF16_NAN, np.uint16)
        buf[..., :D] = x.transpose(0, 2, 1, 3)
        return buf, (bs * H * Dp, Dp, H * Dp)
    buf = np.full((nb, H, bs, Dp), BF16_NAN, np.uint16)
    buf[..., :D] = x
    return buf, (H * bs * Dp, bs * Dp, Dp)


def from_rows(buf, order, D):
    """Logical [nb][H][bs][D] of a row pool."""
    x = buf[..., :D]
    return np.ascontiguousarray(x.transpose(0, 2, 1, 3) if order == "bthd" else x)


def rows_desc(shape, nb, ks, vs, cascade=True, auto_fold=True):
    return fca.make_desc(
        shape.num_q_heads, shape.num_kv_heads, shape.head_dim_qk, shape.head_dim_v, shape.block_size, nb, shape.scale,
        v_aliases_k=shape.v_aliases_k, cascade=cascade, auto_fold=auto_fold, token_rows=True, k_strides=ks,
        v_strides=vs,
    )


def decode_rows(b, vn, layout, cascade, auto_fold=True):
    order, pad = LAYOUTS[layout]
    sh = b.shape
    kr, ks = to_rows(logical_k(vn["k"]), order, pad)
    vd, vs = None, None
    if not sh.v_aliases_k:
        vr, vs = to_rows(logical_v(vn["v"]), order, pad)
        vd = to_device_bf16(vr)
    desc = rows_desc(sh, b.num_blocks, ks, vs, cascade=cascade, auto_fold=auto_fold)
    bt = torch.from_numpy(b.block_tables).cuda()
    sl = torch.from_numpy(b.seq_lens).cuda()
    p = fca.fca_plan(bt, sl, desc)
    out = torch.empty((b.batch, sh.num_q_heads, sh.head_dim_v), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((b.batch, sh.num_q_heads), dtype=torch.float32, device="cuda")
    fca.fca_decode(to_device_bf16(vn["q"]), to_device_bf16(kr), vd, p, out=out, lse=lse)
    torch.cuda.synchronize()
    return p, out, lse


def test_conversions_round_trip():
    """The host rearrangements used here are exact permutations."""
    rng = np.random.default_rng(0)
    k = rng.integers(0, 1 << 15, (3, 2, 16, 16, 8), dtype=np.uint16)
    v = rng.integers(0, 1 << 15, (3, 2, 128, 16), dtype=np.uint16)
    assert (tiles_k(logical_k(k)) == k).all() and (tiles_v(logical_v(v)) == v).all()
    # key (blk, h, t, d) sits at [blk, h, d // 8, t, d % 8]
    assert logical_k(k)[2, 1, 5, 43] == k[2, 1, 5, 5, 3]
    assert logical_v(v)[1, 0, 7, 99] == v[1, 0, 99, 7]
    for order, pad in LAYOUTS.values():
        buf, (sb, sh_, st) = to_rows(logical_k(k), order, pad)
        flat = buf.reshape(-1)
        assert flat[2 * sb + 1 * sh_ + 5 * st + 43] == k[2, 1, 5, 5, 3]
        assert (from_rows(buf, order, 128) == logical_k(k)).all()


@pytest.mark.parametrize("layout", list(LAYOUTS))
@pytest.mark.parametrize("name", ["tiny", "llama3_8b"])
def test_decode_gqa_token_rows(name, layout):
    """GQA decode from row pools against the oracle, with every group kept,
    with the library's fold decision and without the cascade."""
    b = build_batch(CONFIGS[name])
    vn = fill_values_numpy(b, poison=True)
    say("token rows", name, layout)
    ref, ref_lse = A.attend(vn["q"], vn["k"], vn["v"], b.block_tables, b.seq_lens, b.shape)
    for cascade, fold in ((True, False), (True, True), (False, True)):
        p, out, lse = decode_rows(b, vn, layout, cascade, auto_fold=fold)
        rep = assert_close(bf16_tensor_to_f64(out), ref, f"{name} rows {layout} cascade={cascade} fold={fold}")
        assert_lse_close(lse.cpu().numpy(), ref_lse, f"{name} rows {layout}")
        say(name, layout, "cascade", cascade, "fold", fold, rep, "groups", p.info.num_groups)


def test_decode_gqa_token_rows_equals_tiles():
    """One plan's schedule over the same values in both layouts: the row
    kernel gathers exactly the tile kernel's operands, so the outputs are
    bitwise equal."""
    b = build_batch(CONFIGS["llama3_8b"])
    vn = fill_values_numpy(b, poison=True)
    bt = torch.from_numpy(b.block_tables).cuda()
    sl = torch.from_numpy(b.seq_lens).cuda()
    p = fca.fca_plan(bt, sl, fca.desc_from_shape(b.shape, b.num_blocks))
    out_t = fca.fca_decode(to_device_bf16(vn["q"]), to_device_bf16(vn["k"]), to_device_bf16(vn["v"]), p)
    _, out_r, _ = decode_rows(b, vn, "bthd", True)
    torch.cuda.synchronize()
    assert torch.equal(out_t, out_r)


@pytest.mark.parametrize("hq,hkv,layout", [(128, 1, "bthd"), (64, 2, "bthd"), (16, 1, "bthd_padded"),
                                           (64, 2, "bhtd")])
def test_decode_mla_token_rows(hq, hkv, layout):
    """Latent cache in rows of 576 dims: two prompts of 4 and 3 blocks with
    3 samples each plus an unshared request, suffixes from 1 token to
    several blocks."""
    shape = AttnShape(hq, hkv, 576, 512, 64, 1 / math.sqrt(576), v_aliases_k=True)
    cfg = Config(
        name=f"mla_rows_{hq}_{hkv}",
        shape=shape,
        trees=[Node(256, samples=3, suffix=(1, 150)), Node(192, samples=3, suffix=(60, 200))],
        singletons=1,
        singleton_len=(1, 130),
        seed=70 + hq + hkv,
    )
    b = build_batch(cfg)
    vn = fill_values_numpy(b, poison=True)
    say("token rows mla", hq, hkv, layout)
    ref, ref_lse = A.attend(vn["q"], vn["k"], vn["v"], b.block_tables, b.seq_lens, shape)
    for cascade in (True, False):
        _, out, lse = decode_rows(b, vn, layout, cascade, auto_fold=False)
        rep = assert_close(bf16_tensor_to_f64(out), ref, f"mla rows hq={hq} hkv={hkv} {layout} cascade={cascade}")
        assert_lse_close(lse.cpu().numpy(), ref_lse, "mla rows")
        say("mla rows", hq, hkv, layout, "cascade", cascade, rep)


GQA = AttnShape(32, 8, 128, 128, 16, 1 / math.sqrt(128))
MLA = AttnShape(16, 1, 576, 512, 64, 1 / math.sqrt(576), v_aliases_k=True)


@pytest.mark.parametrize("shape,layout", [(GQA, "bthd"), (GQA, "bhtd_pad"), (MLA, "bthd")],
                         ids=["gqa_bthd", "gqa_bhtd_padded", "mla_bthd"])
def test_append_token_rows_bitexact(shape, layout):
    """Three decode steps of appends into row pools, with copy-on-write of
    shared partly filled blocks, fresh blocks where a block is full, and
    in-place writes: the pools (read back into tiles) and the block tables
    equal the oracle's append bit for bit, and the grown cache decodes to
    the oracle's attention."""
    order, pad = ("bhtd", 32) if layout == "bhtd_pad" else (layout, 0)
    bs = shape.block_size
    tables, lens, k, v, free = forked_case(shape, seed=31 + shape.head_dim_qk)
    B = len(lens)
    rng = np.random.default_rng(8)
    kr, ks = to_rows(logical_k(k), order, pad)
    kd = to_device_bf16(kr)
    vd, vs = None, None
    if v is not None:
        vr, vs = to_rows(logical_v(v), order, pad)
        vd = to_device_bf16(vr)
    desc = rows_desc(shape, k.shape[0], ks, vs)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for step in range(3):
        tables, cow = choose_step(tables, lens, bs, free)
        kn, vn = new_rows(rng, shape, B)
        say("append rows", layout, "mla" if shape.v_aliases_k else "gqa", "step", step, "cow", cow.tolist())
        bt = torch.from_numpy(tables).cuda()
        fca.kv_append(
            to_device_bf16(kn), to_device_bf16(vn) if vn is not None else None, kd, vd, bt,
            torch.from_numpy(lens).cuda(), desc, cow_dst=torch.from_numpy(cow).cuda(), status=status,
        )
        torch.cuda.synchronize()
        k, v, tables = KV.append(k, v, tables, lens, kn, vn, bs, cow)
        assert int(status.item()) == 0
        assert (bt.cpu().numpy() == tables).all(), f"step {step}: block tables differ"
        kb = to_bits(kd)
        assert (tiles_k(from_rows(kb, order, shape.head_dim_qk)) == k).all(), f"step {step}: key pool differs"
        if pad:
            assert (kb[..., shape.head_dim_qk:] == BF16_NAN).all(), "row padding was written"
        if v is not None:
            assert (tiles_v(from_rows(to_bits(vd), order, shape.head_dim_v)) == v).all(), f"step {step}: values differ"
        lens = lens + 1
        q = f32_to_bf16_bits(rng.standard_normal((B, shape.num_q_heads, shape.head_dim_qk), dtype=np.float32))
        ref, ref_lse = A.attend(q, k, v, tables, lens, shape)
        p = fca.fca_plan(bt, torch.from_numpy(lens).cuda(), desc)
        out = torch.empty((B, shape.num_q_heads, shape.head_dim_v), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((B, shape.num_q_heads), dtype=torch.float32, device="cuda")
        fca.fca_decode(to_device_bf16(q), kd, vd, p, out=out, lse=lse)
        torch.cuda.synchronize()
        rep = assert_close(bf16_tensor_to_f64(out), ref, f"decode after row append step {step}")
        assert_lse_close(lse.cpu().numpy(), ref_lse, "decode after row append")
        say("step", step, rep)


def test_token_rows_layers_graph_no_alloc_and_append_layers():
    """Token-row pools through the other entry points: two layers decoded by
    one fca_decode_layers call captured in a HIP graph (three replays with
    new queries, each equal to an eager call bit for bit), the no-allocation
    decode equal to fca_decode, and fca_kv_append_layers over both layers'
    pools (bit-exact against the oracle's append), all against the oracle."""
    b = build_batch(CONFIGS["llama3_8b"])
    sh = b.shape
    n_layers = 2
    vns = [fill_values_numpy(b, poison=True) for _ in range(n_layers)]  # batch.rng advances per layer
    caches, descs = [], []
    for vn in vns:
        kr, ks = to_rows(logical_k(vn["k"]), "bthd", 0)
        vr, vs = to_rows(logical_v(vn["v"]), "bthd", 0)
        caches.append((to_device_bf16(kr), to_device_bf16(vr)))
        descs.append(rows_desc(sh, b.num_blocks, ks, vs))
    desc = descs[0]
    bt = torch.from_numpy(b.block_tables).cuda()
    sl = torch.from_numpy(b.seq_lens).cuda()
    p = fca.fca_plan(bt, sl, desc)
    shape_out = (b.batch, sh.num_q_heads, sh.head_dim_v)
    q_static = [to_device_bf16(vn["q"]) for vn in vns]
    outs_g = [torch.empty(shape_out, dtype=torch.bfloat16, device="cuda") for _ in range(n_layers)]
    outs_e = [torch.empty_like(o) for o in outs_g]
    ws = p.decode_workspace(q_static[0].device)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        p.decode_layers(q_static, caches, outs_g, workspace=ws, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        p.decode_layers(q_static, caches, outs_g, workspace=ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(17)
    for rep in range(3):
        q_new = [f32_to_bf16_bits(rng.standard_normal(vn["q"].shape, dtype=np.float32)) for vn in vns]
        for qs_, qn in zip(q_static, q_new):
            qs_.copy_(to_device_bf16(qn))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        p.decode_layers([to_device_bf16(qn) for qn in q_new], caches, outs_e, workspace=torch.empty_like(ws))
        torch.cuda.synchronize()
        for l in range(n_layers):
            assert torch.equal(outs_g[l].view(torch.int16), outs_e[l].view(torch.int16)), f"replay {rep} layer {l}"
    for l in range(n_layers):
        ref, _ = A.attend(q_new[l], vns[l]["k"], vns[l]["v"], b.block_tables, b.seq_lens, sh)
        rep = assert_close(bf16_tensor_to_f64(outs_g[l]), ref, f"rows layers, layer {l}")
        say("rows decode_layers layer", l, rep)
    del graph
    # no allocation: equal to fca_decode on the same plan
    out_w = torch.empty(shape_out, dtype=torch.bfloat16, device="cuda")
    out_s = torch.empty(shape_out, dtype=torch.bfloat16, device="cuda")
    p.decode(q_static[0], caches[0][0], caches[0][1], out=out_w)
    p.decode_no_alloc(q_static[0], caches[0][0], caches[0][1], out_s)
    torch.cuda.synchronize()
    assert torch.equal(out_w.view(torch.int16), out_s.view(torch.int16))
    # one appended token per request into both layers' row pools, no copies
    tables = np.pad(b.block_tables, ((0, 0), (0, 1)))  # room for a block past the longest request
    lens = b.seq_lens.copy()
    free = sorted(set(range(b.num_blocks)) - set(int(x) for x in tables.ravel()))
    for i, L in enumerate(lens):
        if L % sh.block_size == 0:
            tables[i, L // sh.block_size] = free.pop()
    knews = [f32_to_bf16_bits(rng.standard_normal((b.batch, sh.num_kv_heads, 128), dtype=np.float32))
             for _ in range(n_layers)]
    vnews = [f32_to_bf16_bits(rng.standard_normal((b.batch, sh.num_kv_heads, 128), dtype=np.float32))
             for _ in range(n_layers)]
    bt2 = torch.from_numpy(tables).cuda()
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    fca.kv_append_layers([to_device_bf16(k) for k in knews], [to_device_bf16(v) for v in vnews], caches, bt2,
                         torch.from_numpy(lens).cuda(), desc, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for l in range(n_layers):
        k2, v2, t2 = KV.append(vns[l]["k"], vns[l]["v"], tables, lens, knews[l], vnews[l], sh.block_size, None)
        assert (bt2.cpu().numpy() == t2).all()
        assert (tiles_k(from_rows(to_bits(caches[l][0]), "bthd", 128)) == k2).all(), f"layer {l}: keys"
        assert (tiles_v(from_rows(to_bits(caches[l][1]), "bthd", 128)) == v2).all(), f"layer {l}: values"
    say("rows append layers ok")
