"""fca_decode_no_alloc (the decode with the library's static per-device
scratch instead of a workspace) against fca_decode through the C ABI: equal
bit for bit on two calls in a row, the second with a smaller batch, and a
plan too large for the scratch rejected before any launch.  Needs an MI355X."""

from __future__ import annotations

import math
import sys

import numpy as np
import pytest

from workloads import CONFIGS, build_batch
from workloads.forest import AttnShape, Config, Node
from workloads.values import fill_values_torch

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


def case(cfg):
    b = build_batch(cfg)
    vals = fill_values_torch(b, "cuda", seed=cfg.seed, poison=True)
    bt = torch.from_numpy(b.block_tables).cuda()
    sl = torch.from_numpy(b.seq_lens).cuda()
    return b, vals, bt, sl


def both(b, vals, p):
    sh = b.shape
    shape = (b.batch, sh.num_q_heads, sh.head_dim_v)
    out_w = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    lse_w = torch.empty((b.batch, sh.num_q_heads), dtype=torch.float32, device="cuda")
    out_s = torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    lse_s = torch.full((b.batch, sh.num_q_heads), float("nan"), dtype=torch.float32, device="cuda")
    p.decode(vals["q"], vals["k"], vals["v"], out=out_w, lse=lse_w)
    p.decode_no_alloc(vals["q"], vals["k"], vals["v"], out_s, lse_s)
    torch.cuda.synchronize()
    return (out_w, lse_w), (out_s, lse_s)


def test_no_alloc_matches_decode_two_calls_second_smaller():
    for name in ("llama3_8b", "tiny"):  # the second call is the smaller batch
        b, vals, bt, sl = case(CONFIGS[name])
        p = fca.fca_plan(bt, sl, fca.desc_from_shape(b.shape, b.num_blocks))
        say("no-alloc decode", name, "B", b.batch, "scratch bytes", p.info.decode_workspace_bytes)
        (ow, lw), (os_, ls) = both(b, vals, p)
        assert torch.equal(ow.view(torch.int16), os_.view(torch.int16)), f"{name}: output differs"
        assert torch.equal(lw, ls), f"{name}: lse differs"
        del vals


def test_no_alloc_latent_cache_and_float32_output():
    shape = AttnShape(128, 1, 576, 512, 64, 1 / math.sqrt(576), v_aliases_k=True)
    cfg = Config(name="mla_no_alloc", shape=shape, trees=[Node(1024, samples=4, suffix=(1, 150))],
                 singletons=2, singleton_len=(1, 200), seed=61)
    b, vals, bt, sl = case(cfg)
    p = fca.fca_plan(bt, sl, fca.desc_from_shape(shape, b.num_blocks))
    say("no-alloc decode, latent cache, B", b.batch)
    (ow, lw), (os_, ls) = both(b, vals, p)
    assert torch.equal(ow.view(torch.int16), os_.view(torch.int16))
    assert torch.equal(lw, ls)
    b2, vals2, bt2, sl2 = case(CONFIGS["tiny"])
    p2 = fca.fca_plan(bt2, sl2, fca.desc_from_shape(b2.shape, b2.num_blocks, out_f32=True))
    sh = b2.shape
    o1 = torch.empty((b2.batch, sh.num_q_heads, sh.head_dim_v), dtype=torch.float32, device="cuda")
    o2 = torch.empty_like(o1)
    p2.decode(vals2["q"], vals2["k"], vals2["v"], out=o1)
    p2.decode_no_alloc(vals2["q"], vals2["k"], vals2["v"], o2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_no_alloc_rejects_plans_larger_than_the_scratch():
    # 512 unshared latent-cache requests of 8 tokens: 512 x 128 partial rows of
    # 2 KiB, above the 64 MiB scratch
    shape = AttnShape(128, 1, 576, 512, 64, 1 / math.sqrt(576), v_aliases_k=True)
    B = 512
    tables = np.arange(B, dtype=np.int32).reshape(B, 1)
    lens = np.full(B, 8, np.int32)
    p = fca.fca_plan(torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda(),
                     fca.desc_from_shape(shape, B))
    assert p.info.decode_workspace_bytes > 64 << 20
    q = torch.zeros((B, 128, 576), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, 1, 72, 64, 8), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((B, 128, 512), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fca.FcaError) as e:
        p.decode_no_alloc(q, k, None, out)
    assert e.value.status == 3
    torch.cuda.synchronize()
    assert (out.float() == 0).all()  # nothing was launched
