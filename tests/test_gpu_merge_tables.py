"""The two layouts of the plan's merge tables give the same decode, bit for
bit: the fixed-stride table (the default whenever every (request, head) has
at most 64 partial rows, as on all five workloads) and the packed table with
a span per (request, head) (forced here with the FCA_TUNE_MERGE_PACKED
knob; plans whose pairs have more rows use it by themselves).  Needs an
MI355X."""

from __future__ import annotations

import os
import sys

import pytest

from workloads import CONFIGS, build_batch
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


def plan_with(batch, bt, sl, packed):
    old = os.environ.get("FCA_TUNE_MERGE_PACKED")
    try:
        if packed:
            os.environ["FCA_TUNE_MERGE_PACKED"] = "1"
        else:
            os.environ.pop("FCA_TUNE_MERGE_PACKED", None)
        return fca.fca_plan(bt, sl, fca.desc_from_shape(batch.shape, batch.num_blocks))
    finally:
        if old is None:
            os.environ.pop("FCA_TUNE_MERGE_PACKED", None)
        else:
            os.environ["FCA_TUNE_MERGE_PACKED"] = old


@pytest.mark.parametrize("name", ["tiny", "llama3_8b", "long_rl", "forest_mixed", "mla"])
def test_strided_and_packed_merge_tables_agree(name):
    b = build_batch(CONFIGS[name])
    sh = b.shape
    say("merge tables", name)
    vals = fill_values_torch(b, "cuda", seed=11, poison=False)
    bt = torch.from_numpy(b.block_tables).cuda()
    sl = torch.from_numpy(b.seq_lens).cuda()
    res = {}
    for packed in (False, True):
        p = plan_with(b, bt, sl, packed)
        out = torch.empty((b.batch, sh.num_q_heads, sh.head_dim_v), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((b.batch, sh.num_q_heads), dtype=torch.float32, device="cuda")
        fca.fca_decode(vals["q"], vals["k"], vals["v"], p, out=out, lse=lse)
        torch.cuda.synchronize()
        res[packed] = (p.export_schedule()["sources"], out.view(torch.int16).cpu(), lse.view(torch.int32).cpu())
        del p
    assert res[False][0] == res[True][0]  # the same rows, in the same order, for every (request, head)
    assert torch.equal(res[False][1], res[True][1])
    assert torch.equal(res[False][2], res[True][2])
    del vals
    torch.cuda.empty_cache()
