"""C ABI checks that need no GPU: the library loads, exports every declared
symbol, and rejects bad arguments before touching the device."""

import ctypes
import os
import re

import pytest

import shared_prefix_kv_amd as fca

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(fca.LIB_PATH), reason="libfca.so not built")


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "fca.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fca_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    L = fca.lib()
    decl = declared_symbols()
    assert decl, "no declarations parsed"
    for name in decl:
        assert hasattr(L, name), name
    assert sorted(decl) == sorted(fca.EXPORTED)
    assert fca.version() == "0.1.0"


def gqa_desc(**kw):
    args = dict(
        num_q_heads=32, num_kv_heads=8, head_dim_qk=128, head_dim_v=128, block_size=16, num_blocks=100, scale=0.088
    )
    args.update(kw)
    return fca.make_desc(**args)


def status_of(fn, *a):
    return fn(*a)


def test_workspace_size_and_validation():
    n = fca.plan_workspace_size(64, 320, gqa_desc())
    assert n > 64 * 320 * 4
    assert fca.plan_workspace_size(0, 1, gqa_desc()) > 0
    with pytest.raises(fca.FcaError) as e:
        fca.plan_workspace_size(64, 320, gqa_desc(head_dim_qk=96, head_dim_v=96))
    assert e.value.status == 2
    with pytest.raises(fca.FcaError) as e:
        fca.plan_workspace_size(64, 320, gqa_desc(num_q_heads=30))
    assert e.value.status == 1
    with pytest.raises(fca.FcaError) as e:
        fca.plan_workspace_size(64, 320, gqa_desc(num_q_heads=64, num_kv_heads=2))  # ratio 32
    assert e.value.status == 2
    with pytest.raises(fca.FcaError) as e:
        fca.plan_workspace_size(-1, 320, gqa_desc())
    assert e.value.status == 1
    with pytest.raises(fca.FcaError) as e:
        fca.plan_workspace_size(9000, 320, gqa_desc())
    assert e.value.status == 1
    with pytest.raises(fca.FcaError) as e:
        fca.plan_workspace_size(4, 0, gqa_desc())
    assert e.value.status == 1
    d = gqa_desc()
    d.reserved = 3
    with pytest.raises(fca.FcaError):
        fca.plan_workspace_size(4, 4, d)
    d = gqa_desc(scale=float("nan"))
    with pytest.raises(fca.FcaError):
        fca.plan_workspace_size(4, 4, d)
    d = gqa_desc()
    d.flags = 1 << 10
    with pytest.raises(fca.FcaError):
        fca.plan_workspace_size(4, 4, d)
    d = gqa_desc()
    d.k_stride_head = 100  # tiles would overlap
    with pytest.raises(fca.FcaError):
        fca.plan_workspace_size(4, 4, d)


def test_token_row_descriptors():
    """Token-row pools: the default strides of both orders are accepted, and
    mixed, negative, short or misaligned token strides are rejected."""
    d = gqa_desc(token_rows=True)
    assert (d.k_stride_block, d.k_stride_head, d.k_stride_token) == (16 * 8 * 128, 128, 8 * 128)
    assert (d.v_stride_block, d.v_stride_head, d.v_stride_token) == (16 * 8 * 128, 128, 8 * 128)
    fca.plan_workspace_size(4, 4, d)
    fca.plan_workspace_size(4, 4, gqa_desc(token_rows=True, k_strides=(8 * 16 * 128, 16 * 128, 128),
                                           v_strides=(8 * 16 * 128, 16 * 128, 128)))
    tiles = gqa_desc()
    assert tiles.k_stride_token == 0 and tiles.v_stride_token == 0
    bad = []
    d = gqa_desc(token_rows=True)
    d.v_stride_token = 0  # keys in rows, values in tiles
    bad.append(d)
    d = gqa_desc()
    d.v_stride_token = 1024  # the other way round
    bad.append(d)
    d = gqa_desc(token_rows=True)
    d.k_stride_token = -1024
    bad.append(d)
    d = gqa_desc(token_rows=True)
    d.k_stride_token = 64  # shorter than a row
    bad.append(d)
    d = gqa_desc(token_rows=True)
    d.v_stride_token = 1028  # not a multiple of 8 elements
    bad.append(d)
    d = gqa_desc(token_rows=True)
    d.k_stride_head = 0
    bad.append(d)
    for d in bad:
        with pytest.raises(fca.FcaError) as e:
            fca.plan_workspace_size(4, 4, d)
        assert e.value.status == 1
    mla = dict(num_q_heads=128, num_kv_heads=1, head_dim_qk=576, head_dim_v=512, block_size=64, num_blocks=10,
               scale=0.04, v_aliases_k=True, token_rows=True)
    d = fca.make_desc(**mla)
    assert (d.k_stride_block, d.k_stride_head, d.k_stride_token) == (64 * 576, 576, 576)
    assert d.v_stride_token == 0
    fca.plan_workspace_size(4, 4, d)
    for field, value in (("k_stride_token", 520), ("k_stride_token", (1 << 20) + 8), ("k_stride_block", 8),
                         ("k_stride_head", -8)):
        d = fca.make_desc(**mla)
        setattr(d, field, value)
        with pytest.raises(fca.FcaError) as e:
            fca.plan_workspace_size(4, 4, d)
        assert e.value.status == 1, field


def test_create_rejects_bad_args_before_device():
    L = fca.lib()
    d = gqa_desc()
    h = ctypes.c_void_p()
    fake = ctypes.c_void_p(0x1000)
    # NULL tables with batch > 0
    st = L.fca_plan_create(None, 4, fake, 2, 4, ctypes.byref(d), fake, 1 << 20, None, ctypes.byref(h))
    assert st == 1 and b"NULL" in L.fca_last_error()
    # stride smaller than width
    st = L.fca_plan_create(fake, 2, fake, 2, 4, ctypes.byref(d), fake, 1 << 20, None, ctypes.byref(h))
    assert st == 1
    # misaligned workspace
    st = L.fca_plan_create(fake, 4, fake, 2, 4, ctypes.byref(d), ctypes.c_void_p(0x1004), 1 << 20, None, ctypes.byref(h))
    assert st == 3
    # workspace too small
    st = L.fca_plan_create(fake, 4, fake, 2, 4, ctypes.byref(d), fake, 16, None, ctypes.byref(h))
    assert st == 3 and b"needs" in L.fca_last_error()
    # NULL out handle
    st = L.fca_plan_create(fake, 4, fake, 2, 4, ctypes.byref(d), fake, 1 << 20, None, None)
    assert st == 1
    assert not h.value


def test_decode_and_info_reject_null_plan():
    L = fca.lib()
    assert L.fca_decode(None, None, None, None, None, None, None, 0, None) == 1
    assert L.fca_decode_no_alloc(None, None, None, None, None, None, None) == 1
    info = fca.PlanInfo()
    assert L.fca_plan_get_info(None, ctypes.byref(info)) == 1
    assert L.fca_plan_export(None, None, None, None) == 1
    assert L.fca_plan_export_schedule(None, None, None, None, None) == 1
    assert L.fca_profile_enable(None, 1) == 1
    assert L.fca_profile_read(None, None) == 1
    prof = fca.Profile()
    assert L.fca_time_launches(None, None, None, None, 1, 1, None, None, None, 0, None, ctypes.byref(prof)) == 1


def test_merge_states_validation_before_device():
    """fca_merge_states rejects bad arguments without touching the device."""
    L = fca.lib()
    assert L.fca_merge_states(0, None, None, 4, 4, 128, None, None, 0, None) == 1  # no states
    assert L.fca_merge_states(17, None, None, 4, 4, 128, None, None, 0, None) == 1  # too many
    assert L.fca_merge_states(2, None, None, 4, 4, 64, None, None, 0, None) == 2  # head_dim not built
    assert L.fca_merge_states(2, None, None, 4, 4, 128, None, None, 8, None) == 1  # unknown flag
    assert L.fca_merge_states(2, None, None, 4, 4, 128, None, None, 0, None) == 1  # NULL arrays
    assert L.fca_merge_states(2, None, None, 0, 4, 128, None, None, 0, None) == 0  # empty batch: nothing to do
    L.fca_plan_destroy(None)  # no-op


def test_kv_append_validation_before_device():
    """fca_kv_append rejects bad arguments without touching the device; an
    empty batch launches nothing."""
    L = fca.lib()
    d = fca.make_desc(32, 8, 128, 128, 16, 64, 0.088)
    dp = ctypes.byref(d)
    odd = ctypes.c_void_p(0x1008)  # not 16-byte aligned
    ok = ctypes.c_void_p(0x1000)
    assert L.fca_kv_append(None, ok, ok, ok, ok, ok, 4, 4, ok, None, None, 2, None) == 1  # no desc
    assert L.fca_kv_append(dp, ok, ok, ok, ok, ok, 4, 4, ok, None, None, -1, None) == 1  # negative batch
    assert L.fca_kv_append(dp, ok, ok, ok, ok, ok, 4, 4, ok, None, None, 8193, None) == 1  # batch too large
    assert L.fca_kv_append(dp, ok, ok, ok, ok, ok, 4, 0, ok, None, None, 2, None) == 1  # no table width
    assert L.fca_kv_append(dp, ok, ok, ok, ok, ok, 3, 4, ok, None, None, 2, None) == 1  # rows overlap
    assert L.fca_kv_append(dp, ok, None, ok, ok, ok, 4, 4, ok, None, None, 2, None) == 1  # no v_new
    assert L.fca_kv_append(dp, ok, ok, ok, ok, None, 4, 4, ok, None, None, 2, None) == 1  # no table
    assert L.fca_kv_append(dp, odd, ok, ok, ok, ok, 4, 4, ok, None, None, 2, None) == 1  # misaligned row
    assert L.fca_kv_append(dp, ok, ok, ok, odd, ok, 4, 4, ok, None, None, 2, None) == 1  # misaligned pool
    assert L.fca_kv_append(dp, ok, ok, ok, ok, ok, 4, 4, ok, None, None, 0, None) == 0  # nothing to do
    bad = fca.make_desc(32, 8, 64, 64, 16, 64, 0.088)
    assert L.fca_kv_append(ctypes.byref(bad), ok, ok, ok, ok, ok, 4, 4, ok, None, None, 2, None) == 2  # shape
    mla = fca.make_desc(128, 1, 576, 512, 64, 64, 0.07, v_aliases_k=True)
    assert L.fca_kv_append(ctypes.byref(mla), ok, None, ok, None, ok, 4, 4, ok, None, None, 0, None) == 0


def test_struct_layouts_match_header(tmp_path):
    """ctypes mirrors have the sizes and field offsets a C compiler gives the header."""
    import shutil
    import subprocess

    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    structs = {
        "fca_attn_desc": fca.AttnDesc,
        "fca_plan_info": fca.PlanInfo,
        "fca_group_record": fca.GroupRecord,
        "fca_work_item": fca.WorkItem,
        "fca_profile": fca.Profile,
    }
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "fca.h"', "int main(void) {"]
    for cname, py in structs.items():
        lines.append(f'  printf("{cname} %zu\\n", sizeof({cname}));')
        for fname, _ in py._fields_:
            lines.append(f'  printf("{cname}.{fname} %zu\\n", offsetof({cname}, {fname}));')
    lines.append("  return 0; }")
    src = tmp_path / "sizes.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "sizes"
    subprocess.run([cc, "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = dict(l.split() for l in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.splitlines())
    for cname, py in structs.items():
        assert int(got[cname]) == ctypes.sizeof(py), cname
        for fname, _ in py._fields_:
            assert int(got[f"{cname}.{fname}"]) == getattr(py, fname).offset, (cname, fname)


def test_layers_and_probe_validation_before_device():
    """fca_decode_layers, fca_kv_append_layers and the two measurement probes
    reject bad arguments without touching the device; zero layers or an empty
    batch launch nothing."""
    L = fca.lib()
    ok = ctypes.c_void_p(0x1000)
    odd = ctypes.c_void_p(0x1008)
    assert L.fca_decode_layers(None, 1, None, None, None, None, None, None, 0, None) == 1  # no plan
    d = fca.make_desc(32, 8, 128, 128, 16, 64, 0.088)
    dp = ctypes.byref(d)
    one = lambda p: (ctypes.c_void_p * 1)(p)
    arr = one(ok)
    assert L.fca_kv_append_layers(None, 1, arr, arr, arr, arr, ok, 4, 4, ok, None, None, 2, None) == 1  # no desc
    assert L.fca_kv_append_layers(dp, -1, arr, arr, arr, arr, ok, 4, 4, ok, None, None, 2, None) == 1  # n < 0
    assert L.fca_kv_append_layers(dp, 0, None, None, None, None, ok, 4, 4, ok, None, None, 2, None) == 0  # no layers
    assert L.fca_kv_append_layers(dp, 1, None, arr, arr, arr, ok, 4, 4, ok, None, None, 2, None) == 1  # no k_new array
    assert L.fca_kv_append_layers(dp, 1, one(None), arr, arr, arr, ok, 4, 4, ok, None, None, 2, None) == 1  # NULL entry
    assert b"layer 0" in L.fca_last_error()
    assert L.fca_kv_append_layers(dp, 1, arr, arr, one(odd), arr, ok, 4, 4, ok, None, None, 2, None) == 1  # misaligned
    assert L.fca_kv_append_layers(dp, 1, arr, arr, arr, arr, ok, 4, 4, ok, None, None, 0, None) == 0  # empty batch
    g = ctypes.c_double()
    assert L.fca_measure_read_bandwidth(None, 1, 1 << 20, 1, None, ctypes.byref(g)) == 1
    assert L.fca_measure_read_bandwidth(arr, 0, 1 << 20, 1, None, ctypes.byref(g)) == 1
    assert L.fca_measure_read_bandwidth(arr, 1, 1000, 1, None, ctypes.byref(g)) == 1  # not a multiple of 16
    assert L.fca_measure_read_bandwidth(one(odd), 1, 1 << 20, 1, None, ctypes.byref(g)) == 1
    assert L.fca_measure_read_bandwidth(arr, 1, 1 << 20, 0, None, ctypes.byref(g)) == 1
    assert L.fca_measure_mfma_rate(fca.FCA_MFMA_BF16, 16, None, None) == 1  # no result pointer
    assert L.fca_measure_mfma_rate(7, 16, None, ctypes.byref(g)) == 1  # unknown operand type
    assert L.fca_measure_mfma_rate(fca.FCA_MFMA_F16, 0, None, ctypes.byref(g)) == 1
    assert L.fca_measure_mfma_rate(fca.FCA_MFMA_F16, (1 << 20) + 1, None, ctypes.byref(g)) == 1
