"""Python binding of libfca (Forest Cascade Attention decode on gfx950).

Argument marshalling only: every step of the decode path (discovery, grouped
pass, per-request pass, merge) runs in the HIP kernels of libfca.so; torch is
used for device memory and the current stream.  Importing works without a
GPU; calls that reach the device need one.  There is no fallback: if
libfca.so is missing, ``lib()`` raises.
"""

from __future__ import annotations

import ctypes
import time
import os
from dataclasses import dataclass
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfca.so")

FCA_OK = 0
STATUS_NAMES = {
    0: "FCA_OK",
    1: "FCA_ERR_INVALID_ARG",
    2: "FCA_ERR_UNSUPPORTED",
    3: "FCA_ERR_WORKSPACE",
    4: "FCA_ERR_BAD_TABLE",
    5: "FCA_ERR_HIP",
    6: "FCA_ERR_HOST_ALLOC",
}
FCA_PLAN_DISABLE_CASCADE = 1
FCA_PLAN_SEPARATE_PASSES = 2
FCA_PLAN_OUT_F32 = 4
FCA_PLAN_AUTO_FOLD = 8  # the default; accepted, no effect
FCA_PLAN_KEEP_GROUPS = 16
FCA_MERGE_OUT_F32 = 1
FCA_APPEND_BAD_LEN = 1
FCA_APPEND_BAD_BLOCK = 2
FCA_APPEND_BAD_COW = 4

EXPORTED = [
    "fca_plan_workspace_size",
    "fca_plan_create",
    "fca_plan_get_info",
    "fca_decode",
    "fca_decode_layers",
    "fca_decode_no_alloc",
    "fca_plan_export",
    "fca_plan_export_schedule",
    "fca_plan_export_folded",
    "fca_profile_enable",
    "fca_profile_read",
    "fca_time_launches",
    "fca_measure_read_bandwidth",
    "fca_measure_mfma_rate",
    "fca_merge_states",
    "fca_kv_append",
    "fca_kv_append_layers",
    "fca_plan_destroy",
    "fca_last_error",
    "fca_version",
]


class FcaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class AttnDesc(ctypes.Structure):
    _fields_ = [
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim_qk", ctypes.c_int32),
        ("head_dim_v", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("k_stride_block", ctypes.c_int64),
        ("k_stride_head", ctypes.c_int64),
        ("v_stride_block", ctypes.c_int64),
        ("v_stride_head", ctypes.c_int64),
        ("k_stride_token", ctypes.c_int64),
        ("v_stride_token", ctypes.c_int64),
        ("v_aliases_k", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("flags", ctypes.c_uint32),
        ("reserved", ctypes.c_int32),
    ]


class PlanInfo(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_groups", ctypes.c_int32),
        ("max_depth", ctypes.c_int32),
        ("num_grouped_items", ctypes.c_int32),
        ("num_suffix_items", ctypes.c_int32),
        ("num_merge_sources", ctypes.c_int32),
        ("num_partial_rows", ctypes.c_int64),
        ("logical_tokens", ctypes.c_int64),
        ("unique_tokens", ctypes.c_int64),
        ("decode_workspace_bytes", ctypes.c_size_t),
        ("num_folded_groups", ctypes.c_int32),
    ]


class GroupRecord(ctypes.Structure):
    _fields_ = [
        ("depth", ctypes.c_int32),
        ("parent", ctypes.c_int32),
        ("block_begin", ctypes.c_int32),
        ("block_end", ctypes.c_int32),
        ("member_begin", ctypes.c_int32),
        ("member_count", ctypes.c_int32),
    ]


class WorkItem(ctypes.Structure):
    _fields_ = [
        ("request", ctypes.c_int32),
        ("tok_begin", ctypes.c_int32),
        ("tok_end", ctypes.c_int32),
        ("kv_head", ctypes.c_int32),
        ("member_off", ctypes.c_int32),
        ("ncols", ctypes.c_int32),
        ("col0", ctypes.c_int32),
        ("col1", ctypes.c_int32),
        ("part_base", ctypes.c_int32),
        ("kv_heads", ctypes.c_int32),
        ("stripes", ctypes.c_int32),
        ("flags", ctypes.c_int32),
    ]


class Profile(ctypes.Structure):
    _fields_ = [
        ("attention_ms", ctypes.c_double),
        ("grouped_ms", ctypes.c_double),
        ("suffix_ms", ctypes.c_double),
        ("merge_ms", ctypes.c_double),
        ("decode_ms", ctypes.c_double),
        ("calls", ctypes.c_int64),
    ]


_lib = None


def lib():
    """Load libfca.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FileNotFoundError(
                f"{LIB_PATH} is missing: build it with `python -m shared_prefix_kv_amd.build`"
            )
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.fca_plan_workspace_size.argtypes = [i32, i32, ctypes.POINTER(AttnDesc), ctypes.POINTER(sz)]
        L.fca_plan_create.argtypes = [vp, i64, vp, i32, i32, ctypes.POINTER(AttnDesc), vp, sz, vp, ctypes.POINTER(vp)]
        L.fca_plan_get_info.argtypes = [vp, ctypes.POINTER(PlanInfo)]
        L.fca_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.fca_decode_layers.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.fca_decode_no_alloc.argtypes = [vp, vp, vp, vp, vp, vp, vp]
        L.fca_plan_export.argtypes = [vp, vp, vp, vp]
        L.fca_plan_export_schedule.argtypes = [vp, vp, vp, vp, vp]
        L.fca_plan_export_folded.argtypes = [vp, vp]
        L.fca_profile_enable.argtypes = [vp, i32]
        L.fca_profile_read.argtypes = [vp, ctypes.POINTER(Profile)]
        L.fca_time_launches.argtypes = [vp, vp, vp, vp, i32, i32, vp, vp, vp, sz, vp, ctypes.POINTER(Profile)]
        L.fca_measure_read_bandwidth.argtypes = [vp, i32, sz, i32, vp, ctypes.POINTER(ctypes.c_double)]
        L.fca_measure_mfma_rate.argtypes = [i32, i32, vp, ctypes.POINTER(ctypes.c_double)]
        L.fca_merge_states.argtypes = [i32, vp, vp, i32, i32, i32, vp, vp, ctypes.c_uint32, vp]
        L.fca_kv_append.argtypes = [ctypes.POINTER(AttnDesc), vp, vp, vp, vp, vp, i64, i32, vp, vp, vp, i32, vp]
        L.fca_kv_append_layers.argtypes = [ctypes.POINTER(AttnDesc), i32, vp, vp, vp, vp, vp, i64, i32, vp, vp, vp, i32, vp]
        L.fca_plan_destroy.argtypes = [vp]
        L.fca_plan_destroy.restype = None
        L.fca_last_error.restype = ctypes.c_char_p
        L.fca_version.restype = ctypes.c_char_p
        for name in EXPORTED:
            if name not in ("fca_plan_destroy", "fca_last_error", "fca_version"):
                getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status: int):
    if status != FCA_OK:
        raise FcaError(status, lib().fca_last_error().decode())


def make_desc(
    num_q_heads,
    num_kv_heads,
    head_dim_qk,
    head_dim_v,
    block_size,
    num_blocks,
    scale,
    v_aliases_k=False,
    cascade=True,
    k_strides=None,
    v_strides=None,
    separate_passes=False,
    out_f32=False,
    auto_fold=True,
    token_rows=False,
) -> AttnDesc:
    """Descriptor for one of the two documented cache layouts.

    Tiles (default): ``k_strides`` / ``v_strides`` are (block, head) strides,
    default dense pools ``[num_blocks][num_kv_heads][tile]``.
    Token rows (``token_rows=True``): they are (block, head, token) strides,
    default ``[num_blocks][block_size][num_kv_heads][head_dim]``.

    ``auto_fold=False`` keeps every discovered group (FCA_PLAN_KEEP_GROUPS);
    by default the library folds groups that cannot pay for their partial
    rows (GQA caches)."""
    d = AttnDesc()
    d.num_q_heads, d.num_kv_heads = num_q_heads, num_kv_heads
    d.head_dim_qk, d.head_dim_v = head_dim_qk, head_dim_v
    d.block_size, d.num_blocks = block_size, num_blocks

    def strides(given, dim):
        if token_rows:
            return tuple(given) if given else (block_size * num_kv_heads * dim, dim, num_kv_heads * dim)
        return tuple(given) + (0,) if given else (num_kv_heads * dim * block_size, dim * block_size, 0)

    d.k_stride_block, d.k_stride_head, d.k_stride_token = strides(k_strides, head_dim_qk)
    if v_aliases_k:
        d.v_stride_block, d.v_stride_head, d.v_stride_token = d.k_stride_block, d.k_stride_head, 0
    else:
        d.v_stride_block, d.v_stride_head, d.v_stride_token = strides(v_strides, head_dim_v)
    d.v_aliases_k = int(bool(v_aliases_k))
    d.scale = float(scale)
    d.flags = (
        (0 if cascade else FCA_PLAN_DISABLE_CASCADE)
        | (FCA_PLAN_SEPARATE_PASSES if separate_passes else 0)
        | (FCA_PLAN_OUT_F32 if out_f32 else 0)
        | (0 if auto_fold else FCA_PLAN_KEEP_GROUPS)
    )
    d.reserved = 0
    return d


def desc_from_shape(
    shape, num_blocks, cascade=True, separate_passes=False, out_f32=False, auto_fold=True, token_rows=False
) -> AttnDesc:
    return make_desc(
        shape.num_q_heads,
        shape.num_kv_heads,
        shape.head_dim_qk,
        shape.head_dim_v,
        shape.block_size,
        num_blocks,
        shape.scale,
        v_aliases_k=shape.v_aliases_k,
        cascade=cascade,
        separate_passes=separate_passes,
        out_f32=out_f32,
        auto_fold=auto_fold,
        token_rows=token_rows,
    )


def plan_workspace_size(batch: int, max_blocks: int, desc: AttnDesc) -> int:
    n = ctypes.c_size_t()
    _check(lib().fca_plan_workspace_size(batch, max_blocks, ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def _stream_ptr(stream):
    import torch

    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _pool_extent(d: AttnDesc, stride_block, stride_head, stride_token, dim):
    """Elements a pool of ``d.num_blocks`` blocks spans: the end of its last
    tile, or of its last token row."""
    last = (d.num_blocks - 1) * stride_block + (d.num_kv_heads - 1) * stride_head
    if stride_token:
        return last + (d.block_size - 1) * stride_token + dim
    return last + dim * d.block_size


def _span(t):
    """Elements from the tensor's first element to the end of its storage
    (what a kernel given its data pointer may read)."""
    return t.untyped_storage().nbytes() // t.element_size() - t.storage_offset()


def _check_pool(d: AttnDesc, k_cache, v_cache):
    """The pools a call reads or writes: bf16, 16-byte aligned, and large
    enough for every block ID the descriptor allows (the C ABI cannot see
    sizes; a short pool would be read past its end)."""
    import torch

    assert k_cache is not None and k_cache.dtype == torch.bfloat16, "k_cache must be a bf16 tensor"
    assert k_cache.data_ptr() % 16 == 0, "k_cache must be 16-byte aligned"
    need_k = _pool_extent(d, d.k_stride_block, d.k_stride_head, d.k_stride_token, d.head_dim_qk)
    assert _span(k_cache) >= need_k, f"k_cache spans {_span(k_cache)} elements, the descriptor needs {need_k}"
    if not d.v_aliases_k:
        assert v_cache is not None and v_cache.dtype == torch.bfloat16, "v_cache must be a bf16 tensor"
        assert v_cache.data_ptr() % 16 == 0, "v_cache must be 16-byte aligned"
        need_v = _pool_extent(d, d.v_stride_block, d.v_stride_head, d.v_stride_token, d.head_dim_v)
        assert _span(v_cache) >= need_v, f"v_cache spans {_span(v_cache)} elements, the descriptor needs {need_v}"


class Plan:
    """A planned batch: prefix forest + decode schedule (fca_plan_create)."""

    def __init__(self, block_tables, seq_lens, desc: AttnDesc, workspace=None, stream=None):
        import torch

        assert block_tables.dtype == torch.int32 and seq_lens.dtype == torch.int32
        assert block_tables.dim() == 2 and block_tables.stride(1) == 1
        B, W = block_tables.shape
        self.desc = desc
        self.batch, self.max_blocks = int(B), int(W)
        nbytes = plan_workspace_size(self.batch, self.max_blocks, desc)
        if workspace is None:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=block_tables.device)
        self.workspace = workspace  # must outlive the plan
        h = ctypes.c_void_p()
        t0 = time.perf_counter()
        _check(
            lib().fca_plan_create(
                _ptr(block_tables),
                block_tables.stride(0),
                _ptr(seq_lens),
                self.batch,
                self.max_blocks,
                ctypes.byref(desc),
                _ptr(workspace),
                workspace.numel() * workspace.element_size(),
                _stream_ptr(stream),
                ctypes.byref(h),
            )
        )
        # host time of the C call: discovery, its one read-back, planning and
        # the upload; the two table kernels queued last run asynchronously
        self.create_ms = (time.perf_counter() - t0) * 1000.0
        self._h = h
        info = PlanInfo()
        _check(lib().fca_plan_get_info(self._h, ctypes.byref(info)))
        self.info = info
        self._decode_ws = None
        # kept here: at interpreter exit the module's globals may be gone
        # before the plan is collected
        self._destroy = lib().fca_plan_destroy

    def __del__(self):
        h = getattr(self, "_h", None)
        destroy = getattr(self, "_destroy", None)
        if h is not None and h.value and destroy is not None:
            destroy(h)
            self._h = None

    @property
    def handle(self):
        return self._h

    def decode_workspace(self, device):
        import torch

        need = max(int(self.info.decode_workspace_bytes), 256)
        if self._decode_ws is None or self._decode_ws.numel() < need:
            self._decode_ws = torch.empty(need, dtype=torch.uint8, device=device)
        return self._decode_ws

    def decode(self, q, k_cache, v_cache, out=None, lse=None, workspace=None, stream=None):
        """fca_decode of this plan.  Without ``workspace`` the plan's own
        decode workspace is used, so calls of one plan on different streams
        that may overlap must each pass a workspace of their own
        (``torch.empty_like(plan.decode_workspace(device))``)."""
        import torch

        d = self.desc
        assert q.dtype == torch.bfloat16 and q.is_contiguous()
        assert tuple(q.shape) == (self.batch, d.num_q_heads, d.head_dim_qk)
        out_dtype = torch.float32 if d.flags & FCA_PLAN_OUT_F32 else torch.bfloat16
        if out is None:
            out = torch.empty((self.batch, d.num_q_heads, d.head_dim_v), dtype=out_dtype, device=q.device)
        assert out.dtype == out_dtype and out.is_contiguous()
        assert tuple(out.shape) == (self.batch, d.num_q_heads, d.head_dim_v)
        if lse is not None:
            assert lse.dtype == torch.float32 and lse.is_contiguous()
            assert tuple(lse.shape) == (self.batch, d.num_q_heads)
        _check_pool(d, k_cache, v_cache)
        ws = workspace if workspace is not None else self.decode_workspace(q.device)
        _check(
            lib().fca_decode(
                self._h,
                _ptr(q),
                _ptr(k_cache),
                _ptr(v_cache),
                _ptr(out),
                _ptr(lse),
                _ptr(ws),
                ws.numel() * ws.element_size(),
                _stream_ptr(stream),
            )
        )
        return out

    def decode_no_alloc(self, q, k_cache, v_cache, out, lse=None, stream=None):
        """fca_decode_no_alloc: the decode with the partial rows in the
        library's per-device static scratch (no workspace, no allocation;
        calls on one device must not overlap).  ``out`` is required."""
        import torch

        d = self.desc
        assert q.dtype == torch.bfloat16 and q.is_contiguous()
        assert tuple(q.shape) == (self.batch, d.num_q_heads, d.head_dim_qk)
        out_dtype = torch.float32 if d.flags & FCA_PLAN_OUT_F32 else torch.bfloat16
        assert out.dtype == out_dtype and out.is_contiguous()
        assert tuple(out.shape) == (self.batch, d.num_q_heads, d.head_dim_v)
        if lse is not None:
            assert lse.dtype == torch.float32 and lse.is_contiguous()
            assert tuple(lse.shape) == (self.batch, d.num_q_heads)
        _check_pool(d, k_cache, v_cache)
        _check(
            lib().fca_decode_no_alloc(
                self._h, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse), _stream_ptr(stream)
            )
        )
        return out

    def decode_layers(self, qs, caches, outs, lses=None, workspace=None, stream=None):
        """One call decoding several layers with this plan
        (fca_decode_layers): ``qs[l]`` bf16 [B, Hq, Dqk], ``caches[l]`` =
        (k_cache, v_cache), ``outs[l]`` the outputs, ``lses[l]`` float32
        [B, Hq] or None."""
        import torch

        d = self.desc
        n = len(qs)
        assert len(caches) == n and len(outs) == n and (lses is None or len(lses) == n)
        out_dtype = torch.float32 if d.flags & FCA_PLAN_OUT_F32 else torch.bfloat16
        for l in range(n):
            q, out = qs[l], outs[l]
            assert q.dtype == torch.bfloat16 and q.is_contiguous()
            assert tuple(q.shape) == (self.batch, d.num_q_heads, d.head_dim_qk)
            assert out.dtype == out_dtype and out.is_contiguous()
            assert tuple(out.shape) == (self.batch, d.num_q_heads, d.head_dim_v)
            if lses is not None and lses[l] is not None:
                assert lses[l].dtype == torch.float32 and lses[l].is_contiguous()
                assert tuple(lses[l].shape) == (self.batch, d.num_q_heads)
            _check_pool(d, caches[l][0], caches[l][1])
        arr = lambda ts: (ctypes.c_void_p * max(n, 1))(*[(t.data_ptr() if t is not None else 0) for t in ts])
        ws = workspace if workspace is not None else self.decode_workspace(qs[0].device)
        _check(
            lib().fca_decode_layers(
                self._h,
                n,
                arr(qs),
                arr([c[0] for c in caches]),
                arr([c[1] for c in caches]),
                arr(outs),
                arr(lses) if lses is not None else None,
                _ptr(ws),
                ws.numel() * ws.element_size(),
                _stream_ptr(stream),
            )
        )
        return outs

    def profile(self, enable: bool):
        """Record per-pass HIP events in later decode calls (measurement)."""
        _check(lib().fca_profile_enable(self._h, int(bool(enable))))

    def read_profile(self) -> dict:
        p = Profile()
        _check(lib().fca_profile_read(self._h, ctypes.byref(p)))
        return {f: getattr(p, f) for f, _ in Profile._fields_}

    def time_launches(self, q, caches, repeats, out, lse=None, workspace=None, stream=None) -> dict:
        """Average GPU time (ms) of each launch kind of a decode, each issued
        repeats * len(caches) times back to back between two HIP events
        (fca_time_launches).  `caches` is a list of (k_cache, v_cache); out /
        lse end up holding the decode of the last one."""
        import torch

        d = self.desc
        assert q.dtype == torch.bfloat16 and q.is_contiguous()
        assert tuple(q.shape) == (self.batch, d.num_q_heads, d.head_dim_qk)
        assert out.dtype == torch.bfloat16 and out.is_contiguous()
        assert tuple(out.shape) == (self.batch, d.num_q_heads, d.head_dim_v)
        if lse is not None:
            assert lse.dtype == torch.float32 and lse.is_contiguous()
        for k, v in caches:
            _check_pool(d, k, v)
        n = len(caches)
        ks = (ctypes.c_void_p * max(n, 1))(*[k.data_ptr() for k, _ in caches])
        vs = (ctypes.c_void_p * max(n, 1))(*[(v.data_ptr() if v is not None else 0) for _, v in caches])
        ws = workspace if workspace is not None else self.decode_workspace(q.device)
        p = Profile()
        _check(
            lib().fca_time_launches(
                self._h,
                _ptr(q),
                ks,
                vs,
                n,
                int(repeats),
                _ptr(out),
                _ptr(lse),
                _ptr(ws),
                ws.numel() * ws.element_size(),
                _stream_ptr(stream),
                ctypes.byref(p),
            )
        )
        return {f: getattr(p, f) for f, _ in Profile._fields_}

    def export(self):
        """Canonical grouping: dict(groups=[...], requests=[...])."""
        G, B = self.info.num_groups, self.batch
        groups = (GroupRecord * max(G, 1))()
        counts = None
        # members: sum of member_count <= B * (depth + 1); fetch groups first
        _check(lib().fca_plan_export(self._h, groups, None, None))
        total = sum(groups[g].member_count for g in range(G))
        members = (ctypes.c_int32 * max(total, 1))()
        reqs = (ctypes.c_int32 * max(3 * B, 1))()
        _check(lib().fca_plan_export(self._h, None, members, reqs))
        del counts
        out = []
        for g in range(G):
            rec = groups[g]
            mem = tuple(members[rec.member_begin + k] for k in range(rec.member_count))
            out.append(
                dict(
                    depth=rec.depth,
                    parent=rec.parent,
                    block_begin=rec.block_begin,
                    block_end=rec.block_end,
                    members=mem,
                )
            )
        requests = [(reqs[3 * i], reqs[3 * i + 1], reqs[3 * i + 2]) for i in range(B)]
        folded = (ctypes.c_int32 * max(G, 1))()
        _check(lib().fca_plan_export_folded(self._h, folded))
        return dict(groups=out, requests=requests, folded=[int(folded[g]) for g in range(G)])

    def export_schedule(self):
        """Work items of both passes and the merge sources: ``sources[i][h]``
        lists the partial rows query head h of request i merges."""
        ng, ns, B = self.info.num_grouped_items, self.info.num_suffix_items, self.batch
        hq = self.desc.num_q_heads
        gi = (WorkItem * max(ng, 1))()
        si = (WorkItem * max(ns, 1))()
        off = (ctypes.c_int32 * (B * hq + 1))()
        src = (ctypes.c_int32 * max(self.info.num_merge_sources, 1))()
        _check(lib().fca_plan_export_schedule(self._h, gi, si, off, src))

        def items(arr, n):
            names = [f[0] for f in WorkItem._fields_]
            return [{k: getattr(arr[j], k) for k in names} for j in range(n)]

        sources = [[list(src[off[i * hq + h] : off[i * hq + h + 1]]) for h in range(hq)] for i in range(B)]
        return dict(grouped=items(gi, ng), suffix=items(si, ns), sources=sources)


def fca_plan(block_tables, seq_lens, desc: AttnDesc, workspace=None, stream=None) -> Plan:
    """Discover the prefix forest of a batch and schedule its decode."""
    return Plan(block_tables, seq_lens, desc, workspace=workspace, stream=stream)


def fca_decode(q, k_cache, v_cache, plan: Plan, out=None, lse=None, stream=None):
    """Forest Cascade Attention decode for a planned batch; returns `out`."""
    return plan.decode(q, k_cache, v_cache, out=out, lse=lse, stream=stream)


def merge_states(outs, lses, out=None, lse=None, out_f32=False, stream=None):
    """Exact combination of attention states over disjoint key sets
    (fca_merge_states): ``outs`` float32 [B, H, D] normalised outputs, ``lses``
    float32 [B, H] natural log-sum-exps, as fca_decode writes them with
    ``out_f32``.  Returns ``out`` (bf16, or float32 with ``out_f32``)."""
    import torch

    n = len(outs)
    assert n == len(lses) and n >= 1
    B, H, D = outs[0].shape
    for o, l in zip(outs, lses):
        assert o.dtype == torch.float32 and o.is_contiguous() and tuple(o.shape) == (B, H, D)
        assert l.dtype == torch.float32 and l.is_contiguous() and tuple(l.shape) == (B, H)
    dt = torch.float32 if out_f32 else torch.bfloat16
    if out is None:
        out = torch.empty((B, H, D), dtype=dt, device=outs[0].device)
    assert out.dtype == dt and out.is_contiguous() and tuple(out.shape) == (B, H, D)
    if lse is not None:
        assert lse.dtype == torch.float32 and lse.is_contiguous() and tuple(lse.shape) == (B, H)
    po = (ctypes.c_void_p * n)(*[o.data_ptr() for o in outs])
    pl = (ctypes.c_void_p * n)(*[l.data_ptr() for l in lses])
    _check(
        lib().fca_merge_states(
            n, po, pl, B, H, D, _ptr(out), _ptr(lse), FCA_MERGE_OUT_F32 if out_f32 else 0, _stream_ptr(stream)
        )
    )
    return out


def kv_append(k_new, v_new, k_cache, v_cache, block_tables, seq_lens, desc: AttnDesc, cow_dst=None, status=None,
              stream=None):
    """Write one decode token per request into the paged cache, copying a
    shared last block first where ``cow_dst[i] >= 0`` (fca_kv_append).
    ``k_new`` bf16 [B, Hkv, Dqk], ``v_new`` bf16 [B, Hkv, Dv] (None for a
    latent cache), ``block_tables`` int32 [B, W] (updated in place for copied
    requests), ``seq_lens`` int32 [B] (the position of the new token),
    ``cow_dst`` int32 [B] or None, ``status`` int32 [1] or None (bits
    FCA_APPEND_BAD_*, ORed in)."""
    import torch

    assert block_tables.dtype == torch.int32 and block_tables.dim() == 2 and block_tables.stride(1) == 1
    B, W = block_tables.shape
    assert seq_lens.dtype == torch.int32 and seq_lens.is_contiguous() and tuple(seq_lens.shape) == (B,)
    assert k_new.dtype == torch.bfloat16 and k_new.is_contiguous()
    assert tuple(k_new.shape) == (B, desc.num_kv_heads, desc.head_dim_qk)
    if not desc.v_aliases_k:
        assert v_new.dtype == torch.bfloat16 and v_new.is_contiguous()
        assert tuple(v_new.shape) == (B, desc.num_kv_heads, desc.head_dim_v)
    if cow_dst is not None:
        assert cow_dst.dtype == torch.int32 and cow_dst.is_contiguous() and tuple(cow_dst.shape) == (B,)
    if status is not None:
        assert status.dtype == torch.int32 and status.numel() >= 1
    _check_pool(desc, k_cache, None if desc.v_aliases_k else v_cache)
    _check(
        lib().fca_kv_append(
            ctypes.byref(desc),
            _ptr(k_new),
            _ptr(None if desc.v_aliases_k else v_new),
            _ptr(k_cache),
            _ptr(None if desc.v_aliases_k else v_cache),
            _ptr(block_tables),
            block_tables.stride(0),
            W,
            _ptr(seq_lens),
            _ptr(cow_dst),
            _ptr(status),
            B,
            _stream_ptr(stream),
        )
    )


def kv_append_layers(k_news, v_news, caches, block_tables, seq_lens, desc: AttnDesc, cow_dst=None, status=None,
                     stream=None):
    """fca_kv_append_layers: one decode token per request appended to every
    layer's pool (``caches[l]`` = (k_cache, v_cache), ``k_news[l]`` /
    ``v_news[l]`` that layer's new rows), the table entries of copied requests
    rewritten once after all layers."""
    import torch

    assert block_tables.dtype == torch.int32 and block_tables.dim() == 2 and block_tables.stride(1) == 1
    B, W = block_tables.shape
    n = len(caches)
    assert len(k_news) == n and (desc.v_aliases_k or len(v_news) == n)
    assert seq_lens.dtype == torch.int32 and seq_lens.is_contiguous() and tuple(seq_lens.shape) == (B,)
    for l in range(n):
        assert k_news[l].dtype == torch.bfloat16 and k_news[l].is_contiguous()
        assert tuple(k_news[l].shape) == (B, desc.num_kv_heads, desc.head_dim_qk)
        if not desc.v_aliases_k:
            assert v_news[l].dtype == torch.bfloat16 and v_news[l].is_contiguous()
            assert tuple(v_news[l].shape) == (B, desc.num_kv_heads, desc.head_dim_v)
        _check_pool(desc, caches[l][0], None if desc.v_aliases_k else caches[l][1])
    if cow_dst is not None:
        assert cow_dst.dtype == torch.int32 and cow_dst.is_contiguous() and tuple(cow_dst.shape) == (B,)
    if status is not None:
        assert status.dtype == torch.int32 and status.numel() >= 1
    arr = lambda ts: (ctypes.c_void_p * max(n, 1))(*[(t.data_ptr() if t is not None else 0) for t in ts])
    alias = bool(desc.v_aliases_k)
    _check(
        lib().fca_kv_append_layers(
            ctypes.byref(desc),
            n,
            arr(k_news),
            None if alias else arr(v_news),
            arr([c[0] for c in caches]),
            None if alias else arr([c[1] for c in caches]),
            _ptr(block_tables),
            block_tables.stride(0),
            W,
            _ptr(seq_lens),
            _ptr(cow_dst),
            _ptr(status),
            B,
            _stream_ptr(stream),
        )
    )


def measure_read_bandwidth(buffers, repeats=4, stream=None) -> float:
    """HBM read rate (GB/s, 1e9 B/s) of a plain streaming kernel over the
    given device tensors (equal sizes, multiple of 16 bytes), cycled
    ``repeats`` times (fca_measure_read_bandwidth)."""
    n = len(buffers)
    nbytes = buffers[0].numel() * buffers[0].element_size()
    for b in buffers:
        assert b.is_contiguous() and b.numel() * b.element_size() == nbytes
    arr = (ctypes.c_void_p * n)(*[b.data_ptr() for b in buffers])
    g = ctypes.c_double()
    _check(lib().fca_measure_read_bandwidth(arr, n, nbytes, int(repeats), _stream_ptr(stream), ctypes.byref(g)))
    return g.value



FCA_MFMA_BF16 = 0
FCA_MFMA_F16 = 1


def measure_mfma_rate(dtype="bf16", iters=4000, stream=None) -> float:
    """Dense matrix-core rate (TFLOP/s) of a loop of independent 16x16x32
    products, bf16 or fp16 operands (fca_measure_mfma_rate)."""
    code = {"bf16": FCA_MFMA_BF16, "f16": FCA_MFMA_F16}[dtype]
    t = ctypes.c_double()
    _check(lib().fca_measure_mfma_rate(code, int(iters), _stream_ptr(stream), ctypes.byref(t)))
    return t.value


def version() -> str:
    return lib().fca_version().decode()
