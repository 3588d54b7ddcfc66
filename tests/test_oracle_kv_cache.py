"""Pins of the oracle's KV append with copy-on-write (CPU)."""

import numpy as np

from oracle import attention as A
from oracle import kv_cache as KV
from workloads.forest import AttnShape


def _pools(rng, nb, hkv, dq, dv, bs):
    k = rng.integers(0, 2**16, size=(nb, hkv, dq // 8, bs, 8), dtype=np.uint16)
    v = rng.integers(0, 2**16, size=(nb, hkv, dv, bs), dtype=np.uint16)
    return k, v


def test_append_extends_the_gathered_sequence():
    """After the append, each request's gathered keys and values are the old
    ones followed by the new token's (gather_kv reads through the table),
    for empty, mid-block and block-boundary lengths."""
    rng = np.random.default_rng(0)
    bs, hkv, dq, dv, nb = 4, 2, 16, 16, 40
    k, v = _pools(rng, nb, hkv, dq, dv, bs)
    tables = rng.permutation(nb)[:30].reshape(5, 6).astype(np.int32)
    lens = np.array([0, 3, 4, 9, 20], np.int32)
    kn = rng.integers(0, 2**16, size=(5, hkv, dq), dtype=np.uint16)
    vn = rng.integers(0, 2**16, size=(5, hkv, dv), dtype=np.uint16)
    k2, v2, t2 = KV.append(k, v, tables, lens, kn, vn, bs)
    assert (t2 == tables).all()
    for i, L in enumerate(lens):
        K0, V0 = A.gather_kv(k, v, tables[i], int(L), bs, dv, False)
        K1, V1 = A.gather_kv(k2, v2, t2[i], int(L) + 1, bs, dv, False)
        np.testing.assert_array_equal(K1[:L], K0)
        np.testing.assert_array_equal(V1[:L], V0)
        np.testing.assert_array_equal(K1[L], A.widen_bf16(kn[i]))
        np.testing.assert_array_equal(V1[L], A.widen_bf16(vn[i]))


def test_copy_on_write_leaves_the_sharer_unchanged():
    """Two requests share a partly filled block; the one that appends with a
    copy-on-write target gets its own block (old tokens copied, new token
    written), the other still reads the original block untouched."""
    rng = np.random.default_rng(1)
    bs, hkv, dq, dv, nb = 4, 1, 8, 8, 12
    k, v = _pools(rng, nb, hkv, dq, dv, bs)
    tables = np.array([[3, 5, 7], [3, 5, 7]], np.int32)
    lens = np.array([6, 6], np.int32)  # block 5 holds tokens 4, 5 of both
    kn = rng.integers(0, 2**16, size=(2, hkv, dq), dtype=np.uint16)
    vn = rng.integers(0, 2**16, size=(2, hkv, dv), dtype=np.uint16)
    cow = np.array([9, -1], np.int32)
    k2, v2, t2 = KV.append(k, v, tables, lens[:1], kn[:1], vn[:1], bs, cow[:1])
    assert t2[0, 1] == 9 and t2[1, 1] == 5
    np.testing.assert_array_equal(k2[5], k[5])  # the shared block is untouched
    np.testing.assert_array_equal(v2[5], v[5])
    K1, _ = A.gather_kv(k2, v2, t2[0], 7, bs, dv, False)
    K0, _ = A.gather_kv(k, v, tables[0], 6, bs, dv, False)
    np.testing.assert_array_equal(K1[:6], K0)
    np.testing.assert_array_equal(K1[6], A.widen_bf16(kn[0]))
    Kb, _ = A.gather_kv(k2, v2, t2[1], 6, bs, dv, False)
    np.testing.assert_array_equal(Kb, K0)
    # slots after the new token in the copy keep what the target held
    np.testing.assert_array_equal(k2[9, :, :, 3:, :], k[9, :, :, 3:, :])
    np.testing.assert_array_equal(v2[9, :, :, 3:], v[9, :, :, 3:])
    # and blocks no request writes are untouched
    for blk in set(range(nb)) - {9}:
        np.testing.assert_array_equal(k2[blk], k[blk])
        np.testing.assert_array_equal(v2[blk], v[blk])


def test_copy_on_write_for_a_shorter_sharer():
    """A request that shares the first 5 tokens of a block holding 6 (a fork
    at an earlier position) copies only its 5 tokens, and the longer sharer
    appending in place at slot 6 in the same call leaves the copy intact."""
    rng = np.random.default_rng(3)
    bs, hkv, dq, dv, nb = 8, 2, 16, 8, 10
    k, v = _pools(rng, nb, hkv, dq, dv, bs)
    tables = np.array([[1, 2], [1, 2]], np.int32)
    lens = np.array([14, 13], np.int32)  # block 2: slots 0..5 (req 0), 0..4 (req 1)
    kn = rng.integers(0, 2**16, size=(2, hkv, dq), dtype=np.uint16)
    vn = rng.integers(0, 2**16, size=(2, hkv, dv), dtype=np.uint16)
    cow = np.array([-1, 7], np.int32)
    k2, v2, t2 = KV.append(k, v, tables, lens, kn, vn, bs, cow)
    assert t2.tolist() == [[1, 2], [1, 7]]
    K0, V0 = A.gather_kv(k, v, tables[0], 14, bs, dv, False)
    Ka, Va = A.gather_kv(k2, v2, t2[0], 15, bs, dv, False)
    Kb, Vb = A.gather_kv(k2, v2, t2[1], 14, bs, dv, False)
    np.testing.assert_array_equal(Ka[:14], K0)
    np.testing.assert_array_equal(Ka[14], A.widen_bf16(kn[0]))
    np.testing.assert_array_equal(Kb[:13], K0[:13])
    np.testing.assert_array_equal(Vb[:13], V0[:13])
    np.testing.assert_array_equal(Kb[13], A.widen_bf16(kn[1]))
    np.testing.assert_array_equal(Vb[13], A.widen_bf16(vn[1]))
    np.testing.assert_array_equal(k2[7, :, :, 6:, :], k[7, :, :, 6:, :])


def test_latent_cache_append_writes_the_whole_row():
    """With values aliasing the first key dims, only the key row is written
    and the gathered values are its first Dv dims."""
    rng = np.random.default_rng(2)
    bs, dq, dv, nb = 8, 24, 16, 6
    k = rng.integers(0, 2**16, size=(nb, 1, dq // 8, bs, 8), dtype=np.uint16)
    tables = np.array([[2, 4]], np.int32)
    kn = rng.integers(0, 2**16, size=(1, 1, dq), dtype=np.uint16)
    k2, v2, _ = KV.append(k, None, tables, np.array([10]), kn, None, bs)
    assert v2 is None
    K1, V1 = A.gather_kv(k2, None, tables[0], 11, bs, dv, True)
    np.testing.assert_array_equal(K1[10], A.widen_bf16(kn[0]))
    np.testing.assert_array_equal(V1[10], A.widen_bf16(kn[0])[:, :dv])
