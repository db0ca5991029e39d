"""The oracle's append and copy-on-write copy (CPU only).

Append: each new token's K/V rows land in the slot its position maps to
("How PagedAttention works": logical block -> physical block; a growing
request attaches another block, "Paged attention borrows a trick from
operating systems").  Copy-on-write: a diverging candidate gets a private
copy of a shared block ("How PagedAttention works").
"""
import numpy as np
import pytest
import torch

from _paged import TDT, build_pool, rand_rows, sdpa_reference, u16


def _pools(rng, nb=12, hkv=2, bs=8, d=16):
    k = torch.from_numpy(rng.standard_normal((nb, hkv, bs, d), dtype=np.float32)).half()
    v = torch.from_numpy(rng.standard_normal((nb, hkv, bs, d), dtype=np.float32)).half()
    return u16(k).copy(), u16(v).copy()


def test_append_writes_exactly_its_slots(oracle_mod):
    rng = np.random.default_rng(1)
    kp, vp = _pools(rng)
    k0, v0 = kp.copy(), vp.copy()
    T, hkv, d, bs = 5, 2, 16, 8
    key = u16(torch.from_numpy(rng.standard_normal((T, hkv, d), dtype=np.float32)).half())
    val = u16(torch.from_numpy(rng.standard_normal((T, hkv, d), dtype=np.float32)).half())
    slots = np.array([3, -1, 95, 40, -7], dtype=np.int32)
    oracle_mod.reshape_and_cache(key, val, kp, vp, slots)
    touched = np.zeros(kp.shape[:3], dtype=bool)  # [NB][Hkv][bs]
    for i, s in enumerate(slots):
        if s < 0:
            continue
        b, o = divmod(int(s), bs)
        touched[b, :, o] = True
        for h in range(hkv):
            assert np.array_equal(kp[b, h, o], key[i, h])
            assert np.array_equal(vp[b, h, o], val[i, h])
    assert np.array_equal(kp[~touched], k0[~touched])
    assert np.array_equal(vp[~touched], v0[~touched])


def test_append_refuses_duplicate_and_out_of_range_slots(oracle_mod):
    rng = np.random.default_rng(2)
    kp, vp = _pools(rng)
    key = np.zeros((2, 2, 16), np.uint16)
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.reshape_and_cache(key, key, kp, vp, np.array([4, 4], np.int32))
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.reshape_and_cache(key, key, kp, vp, np.array([4, 12 * 8], np.int32))
    # two padding entries are not duplicates
    oracle_mod.reshape_and_cache(key, key, kp, vp, np.array([-1, -1], np.int32))


def test_append_then_decode_equals_contiguous(oracle_mod):
    """Appending the last token of each sequence through its slot and then
    decoding equals attention over the full contiguous rows."""
    rng = np.random.default_rng(3)
    lens, hq, hkv, d, bs, tdt = [17, 9, 5, 1], 4, 2, 32, 8, torch.bfloat16
    Ks = [rand_rows(rng, L, hkv, d, tdt) for L in lens]
    Vs = [rand_rows(rng, L, hkv, d, tdt) for L in lens]
    q = torch.from_numpy(rng.standard_normal((4, hq, d), dtype=np.float32)).to(tdt)
    kp, vp, tb, sl, spare = build_pool([k[:-1] for k in Ks], [v[:-1] for v in Vs], bs, 12,
                                       rng, tdt)
    # a new position that falls past the owned blocks attaches a free block
    tb = np.concatenate([tb, np.full((4, 2), spare, np.int32)], axis=1)
    owned = set(tb[tb != spare].tolist())
    free = [b for b in range(12) if b not in owned and b != spare]
    pos = np.array(lens, np.int32) - 1
    attached = {}
    for s_, p_ in enumerate(pos):
        if p_ % bs == 0:
            tb[s_, p_ // bs] = attached[s_] = free.pop(0)
    assert sorted(attached) == [0, 1, 3]           # 16, 8 and 0 tokens cross a boundary
    slots = oracle_mod.slot_mapping(tb, [0, 1, 2, 3], pos, bs)
    for s_, b_ in attached.items():
        assert slots[s_] == b_ * bs
    assert slots[2] == tb[2, 0] * bs + 4
    K, V = u16(kp).copy(), u16(vp).copy()
    oracle_mod.reshape_and_cache(np.stack([u16(k[-1]) for k in Ks]),
                                 np.stack([u16(v[-1]) for v in Vs]), K, V, slots)
    out = oracle_mod.decode(u16(q), K, V, tb, np.array(lens, np.int32), 0.25, 1)
    np.testing.assert_allclose(out, sdpa_reference(q, Ks, Vs, 0.25), rtol=1e-11, atol=1e-12)


def test_copy_blocks_snapshot_and_repeated_source(oracle_mod):
    rng = np.random.default_rng(4)
    kp, vp = _pools(rng)
    k0, v0 = kp.copy(), vp.copy()
    pairs = np.array([[2, 7], [2, 8], [5, 9]], np.int32)  # a source may repeat
    oracle_mod.copy_blocks(kp, vp, pairs)
    for s, d in pairs:
        assert np.array_equal(kp[d], k0[s]) and np.array_equal(vp[d], v0[s])
    untouched = [b for b in range(12) if b not in (7, 8, 9)]
    assert np.array_equal(kp[untouched], k0[untouched])
    assert np.array_equal(vp[untouched], v0[untouched])


def test_copy_blocks_refuses_chains_and_repeated_destinations(oracle_mod):
    rng = np.random.default_rng(5)
    kp, vp = _pools(rng)
    for bad in ([[1, 2], [2, 3]], [[1, 4], [2, 4]], [[1, 12]], [[-1, 3]]):
        with pytest.raises(oracle_mod.OracleError):
            oracle_mod.copy_blocks(kp, vp, np.array(bad, np.int32))


def test_copy_on_write_then_append_keeps_shared_block(oracle_mod):
    """Two candidates share a partial block; one diverges: after its private
    copy and its append, the shared block is bit-unchanged and the private
    block starts with the shared tokens."""
    rng = np.random.default_rng(6)
    hkv, d, bs = 2, 16, 8
    kp, vp = _pools(rng, nb=6, hkv=hkv, bs=bs, d=d)
    k0, v0 = kp.copy(), vp.copy()
    shared, private = 1, 4
    oracle_mod.copy_blocks(kp, vp, np.array([[shared, private]], np.int32))
    new = u16(torch.from_numpy(rng.standard_normal((1, hkv, d), dtype=np.float32)).half())
    oracle_mod.reshape_and_cache(new, new, kp, vp, np.array([private * bs + 5], np.int32))
    assert np.array_equal(kp[shared], k0[shared]) and np.array_equal(vp[shared], v0[shared])
    assert np.array_equal(kp[private, :, :5], k0[shared, :, :5])
    assert np.array_equal(kp[private, :, 5], new[0])
