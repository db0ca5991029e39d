"""Pins of the CPU oracle against what the pages and the mathematics fix.

CPU only.  Each test names the fact it pins and where it comes from; together
they are chosen so that a plausible mistake in the oracle (a wrong GQA head
map, a swapped block/offset index, a dropped scale, a sign slip in the
softmax, a wrong merge of partitions, a bad widening of a bit pattern) fails
at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from _paged import (TDT, build_pool, default_scale, f32, rand_rows, sdpa_reference, u16)
from conftest import GOLDEN

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ---------------------------------------------------------------- widening

def test_widen_every_f16_pattern(oracle_mod):
    """Exact binary16 -> double for all 65536 patterns vs numpy's decoder."""
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float64)
    got = oracle_mod.widen(pats, oracle_mod.F16)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()
    assert np.array_equal(np.signbit(got[~np.isnan(got)]), np.signbit(ref[~np.isnan(ref)]))


def test_widen_every_bf16_pattern(oracle_mod):
    """Exact bfloat16 -> double for all 65536 patterns vs torch's decoder."""
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(pats.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = oracle_mod.widen(pats, oracle_mod.BF16)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


# ------------------------------------------------- worked block-table example

def test_worked_block_ids_12_87_301_44(oracle_mod):
    """Positions 0..49 held by physical blocks 12, 87, 301, 44 (block 16):
    the paged result equals attention over the contiguous rows, while every
    other pool slot is NaN; position 49 maps to slot 705."""
    ex = json.load(open(os.path.join(GOLDEN, "block_table_example.json")))
    bs, n, ids = ex["block_size"], ex["num_tokens"], ex["physical_blocks"]
    assert -(-n // bs) == ex["logical_blocks"] == len(ids)
    assert n - (len(ids) - 1) * bs == ex["last_block_tokens"]
    rng = np.random.default_rng(1234)
    hkv, hq, d, tdt = 2, 8, 64, torch.float16
    K, V = rand_rows(rng, n, hkv, d, tdt), rand_rows(rng, n, hkv, d, tdt)
    q = torch.from_numpy(rng.standard_normal((1, hq, d), dtype=np.float32)).to(tdt)
    kp, vp, tables, lens, _ = build_pool([K], [V], bs, 302, rng, tdt, ids=[ids])
    assert list(tables[0]) == ids
    sl = oracle_mod.slot_mapping(tables, [0], [ex["derived"]["position"]], bs)
    assert int(sl[0]) == ex["derived"]["slot"]
    sc = default_scale(d)
    got = oracle_mod.decode(u16(q), u16(kp), u16(vp), tables, lens, sc, oracle_mod.F16)
    ref = sdpa_reference(q, [K], [V], sc)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)
    # Attention does not depend on the order of whole blocks, but the table
    # decides which block is the partial one: swapping the partial last block
    # with a full one makes the read reach NaN slots.
    bad = tables.copy()
    bad[0, [0, 3]] = bad[0, [3, 0]]
    got_bad = oracle_mod.decode(u16(q), u16(kp), u16(vp), bad, lens, sc, oracle_mod.F16)
    assert np.isnan(got_bad).all()


# ------------------------------------- reduction to torch's SDPA (contiguous)

CASES = [
    # (lens, Hq, Hkv, d, bs, dtype)
    ([50, 17, 16, 3], 8, 2, 64, 16, 0),
    ([1, 33, 64, 7], 4, 4, 64, 8, 1),      # MHA, bs 8, L = 1 and an exact multiple
    ([31, 97], 16, 2, 128, 32, 1),         # group 8
    ([200], 4, 1, 128, 16, 0),             # MQA
    ([0, 5, 40], 6, 3, 64, 16, 0),         # an empty sequence, group 2
]


@pytest.mark.parametrize("lens,hq,hkv,d,bs,dt", CASES)
def test_paged_equals_contiguous_sdpa(oracle_mod, lens, hq, hkv, d, bs, dt):
    """Paged attention equals torch CPU float64 SDPA on the same rows laid
    out contiguously, KV heads repeated over their query group (the pages:
    the kernel follows the table and keeps positions in order)."""
    rng = np.random.default_rng(hash((tuple(lens), hq, hkv, d, bs, dt)) % 2**32)
    tdt = TDT[dt]
    Ks = [rand_rows(rng, L, hkv, d, tdt) for L in lens]
    Vs = [rand_rows(rng, L, hkv, d, tdt) for L in lens]
    q = torch.from_numpy(rng.standard_normal((len(lens), hq, d), dtype=np.float32)).to(tdt)
    nb = sum(-(-L // bs) for L in lens) + 5
    kp, vp, tables, sl, _ = build_pool(Ks, Vs, bs, nb, rng, tdt)
    sc = f32(0.37)  # not 1/sqrt(d): a dropped or doubled scale must show
    got = oracle_mod.decode(u16(q), u16(kp), u16(vp), tables, sl, sc, dt)
    ref = sdpa_reference(q, Ks, Vs, sc)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


# ------------------------------------------------------------- closed forms

def _one(oracle_mod, rng, L, d=64, hq=4, hkv=2, bs=16, dt=0, kfn=None, vfn=None, qfn=None,
         scale=None):
    tdt = TDT[dt]
    K = rand_rows(rng, L, hkv, d, tdt) if kfn is None else kfn(L, hkv, d, tdt)
    V = rand_rows(rng, L, hkv, d, tdt) if vfn is None else vfn(L, hkv, d, tdt)
    q = torch.from_numpy(rng.standard_normal((1, hq, d), dtype=np.float32)).to(tdt)
    if qfn is not None:
        q = qfn(q)
    kp, vp, tables, sl, _ = build_pool([K], [V], bs, -(-L // bs) + 3, rng, tdt)
    sc = default_scale(d) if scale is None else scale
    out = oracle_mod.decode(u16(q), u16(kp), u16(vp), tables, sl, sc, dt)
    return out[0], K, V


def test_single_token_returns_its_value(oracle_mod):
    """L = 1: softmax over one score is 1, the output is that token's V."""
    out, K, V = _one(oracle_mod, np.random.default_rng(7), 1)
    g = 2
    for h in range(4):
        assert np.array_equal(out[h], V[0, h // g].double().numpy())


def test_constant_value_rows_return_the_constant(oracle_mod):
    """Every V row = c: the weights sum to 1, so the output is exactly c."""
    c = torch.tensor(0.8125)
    out, _, _ = _one(oracle_mod, np.random.default_rng(8), 77,
                     vfn=lambda L, h, d, t: torch.full((L, h, d), float(c)).to(t))
    np.testing.assert_allclose(out, 0.8125, rtol=0, atol=1e-15)


def test_zero_query_gives_mean_of_values(oracle_mod):
    """q = 0 (all scores 0): uniform weights, output = mean of V rows."""
    out, _, V = _one(oracle_mod, np.random.default_rng(9), 45, qfn=lambda q: torch.zeros_like(q))
    mean = V.double().mean(dim=0).numpy()  # [Hkv][d]
    for h in range(4):
        np.testing.assert_allclose(out[h], mean[h // 2], rtol=1e-13, atol=1e-14)


def test_zero_scale_gives_mean_of_values(oracle_mod):
    out, _, V = _one(oracle_mod, np.random.default_rng(10), 30, scale=0.0)
    mean = V.double().mean(dim=0).numpy()
    for h in range(4):
        np.testing.assert_allclose(out[h], mean[h // 2], rtol=1e-13, atol=1e-14)


def test_one_dominant_key_selects_its_value(oracle_mod):
    """A key far better aligned with q than the rest takes (numerically) all
    the weight: output = that token's V.  Fixes the sign of the softmax."""
    rng = np.random.default_rng(11)
    d, L, star = 64, 40, 17
    q = torch.ones((1, 4, d), dtype=torch.float16)

    def keys(L, h, d, t):
        k = torch.zeros((L, h, d))
        k[star] = 1.0
        return k.to(t)
    tdt = torch.float16
    K = keys(L, 2, d, tdt)
    V = rand_rows(rng, L, 2, d, tdt)
    kp, vp, tables, sl, _ = build_pool([K], [V], 16, 6, rng, tdt)
    out = oracle_mod.decode(u16(q), u16(kp), u16(vp), tables, sl, 1.0, 0)[0]
    for h in range(4):
        np.testing.assert_allclose(out[h], V[star, h // 2].double().numpy(), rtol=0, atol=1e-20)


# -------------------------------------------------------------- invariances

def _batch(seed, lens, hq=8, hkv=2, d=64, dt=1):
    rng = np.random.default_rng(seed)
    tdt = TDT[dt]
    Ks = [rand_rows(rng, L, hkv, d, tdt) for L in lens]
    Vs = [rand_rows(rng, L, hkv, d, tdt) for L in lens]
    q = torch.from_numpy(rng.standard_normal((len(lens), hq, d), dtype=np.float32)).to(tdt)
    return rng, q, Ks, Vs


def test_physical_permutation_invariance_bitwise(oracle_mod):
    """Any placement of the physical blocks gives the same result, bit for bit
    (the table, not the physical order, decides the positions)."""
    lens = [50, 129, 16, 1]
    rng, q, Ks, Vs = _batch(21, lens)
    outs = []
    for seed in (1, 2, 3):
        kp, vp, tb, sl, _ = build_pool(Ks, Vs, 16, 40, np.random.default_rng(seed), TDT[1])
        outs.append(oracle_mod.decode(u16(q), u16(kp), u16(vp), tb, sl, 0.125, 1))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_block_size_invariance_bitwise(oracle_mod):
    """The same logical rows at block size 8, 16 and 32 give the same bits."""
    lens = [75, 200, 3]
    rng, q, Ks, Vs = _batch(22, lens)
    outs = []
    for bs in (8, 16, 32):
        nb = sum(-(-L // bs) for L in lens) + 2
        kp, vp, tb, sl, _ = build_pool(Ks, Vs, bs, nb, np.random.default_rng(bs), TDT[1])
        outs.append(oracle_mod.decode(u16(q), u16(kp), u16(vp), tb, sl, 0.125, 1))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_shared_blocks_equal_private_copies(oracle_mod):
    """Sequences that reference the same physical prefix blocks give the same
    result as sequences holding private copies (the pages' shared blocks)."""
    rng, q, Ks, Vs = _batch(23, [96, 96])
    Vs[1] = Vs[0].clone()
    Ks[1] = Ks[0].clone()
    kp, vp, tb, sl, _ = build_pool(Ks, Vs, 16, 20, rng, TDT[1])
    private = oracle_mod.decode(u16(q), u16(kp), u16(vp), tb, sl, 0.125, 1)
    shared_tb = tb.copy()
    shared_tb[1] = tb[0]
    shared = oracle_mod.decode(u16(q), u16(kp), u16(vp), shared_tb, sl, 0.125, 1)
    assert np.array_equal(private, shared)


def test_gqa_equals_mha_with_repeated_kv(oracle_mod):
    """Group g: query head h reads KV head h // g.  The same result comes
    from an MHA pool holding each KV head repeated g times."""
    lens = [37, 64]
    rng, q, Ks, Vs = _batch(24, lens, hq=8, hkv=2)
    kp, vp, tb, sl, _ = build_pool(Ks, Vs, 16, 12, np.random.default_rng(5), TDT[1])
    gqa = oracle_mod.decode(u16(q), u16(kp), u16(vp), tb, sl, 0.2, 1)
    Kr = [k.repeat_interleave(4, dim=1) for k in Ks]
    Vr = [v.repeat_interleave(4, dim=1) for v in Vs]
    kp2, vp2, tb2, sl2, _ = build_pool(Kr, Vr, 16, 12, np.random.default_rng(6), TDT[1])
    mha = oracle_mod.decode(u16(q), u16(kp2), u16(vp2), tb2, sl2, 0.2, 1)
    assert np.array_equal(gqa, mha)


def test_unused_slots_and_entries_are_never_read(oracle_mod):
    """Slots past L and table entries past the last block hold NaN / point at
    a NaN block: the output stays finite and unchanged."""
    lens = [20, 33]
    rng, q, Ks, Vs = _batch(25, lens)
    kp, vp, tb, sl, spare = build_pool(Ks, Vs, 16, 10, np.random.default_rng(3), TDT[1])
    assert (tb == spare).any()
    out_nan = oracle_mod.decode(u16(q), u16(kp), u16(vp), tb, sl, 0.125, 1)
    kp0, vp0, tb0, sl0, _ = build_pool(Ks, Vs, 16, 10, np.random.default_rng(3), TDT[1],
                                       fill=0.0)
    out_zero = oracle_mod.decode(u16(q), u16(kp0), u16(vp0), tb0, sl0, 0.125, 1)
    assert np.isfinite(out_nan).all()
    assert np.array_equal(out_nan, out_zero)


def test_split_by_partitions_equals_unsplit(oracle_mod):
    """Per-partition (m, l, acc) merged by log-sum-exp equals the unsplit
    softmax (an identity of exp; here to double rounding)."""
    lens = [1, 16, 511, 512, 513, 1500]
    rng, q, Ks, Vs = _batch(26, lens, hq=8, hkv=2, d=64)
    kp, vp, tb, sl, _ = build_pool(Ks, Vs, 16, 200, rng, TDT[1])
    full = oracle_mod.decode(u16(q), u16(kp), u16(vp), tb, sl, 0.125, 1)
    for P in (16, 64, 512):
        split = oracle_mod.decode_split(u16(q), u16(kp), u16(vp), tb, sl, 0.125, 1, P)
        np.testing.assert_allclose(split, full, rtol=1e-12, atol=1e-13)


def test_empty_sequence_gives_zeros(oracle_mod):
    rng, q, Ks, Vs = _batch(27, [0, 10])
    kp, vp, tb, sl, _ = build_pool(Ks, Vs, 16, 4, rng, TDT[1])
    out = oracle_mod.decode(u16(q), u16(kp), u16(vp), tb, sl, 0.125, 1)
    assert np.array_equal(out[0], np.zeros_like(out[0]))


def test_sampled_pairs_match_full(oracle_mod):
    rng, q, Ks, Vs = _batch(28, [30, 60, 90])
    kp, vp, tb, sl, _ = build_pool(Ks, Vs, 16, 14, rng, TDT[1])
    full = oracle_mod.decode(u16(q), u16(kp), u16(vp), tb, sl, 0.125, 1)
    pairs = [(0, 3), (2, 7), (1, 0)]
    part = oracle_mod.decode(u16(q), u16(kp), u16(vp), tb, sl, 0.125, 1, pairs=pairs)
    for s, h in pairs:
        assert np.array_equal(part[s, h], full[s, h])
    assert np.isnan(part[0, 0]).all()


def test_out_of_range_table_entry_is_refused(oracle_mod):
    rng, q, Ks, Vs = _batch(29, [20])
    kp, vp, tb, sl, _ = build_pool(Ks, Vs, 16, 4, rng, TDT[1])
    tb[0, 1] = 4
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.decode(u16(q), u16(kp), u16(vp), tb, sl, 0.125, 1)


# ------------------------------------------------------------- brute force

def test_oracle_matches_bruteforce_on_tiny_inputs(oracle_mod):
    """The C oracle against an independent pure-Python implementation."""
    from oracle import bruteforce
    for dt in (0, 1):
        rng, q, Ks, Vs = _batch(30 + dt, [5, 18, 1, 0], hq=4, hkv=2, d=16, dt=dt)
        kp, vp, tb, sl, _ = build_pool(Ks, Vs, 8, 10, rng, TDT[dt])
        got = oracle_mod.decode(u16(q), u16(kp), u16(vp), tb, sl, 0.3, dt)
        ref = np.array(bruteforce.decode(u16(q), u16(kp), u16(vp), tb, sl, 0.3, dt))
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)
