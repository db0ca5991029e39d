"""The seeded input generator (CPU only): determinism, structure of the five
workloads, and its slot mapping / placement checked against the oracle."""
import numpy as np
import pytest
import torch

from oracle import accounting as acc
from paged_kv_cache_400_amd import workload as wl
from paged_kv_cache_400_amd.workload import bits


def test_same_seed_same_bytes():
    a, b = wl.make_tiny(), wl.make_tiny()
    for name in ("q", "k_cache", "v_cache", "new_key", "new_value"):
        assert np.array_equal(bits(getattr(a, name)), bits(getattr(b, name)))
    assert np.array_equal(a.block_tables, b.block_tables)
    assert np.array_equal(a.slot_mapping, b.slot_mapping)


def test_tiny_structure():
    b = wl.make_tiny()
    assert list(b.context_lens) == [50, 17, 16, 3] and list(b.seq_lens) == [51, 18, 17, 4]
    assert b.num_blocks == 64 and b.k_cache.dtype == torch.float16
    owned = [set(r[:acc.blocks_needed(int(L), 16)]) for r, L in zip(b.block_tables, b.seq_lens)]
    assert [len(o) for o in owned] == [4, 2, 2, 1]      # the 16-token one attached a block
    allb = set().union(*owned)
    assert len(allb) == 9 and b.poison_block not in allb
    assert abs(b.scale - 0.125) == 0.0


def test_slot_mapping_matches_oracle(oracle_mod):
    for b in (wl.make_tiny(), wl.make_shared_prefix(num_seqs=6, tail_hi=40)):
        ref = oracle_mod.slot_mapping(b.block_tables, b.append_seq, b.append_pos, b.block_size)
        assert np.array_equal(ref, b.slot_mapping)


def test_worked_example_block_counts():
    b = wl.make_worked_example()
    counts = [(r != b.poison_block).sum() for r in b.block_tables]
    assert counts == [244, 27, 132, 5] and sum(counts) == 408
    used = b.block_tables[b.block_tables != b.poison_block]
    assert len(set(used.tolist())) == 408                 # no block handed out twice
    assert not np.all(np.diff(used) == 1)                 # non-contiguous assignment
    assert b.kv_bytes() == 26_583_040


def test_pool_holds_the_drawn_rows(oracle_mod):
    """Placement check: gathering each sequence's rows back through its table
    (the oracle's slot formula) returns the rows the generator drew."""
    b = wl.make_decode_batch("t", [37, 5, 16], 4, 2, 32, 8, "bf16", seed=9, append=0)
    kp, vp = bits(b.k_cache), bits(b.v_cache)
    for s, L in enumerate(b.seq_lens):
        K, V = wl._seq_rows(9, s, int(L), 2, 32, "bf16")
        slots = oracle_mod.slot_mapping(b.block_tables, [s] * int(L), np.arange(L), 8)
        for t, sl in enumerate(slots):
            assert np.array_equal(kp[sl // 8, :, sl % 8], bits(K[t]))
            assert np.array_equal(vp[sl // 8, :, sl % 8], bits(V[t]))


def test_unused_slots_are_nan():
    b = wl.make_tiny()
    k = b.k_cache.float()
    used = 0
    for s, L in enumerate(b.context_lens):
        used += int(L)
    assert int((~torch.isnan(k[:, 0, :, 0])).sum()) == used


def test_padding_rows_are_skipped_slots():
    b = wl.make_decode_batch("p", [3, 9], 4, 2, 32, 8, "f16", seed=4, append=1, pad_tokens=3)
    assert (b.slot_mapping == -1).sum() == 3 and len(b.slot_mapping) == 5
    assert sorted(b.append_seq[b.slot_mapping >= 0].tolist()) == [0, 1]


def test_shared_prefix_structure():
    b = wl.make_shared_prefix()
    shared = b.info["shared_blocks"]
    r = b.info["r"]
    assert len(shared) == 128 and b.num_seqs == 64
    assert (b.block_tables[:, :127] == shared[:127]).all()          # all share 0..126
    assert (b.block_tables[::2, 127] == shared[127]).all()          # even: 127 too
    odd_last = b.block_tables[1::2, 127]
    assert len(set(odd_last.tolist())) == 32 and shared[127] not in odd_last
    assert len(b.block_mapping) == 32
    assert (b.block_mapping[:, 0] == shared[127]).all()
    assert (r[::2] == 0).all() and ((r[1::2] >= 1) & (r[1::2] <= 15)).all()
    assert (b.context_lens[1::2] % 16 != 0).all()
    assert np.array_equal(b.seq_lens, b.context_lens + b.info["tails"])


@pytest.mark.parametrize("bs", [8, 16, 32])
def test_long_context_logical_data_do_not_depend_on_block_size(bs):
    a = wl.make_decode_batch("x", [40, 70], 8, 2, 16, bs, "bf16", seed=5, append=0)
    ref = wl.make_decode_batch("x", [40, 70], 8, 2, 16, 16, "bf16", seed=5, append=0)
    assert np.array_equal(bits(a.q), bits(ref.q))


def test_fp8_pools_hold_drawn_codes_and_nan_elsewhere():
    b = wl.make_decode_batch("fp8_gen", [50, 17, 16, 3], 8, 2, 64, 16, "bf16", 1, append=1,
                             num_blocks=64, kv="fp8")
    k, v = b.k_cache.numpy(), b.v_cache.numpy()
    assert k.dtype == np.uint8 and b.elem_bytes == 1 and b.k_scale == 2.0 ** -6
    live = np.zeros(k.shape[0] * 16, bool)
    for s, c in enumerate(b.context_lens):
        for p in range(int(c)):
            live[b.block_tables[s, p // 16] * 16 + p % 16] = True
    flat_k = k.transpose(0, 2, 1, 3).reshape(-1, 2 * 64)
    flat_v = v.transpose(0, 2, 1, 3).reshape(-1, 2 * 64)
    assert np.all((flat_k[live] & 0x7F) <= 0x77) and np.all((flat_v[live] & 0x7F) <= 0x77)
    assert np.all(flat_k[~live] == 0x7F) and np.all(flat_v[~live] == 0x7F)
    # both signs and the whole magnitude range appear
    assert (flat_k[live] >> 7).min() == 0 and (flat_k[live] >> 7).max() == 1
    assert (flat_k[live] & 0x7F).max() == 0x77 and (flat_k[live] & 0x7F).min() == 0
    # the appended rows are 16-bit values, one per sequence
    assert b.new_key.dtype == torch.bfloat16 and b.new_key.shape == (4, 2, 64)
    assert b.kv_bytes() == int(b.seq_lens.sum()) * 2 * 2 * 64


def _logical_rows(b, kp, vp):
    """K and V rows of every sequence's positions 0..L-1, read through its table."""
    rows = []
    for s, L in enumerate(b.seq_lens):
        ids = b.block_tables[s]
        t = np.arange(int(L))
        rows.append((kp[ids[t // b.block_size], :, t % b.block_size],
                     vp[ids[t // b.block_size], :, t % b.block_size]))
    return rows


def test_private_prefix_twin_holds_the_same_logical_rows(oracle_mod):
    """make_shared_prefix(private_prefix=True): no copy-on-write pair, no
    shared block, and after the step every sequence reads the same rows as
    with the shared prefix."""
    kw = dict(num_seqs=10, prefix=96, tail_hi=50)
    a, b = wl.make_shared_prefix(**kw), wl.make_shared_prefix(private_prefix=True, **kw)
    assert len(a.block_mapping) == 5 and len(b.block_mapping) == 0
    assert np.array_equal(a.seq_lens, b.seq_lens)
    owned = [set(r[:-(-int(L) // 16)]) for r, L in zip(b.block_tables, b.seq_lens)]
    assert all(not (owned[i] & owned[j]) for i in range(10) for j in range(i))
    pools = []
    for x in (a, b):
        kp, vp = bits(x.k_cache).copy(), bits(x.v_cache).copy()
        oracle_mod.copy_blocks(kp, vp, x.block_mapping)
        oracle_mod.reshape_and_cache(bits(x.new_key), bits(x.new_value), kp, vp, x.slot_mapping)
        pools.append(_logical_rows(x, kp, vp))
    for (ka, va), (kb, vb) in zip(*pools):
        assert np.array_equal(ka, kb) and np.array_equal(va, vb)


def test_fp8_code_range():
    lens = [40, 33, 17]
    a = wl.make_decode_batch("c", lens, 8, 2, 64, 16, "bf16", 3, append=0, kv="fp8")
    b = wl.make_decode_batch("c", lens, 8, 2, 64, 16, "bf16", 3, append=0, kv="fp8",
                             fp8_max_code=wl.FP8_MAX_FINITE_CODE)
    live = lambda x: np.concatenate([r.reshape(-1) for pair in _logical_rows(
        x, x.k_cache.numpy(), x.v_cache.numpy()) for r in pair])
    ca, cb = live(a) & 0x7F, live(b) & 0x7F
    assert ca.max() <= wl.FP8_MAX_MAG_CODE
    assert cb.max() == wl.FP8_MAX_FINITE_CODE and (cb > wl.FP8_MAX_MAG_CODE).any()
    with pytest.raises(ValueError):
        wl.make_decode_batch("c", lens, 8, 2, 64, 16, "bf16", 3, kv="fp8", fp8_max_code=0x7F)


def test_v_mult_scales_only_the_values():
    lens = [20, 7]
    a = wl.make_decode_batch("m", lens, 8, 2, 64, 16, "bf16", 4)
    b = wl.make_decode_batch("m", lens, 8, 2, 64, 16, "bf16", 4, v_mult=64.0)
    assert np.array_equal(bits(a.k_cache), bits(b.k_cache))
    assert np.array_equal(bits(a.q), bits(b.q))
    live = ~torch.isnan(a.v_cache)
    # a power of two commutes with rounding to bf16 (float32's exponent range)
    assert torch.equal(a.v_cache[live].float() * 64, b.v_cache[live].float())
