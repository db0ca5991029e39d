"""Pins of the oracle's chunked-prefill attention (oracle_prefill) to things
outside its own code:

  * one chunk token per sequence is decode: bit for bit the (already
    pinned) decode oracle;
  * a whole prompt (chunk = sequence) equals torch's scaled_dot_product_
    attention in float64 with its causal flag, on the sequence's keys and
    values gathered into contiguous arrays;
  * a chunk that follows a context equals the same library routine with an
    explicit mask letting token i see positions <= context + i (torch's own
    causal flag aligns the mask to the top-left, which is not this reading);
  * every chunk token equals decode over its own prefix (positions 0..p);
  * chunks longer than their sequence, and a query_start that does not end
    at the number of rows, are refused.

The reading pinned ("What problem does PagedAttention solve, and what is
continuous batching?", sections "Why the KV cache becomes the problem" and
"How the two fit together in production"): a chunk's keys and values are in
the pool before its attention, and chunk token i sits at position
L - n + i.
"""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_400_amd import workload as wl
from paged_kv_cache_400_amd.workload import bits


def _batch(ctx, chunks, hq=8, hkv=2, d=64, bs=16, dtype="bf16", seed=3):
    return wl.make_prefill_batch("pin", ctx, chunks, hq, hkv, d, bs, dtype, seed)


def _pools(b):
    kp, vp = bits(b.k_cache).copy(), bits(b.v_cache).copy()
    oracle.reshape_and_cache(bits(b.new_key), bits(b.new_value), kp, vp, b.slot_mapping)
    return kp, vp


def _run(b, kp, vp):
    return oracle.prefill(bits(b.q), kp, vp, b.block_tables, b.seq_lens, b.query_start, b.scale,
                          oracle.BF16 if b.dtype == "bf16" else oracle.F16)


def _gather(b, kp, vp, s):
    """K and V of sequence s as float64 [L][Hkv][d], through its table."""
    L = int(b.seq_lens[s])
    pos = np.arange(L)
    blk, off = b.block_tables[s, pos // b.block_size], pos % b.block_size
    dt = oracle.BF16 if b.dtype == "bf16" else oracle.F16
    return oracle.widen(kp[blk, :, off, :], dt), oracle.widen(vp[blk, :, off, :], dt)


def test_one_token_per_sequence_is_decode():
    b = _batch([50, 17, 0, 3, 200], [1, 1, 1, 1, 1])
    kp, vp = _pools(b)
    got = _run(b, kp, vp)
    ref = oracle.decode(bits(b.q), kp, vp, b.block_tables, b.seq_lens, b.scale, oracle.BF16)
    assert np.array_equal(got, ref)


def _sdpa(q, k, v, scale, mask=None, causal=False):
    # q [n][Hq][d], k/v [L][Hkv][d] float64 -> [n][Hq][d]
    hq, hkv = q.shape[1], k.shape[1]
    kk = torch.from_numpy(np.repeat(k, hq // hkv, axis=1)).permute(1, 0, 2)
    vv = torch.from_numpy(np.repeat(v, hq // hkv, axis=1)).permute(1, 0, 2)
    qq = torch.from_numpy(q).permute(1, 0, 2)
    m = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=m,
                                                         is_causal=causal, scale=scale)
    return o.permute(1, 0, 2).numpy()


def test_whole_prompt_is_causal_attention():
    b = _batch([0, 0], [37, 64])
    kp, vp = _pools(b)
    got = _run(b, kp, vp)
    for s in range(2):
        k, v = _gather(b, kp, vp, s)
        rows = slice(b.query_start[s], b.query_start[s + 1])
        q = oracle.widen(bits(b.q)[rows], oracle.BF16)
        ref = _sdpa(q, k, v, float(np.float32(b.scale)), causal=True)
        np.testing.assert_allclose(got[rows], ref, rtol=1e-12, atol=1e-12)


def test_chunk_after_context_sees_context_plus_its_own_prefix():
    b = _batch([100, 5, 33], [20, 1, 40])
    kp, vp = _pools(b)
    got = _run(b, kp, vp)
    for s in range(3):
        L, n = int(b.seq_lens[s]), int(b.query_start[s + 1] - b.query_start[s])
        k, v = _gather(b, kp, vp, s)
        rows = slice(b.query_start[s], b.query_start[s + 1])
        q = oracle.widen(bits(b.q)[rows], oracle.BF16)
        mask = np.arange(L)[None, :] <= (L - n + np.arange(n))[:, None]
        ref = _sdpa(q, k, v, float(np.float32(b.scale)), mask=mask)
        np.testing.assert_allclose(got[rows], ref, rtol=1e-12, atol=1e-12)


def test_every_token_is_decode_over_its_prefix():
    b = _batch([30, 0], [12, 9], dtype="f16")
    kp, vp = _pools(b)
    got = _run(b, kp, vp)
    for s in range(2):
        L, n = int(b.seq_lens[s]), int(b.query_start[s + 1] - b.query_start[s])
        for i in range(n):
            row = int(b.query_start[s]) + i
            lens = np.array([L - n + i + 1], np.int32)
            ref = oracle.decode(bits(b.q)[row:row + 1], kp, vp, b.block_tables[s:s + 1], lens,
                                b.scale, oracle.F16)
            assert np.array_equal(got[row], ref[0])


def test_contract_errors():
    b = _batch([10, 4], [3, 2])
    kp, vp = _pools(b)
    bad = b.query_start.copy()
    bad[1] = 20                                  # chunk of 20 in a sequence of 13
    with pytest.raises(oracle.OracleError):
        oracle.prefill(bits(b.q), kp, vp, b.block_tables, b.seq_lens, bad, b.scale, oracle.BF16)
    bad = b.query_start.copy()
    bad[-1] = 4                                  # does not end at the number of rows
    with pytest.raises(oracle.OracleError):
        oracle.prefill(bits(b.q), kp, vp, b.block_tables, b.seq_lens, bad, b.scale, oracle.BF16)
