"""GPU parity of pa_prefill (several causal query tokens per sequence,
chunked prefill) against the float64 CPU oracle, through the C ABI.

Each step appends the chunks' keys and values (pa_reshape_and_cache, pools
compared bit for bit) and then runs pa_prefill; outputs are held to the
attention tolerance (max-abs 1e-2 beyond half an ulp of the output type,
mean-abs 1e-3: a chunk's first tokens see few positions, so their outputs
can be as large as the values).

Cases: whole prompts (chunk = sequence), chunks after a context, single-
token chunks (decode), empty chunks, many sequences (more than 64
(sequence, KV head) pairs per XCD, where units are not ordered by context), chunk lengths that are not multiples
of the 16 / G tokens a unit holds, lengths around tile and block
boundaries, every query group, head size, block size and output type; a
chunk longer than its sequence and a block id outside the pool (NaN rows of
that sequence's chunk only); and the benchmark's chunked-prefill step at
full size (32 sequences x 512-token chunks), every row against
oracle.prefill.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_400_amd as pa
from _gpu import compare
from paged_kv_cache_400_amd import workload as wl
from paged_kv_cache_400_amd.workload import bits

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
OD = {"bf16": oracle.BF16, "f16": oracle.F16}


def _step(b):
    dev = wl.to_device(b, DEV)
    pa.reshape_and_cache(dev["new_key"], dev["new_value"], dev["k_cache"], dev["v_cache"],
                         dev["slot_mapping"])
    qs = torch.from_numpy(b.query_start).to(DEV)
    out = pa.prefill(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                     dev["seq_lens"], qs, scale=b.scale)
    torch.cuda.synchronize()
    return out, dev, qs


def _pools(b):
    kp, vp = bits(b.k_cache).copy(), bits(b.v_cache).copy()
    oracle.reshape_and_cache(bits(b.new_key), bits(b.new_value), kp, vp, b.slot_mapping)
    return kp, vp


CASES = [
    # name, context lens, chunk lens, hq, hkv, d, bs, dtype
    ("whole_prompts_g4", [0, 0, 0, 0], [37, 64, 1, 300], 32, 8, 128, 16, "bf16"),
    ("chunks_g4", [100, 5, 33, 500, 0], [20, 1, 40, 77, 16], 32, 8, 128, 16, "bf16"),
    ("g1_d64_bs8", [0, 9, 30, 0], [5, 16, 17, 100], 4, 4, 64, 8, "f16"),
    ("g2_d64_bs16", [15, 16, 17, 0, 1], [1, 31, 33, 48, 2], 8, 4, 64, 16, "f16"),
    ("g8_d128_bs32", [0, 64, 1000, 7], [63, 0, 130, 1], 64, 8, 128, 32, "bf16"),
    ("decode_only", [50, 17, 16, 3, 1000], [1, 1, 1, 1, 1], 16, 4, 128, 16, "bf16"),
    # more than 64 (sequence, KV head) pairs per XCD: units taken in pair order
    # instead of by context length
    ("many_pairs", [int(x) for x in np.random.default_rng(11).integers(0, 120, 70)],
     [int(x) for x in np.random.default_rng(12).integers(0, 40, 70)], 16, 8, 64, 16, "bf16"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_prefill_step_matches_oracle(case):
    name, ctx, chunks, hq, hkv, d, bs, dtype = case
    b = wl.make_prefill_batch(name, ctx, chunks, hq, hkv, d, bs, dtype, seed=41)
    out, dev, _ = _step(b)
    kp, vp = _pools(b)
    assert np.array_equal(bits(dev["k_cache"].cpu()), kp), "K pool differs after the append"
    assert np.array_equal(bits(dev["v_cache"].cpu()), vp), "V pool differs after the append"
    ref = oracle.prefill(bits(b.q), kp, vp, b.block_tables, b.seq_lens, b.query_start, b.scale,
                         OD[dtype])
    compare(out, ref, label=name, round_slack=True)


@pytest.mark.parametrize("what", ["chunk_longer_than_sequence", "block_id"])
def test_contract_violation_gives_nan_rows_of_that_chunk_only(what):
    b = wl.make_prefill_batch("violation", [300, 40, 700, 0], [20, 9, 33, 64], 16, 4, 128, 16,
                              "bf16", seed=42)
    kp, vp = _pools(b)
    dev = wl.to_device(b, DEV)
    pa.reshape_and_cache(dev["new_key"], dev["new_value"], dev["k_cache"], dev["v_cache"],
                         dev["slot_mapping"])
    bad = 1
    lens = dev["seq_lens"].clone()
    bt = dev["block_tables"].clone()
    if what == "chunk_longer_than_sequence":
        lens[bad] = 5          # the chunk has 9 tokens
    else:
        bt[bad, 0] = b.num_blocks + 3
    qs = torch.from_numpy(b.query_start).to(DEV)
    out = pa.prefill(dev["q"], dev["k_cache"], dev["v_cache"], bt, lens, qs, scale=b.scale)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    rows_bad = np.arange(b.query_start[bad], b.query_start[bad + 1])
    assert np.all(np.isnan(got[rows_bad]))
    keep = [s for s in range(b.num_seqs) if s != bad]
    ref = oracle.prefill(bits(b.q), kp, vp, b.block_tables, b.seq_lens, b.query_start, b.scale,
                         oracle.BF16)
    rows = np.concatenate([np.arange(b.query_start[s], b.query_start[s + 1]) for s in keep])
    compare(out[torch.from_numpy(rows).to(DEV)], ref[rows], label=f"violation {what}",
            round_slack=True)


def test_empty_batch_and_empty_chunks_write_nothing():
    b = wl.make_prefill_batch("empties", [10, 20], [0, 3], 8, 2, 64, 16, "bf16", seed=43)
    out, dev, qs = _step(b)
    kp, vp = _pools(b)
    ref = oracle.prefill(bits(b.q), kp, vp, b.block_tables, b.seq_lens, b.query_start, b.scale,
                         oracle.BF16)
    compare(out, ref, label="empty chunk", round_slack=True)
    # total_q = 0: nothing launched, nothing written
    empty = torch.empty((0, 8, 64), dtype=torch.bfloat16, device=DEV)
    zero = torch.zeros(3, dtype=torch.int32, device=DEV)
    pa.prefill(empty, dev["k_cache"], dev["v_cache"], dev["block_tables"], dev["seq_lens"], zero)
    torch.cuda.synchronize()


@pytest.mark.timeout(900)
def test_chunked_prefill_step_full_size_every_row():
    """The benchmark's chunked-prefill step at full size, in the launch the
    benchmark times: every (chunk token, query head) row, 16,384 x 32, against
    oracle.prefill (float64; about 45 s on 16 host cores)."""
    b = wl.make_chunked_prefill()
    out, dev, _ = _step(b)
    kp, vp = _pools(b)
    assert np.array_equal(bits(dev["k_cache"].cpu()), kp)
    assert np.array_equal(bits(dev["v_cache"].cpu()), vp)
    ref = oracle.prefill(bits(b.q), kp, vp, b.block_tables, b.seq_lens, b.query_start, b.scale,
                         oracle.BF16)
    assert ref.shape == (16384, 32, 128)
    compare(out, ref, label="chunked prefill, every row", round_slack=True)
