"""Seeded synthetic paged-KV batches (host side; no attention arithmetic).

This is the one module that both the HIP path's callers (tests, bench) and the
CPU oracle's callers use to build inputs.  It draws lengths, block placements
and N(0, 1) values, lays the values out in a block pool, and produces block
tables, the append's slot mapping and copy-on-write pairs.  It computes no
attention and calls neither the GPU library nor the oracle.

Structure follows "What problem does PagedAttention solve, and what is
continuous batching?" (datarekha), sections "How PagedAttention works" (any
free block can be handed out; a block table maps logical -> physical block;
blocks may be shared, copy-on-write on divergence) and "A concrete memory
example" (the 3900/420/2100/70-token requests), and "Continuous Batching &
Paged Attention" (topicspectrum), section "Paged attention borrows a trick
from operating systems" (a growing request attaches another block).

Random streams (numpy ``default_rng``), one per purpose so that the logical
data do not depend on the block size, the placement or the thread that draws
them:
  * ``[seed, 0]``      lengths, prefix offsets and tail lengths;
  * ``[seed, 1, bs]``  the shuffled free list for block size bs;
  * ``[seed, 2]``      the query, [S][Hq][d];
  * ``[seed, 3, s]``   sequence s's K rows then V rows for every position it
                       holds after the step ([n][Hkv][d] each);
  * ``[seed, 4]``      a shared prefix's K rows then V rows;
  * ``[seed, 5]``      padding rows of the append and their shuffle;
  * ``[seed, 6, s]``   8-bit pools: sequence s's K codes then V codes for
                       the positions already in the pool;
  * ``[seed, 7, s]``   8-bit pools: its 16-bit K rows then V rows for the
                       positions the step appends;
  * ``[seed, 8]``      chunked prefill: the queries of every chunk token,
                       [total_q][Hq][d].
Values are float32 standard normal rounded to fp16/bf16 by
round-to-nearest-even.
Pool slots that hold no token are NaN (0x7E00 fp16, 0x7FC0 bf16); table
entries past a sequence's last block point at a never-allocated NaN block.

8-bit pools (``kv="fp8"``) hold OCP E4M3 codes drawn directly, not made from
values (no quantising happens here): a uniform sign bit and a magnitude code
uniform in 0x00..0x77 (0 to 240), i.e. values up to 3.75 at the default
scale 2^-6, or up to any code through 0x7E (448) on request; slots that hold
no token hold the NaN code 0x7F.  The appended
tokens' rows stay 16-bit N(0, 1) values, which the step's append quantises.
"""
import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np
import torch

DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16}


@dataclass
class PagedBatch:
    """One decode step's inputs, on the host (CPU tensors / numpy arrays).

    The pools hold the state *before* the step's copy-on-write and append.
    A step is: copy_blocks(block_mapping) -> reshape_and_cache(new_key,
    new_value, slot_mapping) -> decode at ``seq_lens``.
    """
    name: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: float
    q: torch.Tensor                  # [S][Hq][d]
    k_cache: torch.Tensor            # [NB][Hkv][bs][d]
    v_cache: torch.Tensor            # [NB][Hkv][bs][d]
    block_tables: np.ndarray         # int32 [S][MB]
    context_lens: np.ndarray         # int32 [S], tokens already in the pool
    seq_lens: np.ndarray             # int32 [S], tokens decode attends over
    new_key: torch.Tensor            # [T][Hkv][d]
    new_value: torch.Tensor          # [T][Hkv][d]
    slot_mapping: np.ndarray         # int32 [T]
    append_seq: np.ndarray           # int32 [T], sequence of each new token
    append_pos: np.ndarray           # int32 [T], its position
    block_mapping: np.ndarray        # int32 [n][2] (src, dst)
    poison_block: int                # a NaN block no sequence owns
    info: Dict = field(default_factory=dict)
    query_start: Optional[np.ndarray] = None  # chunked prefill: int32 [S + 1]; q is [total_q][Hq][d]
    kv: str = "16"                   # "16": pools of `dtype`; "fp8": E4M3 codes (uint8)
    k_scale: float = 1.0             # 8-bit pools: value of a key code = e4m3(code) * k_scale
    v_scale: float = 1.0

    @property
    def num_seqs(self) -> int:
        return int(len(self.seq_lens))

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def elem_bytes(self) -> int:
        return 1 if self.kv == "fp8" else 2

    def kv_bytes(self, lens=None) -> int:
        """Live K+V bytes one decode reads: sum_s L_s * 2 * Hkv * d * 2."""
        lens = self.seq_lens if lens is None else lens
        return int(np.asarray(lens, dtype=np.int64).sum()) * 2 * self.num_kv_heads * \
            self.head_dim * self.elem_bytes


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw 16-bit patterns of a CPU fp16/bf16 tensor as a uint16 array (no copy)."""
    t = t.detach().contiguous()
    return t.view(torch.int16).numpy().view(np.uint16)


def _round(x: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DTYPES[dtype])


def _nan_pool(nb, hkv, bs, d, dtype) -> torch.Tensor:
    return torch.full((nb, hkv, bs, d), float("nan"), dtype=DTYPES[dtype])


def _place(pool: torch.Tensor, ids, rows: torch.Tensor) -> None:
    """Write rows [n][Hkv][d] for positions 0 .. n-1 of a sequence whose
    logical blocks are ``ids``: position p goes to block ids[p // bs], slot
    p % bs.  Whole blocks are written at once, then the partial last one."""
    bs = pool.shape[2]
    n = rows.shape[0]
    full = n // bs
    if full:
        idx = torch.from_numpy(np.asarray(ids[:full], dtype=np.int64))
        pool[idx] = rows[:full * bs].reshape(full, bs, rows.shape[1],
                                             rows.shape[2]).permute(0, 2, 1, 3)
    rem = n - full * bs
    if rem:
        pool[int(ids[full]), :, :rem, :] = rows[full * bs:].permute(1, 0, 2)


def _seq_rows(seed: int, s: int, n: int, hkv: int, d: int, dtype: str, v_mult: float = 1.0):
    """Sequence s's K and V rows from its own stream [seed, 3, s]; the V
    draws are multiplied by v_mult before rounding."""
    rng = np.random.default_rng([seed, 3, s])
    k = _round(rng.standard_normal((n, hkv, d), dtype=np.float32), dtype)
    v = _round(rng.standard_normal((n, hkv, d), dtype=np.float32) * np.float32(v_mult), dtype)
    return k, v


def _all_rows(seed: int, counts, hkv: int, d: int, dtype: str, fn=None, **kw):
    """Rows of every sequence, drawn on a thread pool (numpy releases the GIL)."""
    fn = _seq_rows if fn is None else fn
    workers = max(1, min(16, os.cpu_count() or 1))
    with ThreadPoolExecutor(workers) as ex:
        futs = [ex.submit(fn, seed, s, int(n), hkv, d, dtype, **kw)
                for s, n in enumerate(counts)]
        return [f.result() for f in futs]


FP8_NAN = 0x7F
FP8_MAX_MAG_CODE = 0x77
FP8_DEFAULT_SCALE = 2.0 ** -6


FP8_MAX_FINITE_CODE = 0x7E   # 448, the largest finite E4M3 magnitude


def fp8_codes(rng: np.random.Generator, shape, max_code: int = FP8_MAX_MAG_CODE) -> torch.Tensor:
    """Random E4M3 codes: uniform sign, magnitude code uniform in
    [0, max_code] (at most FP8_MAX_FINITE_CODE: no NaN codes)."""
    if not 0 <= max_code <= FP8_MAX_FINITE_CODE:
        raise ValueError(f"max_code must be in [0, 0x7E], got {max_code:#x}")
    mag = rng.integers(0, max_code + 1, size=shape, dtype=np.uint8)
    sign = rng.integers(0, 2, size=shape, dtype=np.uint8) << 7
    return torch.from_numpy(mag | sign)


def _seq_codes(seed: int, s: int, n: int, hkv: int, d: int, dtype: str,
               max_code: int = FP8_MAX_MAG_CODE):
    """Sequence s's K and V codes for n stored positions, stream [seed, 6, s]."""
    rng = np.random.default_rng([seed, 6, s])
    return fp8_codes(rng, (n, hkv, d), max_code), fp8_codes(rng, (n, hkv, d), max_code)


def _seq_new_rows(seed: int, s: int, n: int, hkv: int, d: int, dtype: str):
    """16-bit K and V rows of the n tokens sequence s appends, stream [seed, 7, s]."""
    rng = np.random.default_rng([seed, 7, s])
    k = _round(rng.standard_normal((n, hkv, d), dtype=np.float32), dtype)
    v = _round(rng.standard_normal((n, hkv, d), dtype=np.float32), dtype)
    return k, v


class _FreeList:
    """Seeded shuffled free list; ``take`` hands out any free block."""

    def __init__(self, num_blocks: int, rng: np.random.Generator):
        self.order = rng.permutation(num_blocks).astype(np.int32)
        self.next = 0

    def take(self, n: int) -> np.ndarray:
        if self.next + n > len(self.order):
            raise RuntimeError("block pool exhausted")
        out = self.order[self.next:self.next + n]
        self.next += n
        return out

    def spare(self) -> int:
        if self.next >= len(self.order):
            raise RuntimeError("no spare block left for the poison entries")
        return int(self.order[-1])


def _blocks(n_tokens: int, bs: int) -> int:
    return -(-n_tokens // bs)


def make_decode_batch(name: str, context_lens, num_q_heads: int, num_kv_heads: int,
                      head_dim: int, block_size: int, dtype: str, seed: int,
                      append: int = 1, num_blocks: Optional[int] = None,
                      pool_slack: float = 0.10, scale: Optional[float] = None,
                      pad_tokens: int = 0, placement_seed: Optional[int] = None,
                      kv: str = "16", k_scale: float = FP8_DEFAULT_SCALE,
                      v_scale: float = FP8_DEFAULT_SCALE, v_mult: float = 1.0,
                      fp8_max_code: int = FP8_MAX_MAG_CODE) -> PagedBatch:
    """A batch of independent sequences (no sharing).

    ``context_lens[s]`` tokens are already in the pool; ``append`` (a count,
    or one count per sequence) new tokens per sequence are appended by the
    step, so decode attends over context + append.  Blocks for the context are taken from the free list in
    sequence order, then blocks attached by the append.  ``pad_tokens`` extra
    new-token rows with slot -1 are interleaved (the append skips them).
    ``placement_seed`` (default ``seed``) changes only where blocks go.
    ``kv="fp8"``: 8-bit pools of E4M3 codes with scales k_scale / v_scale
    (the 16-bit ``dtype`` is then that of q, the new rows and the output),
    magnitude codes drawn up to ``fp8_max_code`` (0x7E: every finite code).
    ``v_mult`` multiplies the 16-bit V draws (values N(0, v_mult^2)).
    """
    if kv not in ("16", "fp8"):
        raise ValueError(f"kv must be '16' or 'fp8', got {kv!r}")
    ctx = np.asarray(context_lens, dtype=np.int32)
    S = len(ctx)
    bs = block_size
    lens = ctx + append
    need = sum(_blocks(int(L), bs) for L in lens)
    if num_blocks is None:
        num_blocks = int(math.ceil((1.0 + pool_slack) * need)) + 1
    rng_place = np.random.default_rng([seed if placement_seed is None else placement_seed, 1, bs])
    free = _FreeList(num_blocks, rng_place)
    MB = max(1, max(_blocks(int(L), bs) for L in lens)) if S else 1
    tables = np.zeros((S, MB), dtype=np.int32)
    owned: List[np.ndarray] = []
    for s in range(S):
        ids = free.take(_blocks(int(ctx[s]), bs))
        owned.append(ids)
    for s in range(S):  # attaches made by the append
        extra = _blocks(int(lens[s]), bs) - len(owned[s])
        if extra > 0:
            owned[s] = np.concatenate([owned[s], free.take(extra)])
    poison = free.spare()
    for s in range(S):
        tables[s, :] = poison
        tables[s, :len(owned[s])] = owned[s]

    d, Hq, Hkv = head_dim, num_q_heads, num_kv_heads
    q = _round(np.random.default_rng([seed, 2]).standard_normal((S, Hq, d), dtype=np.float32),
               dtype)
    new_k, new_v, seqs, poss = [], [], [], []
    if kv == "fp8":
        k_pool = torch.full((num_blocks, Hkv, bs, d), FP8_NAN, dtype=torch.uint8)
        v_pool = torch.full((num_blocks, Hkv, bs, d), FP8_NAN, dtype=torch.uint8)
        codes = _all_rows(seed, ctx, Hkv, d, dtype, _seq_codes, max_code=fp8_max_code)
        fresh = _all_rows(seed, lens - ctx, Hkv, d, dtype, _seq_new_rows)
    else:
        k_pool = _nan_pool(num_blocks, Hkv, bs, d, dtype)
        v_pool = _nan_pool(num_blocks, Hkv, bs, d, dtype)
        rows = _all_rows(seed, lens, Hkv, d, dtype, v_mult=v_mult)
    for s in range(S):
        L = int(lens[s])
        c = int(ctx[s])
        if kv == "fp8":
            K, V = codes[s]
            codes[s] = None
            _place(k_pool, owned[s], K)
            _place(v_pool, owned[s], V)
            K, V = fresh[s]
            base = c
        else:
            K, V = rows[s]
            rows[s] = None
            _place(k_pool, owned[s], K[:c])
            _place(v_pool, owned[s], V[:c])
            base = 0
        for t in range(c, L):
            new_k.append(K[t - base])
            new_v.append(V[t - base])
            seqs.append(s)
            poss.append(t)
    T = len(seqs)
    slot = np.array([int(tables[s, p // bs]) * bs + p % bs for s, p in zip(seqs, poss)],
                    dtype=np.int32).reshape(T)
    if T:
        nk = torch.stack(new_k)
        nv = torch.stack(new_v)
    else:
        nk = torch.zeros((0, Hkv, d), dtype=DTYPES[dtype])
        nv = torch.zeros((0, Hkv, d), dtype=DTYPES[dtype])
    seqs_a = np.asarray(seqs, dtype=np.int32).reshape(T)
    poss_a = np.asarray(poss, dtype=np.int32).reshape(T)
    if pad_tokens:
        # padding rows (slot -1) with junk values, shuffled in among the real ones
        rng_pad = np.random.default_rng([seed, 5])
        junk_k = _round(rng_pad.standard_normal((pad_tokens, Hkv, d), dtype=np.float32), dtype)
        junk_v = _round(rng_pad.standard_normal((pad_tokens, Hkv, d), dtype=np.float32), dtype)
        order = rng_pad.permutation(T + pad_tokens)
        idx = torch.from_numpy(order)
        nk = torch.cat([nk, junk_k])[idx]
        nv = torch.cat([nv, junk_v])[idx]
        minus = np.full(pad_tokens, -1, np.int32)
        slot = np.concatenate([slot, minus])[order]
        seqs_a = np.concatenate([seqs_a, minus])[order]
        poss_a = np.concatenate([poss_a, minus])[order]
    sc = float(np.float32(1.0 / math.sqrt(d))) if scale is None else float(np.float32(scale))
    return PagedBatch(name=name, dtype=dtype, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d,
                      block_size=bs, num_blocks=num_blocks, scale=sc, q=q, k_cache=k_pool,
                      v_cache=v_pool, block_tables=tables, context_lens=ctx,
                      seq_lens=lens.astype(np.int32), new_key=nk.contiguous(),
                      new_value=nv.contiguous(), slot_mapping=slot.astype(np.int32),
                      append_seq=seqs_a, append_pos=poss_a,
                      block_mapping=np.zeros((0, 2), dtype=np.int32), poison_block=poison,
                      kv=kv, k_scale=float(np.float32(k_scale)) if kv == "fp8" else 1.0,
                      v_scale=float(np.float32(v_scale)) if kv == "fp8" else 1.0)


# --------------------------------------------------------------------------
# The five workloads.
# --------------------------------------------------------------------------

def make_tiny(seed: int = 1) -> PagedBatch:
    """4 sequences of 50/17/16/3 tokens, 8 q / 2 KV heads, d 64, fp16, block
    16, pool 64 blocks, scale 1/sqrt(64), one appended token per sequence
    (the 16-token sequence attaches a new block)."""
    return make_decode_batch("tiny", [50, 17, 16, 3], 8, 2, 64, 16, "f16", seed, append=1,
                             num_blocks=64, scale=1.0 / 8.0)


WORKED_EXAMPLE_LENS = (3900, 420, 2100, 70)


def make_worked_example(seed: int = 2) -> PagedBatch:
    """The pages' four requests (3900/420/2100/70 tokens = 244/27/132/5
    blocks of 16) as one layer: 32 q / 8 KV heads, d 128, fp16, pool 4096
    blocks with a seeded non-contiguous assignment.  Decode only."""
    return make_decode_batch("worked_example", list(WORKED_EXAMPLE_LENS), 32, 8, 128, 16,
                             "f16", seed, append=0, num_blocks=4096)


def mixed_lengths(num_seqs: int, lo: int, hi: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng([seed, 0])
    return rng.integers(lo, hi + 1, size=num_seqs).astype(np.int32)


def make_mixed_step(seed: int = 3, num_seqs: int = 256, lo: int = 64, hi: int = 4096,
                    dtype: str = "bf16", kv: str = "16") -> PagedBatch:
    """Continuous-batching decode step: 256 sequences with context lengths
    uniform in [64, 4096], 32 q / 8 KV heads, d 128, bf16, block 16, pool =
    total blocks + 10% from a seeded shuffled free list; the step appends one
    token per sequence, then decodes over context + 1.  ``kv="fp8"``: the
    same step over 8-bit pools."""
    ctx = mixed_lengths(num_seqs, lo, hi, seed)
    b = make_decode_batch("mixed_step" if kv == "16" else "mixed_step_fp8", ctx, 32, 8, 128, 16,
                          dtype, seed, append=1, kv=kv)
    return b


def make_long_context(block_size: int, seed: int = 5, num_seqs: int = 32, lo: int = 8192,
                      hi: int = 32768) -> PagedBatch:
    """Long-context split-K case: 32 sequences of 8192..32768 tokens, 64 q /
    8 KV heads (group 8), d 128, bf16, seeded placement per block size (the
    logical data do not depend on it).  Decode only."""
    lens = mixed_lengths(num_seqs, lo, hi, seed)
    return make_decode_batch(f"long_context_bs{block_size}", lens, 64, 8, 128, block_size,
                             "bf16", seed, append=0)


def make_shared_prefix(seed: int = 4, num_seqs: int = 64, prefix: int = 2048,
                       tail_lo: int = 1, tail_hi: int = 512, num_q_heads: int = 32,
                       num_kv_heads: int = 8, head_dim: int = 128, block_size: int = 16,
                       dtype: str = "f16", private_prefix: bool = False) -> PagedBatch:
    """Shared-prefix / beam case.

    All sequences reference the same physical blocks holding prefix tokens
    0..prefix-1.  In the odd-indexed half a sequence's own prefix stops r_s
    tokens short of the shared one (r_s uniform in [1, bs-1]), so its last
    prefix block is shared but partially its own: the step copies that block
    (copy-on-write) into a private block and appends the sequence's tail from
    offset bs - r_s.  Even-indexed sequences append their tail into fresh
    blocks.  Tails are uniform in [tail_lo, tail_hi] tokens.

    ``private_prefix=True`` builds the same sequences with no sharing: each
    holds its own copy of the prefix blocks (same rows, its own physical
    ids), so the step has no copy-on-write pair; the logical K/V of every
    sequence after the step is the same as with sharing.
    """
    assert prefix % block_size == 0
    bs, d, Hq, Hkv = block_size, head_dim, num_q_heads, num_kv_heads
    rng_len = np.random.default_rng([seed, 0])
    r = np.zeros(num_seqs, dtype=np.int32)
    odd = np.arange(num_seqs) % 2 == 1
    r[odd] = rng_len.integers(1, bs, size=int(odd.sum()))
    tails = rng_len.integers(tail_lo, tail_hi + 1, size=num_seqs).astype(np.int32)
    own_prefix = prefix - r
    lens = own_prefix + tails
    n_shared = prefix // bs
    if private_prefix:
        need = sum(max(_blocks(int(L), bs), n_shared) for L in lens)
    else:
        need = n_shared + int(odd.sum()) + sum(_blocks(int(L), bs) - n_shared for L in lens)
    num_blocks = int(math.ceil(1.1 * need)) + 1
    rng_place = np.random.default_rng([seed, 1, bs])
    free = _FreeList(num_blocks, rng_place)
    shared = None if private_prefix else free.take(n_shared)
    owned, pairs = [], []
    for s in range(num_seqs):
        if private_prefix:
            ids = free.take(n_shared)
        else:
            ids = shared.copy()
        if r[s] > 0 and not private_prefix:  # copy-on-write of the shared partial block
            dst = int(free.take(1)[0])
            pairs.append((int(shared[-1]), dst))
            ids[-1] = dst
        extra = _blocks(int(lens[s]), bs) - n_shared
        if extra > 0:
            ids = np.concatenate([ids, free.take(extra)])
        owned.append(ids)
    poison = free.spare()
    MB = max(len(x) for x in owned)
    tables = np.full((num_seqs, MB), poison, dtype=np.int32)
    for s in range(num_seqs):
        tables[s, :len(owned[s])] = owned[s]

    q = _round(np.random.default_rng([seed, 2]).standard_normal((num_seqs, Hq, d),
                                                                dtype=np.float32), dtype)
    k_pool = _nan_pool(num_blocks, Hkv, bs, d, dtype)
    v_pool = _nan_pool(num_blocks, Hkv, bs, d, dtype)
    rng_pre = np.random.default_rng([seed, 4])
    Kp = _round(rng_pre.standard_normal((prefix, Hkv, d), dtype=np.float32), dtype)
    Vp = _round(rng_pre.standard_normal((prefix, Hkv, d), dtype=np.float32), dtype)
    if private_prefix:
        for s in range(num_seqs):
            _place(k_pool, owned[s][:n_shared], Kp)
            _place(v_pool, owned[s][:n_shared], Vp)
    else:
        _place(k_pool, shared, Kp)
        _place(v_pool, shared, Vp)
    new_k, new_v, seqs, poss = [], [], [], []
    rows = _all_rows(seed, tails, Hkv, d, dtype)
    for s in range(num_seqs):
        Kt, Vt = rows[s]
        for i in range(int(tails[s])):
            new_k.append(Kt[i])
            new_v.append(Vt[i])
            seqs.append(s)
            poss.append(int(own_prefix[s]) + i)
    T = len(seqs)
    slot = np.array([int(tables[s, p // bs]) * bs + p % bs for s, p in zip(seqs, poss)],
                    dtype=np.int32)
    sc = float(np.float32(1.0 / math.sqrt(d)))
    return PagedBatch(name="shared_prefix", dtype=dtype, num_q_heads=Hq, num_kv_heads=Hkv,
                      head_dim=d, block_size=bs, num_blocks=num_blocks, scale=sc, q=q,
                      k_cache=k_pool, v_cache=v_pool, block_tables=tables,
                      context_lens=own_prefix.astype(np.int32), seq_lens=lens.astype(np.int32),
                      new_key=torch.stack(new_k).contiguous(),
                      new_value=torch.stack(new_v).contiguous(), slot_mapping=slot,
                      append_seq=np.asarray(seqs, np.int32), append_pos=np.asarray(poss, np.int32),
                      block_mapping=np.asarray(pairs, dtype=np.int32).reshape(-1, 2),
                      poison_block=poison,
                      info={"shared_blocks": None if shared is None else shared.copy(), "r": r,
                            "tails": tails, "prefix": prefix})


def make_prefill_batch(name: str, context_lens, chunk_lens, num_q_heads: int,
                       num_kv_heads: int, head_dim: int, block_size: int, dtype: str,
                       seed: int, **kw) -> PagedBatch:
    """Chunked prefill: sequence s has context_lens[s] tokens in the pool and
    a chunk of chunk_lens[s] new tokens that the step appends (slot_mapping,
    new_key, new_value) and then attends with, causally: chunk token i sits
    at position context + i.  q holds one row per chunk token, [total_q][Hq]
    [d] from stream [seed, 8]; query_start[s] is sequence s's first row."""
    chunks = np.asarray(chunk_lens, dtype=np.int32)
    b = make_decode_batch(name, context_lens, num_q_heads, num_kv_heads, head_dim, block_size,
                          dtype, seed, append=chunks, **kw)
    T = int(chunks.sum())
    b.q = _round(np.random.default_rng([seed, 8]).standard_normal((T, num_q_heads, head_dim),
                                                                  dtype=np.float32), dtype)
    b.query_start = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    return b


def make_chunked_prefill(seed: int = 6, num_seqs: int = 32, chunk: int = 512, lo: int = 1024,
                         hi: int = 4096, dtype: str = "bf16") -> PagedBatch:
    """Chunked-prefill step: 32 sequences with total lengths uniform in
    [1024, 4096] whose last 512 tokens are this step's chunk, 32 q / 8 KV
    heads, d 128, bf16, block 16, pool of total blocks + 10% from a seeded
    shuffled free list."""
    lens = mixed_lengths(num_seqs, lo, hi, seed)
    chunks = np.full(num_seqs, chunk, dtype=np.int32)
    return make_prefill_batch("chunked_prefill", lens - chunks, chunks, 32, 8, 128, 16, dtype,
                              seed)


WORKLOADS = {
    "tiny": make_tiny,
    "worked_example": make_worked_example,
    "mixed_step": make_mixed_step,
    "shared_prefix": make_shared_prefix,
}


def to_device(b: PagedBatch, device) -> Dict[str, torch.Tensor]:
    """Device copies of every array a step needs."""
    dev = torch.device(device)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    return {
        "q": b.q.to(dev),
        "k_cache": b.k_cache.to(dev),
        "v_cache": b.v_cache.to(dev),
        "block_tables": i32(b.block_tables),
        "seq_lens": i32(b.seq_lens),
        "context_lens": i32(b.context_lens),
        "new_key": b.new_key.to(dev),
        "new_value": b.new_value.to(dev),
        "slot_mapping": i32(b.slot_mapping),
        "block_mapping": i32(b.block_mapping.reshape(-1, 2)),
    }
