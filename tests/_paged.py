"""Small test-side helpers: build a paged pool from contiguous rows, and the
contiguous reference through torch's CPU scaled_dot_product_attention.

Independent of both the product and the oracle; used by the CPU pin tests.
"""
import math

import numpy as np
import torch

TDT = {0: torch.float16, 1: torch.bfloat16}


def rand_rows(rng, n, hkv, d, tdtype):
    return torch.from_numpy(rng.standard_normal((n, hkv, d), dtype=np.float32)).to(tdtype)


def u16(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def build_pool(rows_k, rows_v, bs, num_blocks, rng, tdtype, fill=float("nan"), ids=None):
    """Place each sequence's contiguous rows [L][Hkv][d] into a pool
    [NB][Hkv][bs][d] at shuffled physical blocks (or the given ``ids``).

    Returns (k_pool, v_pool, block_tables, seq_lens, spare) with unused slots
    set to ``fill`` and unused table entries pointing at a spare block."""
    S = len(rows_k)
    hkv, d = rows_k[0].shape[1], rows_k[0].shape[2]
    nbl = [-(-r.shape[0] // bs) for r in rows_k]
    mb = max(1, max(nbl))
    kp = torch.full((num_blocks, hkv, bs, d), fill, dtype=tdtype)
    vp = torch.full((num_blocks, hkv, bs, d), fill, dtype=tdtype)
    order = rng.permutation(num_blocks) if ids is None else None
    spare = int(order[-1]) if ids is None else int(num_blocks - 1)
    tables = np.full((S, mb), spare, dtype=np.int32)
    nxt = 0
    for s in range(S):
        if ids is None:
            my = order[nxt:nxt + nbl[s]]
            nxt += nbl[s]
        else:
            my = np.asarray(ids[s])
        tables[s, :nbl[s]] = my
        for t in range(rows_k[s].shape[0]):
            b, o = int(my[t // bs]), t % bs
            kp[b, :, o, :] = rows_k[s][t]
            vp[b, :, o, :] = rows_v[s][t]
    lens = np.array([r.shape[0] for r in rows_k], dtype=np.int32)
    return kp, vp, tables, lens, spare


def sdpa_reference(q, rows_k, rows_v, scale):
    """float64 torch CPU scaled_dot_product_attention over each sequence's
    contiguous K/V, KV heads repeated for their group of query heads."""
    S, Hq, d = q.shape
    out = np.zeros((S, Hq, d), dtype=np.float64)
    for s in range(S):
        L = rows_k[s].shape[0]
        if L == 0:
            continue
        hkv = rows_k[s].shape[1]
        g = Hq // hkv
        K = rows_k[s].double().permute(1, 0, 2).repeat_interleave(g, dim=0)  # [Hq][L][d]
        V = rows_v[s].double().permute(1, 0, 2).repeat_interleave(g, dim=0)
        Q = q[s].double().unsqueeze(1)  # [Hq][1][d]
        o = torch.nn.functional.scaled_dot_product_attention(
            Q.unsqueeze(0), K.unsqueeze(0), V.unsqueeze(0), scale=float(scale))
        out[s] = o[0, :, 0, :].numpy()
    return out


def f32(x):
    return float(np.float32(x))


def default_scale(d):
    return f32(1.0 / math.sqrt(d))
