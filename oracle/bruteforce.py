"""Second, independent CPU implementation for tiny inputs -- TEST INFRASTRUCTURE.

Pure-Python loops over Python floats (IEEE double) and ``math.exp``; 16-bit
patterns are widened with the ``struct`` module's own binary16 ('e') and
binary32 ('f') decoders.  It shares no code with ``pa_oracle.c``; the tests
use it to pin the C oracle on tiny inputs (it is far too slow for more).

It follows the same reading of the pages as the C oracle (block table maps
logical block -> physical block; position t at offset t % bs of logical block
t // bs; query head h reads KV head h // (Hq // Hkv); softmax attention with
an explicit scale), written the other way round: it first rebuilds each
sequence's contiguous K and V, then applies attention to those rows.
"""
import math
import struct

F16 = 0
BF16 = 1


def _value(bits: int, dtype: int) -> float:
    if dtype == F16:
        return struct.unpack("<e", struct.pack("<H", bits))[0]
    return struct.unpack("<f", struct.pack("<I", bits << 16))[0]


def decode(q, k_cache, v_cache, block_tables, seq_lens, scale, dtype):
    """Nested lists of floats: out[s][h][i].

    q: uint16 array [S][Hq][d]; pools uint16 [NB][Hkv][bs][d];
    block_tables [S][MB]; seq_lens [S]; scale is widened from float32.
    """
    S, Hq, d = q.shape
    NB, Hkv, bs, _ = k_cache.shape
    g = Hq // Hkv
    sc = float(struct.unpack("<f", struct.pack("<f", scale))[0])
    out = []
    for s in range(S):
        L = int(seq_lens[s])
        # contiguous rows of this sequence, gathered position by position
        keys = [[None] * L for _ in range(Hkv)]
        vals = [[None] * L for _ in range(Hkv)]
        for t in range(L):
            phys = int(block_tables[s][t // bs])
            off = t % bs
            for kh in range(Hkv):
                keys[kh][t] = [_value(int(x), dtype) for x in k_cache[phys][kh][off]]
                vals[kh][t] = [_value(int(x), dtype) for x in v_cache[phys][kh][off]]
        rows = []
        for h in range(Hq):
            kh = h // g
            qh = [_value(int(x), dtype) for x in q[s][h]]
            if L == 0:
                rows.append([0.0] * d)
                continue
            scores = []
            for t in range(L):
                acc = 0.0
                for i in range(d):
                    acc += qh[i] * keys[kh][t][i]
                scores.append(sc * acc)
            top = max(scores)
            weights = [math.exp(z - top) for z in scores]
            total = sum(weights)
            row = []
            for i in range(d):
                acc = 0.0
                for t in range(L):
                    acc += weights[t] * vals[kh][t][i]
                row.append(acc / total)
            rows.append(row)
        out.append(rows)
    return out
