"""CPU oracle for paged decode attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (``include/pa.h``,
the HIP library and its Python binding) never imports, links or calls it, and
the two share no code.  The seeded input generator is the one module both
sides use; it holds none of the method's arithmetic.

What is here:
  * ``pa_oracle.c`` (built by ``build.py``): fp64 paged decode attention, its
    split-by-partition form merged by log-sum-exp, the append
    (reshape_and_cache), the copy-on-write block copy and the slot formula;
    for 8-bit pools (OCP E4M3, one scale per pool) the code <-> value maps,
    the quantising append and decode over the dequantised pools; attention
    of several causal query tokens per sequence (chunked prefill).
  * ``block_manager``: a plain-Python model of the host block manager.
  * ``accounting``: block counts and KV byte arithmetic of the worked memory
    example ("What problem does PagedAttention solve ...", section "A
    concrete memory example").
  * ``bruteforce``: a second, independent pure-Python implementation for tiny
    inputs.

Pins (tests marked ``not gpu``): the pages' printed numbers, worked block ids
12/87/301/44, exact widening of every fp16/bf16 bit pattern, torch's CPU
scaled_dot_product_attention in float64 on the contiguous gather, closed forms
(L = 1, constant V, zero query), permutation / sharing / block-size
invariances and the brute force.  Where several readings of the pages were
possible the chosen one is stated where the function is defined.
"""
import ctypes
import os

import numpy as np

from . import build as _build

F16 = 0
BF16 = 1

_lib = None


def lib():
    """Load (building first if needed) the oracle's shared library."""
    global _lib
    if _lib is None:
        path = _build.build(force=False)
        L = ctypes.CDLL(path)
        i32, f32, vp = ctypes.c_int32, ctypes.c_float, ctypes.c_void_p
        L.oracle_decode.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                    f32, i32, vp, i32]
        L.oracle_decode_split.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                          i32, f32, i32, i32]
        L.oracle_reshape_and_cache.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32]
        L.oracle_copy_blocks.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32]
        L.oracle_slot_mapping.argtypes = [vp, vp, vp, vp, i32, i32, i32]
        L.oracle_f16_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_f16_to_double.restype = ctypes.c_double
        L.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_double.restype = ctypes.c_double
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_e4m3_to_double.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_to_double.restype = ctypes.c_double
        L.oracle_e4m3_from_float.argtypes = [f32]
        L.oracle_e4m3_from_float.restype = ctypes.c_uint8
        L.oracle_quantize_e4m3.argtypes = [vp, vp, ctypes.c_int64, i32, f32]
        L.oracle_reshape_and_cache_fp8.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                                   f32, f32, i32]
        L.oracle_decode_fp8.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                        i32, f32, f32, f32, i32, vp, i32]
        L.oracle_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                     i32, i32, f32, i32]
        for name in ("oracle_decode", "oracle_decode_split", "oracle_reshape_and_cache",
                     "oracle_copy_blocks", "oracle_slot_mapping", "oracle_quantize_e4m3",
                     "oracle_reshape_and_cache_fp8", "oracle_decode_fp8", "oracle_prefill"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


class OracleError(RuntimeError):
    pass


_ERRORS = {-1: "bad argument", -2: "table entry out of range", -3: "slot out of range",
           -4: "duplicate slot", -5: "bad copy pair", -6: "out of memory"}


def _check(rc):
    if rc != 0:
        raise OracleError(_ERRORS.get(rc, f"error {rc}"))


def _u16(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"expected raw 16-bit patterns (uint16), got {a.dtype}")
    return a


def _i32(a):
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def widen(bits, dtype):
    """Exact value of each 16-bit pattern as float64 (element-wise)."""
    f = lib().oracle_bf16_to_double if dtype == BF16 else lib().oracle_f16_to_double
    flat = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([f(int(x)) for x in flat], dtype=np.float64).reshape(np.shape(bits))


def decode(q, k_cache, v_cache, block_tables, seq_lens, scale, dtype, pairs=None):
    """fp64 paged decode attention.

    q [S][Hq][d], pools [NB][Hkv][bs][d] as uint16 bit patterns, block_tables
    [S][MB] int32, seq_lens [S] int32, scale a float32 value.  Returns
    out [S][Hq][d] float64.  With ``pairs`` (an [n][2] list of (s, h)) only
    those rows are computed; the other rows are NaN.
    """
    q, k_cache, v_cache = _u16(q), _u16(k_cache), _u16(v_cache)
    bt, sl = _i32(block_tables), _i32(seq_lens)
    S, Hq, d = q.shape
    NB, Hkv, bs, d2 = k_cache.shape
    assert d2 == d and v_cache.shape == k_cache.shape and bt.shape[0] == S and sl.shape == (S,)
    out = np.full((S, Hq, d), np.nan, dtype=np.float64)
    if pairs is not None:
        pr = _i32(np.asarray(pairs).reshape(-1, 2))
        pp, npairs = _p(pr), pr.shape[0]
    else:
        pr, pp, npairs = None, None, 0
    rc = lib().oracle_decode(_p(out), _p(q), _p(k_cache), _p(v_cache), _p(bt), _p(sl), S, Hq,
                             Hkv, d, bs, bt.shape[1], NB, float(np.float32(scale)), dtype, pp,
                             npairs)
    _check(rc)
    return out


def decode_split(q, k_cache, v_cache, block_tables, seq_lens, scale, dtype, partition_size):
    """The same attention merged from per-partition (m, l, acc) by log-sum-exp."""
    q, k_cache, v_cache = _u16(q), _u16(k_cache), _u16(v_cache)
    bt, sl = _i32(block_tables), _i32(seq_lens)
    S, Hq, d = q.shape
    NB, Hkv, bs, _ = k_cache.shape
    out = np.zeros((S, Hq, d), dtype=np.float64)
    rc = lib().oracle_decode_split(_p(out), _p(q), _p(k_cache), _p(v_cache), _p(bt), _p(sl), S,
                                   Hq, Hkv, d, bs, bt.shape[1], NB, float(np.float32(scale)),
                                   dtype, int(partition_size))
    _check(rc)
    return out


def reshape_and_cache(key, value, k_cache, v_cache, slot_mapping):
    """Append in place on host copies of the pools (bit copy)."""
    key, value = _u16(key), _u16(value)
    if not (k_cache.flags["C_CONTIGUOUS"] and v_cache.flags["C_CONTIGUOUS"]):
        raise ValueError("pools must be contiguous")
    _u16(k_cache), _u16(v_cache)
    sm = _i32(slot_mapping)
    T, Hkv, d = key.shape
    NB, Hkv2, bs, d2 = k_cache.shape
    assert Hkv2 == Hkv and d2 == d and sm.shape == (T,)
    _check(lib().oracle_reshape_and_cache(_p(key), _p(value), _p(k_cache), _p(v_cache), _p(sm),
                                          T, Hkv, d, bs, NB))


def copy_blocks(k_cache, v_cache, block_mapping):
    """Copy-on-write block copies in place on host copies of the pools."""
    if not (k_cache.flags["C_CONTIGUOUS"] and v_cache.flags["C_CONTIGUOUS"]):
        raise ValueError("pools must be contiguous")
    _u16(k_cache), _u16(v_cache)
    bm = _i32(np.asarray(block_mapping).reshape(-1, 2))
    NB, Hkv, bs, d = k_cache.shape
    _check(lib().oracle_copy_blocks(_p(k_cache), _p(v_cache), _p(bm), bm.shape[0], Hkv, d, bs,
                                    NB))


def slot_mapping(block_tables, seq_ids, positions, block_size):
    """slot = table[s][pos // bs] * bs + pos % bs for each (s, pos)."""
    bt = _i32(block_tables)
    si, pos = _i32(seq_ids), _i32(positions)
    out = np.zeros(si.shape, dtype=np.int32)
    _check(lib().oracle_slot_mapping(_p(out), _p(bt), _p(si), _p(pos), si.shape[0], bt.shape[1],
                                     int(block_size)))
    return out


# ---- 8-bit (OCP E4M3) KV pools

def _u8(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint8:
        raise TypeError(f"expected E4M3 codes (uint8), got {a.dtype}")
    return a


def e4m3_to_double(codes):
    """Exact value of each E4M3 code as float64 (NaN for the NaN codes)."""
    flat = np.asarray(codes, dtype=np.uint8).ravel()
    f = lib().oracle_e4m3_to_double
    return np.array([f(int(c)) for c in flat], dtype=np.float64).reshape(np.shape(codes))


def e4m3_from_float(y):
    """Nearest E4M3 code (ties to even, saturating) of each float32 value."""
    flat = np.asarray(y, dtype=np.float32).ravel()
    f = lib().oracle_e4m3_from_float
    return np.array([f(float(v)) for v in flat], dtype=np.uint8).reshape(np.shape(y))


def quantize_e4m3(bits, dtype, scale):
    """Codes of x / scale for raw 16-bit patterns x of ``dtype``."""
    x = _u16(bits)
    out = np.empty(x.shape, dtype=np.uint8)
    _check(lib().oracle_quantize_e4m3(_p(out), _p(x), x.size, dtype, float(np.float32(scale))))
    return out


def reshape_and_cache_fp8(key, value, k_cache, v_cache, slot_mapping, k_scale, v_scale, dtype):
    """Quantising append in place on host copies of 8-bit pools."""
    key, value = _u16(key), _u16(value)
    for a in (k_cache, v_cache):
        if a.dtype != np.uint8 or not a.flags["C_CONTIGUOUS"]:
            raise ValueError("pools must be contiguous uint8")
    sm = _i32(slot_mapping)
    T, Hkv, d = key.shape
    NB, Hkv2, bs, d2 = k_cache.shape
    assert Hkv2 == Hkv and d2 == d and sm.shape == (T,) and v_cache.shape == k_cache.shape
    _check(lib().oracle_reshape_and_cache_fp8(_p(key), _p(value), _p(k_cache), _p(v_cache),
                                              _p(sm), T, Hkv, d, bs, NB,
                                              float(np.float32(k_scale)),
                                              float(np.float32(v_scale)), dtype))


def copy_blocks_fp8(k_cache, v_cache, block_mapping):
    """Copy-on-write block copies of 8-bit pools: the same byte copy as
    ``copy_blocks``, run on the pools' bytes two at a time."""
    for a in (k_cache, v_cache):
        if a.dtype != np.uint8 or not a.flags["C_CONTIGUOUS"] or a.shape[-1] % 2:
            raise ValueError("pools must be contiguous uint8 with an even head_dim")
    copy_blocks(k_cache.view(np.uint16), v_cache.view(np.uint16), block_mapping)


def decode_fp8(q, k_cache, v_cache, block_tables, seq_lens, scale, k_scale, v_scale, dtype,
               pairs=None):
    """fp64 paged decode attention over 8-bit pools (codes read as
    e4m3(code) * scale of the pool); otherwise as ``decode``."""
    q, k_cache, v_cache = _u16(q), _u8(k_cache), _u8(v_cache)
    bt, sl = _i32(block_tables), _i32(seq_lens)
    S, Hq, d = q.shape
    NB, Hkv, bs, d2 = k_cache.shape
    assert d2 == d and v_cache.shape == k_cache.shape and bt.shape[0] == S and sl.shape == (S,)
    out = np.full((S, Hq, d), np.nan, dtype=np.float64)
    if pairs is not None:
        pr = _i32(np.asarray(pairs).reshape(-1, 2))
        pp, npairs = _p(pr), pr.shape[0]
    else:
        pr, pp, npairs = None, None, 0
    _check(lib().oracle_decode_fp8(_p(out), _p(q), _p(k_cache), _p(v_cache), _p(bt), _p(sl), S,
                                   Hq, Hkv, d, bs, bt.shape[1], NB, float(np.float32(scale)),
                                   float(np.float32(k_scale)), float(np.float32(v_scale)),
                                   dtype, pp, npairs))
    return out


# ---- several query tokens per sequence (chunked prefill)

def prefill(q, k_cache, v_cache, block_tables, seq_lens, query_start, scale, dtype):
    """fp64 causal attention of chunk tokens: q [total_q][Hq][d] (uint16
    patterns), query_start [S + 1]; token i of sequence s sits at position
    seq_lens[s] - n_s + i and attends to positions <= its own.  Returns out
    [total_q][Hq][d] float64."""
    q, k_cache, v_cache = _u16(q), _u16(k_cache), _u16(v_cache)
    bt, sl, qs = _i32(block_tables), _i32(seq_lens), _i32(query_start)
    T, Hq, d = q.shape
    NB, Hkv, bs, d2 = k_cache.shape
    S = sl.shape[0]
    assert d2 == d and v_cache.shape == k_cache.shape and bt.shape[0] == S and qs.shape == (S + 1,)
    out = np.full((T, Hq, d), np.nan, dtype=np.float64)
    _check(lib().oracle_prefill(_p(out), _p(q), _p(k_cache), _p(v_cache), _p(bt), _p(sl),
                                _p(qs), S, T, Hq, Hkv, d, bs, bt.shape[1], NB,
                                float(np.float32(scale)), dtype))
    return out
