"""Python binding of libpa (include/pa.h): argument marshalling only.

Every function checks the tensors' device, dtype, shape and contiguity,
passes their device pointers and the current HIP stream of their device to
the C ABI, and raises :class:`PaError` with the library's message on a
non-OK status.  No step of the computation runs here; PyTorch supplies the
memory and the stream.  If ``libpa.so`` has not been built the import fails
loudly: there is no fallback.
"""
import ctypes
import os

import torch  # first: libpa binds to the HIP runtime torch has loaded

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")

(PA_OK, PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP,
 PA_ERR_NO_BLOCKS) = range(7)
PA_F16, PA_BF16, PA_FP8_E4M3 = 0, 1, 2
_DT = {torch.float16: PA_F16, torch.bfloat16: PA_BF16}
# pool element types: 16-bit pools hold `dtype` values, 8-bit pools (uint8
# tensors) hold OCP E4M3 codes
_POOL_DT = {torch.float16: PA_F16, torch.bfloat16: PA_BF16, torch.uint8: PA_FP8_E4M3}

# (name, restype, argtypes) for every entry point of include/pa.h, include/pa_probe.h,
# include/pa_block_manager.h and include/pa_scheduler.h
_vp, _i32, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "pa_decode": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                 _i32, _i32, _f32, _i32, ctypes.c_int, _vp, _sz, _vp]),
    "pa_decode_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                         _i32, _i32, _i32, _f32, _i32, ctypes.c_int, _vp]),
    "pa_probe_decode_mfma": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                            _i32, _i32, _i32, _i32, _f32, _i32, ctypes.c_int,
                                            _vp, _sz, _vp]),
    "pa_decode_shared_prefix": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                               _i32, _i32, _i32, _i32, _i32, _f32,
                                               ctypes.c_int, _vp, _sz, _vp]),
    "pa_decode_shared_prefix_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "pa_decode_valu": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                      _i32, _i32, _i32, _f32, _i32, ctypes.c_int, _vp, _sz, _vp]),
    "pa_decode_fp8": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                     _i32, _i32, _i32, _f32, _f32, _f32, ctypes.c_int, _vp, _sz,
                                     _vp]),
    "pa_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_prefill": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                  _i32, _i32, _i32, _f32, ctypes.c_int, _vp]),
    "pa_reshape_and_cache_fp8": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                                _i32, _f32, _f32, ctypes.c_int, _vp]),
    "pa_reshape_and_cache": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                            _i32, ctypes.c_int, _vp]),
    "pa_copy_blocks": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                      ctypes.c_int, _vp]),
    "pa_probe_gather": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                       _i32, _i32, ctypes.c_int, _vp]),
    "pa_probe_stream": (ctypes.c_int, [_vp, _vp, _sz, _vp]),
    "pa_bm_create": (ctypes.c_int, [_i32, _i32, _vp, ctypes.POINTER(_vp)]),
    "pa_bm_destroy": (None, [_vp]),
    "pa_bm_num_free": (_i32, [_vp]),
    "pa_bm_add_sequence": (ctypes.c_int, [_vp, ctypes.c_int64, _vp, _i32, _vp, _vp]),
    "pa_bm_append": (ctypes.c_int, [_vp, ctypes.c_int64, _vp, _i32, _vp, _vp, _i32, _vp]),
    "pa_bm_append_batch": (ctypes.c_int, [_vp, _vp, _vp, _i32, _vp, _vp, _i32, _vp]),
    "pa_bm_fork": (ctypes.c_int, [_vp, ctypes.c_int64, ctypes.c_int64]),
    "pa_bm_free": (ctypes.c_int, [_vp, ctypes.c_int64]),
    "pa_bm_tables": (ctypes.c_int, [_vp, _vp, _i32, _i32, _i32, _vp, _vp]),
    "pa_bm_block_refs": (_i32, [_vp, _i32]),
    "pa_sched_create": (ctypes.c_int, [_i32, _i32, _i32, _i32, _i32, _i32, ctypes.POINTER(_vp)]),
    "pa_sched_destroy": (None, [_vp]),
    "pa_sched_add": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i32]),
    "pa_sched_step": (ctypes.c_int, [_vp, _vp]),
    "pa_sched_active": (ctypes.c_int64, [_vp]),
    "pa_sched_request": (ctypes.c_int, [_vp, ctypes.c_int64, _vp]),
    "pa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pa_last_error": (ctypes.c_char_p, []),
    "pa_abi_version": (ctypes.c_int32, []),
}


class PaError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(f"{_lib.pa_status_string(status).decode()}: {message}")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with paged_kv_cache_400_amd/build.py "
            "(hipcc, gfx950); there is no CPU fallback")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def abi_version() -> int:
    return int(_lib.pa_abi_version())


def _check(status: int):
    if status != PA_OK:
        raise PaError(status, _lib.pa_last_error().decode())


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t, name, dims=None, dtype=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dims is not None and t.dim() != dims:
        raise ValueError(f"{name} must have {dims} dimensions, got shape {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_blocks_per_seq, block_size,
                           partition_size=0) -> int:
    return int(_lib.pa_decode_workspace_bytes(num_seqs, num_q_heads, head_dim,
                                              max_blocks_per_seq, block_size, partition_size))


_DECODE_FN = {"auto": "pa_decode", "valu": "pa_decode_valu", "mfma": "pa_probe_decode_mfma"}


def decode(q, k_cache, v_cache, block_tables, seq_lens, scale=None, partition_size=0, out=None,
           workspace=None, impl="auto"):
    """out[s][h] = softmax(scale * q[s][h] . K) V over the sequence's paged K/V.

    q [S][Hq][d]; k_cache/v_cache [NB][Hkv][bs][d]; block_tables int32
    [S][MB]; seq_lens int32 [S].  ``workspace`` (a uint8 tensor) is allocated
    when needed and not given.  ``impl``: "auto" (pa_decode, the tile wave
    chosen by the query group), "valu" (pa_decode_valu, the vector unit
    alone) or "mfma" (pa_probe_decode_mfma, the matrix cores at every group).
    """
    if impl not in _DECODE_FN:
        raise ValueError(f"impl must be one of {sorted(_DECODE_FN)}, got {impl!r}")
    _need(q, "q", 3)
    dev = q.device
    if q.dtype not in _DT:
        raise ValueError(f"q must be float16 or bfloat16, got {q.dtype}")
    _need(k_cache, "k_cache", 4, q.dtype, dev)
    _need(v_cache, "v_cache", 4, q.dtype, dev)
    _need(block_tables, "block_tables", 2, torch.int32, dev)
    _need(seq_lens, "seq_lens", 1, torch.int32, dev)
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must have the same shape")
    S, Hq, d = q.shape
    NB, Hkv, bs, d2 = k_cache.shape
    if d2 != d or block_tables.shape[0] != S or seq_lens.shape[0] != S:
        raise ValueError("inconsistent shapes between q, the pools, block_tables and seq_lens")
    MB = block_tables.shape[1]
    if scale is None:
        scale = d ** -0.5
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", 3, q.dtype, dev)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    need = decode_workspace_bytes(S, Hq, d, MB, bs, partition_size)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0
    if workspace is not None:
        _need(workspace, "workspace", None, None, dev)
        ws_bytes = workspace.numel() * workspace.element_size()
    fn = getattr(_lib, _DECODE_FN[impl])
    _check(fn(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
              _ptr(block_tables), _ptr(seq_lens), S, Hq, Hkv, d, bs, MB, NB, float(scale),
              int(partition_size), _DT[q.dtype], _ptr(workspace), ws_bytes, _stream(dev)))
    return out


def decode_noalloc(q, k_cache, v_cache, block_tables, seq_lens, out, scale=None,
                   partition_size=0):
    """pa_decode_noalloc: decode with the library's static scratch instead of a
    workspace; ``out`` [S][Hq][d] is required (nothing is allocated here
    either).  Calls that overlap on one GPU race on that scratch."""
    _need(q, "q", 3)
    dev = q.device
    if q.dtype not in _DT:
        raise ValueError(f"q must be float16 or bfloat16, got {q.dtype}")
    _need(k_cache, "k_cache", 4, q.dtype, dev)
    _need(v_cache, "v_cache", 4, q.dtype, dev)
    _need(block_tables, "block_tables", 2, torch.int32, dev)
    _need(seq_lens, "seq_lens", 1, torch.int32, dev)
    _need(out, "out", 3, q.dtype, dev)
    if k_cache.shape != v_cache.shape or out.shape != q.shape:
        raise ValueError("k_cache and v_cache must match, and out must have q's shape")
    S, Hq, d = q.shape
    NB, Hkv, bs, d2 = k_cache.shape
    if d2 != d or block_tables.shape[0] != S or seq_lens.shape[0] != S:
        raise ValueError("inconsistent shapes between q, the pools, block_tables and seq_lens")
    if scale is None:
        scale = d ** -0.5
    _check(_lib.pa_decode_noalloc(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                  _ptr(block_tables), _ptr(seq_lens), S, Hq, Hkv, d, bs,
                                  block_tables.shape[1], NB, float(scale), int(partition_size),
                                  _DT[q.dtype], _stream(dev)))
    return out


def decode_shared_prefix(q, k_cache, v_cache, block_tables, seq_lens, prefix_blocks, scale=None,
                         out=None, workspace=None):
    """pa_decode_shared_prefix: decode of sequences whose block tables all
    start with the same ``prefix_blocks`` physical blocks; the prefix is
    attended once for all of them, the tails per sequence, merged by
    log-sum-exp.  Same tensors as :func:`decode`."""
    _need(q, "q", 3)
    dev = q.device
    if q.dtype not in _DT:
        raise ValueError(f"q must be float16 or bfloat16, got {q.dtype}")
    _need(k_cache, "k_cache", 4, q.dtype, dev)
    _need(v_cache, "v_cache", 4, q.dtype, dev)
    _need(block_tables, "block_tables", 2, torch.int32, dev)
    _need(seq_lens, "seq_lens", 1, torch.int32, dev)
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must have the same shape")
    S, Hq, d = q.shape
    NB, Hkv, bs, d2 = k_cache.shape
    if d2 != d or block_tables.shape[0] != S or seq_lens.shape[0] != S:
        raise ValueError("inconsistent shapes between q, the pools, block_tables and seq_lens")
    if scale is None:
        scale = d ** -0.5
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", 3, q.dtype, dev)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    need = int(_lib.pa_decode_shared_prefix_workspace_bytes(S, Hq, d, int(prefix_blocks), bs))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0
    if workspace is not None:
        _need(workspace, "workspace", None, None, dev)
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(_lib.pa_decode_shared_prefix(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                        _ptr(block_tables), _ptr(seq_lens), S, Hq, Hkv, d, bs,
                                        block_tables.shape[1], NB, int(prefix_blocks),
                                        float(scale), _DT[q.dtype], _ptr(workspace), ws_bytes,
                                        _stream(dev)))
    return out


def decode_shared_prefix_workspace_bytes(num_seqs, num_q_heads, head_dim, prefix_blocks,
                                         block_size) -> int:
    return int(_lib.pa_decode_shared_prefix_workspace_bytes(num_seqs, num_q_heads, head_dim,
                                                            prefix_blocks, block_size))


def prefill(q, k_cache, v_cache, block_tables, seq_lens, query_start, scale=None, out=None):
    """Causal attention of several query tokens per sequence (chunked
    prefill): q [total_q][Hq][d]; query_start int32 [S + 1] (chunk offsets);
    chunk token i of sequence s sits at position seq_lens[s] - n_s + i and
    attends to positions <= its own."""
    _need(q, "q", 3)
    dev = q.device
    if q.dtype not in _DT:
        raise ValueError(f"q must be float16 or bfloat16, got {q.dtype}")
    _need(k_cache, "k_cache", 4, q.dtype, dev)
    _need(v_cache, "v_cache", 4, q.dtype, dev)
    _need(block_tables, "block_tables", 2, torch.int32, dev)
    _need(seq_lens, "seq_lens", 1, torch.int32, dev)
    _need(query_start, "query_start", 1, torch.int32, dev)
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must have the same shape")
    T, Hq, d = q.shape
    NB, Hkv, bs, d2 = k_cache.shape
    S = seq_lens.shape[0]
    if d2 != d or block_tables.shape[0] != S or query_start.shape[0] != S + 1:
        raise ValueError("inconsistent shapes between q, the pools, block_tables, seq_lens and "
                         "query_start")
    if scale is None:
        scale = d ** -0.5
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", 3, q.dtype, dev)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    _check(_lib.pa_prefill(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                           _ptr(seq_lens), _ptr(query_start), S, T, Hq, Hkv, d, bs,
                           block_tables.shape[1], NB, float(scale), _DT[q.dtype], _stream(dev)))
    return out


def decode_fp8(q, k_cache, v_cache, block_tables, seq_lens, k_scale, v_scale, scale=None,
               out=None, workspace=None):
    """pa_decode over 8-bit pools: k_cache/v_cache uint8 [NB][Hkv][bs][d] of
    OCP E4M3 codes standing for e4m3(code) * k_scale (resp. v_scale); q and
    out float16 or bfloat16.  Balanced split always."""
    _need(q, "q", 3)
    dev = q.device
    if q.dtype not in _DT:
        raise ValueError(f"q must be float16 or bfloat16, got {q.dtype}")
    _need(k_cache, "k_cache", 4, torch.uint8, dev)
    _need(v_cache, "v_cache", 4, torch.uint8, dev)
    _need(block_tables, "block_tables", 2, torch.int32, dev)
    _need(seq_lens, "seq_lens", 1, torch.int32, dev)
    if k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must have the same shape")
    S, Hq, d = q.shape
    NB, Hkv, bs, d2 = k_cache.shape
    if d2 != d or block_tables.shape[0] != S or seq_lens.shape[0] != S:
        raise ValueError("inconsistent shapes between q, the pools, block_tables and seq_lens")
    MB = block_tables.shape[1]
    if scale is None:
        scale = d ** -0.5
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", 3, q.dtype, dev)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    need = decode_workspace_bytes(S, Hq, d, MB, bs, 0)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0
    if workspace is not None:
        _need(workspace, "workspace", None, None, dev)
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(_lib.pa_decode_fp8(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                              _ptr(block_tables), _ptr(seq_lens), S, Hq, Hkv, d, bs, MB, NB,
                              float(scale), float(k_scale), float(v_scale), _DT[q.dtype],
                              _ptr(workspace), ws_bytes, _stream(dev)))
    return out


def reshape_and_cache_fp8(key, value, k_cache, v_cache, slot_mapping, k_scale, v_scale):
    """Quantising append: k_cache/v_cache (uint8 E4M3 codes)[slot // bs][:,
    slot % bs] = E4M3(key/value[i] / scale) for slot >= 0."""
    _need(key, "key", 3)
    dev = key.device
    if key.dtype not in _DT:
        raise ValueError(f"key must be float16 or bfloat16, got {key.dtype}")
    _need(value, "value", 3, key.dtype, dev)
    _need(k_cache, "k_cache", 4, torch.uint8, dev)
    _need(v_cache, "v_cache", 4, torch.uint8, dev)
    _need(slot_mapping, "slot_mapping", 1, torch.int32, dev)
    T, Hkv, d = key.shape
    NB, Hkv2, bs, d2 = k_cache.shape
    if value.shape != key.shape or v_cache.shape != k_cache.shape or Hkv2 != Hkv or d2 != d or \
            slot_mapping.shape[0] != T:
        raise ValueError("inconsistent shapes between key/value, the pools and slot_mapping")
    _check(_lib.pa_reshape_and_cache_fp8(_ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache),
                                         _ptr(slot_mapping), T, Hkv, d, bs, NB, float(k_scale),
                                         float(v_scale), _DT[key.dtype], _stream(dev)))


def reshape_and_cache(key, value, k_cache, v_cache, slot_mapping):
    """k_cache/v_cache[slot // bs][:, slot % bs] = key/value[i] for slot >= 0."""
    _need(key, "key", 3)
    dev = key.device
    if key.dtype not in _DT:
        raise ValueError(f"key must be float16 or bfloat16, got {key.dtype}")
    _need(value, "value", 3, key.dtype, dev)
    _need(k_cache, "k_cache", 4, key.dtype, dev)
    _need(v_cache, "v_cache", 4, key.dtype, dev)
    _need(slot_mapping, "slot_mapping", 1, torch.int32, dev)
    T, Hkv, d = key.shape
    NB, Hkv2, bs, d2 = k_cache.shape
    if value.shape != key.shape or v_cache.shape != k_cache.shape or Hkv2 != Hkv or d2 != d or \
            slot_mapping.shape[0] != T:
        raise ValueError("inconsistent shapes between key/value, the pools and slot_mapping")
    _check(_lib.pa_reshape_and_cache(_ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache),
                                     _ptr(slot_mapping), T, Hkv, d, bs, NB, _DT[key.dtype],
                                     _stream(dev)))


def copy_blocks(k_cache, v_cache, block_mapping):
    """For each (src, dst) row of block_mapping: block dst := block src (K and V)."""
    _need(k_cache, "k_cache", 4)
    dev = k_cache.device
    if k_cache.dtype not in _POOL_DT:
        raise ValueError(f"k_cache must be float16, bfloat16 or uint8 (E4M3 codes), got "
                         f"{k_cache.dtype}")
    _need(v_cache, "v_cache", 4, k_cache.dtype, dev)
    _need(block_mapping, "block_mapping", 2, torch.int32, dev)
    if v_cache.shape != k_cache.shape or block_mapping.shape[1] != 2:
        raise ValueError("pools must match and block_mapping must be [n][2]")
    NB, Hkv, bs, d = k_cache.shape
    _check(_lib.pa_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(block_mapping),
                               block_mapping.shape[0], Hkv, d, bs, NB, _POOL_DT[k_cache.dtype],
                               _stream(dev)))


def probe_gather(k_cache, v_cache, block_tables, seq_lens, num_q_heads, sink=None):
    """Measurement support (include/pa_probe.h): read exactly the K/V bytes
    pa_decode's balanced split reads, with the same loads, computing nothing.
    Returns the sink tensor (2 int16 words on the pools' device).  uint8
    pools: what pa_decode_fp8 reads."""
    _need(k_cache, "k_cache", 4)
    dev = k_cache.device
    if k_cache.dtype not in _POOL_DT:
        raise ValueError(f"k_cache must be float16, bfloat16 or uint8, got {k_cache.dtype}")
    _need(v_cache, "v_cache", 4, k_cache.dtype, dev)
    _need(block_tables, "block_tables", 2, torch.int32, dev)
    _need(seq_lens, "seq_lens", 1, torch.int32, dev)
    NB, Hkv, bs, d = k_cache.shape
    S, MB = block_tables.shape
    if sink is None:
        sink = torch.zeros(2, dtype=torch.int16, device=dev)
    _check(_lib.pa_probe_gather(_ptr(sink), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                _ptr(seq_lens), S, num_q_heads, Hkv, d, bs, MB, NB,
                                _POOL_DT[k_cache.dtype], _stream(dev)))
    return sink


def probe_stream(buf, sink=None):
    """Measurement support (include/pa_probe.h): read every byte of the
    device tensor ``buf`` once as a streaming read, computing nothing.
    Returns the sink tensor (2 int16 words on buf's device)."""
    _need(buf, "buf", None, None, None)
    dev = buf.device
    if sink is None:
        sink = torch.zeros(2, dtype=torch.int16, device=dev)
    _check(_lib.pa_probe_stream(_ptr(sink), _ptr(buf), buf.numel() * buf.element_size(),
                                _stream(dev)))
    return sink


class NoBlocks(PaError):
    """The block manager's pool cannot supply the blocks an operation needs."""


def _bm_check(status: int):
    if status == PA_ERR_NO_BLOCKS:
        raise NoBlocks(status, "the pool has too few free blocks")
    _check(status)


def _i32_array(values):
    """(contiguous int32 copy or view, its address).  The address goes to the
    c_void_p argument as a plain integer: numpy's ctypes.data_as costs tens
    of microseconds a call, more than the manager's own work."""
    import numpy as np
    a = np.ascontiguousarray(values, dtype=np.int32)
    return a, a.ctypes.data


class BlockManager:
    """Host-side block manager (include/pa_block_manager.h): free queue,
    reference counts, block tables, copy-on-write and prefix cache.  Numpy
    int32 arrays in and out; no device memory is touched."""

    def __init__(self, num_blocks, block_size, free_order=None):
        import numpy as np
        self._np = np
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)
        order = None
        if free_order is not None:
            order, ptr = _i32_array(free_order)
        else:
            ptr = None
        h = ctypes.c_void_p()
        _check(_lib.pa_bm_create(self.num_blocks, self.block_size, ptr, ctypes.byref(h)))
        self._h = h
        del order

    def close(self):
        if self._h:
            _lib.pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def num_free(self) -> int:
        return int(_lib.pa_bm_num_free(self._h))

    def add_sequence(self, seq_id, tokens):
        """Returns (number of leading tokens found cached, slots int32[n])."""
        np = self._np
        toks, tp = _i32_array(tokens)
        slots = np.empty(len(toks), np.int32)
        nc = ctypes.c_int32()
        _bm_check(_lib.pa_bm_add_sequence(self._h, int(seq_id), tp, len(toks),
                                          slots.ctypes.data,
                                          ctypes.byref(nc)))
        return int(nc.value), slots

    def append(self, seq_id, tokens):
        """Returns (slots int32[n], copy-on-write pairs int32[k][2])."""
        np = self._np
        toks, tp = _i32_array(tokens)
        slots = np.empty(len(toks), np.int32)
        pairs = np.empty((1, 2), np.int32)
        nc = ctypes.c_int32()
        _bm_check(_lib.pa_bm_append(self._h, int(seq_id), tp, len(toks),
                                    slots.ctypes.data,
                                    pairs.ctypes.data, 1, ctypes.byref(nc)))
        return slots, pairs[:nc.value].copy()

    def append_batch(self, seq_ids, tokens):
        """One token per sequence (a decode step) in one call: returns (slots
        int32[S], copy-on-write pairs int32[k][2]); all or nothing."""
        np = self._np
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        toks, tp = _i32_array(tokens)
        if toks.shape != ids.shape:
            raise ValueError("one token per sequence")
        slots = np.empty(len(ids), np.int32)
        pairs = np.empty((max(1, len(ids)), 2), np.int32)
        nc = ctypes.c_int32()
        _bm_check(_lib.pa_bm_append_batch(self._h, ids.ctypes.data, tp,
                                          len(ids), slots.ctypes.data,
                                          pairs.ctypes.data, len(pairs),
                                          ctypes.byref(nc)))
        return slots, pairs[:nc.value].copy()

    def fork(self, parent_id, child_id):
        _bm_check(_lib.pa_bm_fork(self._h, int(parent_id), int(child_id)))

    def free(self, seq_id):
        _bm_check(_lib.pa_bm_free(self._h, int(seq_id)))

    def tables(self, seq_ids, max_blocks_per_seq, pad_block=0, out=None):
        """(block tables int32[S][max_blocks_per_seq], lengths int32[S]).
        ``out``: a (tables, lengths) pair of C-contiguous int32 arrays of those
        shapes to fill instead of new ones (pinned host tensors' numpy views
        serve, for an asynchronous copy to the device)."""
        np = self._np
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        if out is None:
            t = np.empty((len(ids), max_blocks_per_seq), np.int32)
            lens = np.empty(len(ids), np.int32)
        else:
            t, lens = out
            for a, shape in ((t, (len(ids), max_blocks_per_seq)), (lens, (len(ids),))):
                if a.dtype != np.int32 or a.shape != shape or not a.flags["C_CONTIGUOUS"]:
                    raise ValueError(f"out arrays must be C-contiguous int32 of shape {shape}")
        _bm_check(_lib.pa_bm_tables(self._h, ids.ctypes.data, len(ids),
                                    int(max_blocks_per_seq), int(pad_block),
                                    t.ctypes.data,
                                    lens.ctypes.data))
        return t, lens

    def block_refs(self, block) -> int:
        return int(_lib.pa_bm_block_refs(self._h, int(block)))


class _SchedPlan(ctypes.Structure):
    """pa_sched_plan of include/pa_scheduler.h."""
    _p64 = ctypes.POINTER(ctypes.c_int64)
    _fields_ = [("iteration", ctypes.c_int64),
                ("n_prefill", ctypes.c_int32), ("prefill", _p64),
                ("n_decode", ctypes.c_int32), ("decode", _p64),
                ("n_padded", ctypes.c_int32), ("padded", _p64),
                ("n_admitted", ctypes.c_int32), ("admitted", _p64),
                ("n_finished", ctypes.c_int32), ("finished", _p64),
                ("n_preempted", ctypes.c_int32), ("preempted", _p64),
                ("n_released", ctypes.c_int32), ("released", _p64),
                ("running", ctypes.c_int32), ("queued", ctypes.c_int32),
                ("blocks_used", ctypes.c_int64)]


SCHED_MODES = {"static": 0, "reserved": 1, "paged": 2}


class NativeSchedulerHandle:
    """The C scheduler of include/pa_scheduler.h: create, add requests, step.
    step() returns the plan as Python lists (copies; the C arrays are valid
    only until the next step)."""

    def __init__(self, mode, num_blocks, block_size, max_batch, max_step_tokens,
                 reserve_tokens):
        if mode not in SCHED_MODES:
            raise ValueError(f"unknown mode {mode!r}")
        h = ctypes.c_void_p()
        _check(_lib.pa_sched_create(SCHED_MODES[mode], int(num_blocks), int(block_size),
                                    int(max_batch), int(max_step_tokens), int(reserve_tokens),
                                    ctypes.byref(h)))
        self._h = h
        self._plan = _SchedPlan()

    def close(self):
        if self._h:
            _lib.pa_sched_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add(self, rids, arrivals, prompt_lens, gen_lens):
        import numpy as np
        r = np.ascontiguousarray(rids, dtype=np.int64)
        a = np.ascontiguousarray(arrivals, dtype=np.int64)
        p = np.ascontiguousarray(prompt_lens, dtype=np.int32)
        g = np.ascontiguousarray(gen_lens, dtype=np.int32)
        if not (len(r) == len(a) == len(p) == len(g)):
            raise ValueError("one arrival, prompt length and generation length per request")
        _check(_lib.pa_sched_add(self._h, r.ctypes.data, a.ctypes.data, p.ctypes.data,
                                 g.ctypes.data, len(r)))

    def step(self):
        """(iteration, dict of the plan's lists and counts)."""
        pl = self._plan
        st = _lib.pa_sched_step(self._h, ctypes.byref(pl))
        if st != 0:
            raise ValueError("a request is longer than a reservation"
                             if st == 2 else f"pa_sched_step: status {st}")
        def take(n, ptr):
            return ptr[:n] if n else []
        flat = take(3 * pl.n_prefill, pl.prefill)
        return pl.iteration, {
            "prefill": [tuple(flat[i:i + 3]) for i in range(0, len(flat), 3)],
            "decode": take(pl.n_decode, pl.decode),
            "padded": take(pl.n_padded, pl.padded),
            "admitted": take(pl.n_admitted, pl.admitted),
            "finished": take(pl.n_finished, pl.finished),
            "preempted": take(pl.n_preempted, pl.preempted),
            "released": take(pl.n_released, pl.released),
            "running": pl.running, "queued": pl.queued, "blocks_used": pl.blocks_used}

    def active(self) -> int:
        return int(_lib.pa_sched_active(self._h))

    def request(self, rid):
        """(admitted, prefilled, generated, finished, released, preemptions);
        -1 for an iteration that has not happened."""
        out = (ctypes.c_int64 * 6)()
        _check(_lib.pa_sched_request(self._h, int(rid), out))
        return tuple(out)
