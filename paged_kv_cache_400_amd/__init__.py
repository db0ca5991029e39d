"""Paged-KV-cache decode attention for AMD MI355X (gfx950).

The compute lives in ``libpa.so`` (hand-written HIP kernels behind the C ABI
of ``include/pa.h``); :mod:`.binding` is its Python binding.  Importing this
package does not load the library; the first use of one of its names does,
and fails loudly if it has not been built.
"""
_BINDING_NAMES = ("decode", "decode_noalloc", "decode_shared_prefix",
                  "decode_shared_prefix_workspace_bytes", "reshape_and_cache", "copy_blocks",
                  "decode_workspace_bytes", "decode_fp8", "reshape_and_cache_fp8", "prefill",
                  "probe_gather", "probe_stream", "BlockManager", "NoBlocks", "PaError",
                  "abi_version", "LIB_PATH")


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
