"""KV-cache block and byte accounting -- TEST INFRASTRUCTURE ONLY (oracle).

Written from "What problem does PagedAttention solve, and what is continuous
batching?" (datarekha):
  * section "How PagedAttention works": a block holds a fixed number of
    tokens; a request of L tokens needs ceil(L / bs) blocks, the last one
    holding L - (blocks - 1) * bs tokens; the waste is under one block;
  * section "A concrete memory example": raw KV bytes per token are
    2 (K and V) x layers x KV heads x head_dim x element bytes; a request's
    allocation is its whole blocks times the block's bytes; the tail is the
    allocation minus the live bytes; a contiguous design reserves the
    maximum context for every request.
All values are exact integers.
"""


def blocks_needed(num_tokens: int, block_size: int) -> int:
    """ceil(num_tokens / block_size)."""
    if num_tokens < 0 or block_size <= 0:
        raise ValueError("num_tokens >= 0 and block_size > 0 required")
    return -(-num_tokens // block_size)


def last_block_fill(num_tokens: int, block_size: int) -> int:
    """Tokens held by the last (possibly partial) block; 0 when there is none."""
    n = blocks_needed(num_tokens, block_size)
    return 0 if n == 0 else num_tokens - (n - 1) * block_size


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """2 x layers x kv_heads x head_dim x elem_bytes (the 2 is keys + values)."""
    return 2 * layers * kv_heads * head_dim * elem_bytes


def allocated_bytes(num_tokens: int, block_size: int, bytes_per_token: int) -> int:
    return blocks_needed(num_tokens, block_size) * block_size * bytes_per_token


def live_bytes(num_tokens: int, bytes_per_token: int) -> int:
    return num_tokens * bytes_per_token


def tail_tokens(num_tokens: int, block_size: int) -> int:
    """Unused token slots in the last block: 0 <= tail < block_size."""
    return blocks_needed(num_tokens, block_size) * block_size - num_tokens


def tail_bytes(num_tokens: int, block_size: int, bytes_per_token: int) -> int:
    return allocated_bytes(num_tokens, block_size, bytes_per_token) - live_bytes(
        num_tokens, bytes_per_token)


def contiguous_reservation_bytes(max_tokens: int, bytes_per_token: int) -> int:
    """What a design that reserves max_tokens per request hands out."""
    return max_tokens * bytes_per_token


def effective_kv_bytes(seq_lens, kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """Bytes of live K and V one decode layer reads: sum_s L_s x 2 x Hkv x d x e.

    Each live element counted once (a GQA group shares its KV head's read);
    the unused slots of partial blocks are not counted.
    """
    return sum(int(L) for L in seq_lens) * 2 * kv_heads * head_dim * elem_bytes
