"""GPU parity of libpa against the CPU oracle, through the C ABI.

Pools after the append and the copy-on-write copy: bit-exact.  Attention:
max-abs <= 1e-2 and mean-abs <= 1e-3 against the float64 oracle.  The five
workloads run at their full sizes in the launch configuration the benchmark
times (automatic partitioning), and every (sequence, head) row is checked;
the long-context batch also with 512-position partitions.
"""
import numpy as np
import pytest
import torch

from _gpu import compare, gpu_bits, gpu_step, oracle_out, oracle_pools
from paged_kv_cache_400_amd import workload as wl

pytestmark = pytest.mark.gpu


def _check_pools(dev, b):
    kp, vp = oracle_pools(b)
    assert np.array_equal(gpu_bits(dev["k_cache"]), kp), "K pool differs from the oracle"
    assert np.array_equal(gpu_bits(dev["v_cache"]), vp), "V pool differs from the oracle"
    return kp, vp


def test_tiny_before_append():
    b = wl.make_tiny()
    dev = wl.to_device(b, "cuda:0")
    import paged_kv_cache_400_amd as pa
    lens = torch.from_numpy(b.context_lens).cuda()
    out = pa.decode(dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"], lens,
                    scale=b.scale)
    torch.cuda.synchronize()
    from _gpu import oracle_out as oo
    from paged_kv_cache_400_amd.workload import bits
    ref = oo(b, bits(b.k_cache), bits(b.v_cache), lens=b.context_lens)
    compare(out, ref, label="tiny/context")


def test_tiny_step():
    b = wl.make_tiny()
    out, dev = gpu_step(b)
    kp, vp = _check_pools(dev, b)
    compare(out, oracle_out(b, kp, vp), label="tiny/step")


def test_worked_example():
    b = wl.make_worked_example()
    out, dev = gpu_step(b)
    kp, vp = _check_pools(dev, b)
    compare(out, oracle_out(b, kp, vp), label="worked_example")


@pytest.mark.parametrize("impl,part", [("auto", 0), ("valu", 0), ("valu", 512)])
def test_mixed_step_full_size(impl, part):
    b = wl.make_mixed_step()
    out, dev = gpu_step(b, impl=impl, partition_size=part)
    kp, vp = _check_pools(dev, b)
    compare(out, oracle_out(b, kp, vp), label=f"mixed_step {impl} part{part}")


def test_shared_prefix_copy_on_write():
    b = wl.make_shared_prefix()
    out, dev = gpu_step(b)
    kp, vp = _check_pools(dev, b)
    shared = b.info["shared_blocks"]
    # the shared partial block is bit-unchanged; each private copy starts with it
    k0 = wl.bits(b.k_cache)
    assert np.array_equal(kp[shared[-1]], k0[shared[-1]])
    for (src, dst), s in zip(b.block_mapping, range(1, b.num_seqs, 2)):
        keep = 16 - int(b.info["r"][s])
        assert np.array_equal(kp[dst][:, :keep], k0[src][:, :keep])
    compare(out, oracle_out(b, kp, vp), label="shared_prefix")


@pytest.mark.parametrize("bs", [8, 16, 32])
def test_long_context_split(bs):
    b = wl.make_long_context(bs)
    dev = wl.to_device(b, "cuda:0")
    ref = oracle_out(b, wl.bits(b.k_cache), wl.bits(b.v_cache))
    for impl, part in (("auto", 0), ("auto", 512), ("valu", 0), ("valu", 512)):
        out, _ = gpu_step(b, partition_size=part, dev=dev, impl=impl)
        compare(out, ref, label=f"long_context bs{bs} {impl} part{part}")


# ---------------------------------------------------------------- edge cases

EDGE_LENS = [0, 1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 200]


@pytest.mark.parametrize("impl", ["auto", "mfma", "valu"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bs", [8, 16, 32])
@pytest.mark.parametrize("g", [1, 2, 4, 8])
def test_ragged_edges(dtype, d, bs, g, impl):
    """Lengths at and around tile, block and partition edges (partition 64 so
    most sequences split), empty sequences included, every group size."""
    hkv = 2
    b = wl.make_decode_batch("edges", EDGE_LENS, hkv * g, hkv, d, bs, dtype,
                             seed=100 + g + d + bs, append=1)
    for part in (64, 0):
        out, dev = gpu_step(b, partition_size=part, impl=impl)
        kp, vp = _check_pools(dev, b)
        compare(out, oracle_out(b, kp, vp), label=f"edges part{part} {impl}")


def test_empty_and_single_token_sequences():
    b = wl.make_decode_batch("short", [0, 0, 0], 8, 2, 128, 16, "bf16", seed=7, append=1)
    out, dev = gpu_step(b)
    kp, vp = _check_pools(dev, b)
    ref = oracle_out(b, kp, vp)
    compare(out, ref, label="single")
    # L = 1: the output is that token's V row, exactly
    v = dev["new_value"].float().cpu().repeat_interleave(4, dim=1)
    assert torch.equal(out.float().cpu(), v)


@pytest.mark.parametrize("impl", ["auto", "mfma", "valu"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_large_values(dtype, impl):
    """V ~ N(0, 64^2): the softmax weights' rounding must not grow with |V|
    (the matrix-core kernel splits each weight into two 16-bit parts).  The
    plain tolerance, beyond half an ulp of the output (outputs reach tens)."""
    b = wl.make_decode_batch("large_v", [1, 2, 3, 15, 16, 17, 100, 1000, 4097], 32, 8, 128, 16,
                             dtype, seed=9, append=1, v_mult=64.0)
    out, dev = gpu_step(b, impl=impl)
    kp, vp = _check_pools(dev, b)
    compare(out, oracle_out(b, kp, vp), label=f"large values {dtype} {impl}", excess=True)


def test_padding_slots_are_skipped():
    b = wl.make_decode_batch("pad", [5, 40, 16], 8, 2, 64, 16, "f16", seed=8, append=1,
                             pad_tokens=5)
    out, dev = gpu_step(b)
    kp, vp = _check_pools(dev, b)
    compare(out, oracle_out(b, kp, vp), label="padding")
