"""The measurement calls (include/pa_probe.h) run through the C ABI: the
gather-only probe on the benchmark's workload and on edge inputs, without
touching anything but its sink, rejecting bad arguments like pa_decode; the
streaming read over buffers of several sizes, leaving them unchanged."""
import pytest
import torch

import paged_kv_cache_400_amd as pa
from paged_kv_cache_400_amd import workload as wl

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("make", [wl.make_mixed_step, wl.make_tiny,
                                  lambda: wl.make_long_context(8)])
def test_probe_gather_reads_and_writes_nothing_else(make):
    b = make()
    dev = wl.to_device(b, "cuda:0")
    k0, v0 = dev["k_cache"].view(torch.int16).clone(), dev["v_cache"].view(torch.int16).clone()
    sink = pa.probe_gather(dev["k_cache"], dev["v_cache"], dev["block_tables"], dev["seq_lens"],
                           b.num_q_heads)
    torch.cuda.synchronize()
    # bit patterns (unused slots hold NaN)
    assert torch.equal(dev["k_cache"].view(torch.int16), k0)
    assert torch.equal(dev["v_cache"].view(torch.int16), v0)
    assert sink.shape == (2,)


def test_probe_gather_rejects_bad_arguments():
    b = wl.make_tiny()
    dev = wl.to_device(b, "cuda:0")
    with pytest.raises(pa.PaError, match="group"):
        pa.probe_gather(dev["k_cache"], dev["v_cache"], dev["block_tables"], dev["seq_lens"],
                        b.num_kv_heads * 16)


@pytest.mark.parametrize("nbytes", [16, 1008, 1 << 20, (256 << 20) + 48])
def test_probe_stream_reads_and_writes_nothing_else(nbytes):
    buf = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda:0")
    before = buf.clone()
    sink = pa.probe_stream(buf)
    torch.cuda.synchronize()
    assert torch.equal(buf, before)
    assert sink.shape == (2,)
