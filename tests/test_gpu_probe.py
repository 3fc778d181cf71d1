"""The streaming-read probe (a measurement aid of bench.py) runs through the C ABI."""

import ctypes

import pytest
import torch

from decode_attention_verify_amd import binding

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("block", [1024, 4096, 8192])
def test_read_probe_runs(block):
    nblocks = 300
    buf = torch.ones(nblocks * block, dtype=torch.uint8, device="cuda")
    order = torch.randperm(nblocks, device="cuda").to(torch.int32)
    order[5] = -3                                  # clamped on the device, not read out of bounds
    order[7] = nblocks + 9
    sink = torch.zeros(1024, dtype=torch.uint8, device="cuda")
    vp = ctypes.c_void_p
    for waves in (1, 37, 1024):
        st = binding.load().rattn_read_probe(vp(buf.data_ptr()), nblocks, block,
                                             vp(order.data_ptr()), waves, vp(sink.data_ptr()),
                                             vp(torch.cuda.current_stream().cuda_stream))
        assert st == binding.RATTN_OK
    torch.cuda.synchronize()
    assert int(sink.sum()) == 0                    # the data never matches the sink's guard
