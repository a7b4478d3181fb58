"""Measurement helpers of the library: the plain copy used to calibrate the
byte counters, and the streaming read."""

import numpy as np
import pytest
import torch

from gpu_util import DEV
from paged_kv_decode_attention_amd import ops

pytestmark = pytest.mark.gpu


def test_copy_bytes_and_stream_read():
    g = torch.Generator(device=DEV).manual_seed(3)
    src = torch.randint(0, 256, (3 << 20,), dtype=torch.uint8, device=DEV, generator=g)
    dst = torch.zeros_like(src)
    ops.copy_bytes(dst, src)
    sink = torch.zeros(16 * 65536, dtype=torch.uint8, device=DEV)
    ops.stream_read(src, sink)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    # every 16-byte word read exactly once: the XOR over the per-workgroup
    # XORs is the XOR over the buffer
    words = src.view(torch.int32).view(-1, 4).cpu().numpy()
    sw = sink.view(torch.int32).view(-1, 4).cpu().numpy()
    for c in range(4):
        assert np.bitwise_xor.reduce(sw[:, c]) == np.bitwise_xor.reduce(words[:, c])
    # a size that is not a multiple of a workgroup's step: the tail is read too
    tail = src[:(3 << 20) - 16 * 37]
    sink.zero_()
    ops.stream_read(tail, sink)
    torch.cuda.synchronize()
    tw = tail.view(torch.int32).view(-1, 4).cpu().numpy()
    sw = sink.view(torch.int32).view(-1, 4).cpu().numpy()
    for c in range(4):
        assert np.bitwise_xor.reduce(sw[:, c]) == np.bitwise_xor.reduce(tw[:, c])
    with pytest.raises(RuntimeError):
        ops.copy_bytes(dst[1:], src[1:])        # not 16-byte aligned
