"""Measurement helpers of the library: the plain copy used to calibrate the
byte counters, and the streaming read."""

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
    sink = torch.empty(16 * 65536, dtype=torch.uint8, device=DEV)
    ops.stream_read(src, sink)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    with pytest.raises(RuntimeError):
        ops.copy_bytes(dst[1:], src[1:])        # not 16-byte aligned
