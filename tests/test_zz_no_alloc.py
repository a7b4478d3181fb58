"""The no-allocation decode entry point (pa_paged_attention_decode_noalloc,
through the C ABI) against pa_paged_attention_decode with a workspace of its
own: the same kernels, so the outputs must agree bit for bit.  Two calls in
a row, the second with a smaller batch, so that a stale part of the shared
device array from the first call would show; on the balanced schedule and on
fixed partitions; once on a GQA group of 17 heads (two column tiles)."""

import pytest
import torch

from gpu_util import DEV, small_config, upload
from paged_kv_decode_attention_amd import inputs as I
from paged_kv_decode_attention_amd import ops

pytestmark = pytest.mark.gpu


def _pair(cfg, partition_size):
    inp = I.poison_unread(I.generate(cfg))
    d = upload(inp)
    args = (d["query"], d["key_cache"], d["value_cache"], d["block_tables"],
            d["context_lens"])
    ref = ops.paged_attention_decode(*args, partition_size=partition_size)
    got = ops.paged_attention_decode_noalloc(*args, partition_size=partition_size)
    torch.cuda.synchronize()
    return got, ref


@pytest.mark.parametrize("partition_size", [0, 128])
def test_noalloc_matches_decode_twice(partition_size):
    big = I.with_overrides(I.CONFIGS["qwen7b_gqa_bf16"], num_seqs=32, num_blocks=10000)
    small = small_config("bf16", H_kv=4, G=7, lens=(1, 40, 700, 1500, 33), seed=12)
    for cfg, what in ((big, "first call, 32 sequences"), (small, "second call, 5 sequences")):
        print("noalloc %s partition_size=%d" % (what, partition_size), flush=True)
        got, ref = _pair(cfg, partition_size)
        assert torch.isfinite(ref.float()).all()
        assert torch.equal(got, ref), what


def test_noalloc_two_column_tiles_then_smaller():
    wide = small_config("bf16", H_kv=2, G=17, lens=(900, 1, 3000, 257), seed=4)
    narrow = small_config("bf16", H_kv=2, G=3, lens=(64, 5), seed=5)
    for cfg in (wide, narrow):
        got, ref = _pair(cfg, 0)
        assert torch.equal(got, ref)


def test_noalloc_short_partitions_long_histories():
    cfg = small_config("bf16", H_kv=8, G=8, lens=(4096,) * 8, seed=3)
    inp = I.generate(cfg)
    d = upload(inp)
    # fixed partitions of 32 tokens over 4096-token histories: 34 MB of
    # partial states, inside the array
    need = ops.decode_workspace_size(8, 64, 8, 128, 16, 4096, 32, torch.bfloat16)
    assert need <= ops.load_library().pa_noalloc_scratch_bytes()   # this one fits
    got = ops.paged_attention_decode_noalloc(d["query"], d["key_cache"], d["value_cache"],
                                             d["block_tables"], d["context_lens"],
                                             partition_size=32)
    ref = ops.paged_attention_decode(d["query"], d["key_cache"], d["value_cache"],
                                     d["block_tables"], d["context_lens"], partition_size=32)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
