"""Decode steps captured in a HIP graph: every replay equals the eager
result, with eager work and synchronisations between replays."""

import pytest
import torch

from gpu_util import DEV, upload
from paged_kv_decode_attention_amd import inputs as I
from paged_kv_decode_attention_amd import ops

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,partition_size", [("qwen7b_gqa_bf16", 0),
                                                 ("qwen7b_gqa_bf16", 256),
                                                 ("tiny_fp32", 0)])
def test_graph_replays_match_eager(name, partition_size):
    cfg = I.CONFIGS[name]
    inp = I.generate(cfg, new_tokens_at="last" if name != "tiny_fp32" else "free")
    d = upload(inp)
    S, H, D = d["query"].shape
    N, H_kv, BS, _ = d["key_cache"].shape
    W = d["block_tables"].shape[1]
    ws = torch.empty(max(256, ops.decode_workspace_size(S, H, H_kv, D, BS, W * BS,
                                                        partition_size, d["query"].dtype)),
                     dtype=torch.uint8, device=DEV)
    out = torch.empty_like(d["query"])

    def step():
        ops.reshape_and_cache(d["new_key"], d["new_value"], d["key_cache"], d["value_cache"],
                              d["slot_mapping"])
        ops.paged_attention_decode(d["query"], d["key_cache"], d["value_cache"],
                                   d["block_tables"], d["context_lens"],
                                   partition_size=partition_size, out=out, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(float("nan"))                   # eager work between replays
        ws.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), "replay %d differs from the eager step" % rep
        step()                                    # eager step between replays
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
