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


def _replays_match(step, out, ws):
    """Capture step() in a graph; each replay (after eager work that clobbers
    out and the workspace) must equal the eager result bit for bit."""
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
        out.fill_(float("nan"))
        ws.fill_(0xAB)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), "replay %d differs from the eager step" % rep
        step()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)


@pytest.mark.parametrize("partition_size", [0, 64])
def test_graph_verify_replays_match_eager(partition_size):
    """Verify calls in a graph: on the balanced schedule the row map is
    computed inside the decode kernel, on the fixed one a kernel writes it to
    the workspace first; both replay to the eager bits."""
    cfg = I.CONFIGS["qwen7b_gqa_bf16"]
    inp = I.generate(cfg)
    d = upload(inp)
    S, H, D = d["query"].shape
    N, H_kv, BS, _ = d["key_cache"].shape
    W = d["block_tables"].shape[1]
    qs = torch.arange(0, 4 * S + 1, 4, dtype=torch.int32, device=DEV)
    gen = torch.Generator().manual_seed(5)
    q = torch.randn(4 * S, H, D, generator=gen).to(d["query"].dtype).to(DEV)
    need = ops.load_library().pa_verify_workspace_size(4 * S, H, H_kv, D, BS, W * BS,
                                                       partition_size, ops.dtype_code(q.dtype))
    ws = torch.empty(max(256, need), dtype=torch.uint8, device=DEV)
    out = torch.empty_like(q)

    def step():
        ops.paged_attention_verify(q, d["key_cache"], d["value_cache"], d["block_tables"],
                                   d["context_lens"], qs, 4, partition_size=partition_size,
                                   out=out, workspace=ws)

    _replays_match(step, out, ws)


def test_graph_decode_append_replays_match_eager():
    """The fused step of the bench (newest token written inside the decode
    kernel) in a graph."""
    cfg = I.CONFIGS["qwen7b_gqa_bf16"]
    inp = I.generate(cfg, new_tokens_at="last")
    d = upload(inp)
    S, H, D = d["query"].shape
    N, H_kv, BS, _ = d["key_cache"].shape
    W = d["block_tables"].shape[1]
    ws = torch.empty(max(256, ops.decode_workspace_size(S, H, H_kv, D, BS, W * BS, 0,
                                                        d["query"].dtype)),
                     dtype=torch.uint8, device=DEV)
    out = torch.empty_like(d["query"])

    def step():
        ops.decode_append(d["query"], d["new_key"], d["new_value"], d["key_cache"],
                          d["value_cache"], d["block_tables"], d["context_lens"], out=out,
                          workspace=ws)

    _replays_match(step, out, ws)


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_graph_decode_append_8bit_replays_match_eager(fmt):
    """The fused step on 8-bit caches (the newest token quantised inside the
    decode kernel) in a graph.  The caches are restored before each step, so
    every step writes the same codes."""
    cfg = I.with_overrides(I.CONFIGS["qwen7b_gqa_bf16"], num_seqs=16, num_blocks=6000)
    inp = I.generate(cfg, new_tokens_at="last")
    d = upload(inp)
    S, H, D = d["query"].shape
    N, H_kv, BS, _ = d["key_cache"].shape
    W = d["block_tables"].shape[1]
    ks, vs = 1.0 / 24, 1.0 / 20
    dt = torch.uint8 if fmt == "fp8" else torch.int8
    k0 = torch.empty(N, H_kv, BS, D, dtype=dt, device=DEV)
    v0 = torch.empty_like(k0)
    write = ops.reshape_and_cache_fp8 if fmt == "fp8" else ops.reshape_and_cache_i8
    slots = torch.arange(N * BS, dtype=torch.int64, device=DEV)
    write(d["key_cache"].permute(0, 2, 1, 3).reshape(N * BS, H_kv, D).contiguous(),
          d["value_cache"].permute(0, 2, 1, 3).reshape(N * BS, H_kv, D).contiguous(),
          k0, v0, slots, ks, vs)
    kc, vc = k0.clone(), v0.clone()
    ws = torch.empty(max(256, ops.decode_workspace_size(S, H, H_kv, D, BS, W * BS, 0,
                                                        d["query"].dtype)),
                     dtype=torch.uint8, device=DEV)
    out = torch.empty_like(d["query"])
    step_fn = ops.decode_append_fp8 if fmt == "fp8" else ops.decode_append_i8

    def step():
        kc.copy_(k0)
        vc.copy_(v0)
        step_fn(d["query"], d["new_key"], d["new_value"], kc, vc, d["block_tables"],
                d["context_lens"], ks, vs, out=out, workspace=ws)

    _replays_match(step, out, ws)
