"""Seeded synthetic inputs for paged decode attention.

The one module both the HIP path's tests/bench and the oracle's callers use.
It draws numbers and lays out block tables; it holds none of the attention
arithmetic.  Every draw comes from ``numpy.random.default_rng(seed)`` in a
fixed order:

  1. context lengths
  2. the block-table permutation of the physical pool
  3. query
  4. key pool
  5. value pool
  6. new K/V tokens for the cache write, then their slots

Values are drawn as float32 and rounded once to the storage dtype (round to
nearest even, by ``torch.Tensor.to``); those exact tensors go to the GPU and,
upcast, to the oracle.  No dataset is involved: "Qwen-7B" and "LLaMA-7B" name
head shapes only.

The workloads follow the decode settings of the source pages: block size 16
or 32 [MiniPaged-Qwen §6.1; PA-source §五], the [num_blocks, kv_heads,
block_size, head_dim] pool of [MiniPaged-Qwen §8.2], tables that scatter a
sequence over arbitrary physical blocks [MiniPaged-Qwen §6.1], and shared
read-only prefix blocks [MiniPaged-Qwen §9.2 差异 3; vLLM-paging
"Copy-on-write 是共享的正确性边界"].
"""

import concurrent.futures as cf
from dataclasses import dataclass, field, replace
import math
import os

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int            # pool size; 0 = derived (shared-prefix layout)
    max_blocks_per_seq: int
    dtype: str                 # "f32" | "f16" | "bf16"
    value_std: float
    lens_kind: str             # "uniform" | "const" | "list" | "lognormal"
    lens_args: tuple
    seed: int
    prefix_groups: int = 0
    prefix_blocks: int = 0
    new_tokens: int = 0        # tokens for the cache write (0 = one per sequence)

    @property
    def gqa_group_size(self):
        return self.num_heads // self.num_kv_heads

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def max_context_len(self):
        return self.max_blocks_per_seq * self.block_size


CONFIGS = {
    # tiny fp32: S=4, H=H_kv=2, D=64, BS=16, 32 blocks, L ~ U{1..64}
    "tiny_fp32": DecodeConfig(
        "tiny_fp32", 4, 2, 2, 64, 16, 32, 4, "f32", 1.0, "uniform", (1, 64), 1,
        new_tokens=4),
    # Qwen-7B-shaped GQA: S=64, H=28, H_kv=4, D=128, BS=16, 20000 blocks,
    # L ~ U{512..4096}
    "qwen7b_gqa_bf16": DecodeConfig(
        "qwen7b_gqa_bf16", 64, 28, 4, 128, 16, 20000, 256, "bf16", 1.0,
        "uniform", (512, 4096), 2),
    # LLaMA-7B-shaped MHA: S=32, H=H_kv=32, D=128, BS=16, 10000 blocks,
    # L = 4096, values N(0, 0.5)
    "llama7b_mha_fp16": DecodeConfig(
        "llama7b_mha_fp16", 32, 32, 32, 128, 16, 10000, 256, "f16", 0.5,
        "const", (4096,), 3),
    # long context: S=4, H=32, H_kv=8, D=128, BS=32, 12288 blocks,
    # L in {32768, 65536, 98304, 131072}
    "long_ctx_bf16": DecodeConfig(
        "long_ctx_bf16", 4, 32, 8, 128, 32, 12288, 4096, "bf16", 1.0,
        "list", (32768, 65536, 98304, 131072), 4),
    # mixed batch with shared prefixes: S=128, H=32, H_kv=8, D=128, BS=16,
    # lognormal lengths (median 1024, sigma 1) clipped to [1, 8192]; 4 groups
    # of 32 sequences share their first 64 physical blocks
    "mixed_shared_bf16": DecodeConfig(
        "mixed_shared_bf16", 128, 32, 8, 128, 16, 0, 512, "bf16", 1.0,
        "lognormal", (math.log(1024.0), 1.0, 1, 8192), 5,
        prefix_groups=4, prefix_blocks=64),
}

CONFIG_ORDER = ["tiny_fp32", "qwen7b_gqa_bf16", "llama7b_mha_fp16",
                "long_ctx_bf16", "mixed_shared_bf16"]


@dataclass
class DecodeInputs:
    cfg: DecodeConfig
    query: torch.Tensor          # [S, H, D] dtype
    key_cache: torch.Tensor      # [N, H_kv, BS, D] dtype
    value_cache: torch.Tensor    # [N, H_kv, BS, D] dtype
    block_tables: torch.Tensor   # [S, W] int32, unused entries -1
    context_lens: torch.Tensor   # [S] int32
    new_key: torch.Tensor        # [T, H_kv, D] dtype
    new_value: torch.Tensor      # [T, H_kv, D] dtype
    slot_mapping: torch.Tensor   # [T] int64
    free_blocks: np.ndarray      # physical blocks no table references
    extras: dict = field(default_factory=dict)

    @property
    def num_blocks(self):
        return self.key_cache.shape[0]


def _blocks_for(L, bs):
    # layout only: how many table entries a history of L tokens fills
    return -(-int(L) // int(bs))


def _draw_lens(rng, cfg):
    S = cfg.num_seqs
    if cfg.lens_kind == "uniform":
        lo, hi = cfg.lens_args
        return rng.integers(lo, hi + 1, size=S).astype(np.int64)
    if cfg.lens_kind == "const":
        return np.full(S, cfg.lens_args[0], dtype=np.int64)
    if cfg.lens_kind == "list":
        return np.array(cfg.lens_args[:S], dtype=np.int64)
    if cfg.lens_kind == "lognormal":
        mu, sigma, lo, hi = cfg.lens_args
        x = rng.lognormal(mean=mu, sigma=sigma, size=S)
        return np.clip(np.rint(x), lo, hi).astype(np.int64)
    raise ValueError(cfg.lens_kind)


def _draw_pool(rng, shape, std, dtype, chunk_blocks=256):
    """Normal(0, std) pool.  One 63-bit seed is drawn from `rng`; chunk k of
    `chunk_blocks` blocks then comes from its own child stream
    SeedSequence(seed).spawn(...)[k], so chunks can be drawn in parallel and
    the result does not depend on the thread count."""
    out = torch.empty(shape, dtype=DTYPES[dtype])
    n = shape[0]
    starts = list(range(0, n, chunk_blocks))
    children = np.random.SeedSequence(int(rng.integers(0, 2**63 - 1))).spawn(len(starts))

    def fill(k):
        s = starts[k]
        e = min(n, s + chunk_blocks)
        g = np.random.Generator(np.random.PCG64(children[k]))
        x = g.standard_normal((e - s,) + tuple(shape[1:]), dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[s:e] = torch.from_numpy(x).to(DTYPES[dtype])

    workers = max(1, min(16, os.cpu_count() or 1))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(fill, range(len(starts))))
    return out


def _normal(rng, shape, std, dtype):
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return torch.from_numpy(x).to(DTYPES[dtype])


def generate(cfg, seed=None, lens=None, new_tokens_at="free"):
    """Build one seeded workload.

    lens: optional override of the drawn context lengths (the draw still
    happens, so the rest of the stream is unchanged).
    new_tokens_at: "free" -- the new tokens go to distinct slots of blocks no
    table references; "last" -- one token per sequence, at the slot of its
    last history position (the slot that holds position L_b - 1, which is
    rewritten with new data each step; used by the timed decode step).
    """
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    S, H, H_kv, D, BS = (cfg.num_seqs, cfg.num_heads, cfg.num_kv_heads,
                         cfg.head_dim, cfg.block_size)
    W = cfg.max_blocks_per_seq

    # 1. context lengths
    drawn = _draw_lens(rng, cfg)
    L = drawn if lens is None else np.asarray(lens, dtype=np.int64)
    if len(L) != S or L.min() < 0 or L.max() > W * BS:
        raise ValueError("context lengths out of range for this config")
    nblk = [_blocks_for(x, BS) for x in L]

    # 2. block tables from one shuffled permutation of the pool
    tables = np.full((S, W), -1, dtype=np.int64)
    if cfg.prefix_groups:
        G, Pb = cfg.prefix_groups, cfg.prefix_blocks
        per_group = S // G
        private = [max(0, n - Pb) for n in nblk]
        N = G * Pb + sum(private)
        perm = rng.permutation(N)
        shared = [perm[g * Pb:(g + 1) * Pb] for g in range(G)]
        cur = G * Pb
        for b in range(S):
            g = min(b // per_group, G - 1)
            k = min(nblk[b], Pb)
            tables[b, :k] = shared[g][:k]
            tables[b, k:nblk[b]] = perm[cur:cur + private[b]]
            cur += private[b]
        free = np.zeros(0, dtype=np.int64)
        extras = {"shared_blocks": np.stack(shared)}
    else:
        N = cfg.num_blocks
        if sum(nblk) > N:
            raise ValueError("pool too small")
        perm = rng.permutation(N)
        cur = 0
        for b in range(S):
            tables[b, :nblk[b]] = perm[cur:cur + nblk[b]]
            cur += nblk[b]
        free = perm[cur:].copy()
        extras = {}

    # 3-5. query, key pool, value pool
    q = _normal(rng, (S, H, D), cfg.value_std, cfg.dtype)
    kc = _draw_pool(rng, (N, H_kv, BS, D), cfg.value_std, cfg.dtype)
    vc = _draw_pool(rng, (N, H_kv, BS, D), cfg.value_std, cfg.dtype)

    # 6. new tokens and their slots
    T = cfg.new_tokens or S
    nk = _normal(rng, (T, H_kv, D), cfg.value_std, cfg.dtype)
    nv = _normal(rng, (T, H_kv, D), cfg.value_std, cfg.dtype)
    if new_tokens_at == "free":
        if len(free) == 0:
            slots = np.full(T, -1, dtype=np.int64)
        else:
            cand = rng.choice(len(free) * BS, size=min(T, len(free) * BS),
                              replace=False)
            slots = np.array([free[c // BS] * BS + c % BS for c in cand],
                             dtype=np.int64)
            if len(slots) < T:
                slots = np.concatenate([slots, np.full(T - len(slots), -1)])
    elif new_tokens_at == "last":
        if T != S:
            raise ValueError("'last' needs one new token per sequence")
        slots = np.array([tables[b, (L[b] - 1) // BS] * BS + (L[b] - 1) % BS
                          if L[b] > 0 else -1 for b in range(S)], dtype=np.int64)
    else:
        raise ValueError(new_tokens_at)

    return DecodeInputs(
        cfg=cfg, query=q, key_cache=kc, value_cache=vc,
        block_tables=torch.from_numpy(tables.astype(np.int32)),
        context_lens=torch.from_numpy(L.astype(np.int32)),
        new_key=nk, new_value=nv,
        slot_mapping=torch.from_numpy(slots),
        free_blocks=free, extras=extras)


def poison_unread(inp, value=float("nan")):
    """Fill every pool slot no history token occupies (tail slots of last
    blocks, blocks no table references) with `value`, in place.  A correct
    kernel never reads them, so its output does not change."""
    BS = inp.cfg.block_size
    N = inp.num_blocks
    used = np.zeros((N, BS), dtype=bool)
    tables = inp.block_tables.numpy()
    for b, L in enumerate(inp.context_lens.numpy().tolist()):
        n = _blocks_for(L, BS)
        for j in range(n):
            k = BS if j < n - 1 else L - j * BS
            used[tables[b, j], :k] = True
    mask = torch.from_numpy(~used)                      # [N, BS]
    m = mask[:, None, :, None].expand_as(inp.key_cache)
    inp.key_cache.masked_fill_(m, value)
    inp.value_cache.masked_fill_(m, value)
    return inp


def draw_context_lens(cfg, seed=None):
    """The context lengths generate() draws for cfg (the first draw of its
    stream), without building the rest of the workload."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    return _draw_lens(rng, cfg)


def kv_bytes_read(cfg, context_lens):
    """Algorithmic K+V bytes one decode call reads: every history token's K
    and V row of every KV head, once."""
    e = ELEM_BYTES[cfg.dtype]
    return int(np.sum(np.asarray(context_lens, dtype=np.int64))) * \
        cfg.num_kv_heads * cfg.head_dim * e * 2


def with_overrides(cfg, **kw):
    return replace(cfg, **kw)
