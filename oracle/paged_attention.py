"""Plain float64 oracle of single-step decode paged attention.

TEST INFRASTRUCTURE ONLY -- see the package docstring.  Slow and obvious on
purpose: Python loops over sequences, heads and blocks, NumPy for the inner
dot products.  No blocking, fusion or reordering beyond what the cited
definitions state.

Array conventions (all NumPy):
  query         [S, H, D]          any float dtype, upcast to float64 here
  key_cache     [N, H_kv, BS, D]   layout of [MiniPaged-Qwen §8.2]
  value_cache   [N, H_kv, BS, D]
  block_tables  [S, W]             integer; only entries j < ceil(L_b/BS) read
  context_lens  [S]                integer, L_b >= 0

Readings of points the pages leave open (each also listed in the design doc):
  * empty history (L_b == 0): the output row is zero;
  * the scale is an argument (the pages fix 1/sqrt(d));
  * online-update operator: the garbled "l, e^{m-m'}" is a product
    l * e^{m-m'}; the initial state is m = -inf, l = 0, o~ = 0 and the
    rescale factor is 0 while m is still -inf.
"""

import math

import numpy as np

NEG_INF = float("-inf")


# --------------------------------------------------------------------------
# Block arithmetic and address translation
# --------------------------------------------------------------------------

def num_logical_blocks(L, block_size):
    """Blocks a history of L tokens occupies: T = ceil(L / B_s).

    [MiniPaged-Qwen §5, eq. T]; [vLLM-paging "页表与内部碎片", eq. N_block].
    """
    L = int(L)
    block_size = int(block_size)
    if L < 0 or block_size <= 0:
        raise ValueError("need L >= 0 and block_size > 0")
    return (L + block_size - 1) // block_size


def tail_waste(L, block_size):
    """Unused slots in the last block, N_block * P_b - T.

    [vLLM-paging "页表与内部碎片"]: bounded by 0 <= waste < P_b.
    """
    return num_logical_blocks(L, block_size) * int(block_size) - int(L)


def kv_head_of(h, num_heads, num_kv_heads):
    """KV head read by query head h: floor(h / (H_q / H_kv)).

    [MiniPaged-Qwen §9.1, 一致点 4]: contiguous groups of query heads share
    one KV head.
    """
    if num_kv_heads <= 0 or num_heads % num_kv_heads:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    return int(h) // (int(num_heads) // int(num_kv_heads))


def _token_address(block_table_row, pos, block_size):
    """Logical position -> (physical block, offset in block).

    [MiniPaged-Qwen §6.2 steps 2-3, §8.3]: logical_block = pos // block_size,
    off = pos % block_size, pb = block_table[logical_block].
    """
    logical_block = pos // block_size
    off = pos % block_size
    return int(block_table_row[logical_block]), off


def gather_sequence_kv(key_cache, value_cache, block_table_row, L, kv_heads=None):
    """History of one sequence laid out contiguously, per KV head.

    Returns K, V of shape [len(kv_heads), L, D] in the caches' own dtype (a
    pure copy, so bit-exact).  The history is the concatenation of the
    logical blocks K^(0..T-1), block t being key_cache[block_table[t], kvh]
    [MiniPaged-Qwen §5 eqs. K, V, pb_t; §5.1], with the last block cut at L
    tokens [MiniPaged-Qwen §5: the last block may be partly filled].
    """
    N, H_kv, BS, D = key_cache.shape
    if kv_heads is None:
        kv_heads = list(range(H_kv))
    T = num_logical_blocks(L, BS)
    ids = np.asarray(block_table_row[:T], dtype=np.int64)
    if T and (ids.min() < 0 or ids.max() >= N):
        raise IndexError("block table entry outside the pool")
    kvh = np.asarray(kv_heads, dtype=np.int64)
    K = key_cache[ids][:, kvh]            # [T, nh, BS, D]
    V = value_cache[ids][:, kvh]
    K = np.transpose(K, (1, 0, 2, 3)).reshape(len(kvh), T * BS, D)[:, :L]
    V = np.transpose(V, (1, 0, 2, 3)).reshape(len(kvh), T * BS, D)[:, :L]
    return K, V


def _pairs(S, H, pairs):
    if pairs is None:
        return [(b, h) for b in range(S) for h in range(H)]
    return [(int(b), int(h)) for b, h in pairs]


# --------------------------------------------------------------------------
# Path A: contiguous gather, then standard softmax attention
# --------------------------------------------------------------------------

def _softmax(s):
    """p_j = exp(s_j) / sum_u exp(s_u) over the whole history.

    [MiniPaged-Qwen §5.2, eq. p_j].  The maximum is subtracted first, which
    leaves the value unchanged.
    """
    e = np.exp(s - s.max())
    return e / e.sum()


def decode_contiguous(query, key_cache, value_cache, block_tables, context_lens,
                      scale, pairs=None):
    """Path A: o = softmax(scale * q K^T) V over the gathered history.

    [MiniPaged-Qwen §1 eq. o and §5.3]; the same computation as the
    standard_attention sketch of [PA-source §4].  `pairs` optionally
    restricts the work to a list of (sequence, query head); the other rows of
    the result are NaN.
    """
    S, H, D = query.shape
    H_kv = key_cache.shape[1]
    out = np.full((S, H, D), np.nan)
    by_seq = {}
    for b, h in _pairs(S, H, pairs):
        by_seq.setdefault(b, []).append(h)
    for b, heads in by_seq.items():
        L = int(context_lens[b])
        if L == 0:
            out[b, heads] = 0.0
            continue
        kvhs = sorted({kv_head_of(h, H, H_kv) for h in heads})
        K, V = gather_sequence_kv(key_cache, value_cache, block_tables[b], L, kvhs)
        for h in heads:
            i = kvhs.index(kv_head_of(h, H, H_kv))
            Kh = K[i].astype(np.float64)
            Vh = V[i].astype(np.float64)
            s = float(scale) * (Kh @ query[b, h].astype(np.float64))
            out[b, h] = _softmax(s) @ Vh
    return out


# --------------------------------------------------------------------------
# Path B: per-block online softmax walk over the paged cache
# --------------------------------------------------------------------------

def _online_walk(qv, key_cache, value_cache, block_table_row, kvh, t0, t1, scale):
    """Online-softmax state (m, l, o~) over logical tokens [t0, t1).

    Visits the logical blocks overlapping [t0, t1) in order.  For each block
    (addressed by pb = block_table[t], rows cut to the tokens in range, which
    masks the last block past the history [PA-source §4 paged_attention;
    MiniPaged-Qwen §5]) it applies [MiniPaged-Qwen §5.2]:
        m_t = max s^(t);  m' = max(m, m_t);
        l'  = l * e^{m-m'} + sum_j e^{s_j - m'};
        o~' = o~ * e^{m-m'} + sum_j e^{s_j - m'} v_j.
    """
    BS = key_cache.shape[2]
    D = key_cache.shape[3]
    m, l, acc = NEG_INF, 0.0, np.zeros(D)
    if t1 <= t0:
        return m, l, acc
    for t in range(t0 // BS, (t1 - 1) // BS + 1):
        pb = int(block_table_row[t])
        lo = max(t0 - t * BS, 0)
        hi = min(t1 - t * BS, BS)
        Kt = key_cache[pb, kvh, lo:hi].astype(np.float64)
        Vt = value_cache[pb, kvh, lo:hi].astype(np.float64)
        s = float(scale) * (Kt @ qv)
        m_t = float(s.max())
        m_new = max(m, m_t)
        alpha = 0.0 if m == NEG_INF else math.exp(m - m_new)
        e = np.exp(s - m_new)
        l = l * alpha + float(e.sum())
        acc = acc * alpha + e @ Vt
        m = m_new
    return m, l, acc


def decode_online(query, key_cache, value_cache, block_tables, context_lens,
                  scale, pairs=None):
    """Path B: the streamed form of path A, final o = o~ / l.

    [MiniPaged-Qwen §5.2] (equivalent to standard attention, §5.2-5.3), with
    per-token address translation through the block table [§6.2].
    """
    S, H, D = query.shape
    H_kv = key_cache.shape[1]
    out = np.full((S, H, D), np.nan)
    for b, h in _pairs(S, H, pairs):
        L = int(context_lens[b])
        if L == 0:
            out[b, h] = 0.0
            continue
        kvh = kv_head_of(h, H, H_kv)
        m, l, acc = _online_walk(query[b, h].astype(np.float64), key_cache,
                                 value_cache, block_tables[b], kvh, 0, L, scale)
        out[b, h] = acc / l
    return out


# --------------------------------------------------------------------------
# Path C: context partitions, each reduced on its own, then merged
# --------------------------------------------------------------------------

def partition_state(qv, key_cache, value_cache, block_table_row, kvh, t0, t1, scale):
    """(lse, o) of one partition [t0, t1): lse = m + ln l, o = o~ / l.

    One "local reduction" of [MiniPaged-Qwen §10.2 (2)] (several groups take
    different KV shards, reduce locally, then merge).
    """
    m, l, acc = _online_walk(qv, key_cache, value_cache, block_table_row, kvh,
                             t0, t1, scale)
    return m + math.log(l), acc / l


def lse_merge(lses, outs):
    """Global merge of partition results: o = sum_p w_p o_p / sum_p w_p.

    w_p = exp(lse_p - M), M = max_p lse_p.  This is the online update of
    [MiniPaged-Qwen §5.2] applied to whole partitions instead of blocks (the
    update is associative), i.e. the "merge after local reduction" of
    [MiniPaged-Qwen §10.2 (2)].  Summed in partition order.
    """
    lses = np.asarray(lses, dtype=np.float64)
    M = lses.max()
    w = np.exp(lses - M)
    num = np.zeros_like(np.asarray(outs[0], dtype=np.float64))
    for p in range(len(lses)):
        num = num + w[p] * np.asarray(outs[p], dtype=np.float64)
    return num / w.sum()


def decode_partitioned(query, key_cache, value_cache, block_tables, context_lens,
                       scale, partition_size, pairs=None):
    """Path C: partitions [p*P, (p+1)*P) reduced separately, then lse_merge."""
    if partition_size <= 0:
        raise ValueError("partition_size must be positive")
    S, H, D = query.shape
    H_kv = key_cache.shape[1]
    out = np.full((S, H, D), np.nan)
    for b, h in _pairs(S, H, pairs):
        L = int(context_lens[b])
        if L == 0:
            out[b, h] = 0.0
            continue
        kvh = kv_head_of(h, H, H_kv)
        qv = query[b, h].astype(np.float64)
        lses, outs = [], []
        for t0 in range(0, L, partition_size):
            lse, o = partition_state(qv, key_cache, value_cache, block_tables[b],
                                     kvh, t0, min(t0 + partition_size, L), scale)
            lses.append(lse)
            outs.append(o)
        out[b, h] = lse_merge(lses, outs)
    return out


# --------------------------------------------------------------------------
# Cache write
# --------------------------------------------------------------------------

def reshape_and_cache(key, value, key_cache, value_cache, slot_mapping):
    """Store each new token's K/V at its slot; returns new cache arrays.

    [MiniPaged-Qwen §8.1-8.2]: append_token yields a linear slot per new
    token and the cache-write kernel stores its K/V there, so that
    key_cache[pb, kvh, off, :] holds it.  Reading of the linear slot:
    slot = pb * block_size + off (the position -> (block, offset) split of
    §6.2 applied to the pool).  A negative slot marks padding and is skipped.
    key/value: [T, H_kv, D].  Bit-exact for any dtype.
    """
    kc = np.array(key_cache, copy=True)
    vc = np.array(value_cache, copy=True)
    N, H_kv, BS, D = kc.shape
    for i, s in enumerate(np.asarray(slot_mapping).tolist()):
        s = int(s)
        if s < 0:
            continue
        if s >= N * BS:
            raise IndexError("slot outside the pool")
        kc[s // BS, :, s % BS, :] = key[i]
        vc[s // BS, :, s % BS, :] = value[i]
    return kc, vc


# --------------------------------------------------------------------------
# Byte accounting
# --------------------------------------------------------------------------

def kv_cache_bytes(num_layers, num_kv_heads, head_dim, bytes_per_elem, seq_lens):
    """M_KV = 2 * L_layers * b * H_kv * d_h * sum_i T_i.

    [vLLM-paging "为什么连续预留会压低 batch", eq. M_KV].  With one layer and
    the per-sequence context lengths, this is the K+V bytes one decode call
    must read.
    """
    total_tokens = int(sum(int(t) for t in seq_lens))
    return 2 * int(num_layers) * int(bytes_per_elem) * int(num_kv_heads) \
        * int(head_dim) * total_tokens


def kv_cache_bytes_hidden_form(num_layers, seq_len, hidden, batch, bytes_per_elem):
    """2 x layers x seq x hidden x batch x bytes  [KV-principles §2.2]."""
    return 2 * int(num_layers) * int(seq_len) * int(hidden) * int(batch) \
        * int(bytes_per_elem)


def decode_verify(query, key_cache, value_cache, block_tables, context_lens, query_start,
                  scale):
    """Decode with several new query tokens per sequence (the verify step of
    speculative decoding; [vLLM-paging] "Kernel metadata" lists each
    sequence's query range and the verify semantics, "Prefix、beam 与
    speculative": candidate tokens are written to the cache and checked).

    Sequence b owns query rows query_start[b] .. query_start[b+1] - 1 of
    query [total_q, H, D]: its q_b newest tokens, already in the cache as
    history positions L_b - q_b .. L_b - 1.  Row i attends positions
    t <= L_b - q_b + i (causal among the new tokens): the plain decode of
    eq. o over that prefix of the history.  q_b > L_b (a query token outside
    the history) gives NaN rows.
    """
    total_q, H, D = query.shape
    out = np.full((total_q, H, D), np.nan)
    qs = np.asarray(query_start, dtype=np.int64)
    for b in range(len(qs) - 1):
        q_b = int(qs[b + 1] - qs[b])
        L = int(context_lens[b])
        if q_b <= 0 or q_b > L:
            continue
        for i in range(q_b):
            r = int(qs[b]) + i
            Li = L - q_b + i + 1
            one = decode_contiguous(query[r:r + 1], key_cache, value_cache,
                                    np.asarray(block_tables)[b:b + 1],
                                    np.array([Li]), scale)
            out[r] = one[0]
    return out
