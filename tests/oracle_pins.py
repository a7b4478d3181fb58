"""Pins of the oracle: checks against what the pages and mathematics fix.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
something other than itself: a closed form, an invariant, brute force on a
tiny input, a library routine's special case, or a value printed on the
pages (fixtures under tests/golden/).  ``test_oracle.py`` runs every pin;
``test_oracle_mutants.py`` plants plausible mistakes in the oracle and checks
that at least one pin catches each.
"""

import json
import math
import os

import numpy as np
import torch

import oracle
from oracle import paged_attention as pa

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TIGHT = 1e-12


# --------------------------------------------------------------------------
# Test-side construction of paged inputs from a contiguous ground truth
# --------------------------------------------------------------------------

def scatter_into_pool(rng, K_full, V_full, block_size, extra_blocks=3,
                      poison=False):
    """Place per-sequence contiguous K/V [H_kv, L_b, D] into a shuffled pool.

    Returns (key_cache, value_cache, block_tables, context_lens).  Unused
    table entries are -1.  With poison=True every pool slot that does not
    hold a history token (tail slots, unused blocks) is NaN.
    """
    S = len(K_full)
    H_kv, _, D = K_full[0].shape
    lens = [k.shape[1] for k in K_full]
    nblk = [-(-L // block_size) for L in lens]
    N = sum(nblk) + extra_blocks
    W = max(max(nblk), 1)
    fill = np.nan if poison else 0.0
    kc = np.full((N, H_kv, block_size, D), fill)
    vc = np.full((N, H_kv, block_size, D), fill)
    if not poison:
        kc[:] = rng.standard_normal(kc.shape)
        vc[:] = rng.standard_normal(vc.shape)
    perm = rng.permutation(N)
    tables = np.full((S, W), -1, dtype=np.int64)
    cur = 0
    for b in range(S):
        tables[b, :nblk[b]] = perm[cur:cur + nblk[b]]
        cur += nblk[b]
        for pos in range(lens[b]):
            blk = tables[b, pos // block_size]
            kc[blk, :, pos % block_size, :] = K_full[b][:, pos, :]
            vc[blk, :, pos % block_size, :] = V_full[b][:, pos, :]
    return kc, vc, tables, np.array(lens, dtype=np.int64)


def random_problem(seed, S=3, H=6, H_kv=2, D=8, block_size=4, lens=(1, 7, 13),
                   poison=False, scale=None):
    rng = np.random.default_rng(seed)
    K_full = [rng.standard_normal((H_kv, L, D)) for L in lens]
    V_full = [rng.standard_normal((H_kv, L, D)) for L in lens]
    q = rng.standard_normal((S, H, D))
    kc, vc, bt, cl = scatter_into_pool(rng, K_full, V_full, block_size,
                                       poison=poison)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return dict(q=q, kc=kc, vc=vc, bt=bt, cl=cl, scale=scale,
                K_full=K_full, V_full=V_full)


def all_paths(p, partition_sizes=(1, 2, 3, 4, 5, 8, 16)):
    args = (p["q"], p["kc"], p["vc"], p["bt"], p["cl"], p["scale"])
    outs = {"A": oracle.decode_contiguous(*args), "B": oracle.decode_online(*args)}
    for P in partition_sizes:
        outs["C%d" % P] = oracle.decode_partitioned(*args, partition_size=P)
    return outs


def assert_close(a, b, tol=TIGHT, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert np.isfinite(err) and err <= tol, "%s: max abs err %g > %g" % (what, err, tol)


# --------------------------------------------------------------------------
# Pins on attention
# --------------------------------------------------------------------------

def pin_library_sdpa_gqa():
    """Contiguous single-query attention equals torch's SDPA in float64 with
    the KV heads repeated G times (a library routine for the special case
    'one query, contiguous KV'), for every path."""
    for seed, (H, H_kv) in enumerate([(6, 2), (4, 4), (8, 1)]):
        p = random_problem(100 + seed, H=H, H_kv=H_kv, lens=(1, 5, 16, 23)[:3])
        G = H // H_kv
        outs = all_paths(p)
        for b, L in enumerate(p["cl"]):
            qt = torch.from_numpy(p["q"][b]).reshape(1, H, 1, -1)
            kt = torch.from_numpy(p["K_full"][b]).repeat_interleave(G, dim=0)
            vt = torch.from_numpy(p["V_full"][b]).repeat_interleave(G, dim=0)
            ref = torch.nn.functional.scaled_dot_product_attention(
                qt, kt.unsqueeze(0).contiguous(), vt.unsqueeze(0).contiguous(),
                scale=p["scale"]).reshape(H, -1).numpy()
            for name, o in outs.items():
                assert_close(o[b], ref, what="path %s vs SDPA seq %d" % (name, b))


def pin_brute_force_positions():
    """Brute force on a tiny input: walk pos = 0..L-1 one token at a time
    through logical_block -> block_table -> (pb, off) -> cache row (the
    address chain of MiniPaged-Qwen §6.2), scalar math.exp, two passes."""
    p = random_problem(7, S=2, H=4, H_kv=2, D=3, block_size=2, lens=(5, 2))
    outs = all_paths(p, partition_sizes=(1, 2, 3))
    S, H, D = p["q"].shape
    H_kv = p["kc"].shape[1]
    BS = p["kc"].shape[2]
    for b in range(S):
        L = int(p["cl"][b])
        for h in range(H):
            kvh = h * H_kv // H
            scores = []
            for pos in range(L):
                pb = int(p["bt"][b][pos // BS])
                off = pos % BS
                dot = 0.0
                for i in range(D):
                    dot += p["q"][b, h, i] * p["kc"][pb, kvh, off, i]
                scores.append(p["scale"] * dot)
            mx = max(scores)
            w = [math.exp(s - mx) for s in scores]
            den = sum(w)
            ref = []
            for i in range(D):
                acc = 0.0
                for pos in range(L):
                    pb = int(p["bt"][b][pos // BS])
                    acc += w[pos] * p["vc"][pb, kvh, pos % BS, i]
                ref.append(acc / den)
            for name, o in outs.items():
                assert_close(o[b, h], ref, what="path %s brute force (%d,%d)" % (name, b, h))


def pin_paths_agree():
    """Path B (online) and path C (any partition size) equal path A: the
    pages call the streamed form exactly equivalent to standard attention."""
    p = random_problem(11, S=4, H=8, H_kv=2, D=16, block_size=4,
                       lens=(1, 4, 37, 64))
    outs = all_paths(p, partition_sizes=(1, 3, 4, 8, 12, 64, 100))
    for name, o in outs.items():
        assert_close(o, outs["A"], what="path %s vs A" % name)


def pin_single_token_is_v0():
    """L = 1: softmax over one score is 1, so o = v_0 exactly."""
    p = random_problem(3, S=2, lens=(1, 1))
    for name, o in all_paths(p).items():
        for b in range(2):
            for h in range(p["q"].shape[1]):
                kvh = h * p["kc"].shape[1] // p["q"].shape[1]
                assert np.array_equal(o[b, h], p["V_full"][b][kvh, 0]), name


def pin_uniform_weights_give_mean():
    """All keys equal, or q = 0: every weight is 1/L, o = mean of V."""
    for mode in ("equal_keys", "zero_query"):
        p = random_problem(5, lens=(3, 9, 17))
        if mode == "equal_keys":
            for b in range(len(p["K_full"])):
                p["K_full"][b][:] = p["K_full"][b][:, :1, :]
            rng = np.random.default_rng(5)
            p["kc"], p["vc"], p["bt"], p["cl"] = scatter_into_pool(
                rng, p["K_full"], p["V_full"], 4)
        else:
            p["q"][:] = 0.0
        H = p["q"].shape[1]
        H_kv = p["kc"].shape[1]
        for name, o in all_paths(p).items():
            for b in range(len(p["K_full"])):
                for h in range(H):
                    ref = p["V_full"][b][h * H_kv // H].mean(axis=0)
                    assert_close(o[b, h], ref, 1e-13, "%s %s" % (mode, name))


def pin_value_shift():
    """Weights sum to 1, so V + c gives o + c."""
    p = random_problem(9, lens=(2, 6, 31))
    base = all_paths(p)
    p2 = dict(p)
    p2["vc"] = p["vc"] + 2.5
    for name, o in all_paths(p2).items():
        assert_close(o, base[name] + 2.5, 1e-12, "shift %s" % name)


def pin_two_token_closed_form():
    """L = 2: o = sigma(s0 - s1) v0 + sigma(s1 - s0) v1, sigma(x) = 1/(1+e^-x)."""
    p = random_problem(13, S=1, H=2, H_kv=1, D=5, block_size=1, lens=(2,),
                       scale=0.7)
    for name, o in all_paths(p, partition_sizes=(1, 2)).items():
        for h in range(2):
            k = p["K_full"][0][0]
            v = p["V_full"][0][0]
            s0 = p["scale"] * float(k[0] @ p["q"][0, h])
            s1 = p["scale"] * float(k[1] @ p["q"][0, h])
            w0 = 1.0 / (1.0 + math.exp(-(s0 - s1)))
            w1 = 1.0 / (1.0 + math.exp(-(s1 - s0)))
            assert_close(o[0, h], w0 * v[0] + w1 * v[1], 1e-14, name)


def pin_paged_equals_contiguous_any_permutation():
    """Paging does not change the result: the same logical history under
    different block-table permutations and block sizes gives the same o."""
    rng = np.random.default_rng(21)
    lens = (1, 15, 16, 17, 40)
    H_kv, D = 2, 8
    K_full = [rng.standard_normal((H_kv, L, D)) for L in lens]
    V_full = [rng.standard_normal((H_kv, L, D)) for L in lens]
    q = rng.standard_normal((len(lens), 4, D))
    results = []
    for trial, bs in enumerate((4, 4, 16, 32, 1)):
        kc, vc, bt, cl = scatter_into_pool(np.random.default_rng(300 + trial),
                                           K_full, V_full, bs, extra_blocks=5)
        args = (q, kc, vc, bt, cl, 0.3)
        results.append((oracle.decode_contiguous(*args),
                        oracle.decode_online(*args),
                        oracle.decode_partitioned(*args, partition_size=8)))
    for r in results[1:]:
        assert np.array_equal(r[0], results[0][0]), "path A not permutation-exact"
        assert_close(r[1], results[0][1], 1e-14, "path B permutation")
        assert_close(r[2], results[0][2], 1e-14, "path C permutation")


def pin_gqa_equals_mha_with_repeated_kv():
    """A GQA group reads one KV head: the same as MHA whose KV heads are that
    head repeated G times (contiguous groups)."""
    H, H_kv, D, BS = 6, 2, 8, 4
    G = H // H_kv
    p = random_problem(17, H=H, H_kv=H_kv, D=D, block_size=BS, lens=(5, 12, 3))
    gqa = all_paths(p)
    K_rep = [np.repeat(k, G, axis=0) for k in p["K_full"]]
    V_rep = [np.repeat(v, G, axis=0) for v in p["V_full"]]
    kc, vc, bt, cl = scatter_into_pool(np.random.default_rng(4), K_rep, V_rep, BS)
    args = (p["q"], kc, vc, bt, cl, p["scale"])
    mha = {"A": oracle.decode_contiguous(*args), "B": oracle.decode_online(*args)}
    for name in ("A", "B"):
        assert_close(gqa[name], mha[name], 1e-14, "GQA vs MHA " + name)


def pin_masked_slots_never_read():
    """Tail slots past L, unused pool blocks and unused (-1) table entries
    hold NaN; the output is finite and equal to the clean problem's."""
    clean = random_problem(23, lens=(1, 6, 13), block_size=4)
    rng = np.random.default_rng(0)
    kc, vc, bt, cl = scatter_into_pool(rng, clean["K_full"], clean["V_full"], 4,
                                       poison=True)
    dirty = dict(clean, kc=kc, vc=vc, bt=bt, cl=cl)
    a = all_paths(clean)
    d = all_paths(dirty)
    for name in a:
        assert np.all(np.isfinite(d[name])), name
        assert_close(d[name], a[name], 1e-14, "masked " + name)


def pin_convex_hull():
    """Each output element lies between the min and max of V over the history."""
    p = random_problem(29, lens=(3, 8, 20))
    H = p["q"].shape[1]
    H_kv = p["kc"].shape[1]
    for name, o in all_paths(p).items():
        for b in range(3):
            for h in range(H):
                V = p["V_full"][b][h * H_kv // H]
                assert np.all(o[b, h] >= V.min(axis=0) - 1e-15), name
                assert np.all(o[b, h] <= V.max(axis=0) + 1e-15), name


def pin_score_shift_and_large_logits():
    """Adding a constant to every score leaves o unchanged (softmax shift
    invariance); with scores near 1e4 the result stays finite.  Built by an
    extra key dimension that is constant c for every token, with q = 1 there."""
    base = random_problem(31, D=6, lens=(4, 9, 2))
    ref = all_paths(base)
    for c in (50.0, 1.0e4, -1.0e4):
        K_aug = [np.concatenate([k, np.full(k.shape[:2] + (1,), c)], axis=2)
                 for k in base["K_full"]]
        V_aug = [np.concatenate([v, np.zeros(v.shape[:2] + (1,))], axis=2)
                 for v in base["V_full"]]
        q_aug = np.concatenate([base["q"], np.ones(base["q"].shape[:2] + (1,))], axis=2)
        kc, vc, bt, cl = scatter_into_pool(np.random.default_rng(2), K_aug, V_aug, 4)
        outs = all_paths(dict(q=q_aug, kc=kc, vc=vc, bt=bt, cl=cl, scale=base["scale"]))
        for name, o in outs.items():
            assert np.all(np.isfinite(o)), (c, name)
            assert_close(o[..., :-1], ref[name], 1e-9, "shift %g %s" % (c, name))


def pin_empty_history_is_zero():
    """L = 0 (reading: nothing to attend to) gives a zero output row."""
    p = random_problem(37, lens=(0, 5, 0))
    for name, o in all_paths(p).items():
        assert np.array_equal(o[0], np.zeros_like(o[0])), name
        assert np.array_equal(o[2], np.zeros_like(o[2])), name
        assert np.all(np.isfinite(o[1])), name


def pin_pairs_subset():
    """Restricting to a list of (sequence, head) pairs computes the same rows."""
    p = random_problem(41, lens=(5, 9, 3))
    args = (p["q"], p["kc"], p["vc"], p["bt"], p["cl"], p["scale"])
    pairs = [(0, 1), (2, 5), (1, 0)]
    for fn in (oracle.decode_contiguous, oracle.decode_online):
        full = fn(*args)
        sub = fn(*args, pairs=pairs)
        for b, h in pairs:
            assert np.array_equal(sub[b, h], full[b, h])
    full = oracle.decode_partitioned(*args, partition_size=4)
    sub = oracle.decode_partitioned(*args, partition_size=4, pairs=pairs)
    for b, h in pairs:
        assert np.array_equal(sub[b, h], full[b, h])


# --------------------------------------------------------------------------
# Pins on block arithmetic, cache write and gather
# --------------------------------------------------------------------------

def pin_block_count_and_waste_bound():
    """T is the least n with n * B_s >= L, and 0 <= n*B_s - L < B_s
    (vLLM-paging '页表与内部碎片')."""
    for bs in (1, 2, 3, 4, 16, 32):
        assert oracle.num_logical_blocks(0, bs) == 0
        for L in range(1, 200):
            n = next(k for k in range(L + 1) if k * bs >= L)
            assert oracle.num_logical_blocks(L, bs) == n, (L, bs)
            w = oracle.tail_waste(L, bs)
            assert 0 <= w < bs, (L, bs, w)


def pin_printed_block_mapping():
    """Replays the FIFO allocator of PA-source §三 on the mapping example of
    §二: 32, 16, 48 tokens at block size 16 -> [0,1], [2], [3,4,5]."""
    with open(os.path.join(GOLDEN, "pa_source_block_mapping.json")) as f:
        g = json.load(f)
    free = list(range(64))
    for r in g["requests"]:
        n = oracle.num_logical_blocks(r["tokens"], g["block_size"])
        got = [free.pop(0) for _ in range(n)]
        assert got == r["blocks"], (r, got)
    assert free[:3] == g["free_head_after"]


def pin_printed_kv_sizes():
    """KV-size worked examples printed on the pages, in both byte formulas."""
    with open(os.path.join(GOLDEN, "kv_cache_sizes.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        hidden_form = oracle.kv_cache_bytes_hidden_form(
            c["num_layers"], c["seq_len"], c["hidden"], c["batch"], c["bytes_per_elem"])
        # M_KV with MHA: H_kv * d_h = hidden (32 heads of 128)
        mkv = oracle.kv_cache_bytes(c["num_layers"], 32, c["hidden"] // 32,
                                    c["bytes_per_elem"], [c["seq_len"]] * c["batch"])
        assert hidden_form == mkv
        shown = round(hidden_form / c["unit_bytes"], c["printed_decimals"])
        assert shown == c["printed"], (c["source"], hidden_form, shown)


def pin_kv_head_map():
    """Contiguous groups: each KV head serves exactly G consecutive query heads."""
    for H, H_kv in ((28, 4), (32, 8), (32, 32), (7, 1)):
        G = H // H_kv
        m = [oracle.kv_head_of(h, H, H_kv) for h in range(H)]
        assert m == sorted(m)
        assert all(m.count(k) == G for k in range(H_kv))
    try:
        oracle.kv_head_of(0, 28, 5)
    except ValueError:
        pass
    else:
        raise AssertionError("H % H_kv != 0 must be rejected")


def pin_cache_write_round_trip():
    """Tokens written at the slots of positions 0..L-1 of a sequence come
    back, in order, from the block-wise gather; every other element of the
    pool keeps its bits; negative slots write nothing."""
    rng = np.random.default_rng(43)
    N, H_kv, BS, D = 9, 2, 4, 3
    for dt in (np.float64, np.float32, np.uint16):
        kc0 = rng.integers(0, 60000, size=(N, H_kv, BS, D)).astype(dt)
        vc0 = rng.integers(0, 60000, size=(N, H_kv, BS, D)).astype(dt)
        kc0_before = kc0.copy()
        table = rng.permutation(N)[:3]
        L = 10
        keys = rng.integers(0, 60000, size=(L, H_kv, D)).astype(dt)
        vals = rng.integers(0, 60000, size=(L, H_kv, D)).astype(dt)
        # slots of positions 0..L-1 (the append flow of MiniPaged-Qwen §8.1),
        # with two padding entries mixed in
        slots = [int(table[pos // BS]) * BS + pos % BS for pos in range(L)]
        slots_pad = slots[:4] + [-1] + slots[4:] + [-7]
        keys_pad = np.concatenate([keys[:4], keys[:1], keys[4:], keys[:1]])
        vals_pad = np.concatenate([vals[:4], vals[:1], vals[4:], vals[:1]])
        kc, vc = oracle.reshape_and_cache(keys_pad, vals_pad, kc0, vc0, slots_pad)
        assert kc.dtype == dt and vc.dtype == dt
        K, V = oracle.gather_sequence_kv(kc, vc, table, L)
        assert np.array_equal(K, np.transpose(keys, (1, 0, 2)))
        assert np.array_equal(V, np.transpose(vals, (1, 0, 2)))
        touched = np.zeros((N, BS), dtype=bool)
        for s in slots:
            touched[s // BS, s % BS] = True
        for blk in range(N):
            for off in range(BS):
                if not touched[blk, off]:
                    assert np.array_equal(kc[blk, :, off], kc0[blk, :, off])
                    assert np.array_equal(vc[blk, :, off], vc0[blk, :, off])
        assert np.array_equal(kc0, kc0_before)  # input untouched (copy semantics)


def pin_gather_is_bit_exact():
    """The gather copies bits: uint16 (bf16/fp16 payload) round-trips, rows
    come from block_table[pos // BS] at offset pos % BS."""
    rng = np.random.default_rng(47)
    N, H_kv, BS, D = 6, 3, 4, 5
    kc = rng.integers(0, 65536, size=(N, H_kv, BS, D)).astype(np.uint16)
    vc = rng.integers(0, 65536, size=(N, H_kv, BS, D)).astype(np.uint16)
    table = np.array([4, 0, 5, -1])
    L = 9
    K, V = oracle.gather_sequence_kv(kc, vc, table, L)
    assert K.shape == (H_kv, L, D) and K.dtype == np.uint16
    for pos in range(L):
        blk = int(table[pos // BS])
        assert np.array_equal(K[:, pos], kc[blk, :, pos % BS])
        assert np.array_equal(V[:, pos], vc[blk, :, pos % BS])


ALL_PINS = [
    pin_library_sdpa_gqa,
    pin_brute_force_positions,
    pin_paths_agree,
    pin_single_token_is_v0,
    pin_uniform_weights_give_mean,
    pin_value_shift,
    pin_two_token_closed_form,
    pin_paged_equals_contiguous_any_permutation,
    pin_gqa_equals_mha_with_repeated_kv,
    pin_masked_slots_never_read,
    pin_convex_hull,
    pin_score_shift_and_large_logits,
    pin_empty_history_is_zero,
    pin_pairs_subset,
    pin_block_count_and_waste_bound,
    pin_printed_block_mapping,
    pin_printed_kv_sizes,
    pin_kv_head_map,
    pin_cache_write_round_trip,
    pin_gather_is_bit_exact,
]
