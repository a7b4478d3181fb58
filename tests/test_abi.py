"""The C-ABI boundary on the CPU: the library loads, exports every symbol
include/pagedattn.h declares, and rejects invalid arguments on the host with
the documented status before anything is launched (no GPU needed; these
calls never reach a kernel)."""

import ctypes
import os
import re

import pytest

from paged_kv_decode_attention_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagedattn.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3
FAKE = 0x10000            # a 16-byte aligned non-null address, never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ops.LIB_PATH):
        from paged_kv_decode_attention_amd import build
        build.build()
    return ops.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(ops._SIGNATURES), "binding and header disagree"


def test_version_and_status_strings(lib):
    assert lib.pa_version() == 100
    for s, text in ((OK, b"ok"), (INVALID, b"invalid argument"),
                    (UNSUPPORTED, b"unsupported configuration"),
                    (-5, b"KV pool exhausted")):
        assert lib.pa_status_string(s) == text
    assert lib.pa_status_string(12345) == b"unknown status"


def _decode(lib, **kw):
    a = dict(out=FAKE, query=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, cl=FAKE, S=2, H=28, H_kv=4,
             G=7, D=128, BS=16, N=100, W=8, max_ctx=128, scale=0.088, dtype=ops.PA_BF16,
             P=0, ws=0, ws_bytes=0, stream=0)
    a.update(kw)
    vp = ctypes.c_void_p
    return lib.pa_paged_attention_decode(
        vp(a["out"]), vp(a["query"]), vp(a["kc"]), vp(a["vc"]), vp(a["bt"]), vp(a["cl"]),
        a["S"], a["H"], a["H_kv"], a["G"], a["D"], a["BS"], a["N"], a["W"], a["max_ctx"],
        a["scale"], a["dtype"], a["P"], vp(a["ws"]), a["ws_bytes"], vp(a["stream"]))


@pytest.mark.parametrize("kw,status", [
    (dict(H=30, H_kv=4, G=7), INVALID),          # H % H_kv != 0
    (dict(G=4), INVALID),                        # group size mismatch
    (dict(H_kv=0), INVALID),
    (dict(S=-1), INVALID),
    (dict(dtype=7), INVALID),
    (dict(D=96), UNSUPPORTED),
    (dict(BS=12), UNSUPPORTED),
    (dict(max_ctx=129), INVALID),                # > W * BS
    (dict(max_ctx=-1), INVALID),
    (dict(scale=float("inf")), INVALID),
    (dict(N=0), INVALID),
    (dict(query=0), INVALID),                    # null pointer
    (dict(kc=FAKE + 8), INVALID),                # misaligned
    (dict(P=48), INVALID),                       # not a multiple of 32
    (dict(P=2048), INVALID),                     # > 64 * block_size
    (dict(max_ctx=128, P=32), WORKSPACE),        # 4 partitions, no workspace
    (dict(max_ctx=128, P=32, ws=FAKE, ws_bytes=16), WORKSPACE),
    (dict(max_ctx=128, P=32, ws=FAKE + 16, ws_bytes=1 << 30), INVALID),  # not 256-aligned
])
def test_decode_rejects_on_host(lib, kw, status):
    assert _decode(lib, **kw) == status
    assert lib.pa_last_error() != b""


def test_noalloc_decode_rejects_on_host(lib):
    """The no-allocation decode: its device array's size, and sizes that are
    invalid or need more workspace than the array holds are refused before
    any HIP call (the array's address is looked up only for a call that runs)."""
    vp = ctypes.c_void_p
    assert lib.pa_noalloc_scratch_bytes() == 40 << 20

    def call(**kw):
        a = dict(S=2, H=28, H_kv=4, G=7, D=128, BS=16, N=100, W=8, max_ctx=128, P=0,
                 dtype=ops.PA_BF16)
        a.update(kw)
        return lib.pa_paged_attention_decode_noalloc(
            vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), a["S"], a["H"],
            a["H_kv"], a["G"], a["D"], a["BS"], a["N"], a["W"], a["max_ctx"], 0.088,
            a["dtype"], a["P"], vp(0))
    assert call(H=30) == INVALID                       # H % H_kv != 0
    assert call(D=96) == INVALID                       # no workspace size for this shape
    # fixed partitions of 32 tokens over 2048 sequences x 64 heads x 4096 tokens:
    # 2048 * 64 * 128 * 129 * 4 bytes of partial states, beyond 40 MiB
    assert call(S=2048, H=64, H_kv=8, G=8, W=256, max_ctx=4096, P=32) == WORKSPACE
    assert b"workspace" in lib.pa_last_error()
    assert lib.pa_decode_workspace_size(2048, 64, 8, 128, 16, 4096, 32, ops.PA_BF16) > 40 << 20


def test_decode_empty_batch_is_noop(lib):
    assert _decode(lib, S=0, out=0, query=0) == OK


def test_workspace_size_arithmetic(lib):
    f = lib.pa_decode_workspace_size
    # one partition of the vector-ALU kernel (float32 at head_dim 256): no workspace
    assert f(4, 2, 2, 256, 16, 64, 0, ops.PA_F32) == 0
    # S=2, H=4, P=32, max 128 -> 4 partitions: lse 2*4*4 floats, out
    # 2*4*4*D floats, each region 256-byte aligned
    up = lambda x: (x + 255) // 256 * 256
    rows = 2 * 4 * 4
    want = up(rows * 4) + up(rows * 128 * 4)
    assert f(2, 4, 2, 128, 16, 128, 32, ops.PA_BF16) == want
    assert f(2, 4, 3, 128, 16, 128, 32, ops.PA_BF16) == ctypes.c_size_t(-1).value
    assert f(2, 4, 2, 128, 16, 128, 40, ops.PA_BF16) == ctypes.c_size_t(-1).value


def test_balanced_workspace_follows_the_pass_width(lib):
    """Balanced-schedule slots hold 16 columns, or 32 when a pass serves more
    than 16 heads; the pass width is ceil(G / passes) with the fewest passes
    of <= 32 heads (<= 16 at head_dim 256)."""
    f = lib.pa_decode_workspace_size
    up = lambda x: (x + 255) // 256 * 256
    W = 1024                                   # workgroups the layout is sized for

    def bal(cols, D):
        rows = W * 2 * cols
        return up(rows * 4) + up(rows * D * 4) + up(W * 4 * 4)
    # one sequence of 64 tokens: the fixed layout needs nothing, so the size
    # is the balanced layout's
    for G, D, cols in ((7, 128, 16), (24, 128, 32), (33, 128, 32), (37, 128, 32),
                       (96, 128, 32), (17, 256, 16), (37, 256, 16), (40, 64, 32)):
        assert f(1, G, 1, D, 16, 64, 0, ops.PA_BF16) == bal(cols, D), (G, D)
    # float32 rows: passes of at most 16 heads, one column tile
    for G, D in ((7, 128), (24, 128), (33, 64)):
        assert f(1, G, 1, D, 16, 64, 0, ops.PA_F32) == bal(16, D), (G, D)


def test_partition_heuristic_is_valid(lib):
    for S, H_kv, BS, L in ((64, 4, 16, 4096), (32, 32, 16, 4096), (4, 8, 32, 131072),
                           (128, 8, 16, 8192), (4, 2, 16, 64), (1, 1, 32, 1)):
        P = lib.pa_decode_partition_size(S, H_kv, 7, 128, BS, L, ops.PA_BF16)
        assert P > 0 and P % 32 == 0 and P % BS == 0 and P <= 64 * BS
    assert lib.pa_decode_partition_size(4, 0, 1, 128, 16, 64, ops.PA_BF16) == 0


def test_reshape_and_cache_rejects_on_host(lib):
    vp = ctypes.c_void_p
    f = lib.pa_reshape_and_cache
    assert f(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), 0, 2, 64, 16, 4, ops.PA_F32,
             vp(0)) == OK                                               # no tokens
    assert f(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(0), 4, 2, 64, 16, 4, ops.PA_F32,
             vp(0)) == INVALID                                          # null slots
    assert f(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), 4, 2, 6, 16, 4, ops.PA_F16,
             vp(0)) == UNSUPPORTED                                      # 12-byte rows
    assert f(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), 4, 2, 64, 16, 4, 9,
             vp(0)) == INVALID


def test_copy_blocks_rejects_on_host(lib):
    vp = ctypes.c_void_p
    f = lib.pa_copy_blocks
    assert f(vp(FAKE), vp(FAKE), vp(FAKE), 0, 2, 64, 16, 4, ops.PA_F32, vp(0)) == OK   # no pairs
    assert f(vp(FAKE), vp(FAKE), vp(0), 3, 2, 64, 16, 4, ops.PA_F32, vp(0)) == INVALID
    assert f(vp(FAKE), vp(FAKE), vp(FAKE), -1, 2, 64, 16, 4, ops.PA_F32, vp(0)) == INVALID
    assert f(vp(FAKE), vp(FAKE), vp(FAKE), 3, 2, 6, 16, 4, ops.PA_F16, vp(0)) == UNSUPPORTED
    assert f(vp(FAKE + 8), vp(FAKE), vp(FAKE), 3, 2, 64, 16, 4, ops.PA_F32, vp(0)) == INVALID
    assert f(vp(FAKE), vp(FAKE), vp(FAKE), 3, 2, 64, 16, 0, ops.PA_F32, vp(0)) == INVALID


@pytest.mark.parametrize("fmt", ["fp8", "i8"])
def test_8bit_entry_points_reject_on_host(lib, fmt):
    vp, f32 = ctypes.c_void_p, ctypes.c_float
    f = getattr(lib, "pa_reshape_and_cache_" + fmt)
    args = lambda ks, vs, T=4, D=128: (vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), T, 2, D,
                                       16, 4, ops.PA_BF16, f32(ks), f32(vs), vp(0))
    assert f(*args(1.0, 1.0, T=0)) == OK                       # no tokens
    assert f(*args(0.0, 1.0)) == INVALID                       # scale must be > 0
    assert f(*args(1.0, float("inf"))) == INVALID
    assert f(*args(1.0, 1.0, D=24)) == UNSUPPORTED             # head_dim not a multiple of 16
    d = getattr(lib, "pa_paged_attention_decode_" + fmt)
    base = dict(S=2, H=28, H_kv=4, G=7, D=128, BS=16, dtype=ops.PA_BF16, ks=0.5, vs=0.5)

    def call(**kw):
        a = dict(base, **kw)
        return d(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), a["S"], a["H"],
                 a["H_kv"], a["G"], a["D"], a["BS"], 64, 16, 256, f32(0.1), a["dtype"],
                 f32(a["ks"]), f32(a["vs"]), 0, vp(FAKE), ctypes.c_size_t(1 << 30), vp(0))
    assert call(ks=-1.0) == INVALID
    assert call(vs=float("nan")) == INVALID
    assert call(G=37, H=148, S=0) == OK                        # 37: passes of 19 and 18 heads
    assert call(G=160, H=160, H_kv=1, S=0) == OK               # 5 passes of 32
    # the fused 8-bit append takes groups of one pass only
    a8 = getattr(lib, "pa_decode_append_" + fmt)
    assert a8(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE),
              2, 64, 1, 64, 128, 16, 64, 16, 256, f32(0.1), ops.PA_BF16, f32(0.5), f32(0.5), 0,
              vp(FAKE), ctypes.c_size_t(1 << 30), vp(0)) == UNSUPPORTED
    assert b"fused append" in lib.pa_last_error()
    assert call(G=33, H=132, S=0) == OK                        # 33: passes of 17 and 16 heads
    assert call(dtype=ops.PA_F32) == UNSUPPORTED               # 8-bit codes: 16-bit queries
    assert call(S=0) == OK
    # the fused append needs the new key and value
    a = getattr(lib, "pa_decode_append_" + fmt)
    assert a(vp(FAKE), vp(FAKE), vp(0), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE),
             2, 28, 4, 7, 128, 16, 64, 16, 256, f32(0.1), ops.PA_BF16, f32(0.5), f32(0.5), 0,
             vp(FAKE), ctypes.c_size_t(1 << 30), vp(0)) == INVALID


def test_decode_kernel_choice(lib):
    """Which family serves a shape, under each selection setting (host only)."""
    f = lib.pa_decode_kernel
    MFMA, GEN = 2, 1
    assert f(128, 16, 7, ops.PA_BF16) == MFMA
    assert f(64, 64, 16, ops.PA_F16) == MFMA
    assert f(128, 8, 7, ops.PA_BF16) == MFMA
    assert f(256, 16, 7, ops.PA_BF16) == MFMA
    # groups beyond one pass: the fewest passes of <= 32 heads (<= 16 at
    # head_dim 256), the last holding the remainder -- every bf16/f16 group
    assert f(128, 16, 64, ops.PA_BF16) == MFMA
    assert f(64, 16, 48, ops.PA_F16) == MFMA
    assert f(256, 16, 32, ops.PA_BF16) == MFMA
    assert f(128, 16, 37, ops.PA_BF16) == MFMA       # passes of 19 and 18
    assert f(128, 16, 160, ops.PA_BF16) == MFMA      # 5 passes of 32
    assert f(256, 16, 17, ops.PA_BF16) == MFMA       # passes of 9 and 8
    assert f(256, 8, 257, ops.PA_F16) == MFMA        # 17 passes of 16, the last of 1
    assert f(128, 16, 17, ops.PA_BF16) == MFMA       # groups of 17..32: two column tiles
    assert f(64, 8, 32, ops.PA_F16) == MFMA
    assert f(128, 16, 33, ops.PA_BF16) == MFMA       # passes of 17 and 16
    assert f(256, 16, 18, ops.PA_BF16) == MFMA       # two passes of 9 at head_dim 256
    assert f(128, 16, 7, ops.PA_F32) == MFMA         # float32 rows: 16x16x4 f32 MFMA
    assert f(64, 8, 16, ops.PA_F32) == MFMA
    assert f(128, 16, 17, ops.PA_F32) == MFMA        # passes of 9 and 8 (16 columns)
    assert f(256, 16, 7, ops.PA_F32) == GEN          # head_dim 256: vector ALU
    assert f(96, 16, 7, ops.PA_BF16) == UNSUPPORTED
    assert f(128, 16, 0, ops.PA_BF16) == INVALID
    assert f(128, 16, 7, 9) == INVALID
    prev = lib.pa_debug_select_kernel(1)
    try:
        assert f(128, 16, 7, ops.PA_BF16) == GEN
        lib.pa_debug_select_kernel(2)
        assert f(128, 16, 7, ops.PA_BF16) == MFMA
        assert f(128, 8, 37, ops.PA_BF16) == MFMA
        assert f(256, 8, 7, ops.PA_F32) == UNSUPPORTED      # f32 at 256: vector-ALU only
    finally:
        lib.pa_debug_select_kernel(prev)


def test_select_kernel_validates(lib):
    assert lib.pa_debug_select_kernel(5) == INVALID
    prev = lib.pa_debug_select_kernel(1)
    assert lib.pa_debug_select_kernel(prev) == 1


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(2, 4, 64)
    kc = torch.zeros(8, 2, 16, 64)
    with pytest.raises(ValueError):
        ops.paged_attention_decode(q, kc, kc, torch.zeros(2, 1, dtype=torch.int32),
                                   torch.zeros(2, dtype=torch.int32))


def test_8bit_bindings_refuse_cpu_tensors():
    """Every 8-bit binding checks its tensors before calling the library: host
    tensors are refused on a machine without a GPU as on one with it."""
    import torch
    q = torch.zeros(2, 4, 64, dtype=torch.bfloat16)
    bt, cl = torch.zeros(2, 1, dtype=torch.int32), torch.zeros(2, dtype=torch.int32)
    kv = torch.zeros(2, 2, 64, dtype=torch.bfloat16)
    slots = torch.zeros(2, dtype=torch.int64)
    for fmt, dt in (("fp8", torch.uint8), ("i8", torch.int8)):
        kc = torch.zeros(8, 2, 16, 64, dtype=dt)
        with pytest.raises(ValueError):
            getattr(ops, "paged_attention_decode_" + fmt)(q, kc, kc, bt, cl, 1.0, 1.0)
        with pytest.raises(ValueError):
            getattr(ops, "decode_append_" + fmt)(q, kv, kv, kc, kc, bt, cl, 1.0, 1.0)
        with pytest.raises(ValueError):
            getattr(ops, "reshape_and_cache_" + fmt)(kv, kv, kc, kc, slots, 1.0, 1.0)
