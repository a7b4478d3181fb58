"""Pins of the INT8 KV-cache oracle: the code's definition (two's complement
bytes), exhaustive round trips, PyTorch's round-half-to-even (a library
special case) over every bf16 bit pattern, brute-force nearest integers,
ties and saturation, and the cache write."""

import numpy as np
import torch

from oracle import int8


def torch_codes(x):
    """round half to even, clamp, two's complement byte (torch.round rounds
    halves to even)."""
    t = torch.from_numpy(np.asarray(x, dtype=np.float32)).double()
    t = torch.nan_to_num(t, nan=0.0).clamp(-127.0, 127.0)
    return torch.round(t).to(torch.int64).to(torch.int8).view(torch.uint8).numpy()


def test_decode_is_twos_complement():
    c = np.arange(256, dtype=np.uint8)
    want = c.view(np.int8).astype(np.float64)
    assert np.array_equal(int8.i8_decode(c), want)


def test_every_code_but_minus_128_round_trips():
    c = np.array([x for x in range(256) if x != 0x80], dtype=np.uint8)
    assert np.array_equal(int8.i8_encode(int8.i8_decode(c).astype(np.float32)), c)


def test_encode_matches_torch_round_on_every_bf16_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    x = bits.view(np.float32)
    x = x[~np.isnan(x)]
    assert np.array_equal(int8.i8_encode(x), torch_codes(x))


def test_ties_go_to_the_even_integer():
    k = np.arange(-127, 127)
    mids = (k + 0.5).astype(np.float32)
    codes = int8.i8_decode(int8.i8_encode(mids)).astype(int)
    assert np.array_equal(codes, np.where(k % 2 == 0, k, k + 1))


def test_saturation_and_specials():
    enc = int8.i8_encode
    assert enc([127.0, 127.4, 127.5, 128.0, 1e30, np.inf]).tolist() == [127] * 6
    assert enc([-127.0, -127.5, -128.0, -1e30, -np.inf]).tolist() == [0x81] * 5
    assert enc([np.nan, 0.0, -0.0, 0.49, -0.49]).tolist() == [0] * 5
    assert enc([0.51, -0.51]).tolist() == [1, 0xFF]


def test_brute_force_nearest():
    ks = np.arange(-127, 128, dtype=np.float64)
    rng = np.random.default_rng(1)
    x = rng.uniform(-126.9, 126.9, 5000).astype(np.float32)
    for xi, c in zip(x, int8.i8_decode(int8.i8_encode(x))):
        d = np.abs(ks - float(xi))
        best = ks[d == d.min()]
        assert c in best and (len(best) == 1 or c % 2 == 0)


def test_quantize_is_one_fp32_product_then_round():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(10000).astype(np.float32)
    for scale in (1.0, 0.037, 3.5, 1 / 127):
        inv = np.float32(1.0 / scale)
        assert np.array_equal(int8.quantize(x, scale), int8.i8_encode(x * inv))
    # error of the round trip inside the range: at most half a code step
    y = int8.dequantize(int8.quantize(x, 0.05), 0.05)
    inside = np.abs(x) <= 0.05 * 126
    assert np.all(np.abs(y - x)[inside] <= 0.025 * (1 + 1e-6))


def test_int8_cache_write_round_trip():
    rng = np.random.default_rng(3)
    T, H_kv, D, N, BS = 5, 2, 16, 6, 4
    k = rng.standard_normal((T, H_kv, D)).astype(np.float32)
    v = rng.standard_normal((T, H_kv, D)).astype(np.float32)
    kc = np.full((N, H_kv, BS, D), 0x80, np.uint8)
    vc = kc.copy()
    slots = np.array([0, 7, -1, 22, 13])
    k2, v2 = int8.reshape_and_cache_i8(k, v, kc, vc, slots, 0.02, 0.03)
    for i, s in enumerate(slots):
        if s < 0:
            continue
        assert np.array_equal(k2[s // BS, :, s % BS], int8.quantize(k[i], 0.02))
        assert np.array_equal(v2[s // BS, :, s % BS], int8.quantize(v[i], 0.03))
    written = {(s // BS, s % BS) for s in slots if s >= 0}
    for b in range(N):
        for o in range(BS):
            if (b, o) not in written:
                assert np.all(k2[b, :, o] == 0x80) and np.all(v2[b, :, o] == 0x80)
