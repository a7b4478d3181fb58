"""Oracle of the 8-bit floating-point KV cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name a quantised KV cache as the lever once KV memory binds
([KV-principles] §3.3: K and V stored in fewer bits, INT8 or INT4, at some
accuracy cost; its tuning Q&A names an FP8 KV cache; [vLLM-paging] "Kernel
metadata" lists the KV dtype and quantisation scales among what a kernel
must be told explicitly).  They fix neither the format nor the scale
granularity.  Reading taken here:

* codes are OCP FP8 E4M3 ("e4m3fn"): sign, 4 exponent bits (bias 7),
  3 mantissa bits; no infinities; S.1111.111 is NaN; largest finite 448;
  subnormals m * 2^-9;
* one scale per cache tensor (k_scale for keys, v_scale for values), passed
  with every call: the stored code of x is E4M3(fp32(x) * fp32(1 / scale)),
  and the value a code stands for is decode(code) * scale;
* E4M3(y) rounds y to the nearest representable value, ties to the even
  code, and saturates to +-448 when |y| exceeds 448 (no NaN from overflow);
  NaN stays NaN.

The decode on an FP8 cache is then the plain decode (paged_attention) on the
dequantised caches, computed in float64.
"""

import numpy as np

MAX_E4M3 = 448.0
NAN_CODE = 0x7F


def e4m3_decode(codes):
    """float64 value of each E4M3 code (uint8 array)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = m * 2.0 ** -9
    v = sign * np.where(e == 0, sub, normal)
    return np.where((e == 15) & ((c & 7) == 7), np.nan, v)


# the non-negative finite values and their codes, in increasing order
_POS_CODES = np.arange(0, 0x7F, dtype=np.uint8)          # 0x00 .. 0x7E
_POS_VALUES = e4m3_decode(_POS_CODES)


def e4m3_encode(y):
    """Codes of float32 values y: nearest representable value, ties to the
    even code, saturating to +-448; NaN -> 0x7F."""
    y = np.asarray(y, dtype=np.float32).astype(np.float64)
    a = np.abs(y)
    # index of the largest value <= a (a >= 0), then compare with the next
    lo = np.searchsorted(_POS_VALUES, np.minimum(a, MAX_E4M3), side="right") - 1
    lo = np.clip(lo, 0, len(_POS_VALUES) - 1)
    hi = np.minimum(lo + 1, len(_POS_VALUES) - 1)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi != lo) & (_POS_CODES[lo] % 2 == 1))
    code = np.where(take_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.int64)
    code = np.where(a >= MAX_E4M3, 0x7E, code)
    code = np.where(np.signbit(y), code | 0x80, code)
    code = np.where(np.isnan(y), NAN_CODE, code)
    return code.astype(np.uint8)


def inverse_scale(scale):
    """The float32 multiplier the encoder applies: fp32(1 / scale)."""
    return np.float32(1.0 / float(scale))


def quantize(x, scale):
    """E4M3 codes of fp32(x) * fp32(1 / scale) (x: float32-exact values)."""
    with np.errstate(over="ignore", invalid="ignore"):      # inf/NaN inputs are legal
        prod = np.asarray(x, dtype=np.float32) * inverse_scale(scale)   # one fp32 rounding
    return e4m3_encode(prod.astype(np.float32))


def dequantize(codes, scale):
    return e4m3_decode(codes) * float(scale)


def reshape_and_cache_fp8(key, value, key_cache, value_cache, slot_mapping, k_scale, v_scale):
    """The cache write of [MiniPaged-Qwen] §8.1-8.2 into E4M3 caches: token i's
    quantised rows go to slot s = slot_mapping[i] (s < 0 skipped).  key, value:
    float32-exact arrays [T, H_kv, D]; caches: uint8 [N, H_kv, BS, D]."""
    kc = np.array(key_cache, dtype=np.uint8, copy=True)
    vc = np.array(value_cache, dtype=np.uint8, copy=True)
    BS = kc.shape[2]
    qk = quantize(key, k_scale)
    qv = quantize(value, v_scale)
    for i, s in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if s < 0:
            continue
        kc[s // BS, :, s % BS, :] = qk[i]
        vc[s // BS, :, s % BS, :] = qv[i]
    return kc, vc
