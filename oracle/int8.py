"""Oracle of the 8-bit integer KV cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages' own example of a quantised KV cache is INT8 (or INT4) K and V in
place of FP16, half (a quarter) of the memory at a small accuracy cost
([KV-principles] §3.3); [vLLM-paging] "Kernel metadata" lists the
quantisation scales among what a kernel must be told explicitly.  They fix
neither the code range, the rounding nor the scale granularity.  Reading
taken here (the plain symmetric scheme, with the same scale handling as the
FP8 cache in fp8.py):

* codes are signed 8-bit integers (two's complement bytes) in [-127, 127];
  -128 is never written, so the range is symmetric (a stored -128 still
  reads as -128);
* one scale per cache tensor (k_scale for keys, v_scale for values), passed
  with every call: the stored code of x is Q(fp32(x) * fp32(1 / scale)), and
  a code c stands for c * scale;
* Q(y) is y rounded to the nearest integer, ties to the even integer,
  saturated to [-127, 127] (infinities too); NaN, which no integer code can
  hold, is stored as 0.

The decode on an INT8 cache is then the plain decode (paged_attention) on the
dequantised caches, computed in float64.
"""

import numpy as np

MAX_I8 = 127


def i8_decode(codes):
    """float64 integer value of each code (uint8 array of two's complement
    bytes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    return np.where(c >= 128, c - 256, c).astype(np.float64)


def i8_encode(y):
    """Codes of float32 values y: the nearest integer, ties to the even one,
    saturated to +-127; NaN -> 0."""
    y = np.asarray(y, dtype=np.float32).astype(np.float64)
    a = np.minimum(np.abs(np.nan_to_num(y, nan=0.0)), float(MAX_I8))
    lo = np.floor(a)
    frac = a - lo
    up = (frac > 0.5) | ((frac == 0.5) & (lo % 2 == 1))
    k = (lo + up).astype(np.int64)                 # nearest integer to |y|, ties to even
    k = np.where(np.signbit(y) & ~np.isnan(y), -k, k)
    return (k & 0xFF).astype(np.uint8)


def inverse_scale(scale):
    """The float32 multiplier the encoder applies: fp32(1 / scale)."""
    return np.float32(1.0 / float(scale))


def quantize(x, scale):
    """INT8 codes of fp32(x) * fp32(1 / scale) (x: float32-exact values)."""
    with np.errstate(over="ignore", invalid="ignore"):      # inf/NaN inputs are legal
        prod = np.asarray(x, dtype=np.float32) * inverse_scale(scale)   # one fp32 rounding
    return i8_encode(prod.astype(np.float32))


def dequantize(codes, scale):
    return i8_decode(codes) * float(scale)


def reshape_and_cache_i8(key, value, key_cache, value_cache, slot_mapping, k_scale, v_scale):
    """The cache write of [MiniPaged-Qwen] §8.1-8.2 into INT8 caches: token i's
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
