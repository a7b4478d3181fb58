// Device-side helpers shared by the kernels of libpagedattn.so: element
// conversions, 16-byte vector loads and the paged-cache address function.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// Row index (in units of head_dim elements) of token slot `off` of physical
// block `pb`, KV head `kvh`, in a [num_blocks, num_kv_heads, block_size,
// head_dim] pool: key_cache[pb, kvh, off, :] of [MiniPaged-Qwen] §8.2, the
// last step of the position -> block -> slot translation of §6.2.  64-bit so
// pools beyond 4 GiB address correctly.
__device__ __forceinline__ uint64_t kv_row(int pb, int kvh, int off,
                                           int num_kv_heads, int block_size) {
    return ((uint64_t)(uint32_t)pb * (uint32_t)num_kv_heads + (uint32_t)kvh) *
               (uint32_t)block_size + (uint32_t)off;
}

// ---- element types -------------------------------------------------------
// Tags for the three storage types; 16-bit types travel as raw bits.
struct F32 {
    static constexpr int kBytes = 4;
};
struct F16 {
    static constexpr int kBytes = 2;
};
struct BF16 {
    static constexpr int kBytes = 2;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// Two float32 -> two 16-bit values packed in one dword (low = a), rounded to
// nearest even.
__device__ __forceinline__ uint32_t pack2(BF16, float a, float b) {
    bf16x2 v = __builtin_convertvector((f32x2){a, b}, bf16x2);
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint32_t pack2(F16, float a, float b) {
    f16x2 v = __builtin_convertvector((f32x2){a, b}, f16x2);
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float unpack_lo(BF16, uint32_t w) { return bf16_lo(w); }
__device__ __forceinline__ float unpack_hi(BF16, uint32_t w) { return bf16_hi(w); }
__device__ __forceinline__ float unpack_lo(F16, uint32_t w) { return f16_lo(w); }
__device__ __forceinline__ float unpack_hi(F16, uint32_t w) { return f16_hi(w); }

// Store one float32 as the storage type (round to nearest even).
__device__ __forceinline__ void store_elem(F32, void* base, uint64_t i, float v) {
    reinterpret_cast<float*>(base)[i] = v;
}
__device__ __forceinline__ void store_elem(BF16, void* base, uint64_t i, float v) {
    reinterpret_cast<__bf16*>(base)[i] = (__bf16)v;
}
__device__ __forceinline__ void store_elem(F16, void* base, uint64_t i, float v) {
    reinterpret_cast<_Float16*>(base)[i] = (_Float16)v;
}

// Store four float32 as elements i .. i + 3 of the storage type in one
// instruction (i a multiple of 4; base 16-byte aligned).
__device__ __forceinline__ void store4(F32, void* base, uint64_t i, f32x4 v) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(base) + i) = v;
}
template <typename Tag>
__device__ __forceinline__ void store4(Tag t, void* base, uint64_t i, f32x4 v) {
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(base) + i) =
        (u32x2){pack2(t, v[0], v[1]), pack2(t, v[2], v[3])};
}

// OCP FP8 E4M3 code of a float32 (sign, 4 exponent bits of bias 7, 3
// mantissa bits; no infinities; 0x7F is NaN; largest finite 448): nearest
// representable value, ties to the even code, saturating to +-448.
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
    const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
    const float a = fabsf(y);
    if (!(a == a)) return 0x7Fu;                       // NaN
    uint32_t code;
    if (a >= 448.0f) {
        code = 0x7Eu;
    } else if (a < 0.015625f) {
        // below the least normal 2^-6: multiples of 2^-9 (8 is 2^-6 itself)
        code = (uint32_t)__builtin_rintf(a * 512.0f);
    } else {
        // keep 3 mantissa bits, rounding the 20 dropped ones to nearest even;
        // exponent bias 127 -> 7
        const uint32_t u = __float_as_uint(a);
        code = ((u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20) - (120u << 3);
        if (code > 0x7Eu) code = 0x7Eu;
    }
    return code | sign;
}

// Signed 8-bit code (two's complement byte) of a float32: the nearest
// integer, ties to the even one, saturated to +-127; NaN, which no integer
// code holds, is stored as 0.
__device__ __forceinline__ uint32_t i8_encode(float y) {
    if (y != y) return 0u;
    const float r = __builtin_rintf(fminf(fmaxf(y, -127.0f), 127.0f));
    return (uint32_t)(int)r & 0xFFu;
}

// 16 bytes -> float32 values (4 for F32, 8 for the 16-bit types).
__device__ __forceinline__ void to_float(F32, u32x4 w, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
}
__device__ __forceinline__ void to_float(BF16, u32x4 w, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf16_lo(w[i]);
        f[2 * i + 1] = bf16_hi(w[i]);
    }
}
__device__ __forceinline__ void to_float(F16, u32x4 w, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = f16_lo(w[i]);
        f[2 * i + 1] = f16_hi(w[i]);
    }
}

__device__ __forceinline__ u32x4 load16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

// exp2 on the hardware transcendental unit; exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Weight of a partial state with running max m against the merged max M,
// 0 for an empty state (m = -inf).
__device__ __forceinline__ float rescale_weight(float m, float M) {
    return m == -INFINITY ? 0.0f : fast_exp2(m - M);
}

// Verify mode's row map, for query row r: the sequence b with qs[b] <= r <
// qs[b + 1] (qs: query_start, nsrc + 1 entries, in LDS or global memory) is
// found by binary search; its token i = r - qs[b] of q_b sits at history
// position L_b - q_b + i (L_b = lens(b)).  Rows are grouped u at a time: the
// row at a group's start carries n = min(u, q_b - i) query rows and the
// length of its last one, L_b - q_b + i + n; the group's other rows carry
// none (length 0).  A row whose sequence cannot be found, whose q_b exceeds
// max_query_len or L_b, or whose L_b is invalid carries itself with length
// -1 (a NaN row) and table row 0.
struct VerifyRow {
    int table_row;   // block-table row
    int len;         // history length the decode row attends (its last row's)
    int ntok;        // query rows it carries
};

template <typename QS, typename Lens>
__device__ __forceinline__ VerifyRow verify_row(QS qs, Lens lens, int nsrc, int max_query_len,
                                                int max_context_len, int u, int r) {
    int lo = 0, hi = nsrc - 1;   // largest b with qs[b] <= r
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (qs(mid) <= r) lo = mid; else hi = mid - 1;
    }
    const int b = lo;
    const int q0 = qs(b);
    const int q1 = qs(b + 1);
    const int L = lens(b);
    const int qb = q1 - q0;
    const bool ok = q0 <= r && r < q1 && qb <= max_query_len && L >= qb && L <= max_context_len;
    const int i = r - q0;
    const int n = !ok ? 1 : i % u == 0 ? min(u, qb - i) : 0;
    return VerifyRow{ok ? b : 0, !ok ? -1 : n > 0 ? L - qb + i + n : 0, n};
}

}  // namespace pa
