// Cache write, block copy and the debug gather: pure 16-byte copies,
// bit-exact for every dtype (they move bytes, never values).
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kCopyThreads = 256;

// Token i, KV head h, 16-byte column c:  key[i, h, c] -> key_cache[pb, h, off, c]
// with pb = slot / block_size, off = slot % block_size ([MiniPaged-Qwen] §8.1
// linear slot of an appended token; §8.2 pool layout).  Negative slots are
// padding; slots past the pool are dropped, never written out of bounds.
__global__ __launch_bounds__(kCopyThreads) void reshape_and_cache_kernel(
    const char* __restrict__ key, const char* __restrict__ value, char* key_cache,
    char* value_cache, const int64_t* __restrict__ slots, int num_tokens, int num_kv_heads,
    int row_bytes, int block_size, int num_blocks) {
    const int cols = row_bytes / 16;
    const uint64_t total = (uint64_t)num_tokens * num_kv_heads * cols;
    const uint64_t idx = (uint64_t)blockIdx.x * kCopyThreads + threadIdx.x;
    if (idx >= total) return;
    const int c = (int)(idx % cols);
    const uint64_t th = idx / cols;              // token * H_kv + h
    const int h = (int)(th % num_kv_heads);
    const uint64_t i = th / num_kv_heads;
    // the row loads do not depend on the slot: issue all three together
    const uint64_t src = th * row_bytes + c * 16;
    const u32x4 kv = load16(key + src);
    const u32x4 vv = load16(value + src);
    const int64_t slot = slots[i];
    if (slot < 0 || slot >= (int64_t)num_blocks * block_size) return;
    const int pb = (int)(slot / block_size);
    const int off = (int)(slot - (int64_t)pb * block_size);
    const uint64_t dst = kv_row(pb, h, off, num_kv_heads, block_size) * row_bytes + c * 16;
    *reinterpret_cast<u32x4*>(key_cache + dst) = kv;
    *reinterpret_cast<u32x4*>(value_cache + dst) = vv;
}

// Cache write into 8-bit caches: 8 consecutive values of token i, KV head h
// (column group c) -> 8 codes at key_cache[pb, h, off, 8c .. +8], each
// Q(fp32(x) * inv_scale) with Q = OCP FP8 E4M3 (kI8 false) or INT8 (kI8
// true) -- the quantised form of the cache write above, with one scale per
// cache.
template <typename Tag>
__device__ __forceinline__ void load8_f32(const char* src, float* f) {
    if constexpr (Tag::kBytes == 4) {
        to_float(Tag(), load16(src), f);
        to_float(Tag(), load16(src + 16), f + 4);
    } else {
        to_float(Tag(), load16(src), f);
    }
}

template <typename Tag, bool kI8>
__global__ __launch_bounds__(kCopyThreads) void reshape_and_cache_q8_kernel(
    const char* __restrict__ key, const char* __restrict__ value, uint8_t* key_cache,
    uint8_t* value_cache, const int64_t* __restrict__ slots, int num_tokens, int num_kv_heads,
    int head_dim, int block_size, int num_blocks, float k_inv, float v_inv) {
    const int cols = head_dim / 8;
    const uint64_t total = (uint64_t)num_tokens * num_kv_heads * cols;
    const uint64_t idx = (uint64_t)blockIdx.x * kCopyThreads + threadIdx.x;
    if (idx >= total) return;
    const int c = (int)(idx % cols);
    const uint64_t th = idx / cols;              // token * H_kv + h
    const int h = (int)(th % num_kv_heads);
    const uint64_t i = th / num_kv_heads;
    const uint64_t src = (th * head_dim + 8 * c) * Tag::kBytes;
    float fk[8], fv[8];
    load8_f32<Tag>(key + src, fk);
    load8_f32<Tag>(value + src, fv);
    const int64_t slot = slots[i];
    if (slot < 0 || slot >= (int64_t)num_blocks * block_size) return;
    const int pb = (int)(slot / block_size);
    const int off = (int)(slot - (int64_t)pb * block_size);
    uint32_t ck[8], cv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        ck[e] = kI8 ? i8_encode(fk[e] * k_inv) : e4m3_encode(fk[e] * k_inv);
        cv[e] = kI8 ? i8_encode(fv[e] * v_inv) : e4m3_encode(fv[e] * v_inv);
    }
    const uint64_t dst = kv_row(pb, h, off, num_kv_heads, block_size) * head_dim + 8 * c;
    *reinterpret_cast<u32x2*>(key_cache + dst) =
        (u32x2){ck[0] | ck[1] << 8 | ck[2] << 16 | ck[3] << 24,
                ck[4] | ck[5] << 8 | ck[6] << 16 | ck[7] << 24};
    *reinterpret_cast<u32x2*>(value_cache + dst) =
        (u32x2){cv[0] | cv[1] << 8 | cv[2] << 16 | cv[3] << 24,
                cv[4] | cv[5] << 8 | cv[6] << 16 | cv[7] << 24};
}

// Verify mode's row map (verify_row) of every query row, for the kernels
// that read it from memory (the fixed schedule and the vector-ALU kernel;
// the balanced schedule computes it in its own prologue).  Every row is
// written on every call.
__global__ __launch_bounds__(kCopyThreads) void verify_rows_kernel(
    const int32_t* __restrict__ query_start, const int32_t* __restrict__ context_lens,
    int num_seqs, int total_queries, int max_query_len, int max_context_len, int u,
    int32_t* table_rows, int32_t* lens, int32_t* row_tokens) {
    const int r = blockIdx.x * kCopyThreads + threadIdx.x;
    if (r >= total_queries) return;
    const VerifyRow v = verify_row([=](int i) { return query_start[i]; },
                                   [=](int i) { return context_lens[i]; }, num_seqs,
                                   max_query_len, max_context_len, u, r);
    table_rows[r] = v.table_row;
    lens[r] = v.len;
    row_tokens[r] = v.ntok;
}

// Sequence b's newest token (history position L_b - 1): key[b, h, c] ->
// key_cache[pb, h, off, c] with pb = block_tables[b, (L_b-1) / block_size],
// off = (L_b-1) % block_size -- the append step of [MiniPaged-Qwen] §8.1 with
// the slot taken from the table.  Empty or invalid lengths and table entries
// outside the pool write nothing.
__global__ __launch_bounds__(kCopyThreads) void append_tokens_kernel(
    const char* __restrict__ key, const char* __restrict__ value, char* key_cache,
    char* value_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ context_lens, int num_seqs, int num_kv_heads, int row_bytes,
    int block_size, int num_blocks, int max_blocks_per_seq, int max_context_len) {
    const int cols = row_bytes / 16;
    const uint64_t total = (uint64_t)num_seqs * num_kv_heads * cols;
    const uint64_t idx = (uint64_t)blockIdx.x * kCopyThreads + threadIdx.x;
    if (idx >= total) return;
    const int c = (int)(idx % cols);
    const uint64_t th = idx / cols;              // sequence * H_kv + h
    const int h = (int)(th % num_kv_heads);
    const uint64_t b = th / num_kv_heads;
    const uint64_t src = th * row_bytes + c * 16;
    const u32x4 kv = load16(key + src);
    const u32x4 vv = load16(value + src);
    const int L = context_lens[b];
    if (L <= 0 || L > max_context_len) return;
    const int pos = L - 1;
    const int pb = block_tables[b * max_blocks_per_seq + pos / block_size];
    if ((unsigned)pb >= (unsigned)num_blocks) return;
    const uint64_t dst = kv_row(pb, h, pos % block_size, num_kv_heads, block_size) * row_bytes + c * 16;
    *reinterpret_cast<u32x4*>(key_cache + dst) = kv;
    *reinterpret_cast<u32x4*>(value_cache + dst) = vv;
}

// Block copy for copy-on-write: 16-byte column c of pair i's block slab
// (num_kv_heads * block_size * head_dim elements, contiguous in the
// [N, H_kv, BS, D] layout), for the key cache (blockIdx.y = 0) or the value
// cache (blockIdx.y = 1).  Pairs with an index outside the pool, or with
// src == dst, are skipped.
__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(
    char* key_cache, char* value_cache, const int32_t* __restrict__ pairs, int num_pairs,
    int block_bytes, int num_blocks) {
    const int cols = block_bytes / 16;
    const uint64_t idx = (uint64_t)blockIdx.x * kCopyThreads + threadIdx.x;
    if (idx >= (uint64_t)num_pairs * cols) return;
    const int i = (int)(idx / cols);
    const int c = (int)(idx - (uint64_t)i * cols);
    const int src = pairs[2 * i];
    const int dst = pairs[2 * i + 1];
    if ((unsigned)src >= (unsigned)num_blocks || (unsigned)dst >= (unsigned)num_blocks ||
        src == dst)
        return;
    char* base = blockIdx.y == 0 ? key_cache : value_cache;
    const u32x4 v = load16(base + (uint64_t)src * block_bytes + c * 16);
    *reinterpret_cast<u32x4*>(base + (uint64_t)dst * block_bytes + c * 16) = v;
}

// History row t of sequence `seq`, KV head h -> k_out[h, t, :], through the
// decode kernels' address function.
__global__ __launch_bounds__(kCopyThreads) void gather_kernel(
    char* k_out, char* v_out, const char* key_cache, const char* value_cache,
    const int32_t* block_tables, const int32_t* context_lens, int seq, int num_kv_heads,
    int row_bytes, int block_size, int num_blocks, int max_blocks_per_seq,
    int max_context_len) {
    const int cols = row_bytes / 16;
    const int h = blockIdx.y;
    const uint64_t idx = (uint64_t)blockIdx.x * kCopyThreads + threadIdx.x;
    const int t = (int)(idx / cols);
    const int c = (int)(idx % cols);
    int L = context_lens[seq];
    L = L < 0 ? 0 : (L > max_context_len ? max_context_len : L);
    if (t >= L) return;
    const int pb = block_tables[(uint64_t)seq * max_blocks_per_seq + t / block_size];
    const uint64_t dst = ((uint64_t)h * max_context_len + t) * row_bytes + c * 16;
    if ((unsigned)pb >= (unsigned)num_blocks) {
        const u32x4 ones = {~0u, ~0u, ~0u, ~0u};
        *reinterpret_cast<u32x4*>(k_out + dst) = ones;
        *reinterpret_cast<u32x4*>(v_out + dst) = ones;
        return;
    }
    const uint64_t src = kv_row(pb, h, t % block_size, num_kv_heads, block_size) * row_bytes + c * 16;
    *reinterpret_cast<u32x4*>(k_out + dst) = load16(key_cache + src);
    *reinterpret_cast<u32x4*>(v_out + dst) = load16(value_cache + src);
}

}  // namespace

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* key_cache,
                                    void* value_cache, const int64_t* slots, int num_tokens,
                                    int num_kv_heads, int row_bytes, int block_size,
                                    int num_blocks, hipStream_t s) {
    const uint64_t total = (uint64_t)num_tokens * num_kv_heads * (row_bytes / 16);
    if (total == 0) return hipSuccess;
    const unsigned grid = (unsigned)((total + kCopyThreads - 1) / kCopyThreads);
    hipLaunchKernelGGL(reshape_and_cache_kernel, dim3(grid), dim3(kCopyThreads), 0, s,
                       static_cast<const char*>(key), static_cast<const char*>(value),
                       static_cast<char*>(key_cache), static_cast<char*>(value_cache), slots,
                       num_tokens, num_kv_heads, row_bytes, block_size, num_blocks);
    return hipGetLastError();
}

hipError_t launch_reshape_and_cache_q8(const void* key, const void* value, void* key_cache,
                                       void* value_cache, const int64_t* slots, int num_tokens,
                                       int num_kv_heads, int head_dim, int block_size,
                                       int num_blocks, pa_dtype src_dtype, bool int8,
                                       float k_inv_scale, float v_inv_scale, hipStream_t s) {
    const uint64_t total = (uint64_t)num_tokens * num_kv_heads * (head_dim / 8);
    if (total == 0) return hipSuccess;
    const unsigned grid = (unsigned)((total + kCopyThreads - 1) / kCopyThreads);
    auto go = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, dim3(grid), dim3(kCopyThreads), 0, s,
                           static_cast<const char*>(key), static_cast<const char*>(value),
                           static_cast<uint8_t*>(key_cache), static_cast<uint8_t*>(value_cache),
                           slots, num_tokens, num_kv_heads, head_dim, block_size, num_blocks,
                           k_inv_scale, v_inv_scale);
    };
    switch (src_dtype) {
        case PA_F32:
            int8 ? go(reshape_and_cache_q8_kernel<F32, true>)
                 : go(reshape_and_cache_q8_kernel<F32, false>);
            break;
        case PA_F16:
            int8 ? go(reshape_and_cache_q8_kernel<F16, true>)
                 : go(reshape_and_cache_q8_kernel<F16, false>);
            break;
        default:
            int8 ? go(reshape_and_cache_q8_kernel<BF16, true>)
                 : go(reshape_and_cache_q8_kernel<BF16, false>);
            break;
    }
    return hipGetLastError();
}

hipError_t launch_verify_rows(const int32_t* query_start, const int32_t* context_lens,
                              int num_seqs, int total_queries, int max_query_len,
                              int max_context_len, int tokens_per_row, int32_t* table_rows,
                              int32_t* lens, int32_t* row_tokens, hipStream_t s) {
    if (total_queries == 0) return hipSuccess;
    if (tokens_per_row < 1) return hipErrorInvalidValue;
    const unsigned grid = (unsigned)((total_queries + kCopyThreads - 1) / kCopyThreads);
    hipLaunchKernelGGL(verify_rows_kernel, dim3(grid), dim3(kCopyThreads), 0, s, query_start,
                       context_lens, num_seqs, total_queries, max_query_len, max_context_len,
                       tokens_per_row, table_rows, lens, row_tokens);
    return hipGetLastError();
}

hipError_t launch_append_tokens(const void* key, const void* value, void* key_cache,
                                void* value_cache, const int32_t* block_tables,
                                const int32_t* context_lens, int num_seqs, int num_kv_heads,
                                int row_bytes, int block_size, int num_blocks,
                                int max_blocks_per_seq, int max_context_len, hipStream_t s) {
    const uint64_t total = (uint64_t)num_seqs * num_kv_heads * (row_bytes / 16);
    if (total == 0) return hipSuccess;
    const unsigned grid = (unsigned)((total + kCopyThreads - 1) / kCopyThreads);
    hipLaunchKernelGGL(append_tokens_kernel, dim3(grid), dim3(kCopyThreads), 0, s,
                       static_cast<const char*>(key), static_cast<const char*>(value),
                       static_cast<char*>(key_cache), static_cast<char*>(value_cache),
                       block_tables, context_lens, num_seqs, num_kv_heads, row_bytes, block_size,
                       num_blocks, max_blocks_per_seq, max_context_len);
    return hipGetLastError();
}

hipError_t launch_copy_blocks(void* key_cache, void* value_cache, const int32_t* pairs,
                              int num_pairs, int block_bytes, int num_blocks, hipStream_t s) {
    const uint64_t total = (uint64_t)num_pairs * (block_bytes / 16);
    if (total == 0) return hipSuccess;
    dim3 grid((unsigned)((total + kCopyThreads - 1) / kCopyThreads), 2);
    hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(kCopyThreads), 0, s,
                       static_cast<char*>(key_cache), static_cast<char*>(value_cache), pairs,
                       num_pairs, block_bytes, num_blocks);
    return hipGetLastError();
}

hipError_t launch_gather(void* k_out, void* v_out, const void* key_cache,
                         const void* value_cache, const int32_t* block_tables,
                         const int32_t* context_lens, int seq, int num_kv_heads,
                         int row_bytes, int block_size, int num_blocks,
                         int max_blocks_per_seq, int max_context_len, hipStream_t s) {
    const uint64_t per_head = (uint64_t)max_context_len * (row_bytes / 16);
    if (per_head == 0) return hipSuccess;
    dim3 grid((unsigned)((per_head + kCopyThreads - 1) / kCopyThreads), num_kv_heads);
    hipLaunchKernelGGL(gather_kernel, grid, dim3(kCopyThreads), 0, s, static_cast<char*>(k_out),
                       static_cast<char*>(v_out), static_cast<const char*>(key_cache),
                       static_cast<const char*>(value_cache), block_tables, context_lens, seq,
                       num_kv_heads, row_bytes, block_size, num_blocks, max_blocks_per_seq,
                       max_context_len);
    return hipGetLastError();
}

}  // namespace pa
