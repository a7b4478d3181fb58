// Host side of libpagedattn.so: argument validation, partition sizing,
// workspace layout and kernel dispatch behind the C ABI of pagedattn.h.
#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>

#include "pa_internal.h"

namespace {

thread_local std::string g_last_error;
std::atomic<int> g_kernel_kind{pa::kAuto};

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

}  // namespace

int pa::report_error(int status, const char* msg) {
    g_last_error = msg;
    return status;
}

namespace {

int hip_fail(hipError_t e, const char* what) {
    return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(pa_dtype dt) {
    switch (dt) {
        case PA_F32: return 4;
        case PA_F16: return 2;
        case PA_BF16: return 2;
        default: return 0;
    }
}

int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Partition length heuristic.  Histories longer than one partition are
// reduced in parallel pieces and merged; the launch has
// num_seqs * num_kv_heads * ceil(max_context_len / P) workgroups (those past a
// sequence's own length exit at once).  Aim for >= 2048 launched workgroups
// (8 per compute unit) with partitions no shorter than 128 tokens, so each
// wavefront still streams at least one 32-token chunk.
int heuristic_partition(int num_seqs, int num_kv_heads, int block_size, int max_context_len) {
    const int unit = block_size > 32 ? block_size : 32;
    int P = 512;
    const int64_t pairs = (int64_t)num_seqs * num_kv_heads;
    while (P > 128 && pairs * ceil_div(max_context_len, P) < 2048) P /= 2;
    P = (P + unit - 1) / unit * unit;
    if (P > 64 * block_size) P = 64 * block_size;
    return P;
}

bool valid_partition(int P, int block_size) {
    return P > 0 && P % 32 == 0 && P % block_size == 0 && P <= 64 * block_size;
}

// A small call -- histories of at most 16 chunks (512 tokens) and at most
// 8192 (sequence, KV head pass, chunk) work items -- runs on the fixed
// schedule with one partition covering every history: one launch, no merge
// kernel, one workgroup per (sequence, KV head pass).  The balanced
// schedule's prologue, edge merge and merge launch cost more than such a
// call streams.  Measured (bf16, 28/4 heads, head_dim 128; balanced against
// one partition): 4 x 64-token histories 9.8 vs 3.4 us, 64 x U[32, 255]
// 12.5 vs 8.7, 256 x U[32, 255] 24.1 vs 22.2, 64 x U[256, 511] 17.2 vs
// 13.3; past the bounds the balanced schedule wins: 512 x U[32, 255] 37.2
// vs 38.3, 16 x U[768, 1023] 14.8 vs 18.4.  Returns that partition, or 0.
int small_call_partition(int num_seqs, int kv_passes, int block_size, int max_context_len) {
    const int chunks = ceil_div(max_context_len, pa::kChunk);
    if (max_context_len <= 0 || chunks > 16 ||
        (int64_t)num_seqs * kv_passes * chunks > 8192)
        return 0;
    const int unit = block_size > 32 ? block_size : 32;
    const int P = ceil_div(max_context_len, unit) * unit;
    return valid_partition(P, block_size) ? P : 0;
}

struct Layout {
    int part_len = 0;
    int num_parts = 0;
    size_t lse_off = 0, out_off = 0, meta_off = 0, bytes = 0;
};

// Fixed schedule: states [S, H, num_parts] (lse) and [S, H, num_parts, D].
Layout fixed_layout(int num_seqs, int num_heads, int head_dim, int max_context_len,
                    int part_len) {
    Layout l;
    l.part_len = part_len;
    l.num_parts = max_context_len > 0 ? ceil_div(max_context_len, part_len) : 1;
    if (l.num_parts <= 1) return l;   // single partition: no workspace
    const size_t rows = (size_t)num_seqs * num_heads * l.num_parts;
    l.lse_off = 0;
    l.out_off = align256(rows * sizeof(float));
    l.bytes = l.out_off + align256(rows * head_dim * sizeof(float));
    return l;
}

// Balanced schedule: two slots per workgroup of `cols` columns each (16, or
// 32 for verify rows with two column tiles), and one 16-byte record per
// workgroup.
Layout balanced_layout(int head_dim, int cols = pa::kMaxGroup) {
    Layout l;
    const size_t rows = (size_t)pa::kMaxBalancedWg * 2 * cols;
    l.lse_off = 0;
    l.out_off = align256(rows * sizeof(float));
    l.meta_off = l.out_off + align256(rows * head_dim * sizeof(float));
    l.bytes = l.meta_off + align256((size_t)pa::kMaxBalancedWg * 4 * sizeof(int));
    return l;
}

// Workgroups of the balanced schedule: pa::mfma_workgroups_per_cu per compute
// unit of the current device, all resident at once.
int balanced_workgroups(int head_dim) {
    // compute units per device, queried once (calls may come from any thread)
    static std::atomic<int> cached[64];
    int dev = 0;
    int cus = 256;
    if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64) {
        cus = cached[dev].load(std::memory_order_relaxed);
        if (cus == 0) {
            int n = 0;
            if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
                    hipSuccess || n <= 0)
                n = 256;
            cached[dev].store(n, std::memory_order_relaxed);
            cus = n;
        }
    }
    const int wgs = cus * pa::mfma_workgroups_per_cu(head_dim);
    return wgs > pa::kMaxBalancedWg ? pa::kMaxBalancedWg : wgs;
}

// Verify rows (several query rows of a sequence in one pass) run on the
// matrix-core kernel with 16-bit rows and a group it serves in one pass; the
// rest on the vector-ALU kernel.
bool verify_on_mfma(pa_dtype dt, int head_dim, int block_size, int group) {
    return dt != PA_F32 && pa::mfma_supported(dt, head_dim, block_size, group);
}

// The balanced schedule serves the matrix-core kernel when no partition
// size is forced, the prefix table of context lengths fits in LDS, its
// work-unit sums fit in 32 bits and there can be history to read.
bool use_balanced(bool mfma, int partition_size, int num_seqs, int max_context_len) {
    const int64_t units = (int64_t)num_seqs *
                          (pa::kMaxStartUnits + (int64_t)pa::kChunkUnits *
                                               (((int64_t)max_context_len + pa::kChunk - 1) / pa::kChunk));
    return mfma && partition_size == 0 && num_seqs <= pa::kMaxBalancedSeqs &&
           max_context_len > 0 && units <= INT32_MAX;
}

bool supported_shape(int head_dim, int block_size) {
    return (head_dim == 64 || head_dim == 128 || head_dim == 256) &&
           (block_size == 8 || block_size == 16 || block_size == 32 || block_size == 64);
}

}  // namespace

extern "C" {

int pa_version(void) { return 100; }

const char* pa_status_string(int status) {
    switch (status) {
        case PA_OK: return "ok";
        case PA_ERR_INVALID_ARG: return "invalid argument";
        case PA_ERR_UNSUPPORTED: return "unsupported configuration";
        case PA_ERR_WORKSPACE: return "workspace missing or too small";
        case PA_ERR_HIP: return "HIP runtime error";
        case PA_ERR_POOL_EXHAUSTED: return "KV pool exhausted";
        default: return "unknown status";
    }
}

const char* pa_last_error(void) { return g_last_error.c_str(); }

int pa_debug_select_kernel(int kind) {
    if (kind != pa::kAuto && kind != pa::kGeneric && kind != pa::kMfma)
        return fail(PA_ERR_INVALID_ARG, "kernel kind %d not in {0,1,2}", kind);
    return g_kernel_kind.exchange(kind);
}

int pa_decode_kernel(int head_dim, int block_size, int gqa_group_size, pa_dtype dtype) {
    if (elem_bytes(dtype) == 0 || gqa_group_size < 1)
        return fail(PA_ERR_INVALID_ARG, "unknown dtype %d or gqa_group_size %d < 1", (int)dtype,
                    gqa_group_size);
    if (!supported_shape(head_dim, block_size))
        return fail(PA_ERR_UNSUPPORTED, "head_dim %d with block_size %d not built", head_dim,
                    block_size);
    const int kind = g_kernel_kind.load();
    const bool mfma_ok = pa::mfma_split(dtype, head_dim, block_size, gqa_group_size) > 0;
    if (kind == pa::kMfma && !mfma_ok)
        return fail(PA_ERR_UNSUPPORTED, "matrix-core kernel selected but not built for this shape");
    return mfma_ok && kind != pa::kGeneric ? pa::kMfma : pa::kGeneric;
}

int pa_decode_partition_size(int num_seqs, int num_kv_heads, int gqa_group_size, int head_dim,
                             int block_size, int max_context_len, pa_dtype dtype) {
    if (num_seqs < 0 || num_kv_heads <= 0 || gqa_group_size <= 0 || max_context_len < 0 ||
        !supported_shape(head_dim, block_size) || elem_bytes(dtype) == 0)
        return 0;
    const int split = pa::mfma_split(dtype, head_dim, block_size, gqa_group_size);
    const int ps = small_call_partition(num_seqs, num_kv_heads * (split > 0 ? split : 1),
                                        block_size, max_context_len);
    return ps > 0 ? ps : heuristic_partition(num_seqs, num_kv_heads, block_size, max_context_len);
}

size_t pa_decode_workspace_size(int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                                int block_size, int max_context_len, int partition_size,
                                pa_dtype dtype) {
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads ||
        max_context_len < 0 || !supported_shape(head_dim, block_size) || elem_bytes(dtype) == 0)
        return (size_t)-1;
    int P = partition_size;
    if (P == 0) P = heuristic_partition(num_seqs, num_kv_heads, block_size, max_context_len);
    if (!valid_partition(P, block_size)) return (size_t)-1;
    size_t bytes = fixed_layout(num_seqs, num_heads, head_dim, max_context_len, P).bytes;
    // enough for either kernel family (pa_debug_select_kernel may force one)
    const int group = num_heads / num_kv_heads;
    const int split = pa::mfma_split(dtype, head_dim, block_size, group);
    if (use_balanced(split > 0, partition_size, num_seqs, max_context_len)) {
        // groups (per pass) of more than 16 heads take two 16-column tiles per slot
        const int slot_cols =
            pa::mfma_pass_group(group, split) > pa::kMaxGroup ? 2 * pa::kMaxGroup : pa::kMaxGroup;
        const size_t bal = balanced_layout(head_dim, slot_cols).bytes;
        if (bal > bytes) bytes = bal;
    }
    return bytes;
}

}  // extern "C"

// Verify rows whose row map the balanced decode kernel computes itself.
struct VerifyFold {
    const int32_t* query_start;
    const int32_t* src_lens;
    int num_src_seqs, max_query_len, u;
};

static int decode_impl(void* out, const void* query, const void* new_key,
                       const void* new_value, const void* key_cache, const void* value_cache,
                       const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                       int num_heads, int num_kv_heads, int gqa_group_size, int head_dim,
                       int block_size, int num_blocks, int max_blocks_per_seq,
                       int max_context_len, float scale, pa_dtype dtype, int partition_size,
                       void* workspace, size_t workspace_bytes, void* hip_stream,
                       int kv_format = pa::kKvSame, float k_scale = 1.0f, float v_scale = 1.0f,
                       const int32_t* table_rows = nullptr, const int32_t* row_tokens = nullptr,
                       int kernel_kind = -1, int col_tiles = 1,
                       const VerifyFold* fold = nullptr) {
    if (num_seqs < 0) return fail(PA_ERR_INVALID_ARG, "num_seqs %d < 0", num_seqs);
    if (kv_format != pa::kKvSame && kv_format != pa::kKvE4M3 && kv_format != pa::kKvI8)
        return fail(PA_ERR_INVALID_ARG, "internal: unknown cache format %d", kv_format);
    const bool q8 = kv_format != pa::kKvSame;     // 8-bit codes with one scale per cache
    if (q8 && !(std::isfinite(k_scale) && k_scale > 0.0f && std::isfinite(v_scale) &&
                  v_scale > 0.0f))
        return fail(PA_ERR_INVALID_ARG, "k_scale and v_scale must be finite and positive");
    if (num_heads <= 0 || num_kv_heads <= 0)
        return fail(PA_ERR_INVALID_ARG, "num_heads %d / num_kv_heads %d must be positive",
                    num_heads, num_kv_heads);
    if (num_heads % num_kv_heads)
        return fail(PA_ERR_INVALID_ARG, "num_heads %d not a multiple of num_kv_heads %d",
                    num_heads, num_kv_heads);
    if (gqa_group_size != num_heads / num_kv_heads)
        return fail(PA_ERR_INVALID_ARG, "gqa_group_size %d != num_heads/num_kv_heads = %d",
                    gqa_group_size, num_heads / num_kv_heads);
    if (elem_bytes(dtype) == 0) return fail(PA_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
    if (num_blocks <= 0 || max_blocks_per_seq <= 0)
        return fail(PA_ERR_INVALID_ARG, "num_blocks %d / max_blocks_per_seq %d must be positive",
                    num_blocks, max_blocks_per_seq);
    if (head_dim <= 0 || block_size <= 0)
        return fail(PA_ERR_INVALID_ARG, "head_dim %d / block_size %d must be positive",
                    head_dim, block_size);
    if (!supported_shape(head_dim, block_size))
        return fail(PA_ERR_UNSUPPORTED, "head_dim %d with block_size %d not built "
                    "(head_dim 64/128/256, block_size 8/16/32/64)", head_dim, block_size);
    if (max_context_len < 0 || (int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
        return fail(PA_ERR_INVALID_ARG, "max_context_len %d outside [0, %lld]", max_context_len,
                    (long long)max_blocks_per_seq * block_size);
    if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale is not finite");
    if ((int64_t)num_blocks * num_kv_heads * block_size * head_dim > ((int64_t)1 << 46))
        return fail(PA_ERR_INVALID_ARG, "pool too large");
    if (num_seqs == 0) return PA_OK;
    if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens)
        return fail(PA_ERR_INVALID_ARG, "null tensor pointer");
    if (!aligned16(out) || !aligned16(query) || !aligned16(key_cache) || !aligned16(value_cache))
        return fail(PA_ERR_INVALID_ARG, "query/out/cache pointers must be 16-byte aligned");
    const bool append = new_key != nullptr || new_value != nullptr;
    if (append && (!new_key || !new_value || !aligned16(new_key) || !aligned16(new_value)))
        return fail(PA_ERR_INVALID_ARG, "new key/value must be non-null and 16-byte aligned");
    if (partition_size != 0 && !valid_partition(partition_size, block_size))
        return fail(PA_ERR_INVALID_ARG, "partition_size %d must be a positive multiple of 32 "
                    "and of block_size, at most 64*block_size", partition_size);

    int kind = kernel_kind >= 0 ? kernel_kind : g_kernel_kind.load();
    if (q8 && dtype == PA_F32)
        return fail(PA_ERR_UNSUPPORTED, "8-bit caches take bf16 or f16 queries");
    // verify rows (a row map or a fold) take the matrix-core kernel in one
    // pass only, with 16-bit rows
    const bool rows_mapped = table_rows != nullptr || fold != nullptr;
    const int split = rows_mapped
                          ? (verify_on_mfma(dtype, head_dim, block_size, gqa_group_size) ? 1 : 0)
                          : pa::mfma_split(dtype, head_dim, block_size, gqa_group_size);
    const bool mfma_ok = split > 0;
    if (kind == pa::kMfma && !mfma_ok)
        return fail(PA_ERR_UNSUPPORTED, "matrix-core kernel selected but not built for this shape");
    // A small call left to the library takes one partition covering every
    // history (see small_call_partition); float32 rows then take the
    // vector-ALU kernel, whose single launch is the shortest (the tiny
    // float32 workload: 3.7 against 4.5 us on the matrix cores).
    if (partition_size == 0 && !rows_mapped) {
        const int ps = small_call_partition(num_seqs, num_kv_heads * (mfma_ok ? split : 1),
                                            block_size, max_context_len);
        if (ps > 0) {
            partition_size = ps;
            if (dtype == PA_F32 && kind == pa::kAuto) kind = pa::kGeneric;
        }
    }
    const bool use_mfma = mfma_ok && kind != pa::kGeneric;
    if (q8 && !use_mfma)
        return fail(PA_ERR_UNSUPPORTED, "8-bit caches are served by the matrix-core kernel only "
                    "(bf16/f16 queries, head_dim 64/128/256, block_size 8/16/32/64)");
    // a row map held in memory is read by the fixed schedule's kernels only
    const bool balanced = table_rows == nullptr &&
                          use_balanced(use_mfma, partition_size, num_seqs, max_context_len);
    if (fold && !balanced)
        return fail(PA_ERR_INVALID_ARG, "internal: verify row map folded off the balanced path");

    const int P = partition_size ? partition_size
                                 : heuristic_partition(num_seqs, num_kv_heads, block_size,
                                                       max_context_len);
    // a group too large for one pass runs as `split` passes of smaller ones
    const int kv_split = use_mfma ? split : 1;
    const int pass_group = pa::mfma_pass_group(gqa_group_size, kv_split);
    // the passes of a split group all read the newest token, so its append
    // runs in a kernel of its own first -- built for 16-bit and f32 rows only
    if (append && q8 && kv_split > 1)
        return fail(PA_ERR_UNSUPPORTED, "the fused append into 8-bit caches needs a group of at "
                    "most 16 heads (32 at head_dim 64/128); store the token with "
                    "pa_reshape_and_cache_fp8/_i8, then call the 8-bit decode");
    // groups of more than 16 heads always take two column tiles
    if (use_mfma && pass_group > pa::kMaxGroup) col_tiles = 2;
    if (col_tiles != 1 && !(col_tiles == 2 && use_mfma && head_dim <= 128))
        return fail(PA_ERR_INVALID_ARG, "two column tiles serve the matrix-core kernel at "
                    "head_dim 64/128 only");
    const Layout lay = balanced ? balanced_layout(head_dim, pa::kMaxGroup * col_tiles)
                                : fixed_layout(num_seqs, num_heads, head_dim, max_context_len, P);
    const bool needs_ws = lay.bytes > 0;
    if (needs_ws) {
        if (!workspace || workspace_bytes < lay.bytes)
            return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", lay.bytes,
                        workspace ? workspace_bytes : (size_t)0);
        if (reinterpret_cast<uintptr_t>(workspace) & 255u)
            return fail(PA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    }

    pa::DecodeArgs a{};
    a.out = out;
    a.query = query;
    a.key_cache = key_cache;
    a.value_cache = value_cache;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.table_rows = table_rows;
    a.row_tokens = row_tokens;
    if (fold) {
        a.query_start = fold->query_start;
        a.src_lens = fold->src_lens;
        a.num_src_seqs = fold->num_src_seqs;
        a.max_query_len = fold->max_query_len;
        a.row_group = fold->u;
    }
    a.ws_lse = needs_ws ? reinterpret_cast<float*>(static_cast<char*>(workspace) + lay.lse_off)
                        : nullptr;
    a.ws_out = needs_ws ? reinterpret_cast<float*>(static_cast<char*>(workspace) + lay.out_off)
                        : nullptr;
    a.ws_meta = needs_ws && balanced
                    ? reinterpret_cast<int*>(static_cast<char*>(workspace) + lay.meta_off)
                    : nullptr;
    a.num_seqs = num_seqs;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads * kv_split;
    a.group = pass_group;
    a.kv_split = kv_split;
    a.kv_heads_mem = num_kv_heads;
    a.group_mem = gqa_group_size;
    a.head_dim = head_dim;
    a.block_size = block_size;
    a.num_blocks = num_blocks;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.max_context_len = max_context_len;
    a.part_len = P;
    a.num_parts = balanced ? 1 : lay.num_parts;
    a.schedule = balanced ? pa::kBalanced : pa::kFixed;
    a.num_wg = balanced ? balanced_workgroups(head_dim) : 0;
    a.col_tiles = col_tiles;
    // scale * log2(e), and the key scale of an 8-bit cache folded into it
    a.scale_log2 = (float)((double)scale * 1.4426950408889634 * (q8 ? (double)k_scale : 1.0));
    a.kv_format = kv_format;
    a.out_scale = q8 ? v_scale : 1.0f;
    a.k_inv_scale = q8 ? (float)(1.0 / (double)k_scale) : 1.0f;
    a.v_inv_scale = q8 ? (float)(1.0 / (double)v_scale) : 1.0f;

    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    hipError_t e = hipSuccess;
    if (append && use_mfma && kv_split == 1 && dtype != PA_F32) {
        // the matrix-core kernel stores each newest token itself (with a
        // split group, several passes read that token, and float32 rows
        // have no in-kernel append: a kernel of its own stores it first)
        a.new_key = new_key;
        a.new_value = new_value;
    } else if (append) {
        e = pa::launch_append_tokens(new_key, new_value, const_cast<void*>(key_cache),
                                     const_cast<void*>(value_cache), block_tables, context_lens,
                                     num_seqs, num_kv_heads, head_dim * elem_bytes(dtype),
                                     block_size, num_blocks, max_blocks_per_seq,
                                     max_context_len, s);
        if (e != hipSuccess) return hip_fail(e, "append kernel launch");
    }
    e = use_mfma ? pa::launch_decode_mfma(a, dtype, s) : pa::launch_decode_generic(a, dtype, s);
    if (e != hipSuccess) return hip_fail(e, "decode partition kernel launch");
    if (balanced || lay.num_parts > 1) {
        e = pa::launch_lse_merge(a, dtype, s);
        if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
    }
    return PA_OK;
}

extern "C" {

int pa_paged_attention_decode(void* out, const void* query, const void* key_cache,
                              const void* value_cache, const int32_t* block_tables,
                              const int32_t* context_lens, int num_seqs, int num_heads,
                              int num_kv_heads, int gqa_group_size, int head_dim,
                              int block_size, int num_blocks, int max_blocks_per_seq,
                              int max_context_len, float scale, pa_dtype dtype,
                              int partition_size, void* workspace, size_t workspace_bytes,
                              void* hip_stream) {
    return decode_impl(out, query, nullptr, nullptr, key_cache, value_cache, block_tables,
                       context_lens, num_seqs, num_heads, num_kv_heads, gqa_group_size, head_dim,
                       block_size, num_blocks, max_blocks_per_seq, max_context_len, scale, dtype,
                       partition_size, workspace, workspace_bytes, hip_stream);
}

int pa_decode_append(void* out, const void* query, const void* key, const void* value,
                     void* key_cache, void* value_cache, const int32_t* block_tables,
                     const int32_t* context_lens, int num_seqs, int num_heads, int num_kv_heads,
                     int gqa_group_size, int head_dim, int block_size, int num_blocks,
                     int max_blocks_per_seq, int max_context_len, float scale, pa_dtype dtype,
                     int partition_size, void* workspace, size_t workspace_bytes,
                     void* hip_stream) {
    if (num_seqs > 0 && (!key || !value))
        return fail(PA_ERR_INVALID_ARG, "null key/value pointer");
    return decode_impl(out, query, key, value, key_cache, value_cache, block_tables,
                       context_lens, num_seqs, num_heads, num_kv_heads, gqa_group_size, head_dim,
                       block_size, num_blocks, max_blocks_per_seq, max_context_len, scale, dtype,
                       partition_size, workspace, workspace_bytes, hip_stream);
}

int pa_paged_attention_decode_fp8(void* out, const void* query, const void* key_cache,
                                  const void* value_cache, const int32_t* block_tables,
                                  const int32_t* context_lens, int num_seqs, int num_heads,
                                  int num_kv_heads, int gqa_group_size, int head_dim,
                                  int block_size, int num_blocks, int max_blocks_per_seq,
                                  int max_context_len, float scale, pa_dtype dtype, float k_scale,
                                  float v_scale, int partition_size, void* workspace,
                                  size_t workspace_bytes, void* hip_stream) {
    return decode_impl(out, query, nullptr, nullptr, key_cache, value_cache, block_tables,
                       context_lens, num_seqs, num_heads, num_kv_heads, gqa_group_size, head_dim,
                       block_size, num_blocks, max_blocks_per_seq, max_context_len, scale, dtype,
                       partition_size, workspace, workspace_bytes, hip_stream, pa::kKvE4M3,
                       k_scale, v_scale);
}

int pa_decode_append_fp8(void* out, const void* query, const void* key, const void* value,
                         void* key_cache, void* value_cache, const int32_t* block_tables,
                         const int32_t* context_lens, int num_seqs, int num_heads,
                         int num_kv_heads, int gqa_group_size, int head_dim, int block_size,
                         int num_blocks, int max_blocks_per_seq, int max_context_len, float scale,
                         pa_dtype dtype, float k_scale, float v_scale, int partition_size,
                         void* workspace, size_t workspace_bytes, void* hip_stream) {
    if (!key || !value) return fail(PA_ERR_INVALID_ARG, "new key/value must be non-null");
    return decode_impl(out, query, key, value, key_cache, value_cache, block_tables,
                       context_lens, num_seqs, num_heads, num_kv_heads, gqa_group_size, head_dim,
                       block_size, num_blocks, max_blocks_per_seq, max_context_len, scale, dtype,
                       partition_size, workspace, workspace_bytes, hip_stream, pa::kKvE4M3,
                       k_scale, v_scale);
}

}  // extern "C"

static int reshape_and_cache_q8(const void* key, const void* value, void* key_cache,
                                void* value_cache, const int64_t* slot_mapping, int num_tokens,
                                int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                pa_dtype dtype, float k_scale, float v_scale, bool int8,
                                void* hip_stream) {
    const int e = elem_bytes(dtype);
    if (e == 0) return fail(PA_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
    if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
        return fail(PA_ERR_INVALID_ARG, "sizes must be positive (num_tokens >= 0)");
    if (head_dim % 16)
        return fail(PA_ERR_UNSUPPORTED, "head_dim must be a multiple of 16");
    if (!(std::isfinite(k_scale) && k_scale > 0.0f && std::isfinite(v_scale) && v_scale > 0.0f))
        return fail(PA_ERR_INVALID_ARG, "k_scale and v_scale must be finite and positive");
    if (num_tokens == 0) return PA_OK;
    if (!key || !value || !key_cache || !value_cache || !slot_mapping)
        return fail(PA_ERR_INVALID_ARG, "null tensor pointer");
    if (!aligned16(key) || !aligned16(value) || !aligned16(key_cache) || !aligned16(value_cache))
        return fail(PA_ERR_INVALID_ARG, "key/value/cache pointers must be 16-byte aligned");
    hipError_t err = pa::launch_reshape_and_cache_q8(
        key, value, key_cache, value_cache, slot_mapping, num_tokens, num_kv_heads, head_dim,
        block_size, num_blocks, dtype, int8, (float)(1.0 / (double)k_scale),
        (float)(1.0 / (double)v_scale), static_cast<hipStream_t>(hip_stream));
    if (err != hipSuccess)
        return hip_fail(err, int8 ? "int8 cache write kernel launch" : "fp8 cache write kernel launch");
    return PA_OK;
}

extern "C" {

int pa_reshape_and_cache_fp8(const void* key, const void* value, void* key_cache,
                             void* value_cache, const int64_t* slot_mapping, int num_tokens,
                             int num_kv_heads, int head_dim, int block_size, int num_blocks,
                             pa_dtype dtype, float k_scale, float v_scale, void* hip_stream) {
    return reshape_and_cache_q8(key, value, key_cache, value_cache, slot_mapping, num_tokens,
                                num_kv_heads, head_dim, block_size, num_blocks, dtype, k_scale,
                                v_scale, false, hip_stream);
}

int pa_paged_attention_decode_i8(void* out, const void* query, const void* key_cache,
                                 const void* value_cache, const int32_t* block_tables,
                                 const int32_t* context_lens, int num_seqs, int num_heads,
                                 int num_kv_heads, int gqa_group_size, int head_dim,
                                 int block_size, int num_blocks, int max_blocks_per_seq,
                                 int max_context_len, float scale, pa_dtype dtype, float k_scale,
                                 float v_scale, int partition_size, void* workspace,
                                 size_t workspace_bytes, void* hip_stream) {
    return decode_impl(out, query, nullptr, nullptr, key_cache, value_cache, block_tables,
                       context_lens, num_seqs, num_heads, num_kv_heads, gqa_group_size, head_dim,
                       block_size, num_blocks, max_blocks_per_seq, max_context_len, scale, dtype,
                       partition_size, workspace, workspace_bytes, hip_stream, pa::kKvI8,
                       k_scale, v_scale);
}

int pa_decode_append_i8(void* out, const void* query, const void* key, const void* value,
                        void* key_cache, void* value_cache, const int32_t* block_tables,
                        const int32_t* context_lens, int num_seqs, int num_heads,
                        int num_kv_heads, int gqa_group_size, int head_dim, int block_size,
                        int num_blocks, int max_blocks_per_seq, int max_context_len, float scale,
                        pa_dtype dtype, float k_scale, float v_scale, int partition_size,
                        void* workspace, size_t workspace_bytes, void* hip_stream) {
    if (!key || !value) return fail(PA_ERR_INVALID_ARG, "new key/value must be non-null");
    return decode_impl(out, query, key, value, key_cache, value_cache, block_tables,
                       context_lens, num_seqs, num_heads, num_kv_heads, gqa_group_size, head_dim,
                       block_size, num_blocks, max_blocks_per_seq, max_context_len, scale, dtype,
                       partition_size, workspace, workspace_bytes, hip_stream, pa::kKvI8,
                       k_scale, v_scale);
}

int pa_reshape_and_cache_i8(const void* key, const void* value, void* key_cache,
                            void* value_cache, const int64_t* slot_mapping, int num_tokens,
                            int num_kv_heads, int head_dim, int block_size, int num_blocks,
                            pa_dtype dtype, float k_scale, float v_scale, void* hip_stream) {
    return reshape_and_cache_q8(key, value, key_cache, value_cache, slot_mapping, num_tokens,
                                num_kv_heads, head_dim, block_size, num_blocks, dtype, k_scale,
                                v_scale, true, hip_stream);
}

size_t pa_verify_workspace_size(int total_queries, int num_heads, int num_kv_heads,
                                int head_dim, int block_size, int max_context_len,
                                int partition_size, pa_dtype dtype) {
    if (total_queries < 0) return (size_t)-1;
    const size_t dec = pa_decode_workspace_size(total_queries, num_heads, num_kv_heads, head_dim,
                                                block_size, max_context_len, partition_size,
                                                dtype);
    if (dec == (size_t)-1) return dec;
    // room for the 32-column slots of two column tiles (head_dim <= 128)
    const size_t bal = head_dim <= 128 && partition_size == 0 && max_context_len > 0
                           ? balanced_layout(head_dim, 2 * pa::kMaxGroup).bytes
                           : 0;
    return align256(std::max(dec, bal)) + 3 * align256((size_t)total_queries * sizeof(int32_t));
}

int pa_paged_attention_verify(void* out, const void* query, const void* key_cache,
                              const void* value_cache, const int32_t* block_tables,
                              const int32_t* context_lens, const int32_t* query_start,
                              int num_seqs, int total_queries, int max_query_len, int num_heads,
                              int num_kv_heads, int gqa_group_size, int head_dim, int block_size,
                              int num_blocks, int max_blocks_per_seq, int max_context_len,
                              float scale, pa_dtype dtype, int partition_size, void* workspace,
                              size_t workspace_bytes, void* hip_stream) {
    if (num_seqs < 0 || total_queries < 0 || max_query_len < 1)
        return fail(PA_ERR_INVALID_ARG, "num_seqs, total_queries >= 0 and max_query_len >= 1");
    if (total_queries > 0 && num_seqs == 0)
        return fail(PA_ERR_INVALID_ARG, "query rows without sequences");
    if (total_queries == 0) return PA_OK;
    if (!query_start) return fail(PA_ERR_INVALID_ARG, "null query_start");
    const size_t need = pa_verify_workspace_size(total_queries, num_heads, num_kv_heads,
                                                 head_dim, block_size, max_context_len,
                                                 partition_size, dtype);
    if (need == (size_t)-1) return fail(PA_ERR_INVALID_ARG, "invalid sizes");
    if (!workspace || workspace_bytes < need)
        return fail(PA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
        return fail(PA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    const size_t arr = align256((size_t)total_queries * sizeof(int32_t));
    const size_t dec = need - 3 * arr;
    char* base = static_cast<char*>(workspace);
    int32_t* rows = reinterpret_cast<int32_t*>(base + dec);
    int32_t* lens = reinterpret_cast<int32_t*>(base + dec + arr);
    int32_t* toks = reinterpret_cast<int32_t*>(base + dec + 2 * arr);
    if (!context_lens) return fail(PA_ERR_INVALID_ARG, "null context_lens");
    if (gqa_group_size < 1) return fail(PA_ERR_INVALID_ARG, "gqa_group_size must be positive");
    // The matrix-core kernel serves up to 16 / G query rows of a sequence in
    // one pass over its K/V (their (row, head) pairs fill its 16 columns), or
    // 32 / G with two column tiles when a sequence may hold more (head_dim
    // 64 and 128); the vector-ALU kernel takes one row per pass.  The kernel
    // family is chosen once here, so the grouping and the decode launch
    // agree.
    const int kind = g_kernel_kind.load();
    const bool mfma =
        verify_on_mfma(dtype, head_dim, block_size, gqa_group_size) && kind != pa::kGeneric;
    const int nt = mfma && head_dim <= 128 &&
                           (int64_t)max_query_len * gqa_group_size > pa::kMaxGroup
                       ? 2
                       : 1;
    const int u = mfma ? std::max(1, pa::kMaxGroup * nt / gqa_group_size) : 1;
    // On the balanced schedule the decode kernel computes the row map in its
    // prologue (one launch fewer); otherwise a kernel writes it to the
    // workspace for the fixed schedule's kernels.
    if (mfma && use_balanced(true, partition_size, total_queries, max_context_len) &&
        num_seqs <= pa::kMaxVerifyFoldSeqs) {
        const VerifyFold fold{query_start, context_lens, num_seqs, max_query_len, u};
        return decode_impl(out, query, nullptr, nullptr, key_cache, value_cache, block_tables,
                           context_lens, total_queries, num_heads, num_kv_heads, gqa_group_size,
                           head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len,
                           scale, dtype, partition_size, dec > 0 ? workspace : nullptr, dec,
                           hip_stream, pa::kKvSame, 1.0f, 1.0f, nullptr, nullptr, kind, nt,
                           &fold);
    }
    hipError_t e = pa::launch_verify_rows(query_start, context_lens, num_seqs, total_queries,
                                          max_query_len, max_context_len, u, rows, lens, toks,
                                          static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return hip_fail(e, "verify row kernel launch");
    return decode_impl(out, query, nullptr, nullptr, key_cache, value_cache, block_tables, lens,
                       total_queries, num_heads, num_kv_heads, gqa_group_size, head_dim,
                       block_size, num_blocks, max_blocks_per_seq, max_context_len, scale, dtype,
                       partition_size, dec > 0 ? workspace : nullptr, dec, hip_stream,
                       pa::kKvSame, 1.0f, 1.0f, rows, toks, kind, nt);
}

int pa_reshape_and_cache(const void* key, const void* value, void* key_cache, void* value_cache,
                         const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                         int head_dim, int block_size, int num_blocks, pa_dtype dtype,
                         void* hip_stream) {
    const int e = elem_bytes(dtype);
    if (e == 0) return fail(PA_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
    if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
        return fail(PA_ERR_INVALID_ARG, "sizes must be positive (num_tokens >= 0)");
    if ((head_dim * e) % 16)
        return fail(PA_ERR_UNSUPPORTED, "head_dim * element size must be a multiple of 16 bytes");
    if (num_tokens == 0) return PA_OK;
    if (!key || !value || !key_cache || !value_cache || !slot_mapping)
        return fail(PA_ERR_INVALID_ARG, "null tensor pointer");
    if (!aligned16(key) || !aligned16(value) || !aligned16(key_cache) || !aligned16(value_cache))
        return fail(PA_ERR_INVALID_ARG, "key/value/cache pointers must be 16-byte aligned");
    hipError_t err = pa::launch_reshape_and_cache(key, value, key_cache, value_cache, slot_mapping,
                                                  num_tokens, num_kv_heads, head_dim * e,
                                                  block_size, num_blocks,
                                                  static_cast<hipStream_t>(hip_stream));
    if (err != hipSuccess) return hip_fail(err, "cache write kernel launch");
    return PA_OK;
}

int pa_copy_blocks(void* key_cache, void* value_cache, const int32_t* block_pairs,
                   int num_pairs, int num_kv_heads, int head_dim, int block_size,
                   int num_blocks, pa_dtype dtype, void* hip_stream) {
    const int e = elem_bytes(dtype);
    if (e == 0) return fail(PA_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
    if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
        return fail(PA_ERR_INVALID_ARG, "sizes must be positive (num_pairs >= 0)");
    if ((head_dim * e) % 16)
        return fail(PA_ERR_UNSUPPORTED, "head_dim * element size must be a multiple of 16 bytes");
    const int64_t block_bytes = (int64_t)num_kv_heads * block_size * head_dim * e;
    if (block_bytes > (int64_t)1 << 30)
        return fail(PA_ERR_UNSUPPORTED, "blocks of %lld bytes are too large", (long long)block_bytes);
    if (num_pairs == 0) return PA_OK;
    if (!key_cache || !value_cache || !block_pairs)
        return fail(PA_ERR_INVALID_ARG, "null pointer");
    if (!aligned16(key_cache) || !aligned16(value_cache))
        return fail(PA_ERR_INVALID_ARG, "cache pointers must be 16-byte aligned");
    hipError_t err = pa::launch_copy_blocks(key_cache, value_cache, block_pairs, num_pairs,
                                            (int)block_bytes, num_blocks,
                                            static_cast<hipStream_t>(hip_stream));
    if (err != hipSuccess) return hip_fail(err, "block copy kernel launch");
    return PA_OK;
}

int pa_debug_gather_kv(void* k_out, void* v_out, const void* key_cache, const void* value_cache,
                       const int32_t* block_tables, const int32_t* context_lens, int seq,
                       int num_seqs, int num_kv_heads, int head_dim, int block_size,
                       int num_blocks, int max_blocks_per_seq, int max_context_len,
                       pa_dtype dtype, void* hip_stream) {
    const int e = elem_bytes(dtype);
    if (e == 0) return fail(PA_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
    if (seq < 0 || seq >= num_seqs)
        return fail(PA_ERR_INVALID_ARG, "seq %d outside [0, %d)", seq, num_seqs);
    if (num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0 ||
        max_blocks_per_seq <= 0 || max_context_len < 0 ||
        (int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
        return fail(PA_ERR_INVALID_ARG, "invalid sizes");
    if ((head_dim * e) % 16)
        return fail(PA_ERR_UNSUPPORTED, "head_dim * element size must be a multiple of 16 bytes");
    if (!k_out || !v_out || !key_cache || !value_cache || !block_tables || !context_lens)
        return fail(PA_ERR_INVALID_ARG, "null tensor pointer");
    if (!aligned16(k_out) || !aligned16(v_out) || !aligned16(key_cache) || !aligned16(value_cache))
        return fail(PA_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
    hipError_t err = pa::launch_gather(k_out, v_out, key_cache, value_cache, block_tables,
                                       context_lens, seq, num_kv_heads, head_dim * e, block_size,
                                       num_blocks, max_blocks_per_seq, max_context_len,
                                       static_cast<hipStream_t>(hip_stream));
    if (err != hipSuccess) return hip_fail(err, "gather kernel launch");
    return PA_OK;
}

int pa_bench_stream_read(const void* src, size_t bytes, void* sink, void* hip_stream) {
    if (!src || !sink || bytes % 16 || !aligned16(src) || !aligned16(sink))
        return fail(PA_ERR_INVALID_ARG, "stream read needs 16-byte aligned buffers and sizes");
    hipError_t err = pa::launch_stream_read(src, bytes, sink, static_cast<hipStream_t>(hip_stream));
    if (err != hipSuccess) return hip_fail(err, "stream read kernel launch");
    return PA_OK;
}

int pa_bench_copy(void* dst, const void* src, size_t bytes, void* hip_stream) {
    if (!src || !dst || bytes % 16 || !aligned16(src) || !aligned16(dst))
        return fail(PA_ERR_INVALID_ARG, "copy needs 16-byte aligned buffers and sizes");
    hipError_t err = pa::launch_copy(dst, src, bytes, static_cast<hipStream_t>(hip_stream));
    if (err != hipSuccess) return hip_fail(err, "copy kernel launch");
    return PA_OK;
}

}  // extern "C"
