/*
 * pagedattn.h -- C ABI of the MI355X (gfx950) paged KV decode attention
 * library, libpagedattn.so.
 *
 * Two operations make up one decode step of one attention layer:
 *
 *   pa_reshape_and_cache      store the new tokens' K/V into the paged pool at
 *                             the slots the block manager handed out;
 *   pa_paged_attention_decode attend each sequence's single new query (one per
 *                             query head) over its whole paged history;
 *
 * (pa_decode_append does both in one call), and the write side of shared
 * blocks:
 *
 *   pa_pool_*                 a host-side block pool with reference counts
 *                             and copy-on-write of shared partial blocks;
 *   pa_copy_blocks            the device copy that copy-on-write asks for.
 *
 * Sources, cited by page title and section:
 *   [MiniPaged-Qwen]  "MiniPaged-Qwen: 把 Paged Attention 讲清楚"
 *   [PA-source]       "PagedAttention 源码解析: KV Cache 怎么管理"
 *   [vLLM-paging]     "vLLM 与 PagedAttention: 把 KV Cache 变成分页状态"
 *   [KV-principles]   "2.1 KV Cache 与 PagedAttention 原理"
 *
 * Conventions for every entry point
 *   - All tensor arguments are DEVICE pointers to dense row-major arrays owned
 *     by the caller; the library never allocates, frees or keeps them.
 *   - Work is enqueued on `hip_stream` (a hipStream_t; NULL = the default
 *     stream) and runs asynchronously; no call synchronises the device.
 *   - The return value is a pa_status.  Every argument check happens on the
 *     host before anything is enqueued, so a non-zero status means nothing was
 *     launched.  pa_status_string() describes a status; pa_last_error() gives
 *     the text of the last failure on the calling thread.
 *   - Preconditions on device-resident data (context lengths, table entries,
 *     slots) cannot be checked without a sync; they are stated per call with
 *     what the kernels do when they are broken.  The kernels never access
 *     memory outside the arrays described here.
 *   - Thread safety: the library has no mutable global state apart from the
 *     thread-local error text and the test-only kernel selection below.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of query, caches, new K/V and output (all the same). */
typedef enum {
    PA_F32 = 0,
    PA_F16 = 1,
    PA_BF16 = 2
} pa_dtype;

typedef enum {
    PA_OK = 0,
    PA_ERR_INVALID_ARG = -1,   /* null/misaligned pointer, bad size, H % H_kv != 0 ... */
    PA_ERR_UNSUPPORTED = -2,   /* valid but not built: dtype, head_dim, block_size */
    PA_ERR_WORKSPACE = -3,     /* workspace missing or smaller than required */
    PA_ERR_HIP = -4,           /* a HIP runtime call failed (text in pa_last_error) */
    PA_ERR_POOL_EXHAUSTED = -5 /* the block pool has too few free blocks */
} pa_status;

/* Library ABI version (major*100 + minor). */
int pa_version(void);

/* Static text for a status code. */
const char* pa_status_string(int status);

/* Text of the last non-OK status returned on this thread ("" if none). */
const char* pa_last_error(void);

/*
 * pa_decode_partition_size -- context partition length (tokens) the decode
 * call uses for these sizes when called with partition_size = 0 and it runs
 * on partitions: a small call (histories of at most 512 tokens, at most 8192
 * (sequence, KV head pass, 32-token chunk) items) always does, with one
 * partition covering max_context_len; otherwise the vector-ALU kernel does,
 * and the matrix-core kernel uses its balanced schedule (no partitions).
 *
 * Long histories are split into partitions that are reduced independently and
 * merged by log-sum-exp ([MiniPaged-Qwen] §10.2 (2): shards reduced locally,
 * then merged globally).  The result is a multiple of 32 and of block_size.
 * Returns 0 for invalid sizes.
 */
int pa_decode_partition_size(int num_seqs, int num_kv_heads, int gqa_group_size,
                             int head_dim, int block_size, int max_context_len,
                             pa_dtype dtype);

/*
 * pa_decode_workspace_size -- bytes of device workspace pa_paged_attention_decode
 * needs for these sizes (0 if it needs none).  partition_size = 0 selects
 * pa_decode_partition_size().  The workspace holds the float32
 * per-partition states (log-sum-exp and normalised output of every (sequence,
 * head, partition)); contents need no initialisation and are meaningless
 * between calls.  Calls that share one workspace must not overlap in time
 * (use one per stream).  Returns (size_t)-1 for invalid sizes.
 */
size_t pa_decode_workspace_size(int num_seqs, int num_heads, int num_kv_heads,
                                int head_dim, int block_size, int max_context_len,
                                int partition_size, pa_dtype dtype);

/*
 * pa_paged_attention_decode -- single-step decode attention over a paged cache.
 *
 * Computes, for every sequence b and query head h,
 *     out[b,h,:] = sum_j softmax_j(scale * q[b,h,:] . k_j) v_j,  j = 0..L_b-1
 * ([MiniPaged-Qwen] §1, eq. o; normalised over the whole history, §5.2), where
 * history token j lives at key_cache[pb, kvh, off, :] / value_cache[...] with
 * pb = block_tables[b, j / block_size], off = j % block_size ([MiniPaged-Qwen]
 * §6.2 steps 1-4, [vLLM-paging] "Attention kernel 如何读取分页 KV") and
 * kvh = h / gqa_group_size ([MiniPaged-Qwen] §9.1, 一致点 4).  The sum is
 * evaluated as an online softmax (running max, rescaled denominator and
 * accumulator, [MiniPaged-Qwen] §5.2) in float32, with one rounding to the
 * output dtype at the end.
 *
 *   out            [num_seqs, num_heads, head_dim]                dtype, written
 *   query          [num_seqs, num_heads, head_dim]                dtype
 *   key_cache      [num_blocks, num_kv_heads, block_size, head_dim] dtype
 *   value_cache    [num_blocks, num_kv_heads, block_size, head_dim] dtype
 *                  (layout of [MiniPaged-Qwen] §8.2)
 *   block_tables   [num_seqs, max_blocks_per_seq] int32; entries j with
 *                  j*block_size >= L_b are never read (may hold anything)
 *   context_lens   [num_seqs] int32, L_b
 *   num_heads      H = num_kv_heads * gqa_group_size
 *   max_context_len host-side upper bound of every L_b; sizes the launch;
 *                  must be <= max_blocks_per_seq * block_size
 *   scale          score scale (1/sqrt(head_dim) in the sources)
 *   partition_size 0 = pa_decode_partition_size(); else a positive multiple
 *                  of 32 and of block_size (forces the partitioned path)
 *   workspace      device buffer of at least pa_decode_workspace_size() bytes,
 *                  256-byte aligned (may be NULL when that size is 0)
 *
 * Supported: dtype f32, f16, bf16; head_dim 64, 128 or 256; block_size 8,
 * 16, 32 or 64; any gqa_group_size >= 1 (other head_dim / block_size values
 * return PA_ERR_UNSUPPORTED).  bf16/f16 run on the matrix-core kernel
 * (pa_decode_kernel tells): a group of <= 16 heads, or <= 32 at head_dim 64
 * or 128, in one pass over each KV head's history; a larger group in the
 * fewest passes of at most that many heads, ceil(G / passes) heads each and
 * the remainder in the last, each pass over the whole history.  f32 runs on
 * the vector-ALU kernel.  Pointers to query/out/caches must be 16-byte
 * aligned.
 *
 * Device-data preconditions and what happens when they are broken:
 *   0 <= L_b <= max_context_len      otherwise out[b] is all NaN
 *   0 <= block_tables[b,j] < num_blocks for j*block_size < L_b
 *                                    otherwise the rows of the (b, kv-head)
 *                                    groups whose partitions read it are NaN
 *   L_b == 0                         out[b] is zero (empty history)
 */
int pa_paged_attention_decode(void* out, const void* query,
                              const void* key_cache, const void* value_cache,
                              const int32_t* block_tables,
                              const int32_t* context_lens,
                              int num_seqs, int num_heads, int num_kv_heads,
                              int gqa_group_size, int head_dim, int block_size,
                              int num_blocks, int max_blocks_per_seq,
                              int max_context_len, float scale, pa_dtype dtype,
                              int partition_size, void* workspace,
                              size_t workspace_bytes, void* hip_stream);

/*
 * pa_paged_attention_decode_noalloc -- pa_paged_attention_decode with no
 * workspace argument and no device allocation, for callers that cannot
 * allocate: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.
 *
 * Same arguments, results (bit for bit), supported shapes and errors as
 * pa_paged_attention_decode, minus workspace / workspace_bytes.  The
 * workspace is a device array of pa_noalloc_scratch_bytes() bytes (40 MiB)
 * that the library holds, one per GPU, from the first call made with that
 * GPU current until the process ends.  Nothing in it needs to start at zero:
 * every call writes what it reads.  Sizes whose
 * pa_decode_workspace_size() exceeds that return PA_ERR_WORKSPACE (use
 * pa_paged_attention_decode with a workspace of your own); the balanced
 * schedule of the matrix-core kernel needs at most about 34 MB, so every call
 * on it fits.  All calls on one GPU share its array: calls that overlap in
 * time on one GPU (different streams, or several host threads) race and
 * give wrong results -- serialise them.  PA_ERR_HIP if the array's device
 * address cannot be found (no current device).
 */
int pa_paged_attention_decode_noalloc(void* out, const void* query,
                                      const void* key_cache, const void* value_cache,
                                      const int32_t* block_tables,
                                      const int32_t* context_lens,
                                      int num_seqs, int num_heads, int num_kv_heads,
                                      int gqa_group_size, int head_dim, int block_size,
                                      int num_blocks, int max_blocks_per_seq,
                                      int max_context_len, float scale, pa_dtype dtype,
                                      int partition_size, void* hip_stream);

/* Bytes of the per-GPU device array pa_paged_attention_decode_noalloc works in. */
size_t pa_noalloc_scratch_bytes(void);

/*
 * pa_decode_append -- one decode step: append each sequence's newest token to
 * its paged history, then attend over the whole history (the step of
 * [MiniPaged-Qwen] §8.1 -- append_token gives the new token's slot, the
 * cache-write kernel stores it -- followed by §8.3's decode attention).
 *
 * context_lens already count the new token: sequence b's new token is its
 * history position L_b - 1, stored at
 *     key_cache  [block_tables[b, (L_b-1)/block_size], h, (L_b-1) % block_size, :] = key  [b, h, :]
 *     value_cache[...]                                                       = value[b, h, :]
 * for every KV head h, and then out is exactly what pa_paged_attention_decode
 * returns on the updated caches (bit for bit).  Equivalent to
 * pa_reshape_and_cache with those slots followed by pa_paged_attention_decode;
 * the matrix-core path does both in one launch.
 *
 *   key, value     [num_seqs, num_kv_heads, head_dim] dtype, 16-byte aligned
 *   key_cache,
 *   value_cache    written at the new tokens' slots
 *   all other arguments as for pa_paged_attention_decode.
 *
 * Precondition: the block that receives a sequence's new token is not read by
 * any other sequence in the same call (the tail block of a sequence being
 * appended to is private to it -- copy-on-write, [vLLM-paging]
 * "Copy-on-write 是共享的正确性边界").  L_b = 0 appends nothing; an invalid
 * length or a table entry outside the pool writes nothing and yields NaN
 * rows, as for the decode call.
 */
int pa_decode_append(void* out, const void* query, const void* key, const void* value,
                     void* key_cache, void* value_cache, const int32_t* block_tables,
                     const int32_t* context_lens, int num_seqs, int num_heads, int num_kv_heads,
                     int gqa_group_size, int head_dim, int block_size, int num_blocks,
                     int max_blocks_per_seq, int max_context_len, float scale, pa_dtype dtype,
                     int partition_size, void* workspace, size_t workspace_bytes,
                     void* hip_stream);

/*
 * pa_reshape_and_cache -- store new tokens' K/V into their cache slots.
 *
 * For every token i with s = slot_mapping[i] >= 0:
 *     key_cache  [s / block_size, h, s % block_size, :] = key  [i, h, :]
 *     value_cache[s / block_size, h, s % block_size, :] = value[i, h, :]
 * for all h < num_kv_heads ([MiniPaged-Qwen] §8.1: the block manager returns
 * the linear slot of each appended token; §8.2: the cache-write kernel stores
 * its K/V there).  The linear slot is read as pb * block_size + offset.  A
 * pure copy: bit-exact.
 *
 *   key, value     [num_tokens, num_kv_heads, head_dim] dtype
 *   key_cache,
 *   value_cache    [num_blocks, num_kv_heads, block_size, head_dim] dtype
 *   slot_mapping   [num_tokens] int64
 *
 * Supported: dtype f32, f16, bf16; head_dim * element size a multiple of 16
 * bytes; any block_size >= 1.  num_tokens = 0 is a no-op.
 *
 * Device-data preconditions:
 *   slot < 0                      padding: the token is skipped
 *   slot >= num_blocks*block_size the token is skipped (never written out of
 *                                 bounds); this is a caller error
 *   slots distinct                duplicate slots race; the stored row is one
 *                                 of the candidates
 */
int pa_reshape_and_cache(const void* key, const void* value,
                         void* key_cache, void* value_cache,
                         const int64_t* slot_mapping,
                         int num_tokens, int num_kv_heads, int head_dim,
                         int block_size, int num_blocks, pa_dtype dtype,
                         void* hip_stream);

/*
 * pa_check_slot_mapping -- host-side check of a cache write's slot mapping
 * against the preconditions above (the write kernels do not check them).
 *   slot_mapping   HOST [num_tokens] int64
 *   num_slots      num_blocks * block_size of the caches the write targets
 * Returns PA_OK when every non-negative slot is below num_slots and no two
 * tokens share a slot; otherwise PA_ERR_INVALID_ARG, and pa_last_error()
 * names the first offending token (past the pool) or slot (given twice).
 * Negative slots are padding and pass.  Reads only; O(n log n) host time.
 */
int pa_check_slot_mapping(const int64_t* slot_mapping, int num_tokens, int64_t num_slots);

/*
 * pa_paged_attention_verify -- decode with several new query tokens per
 * sequence: the verify step of speculative decoding, or multi-token decode
 * ([vLLM-paging] "Kernel metadata": each sequence's query range and the
 * verify semantics are passed explicitly; "Prefix、beam 与 speculative":
 * candidate tokens are written to the cache, then checked).
 *
 * Sequence b owns the query rows query_start[b] .. query_start[b+1] - 1 of
 * query and out [total_queries, num_heads, head_dim]: its q_b newest tokens,
 * already stored in the caches as history positions L_b - q_b .. L_b - 1
 * (context_lens count them).  Row i of the sequence attends positions
 * t <= L_b - q_b + i: causal among the new tokens, the plain decode of
 * pa_paged_attention_decode over that prefix.
 *
 *   query_start    DEVICE [num_seqs + 1] int32, non-decreasing, starting at 0
 *   max_query_len  host-side bound on every q_b
 *   block_tables   [num_seqs, max_blocks_per_seq]; context_lens [num_seqs]
 *   workspace      at least pa_verify_workspace_size() bytes, 256-byte aligned
 *   other arguments as for pa_paged_attention_decode (same support matrix).
 *
 * Rows of a sequence with q_b > max_query_len, q_b > L_b or an invalid L_b,
 * and rows outside every sequence's range, are NaN.  On the matrix-core
 * kernel up to u = 16 / G query rows of a sequence share one pass over its
 * K/V (their (row, head) pairs are the 16 columns of its tiles, each column
 * masked at its own causal end), or u = 32 / G with two column tiles when
 * max_query_len * G > 16 and head_dim is 64 or 128; the K/V of a sequence
 * is read ceil(q_b / u) times.  The vector-ALU kernel reduces each query
 * row on its own.
 */
size_t pa_verify_workspace_size(int total_queries, int num_heads, int num_kv_heads,
                                int head_dim, int block_size, int max_context_len,
                                int partition_size, pa_dtype dtype);
int pa_paged_attention_verify(void* out, const void* query, const void* key_cache,
                              const void* value_cache, const int32_t* block_tables,
                              const int32_t* context_lens, const int32_t* query_start,
                              int num_seqs, int total_queries, int max_query_len, int num_heads,
                              int num_kv_heads, int gqa_group_size, int head_dim, int block_size,
                              int num_blocks, int max_blocks_per_seq, int max_context_len,
                              float scale, pa_dtype dtype, int partition_size, void* workspace,
                              size_t workspace_bytes, void* hip_stream);

/*
 * FP8 KV cache.  The caches hold OCP FP8 E4M3 codes (one byte per value:
 * sign, 4 exponent bits of bias 7, 3 mantissa bits; no infinities; 0x7F and
 * 0xFF are NaN; largest finite 448), in the same [num_blocks, num_kv_heads,
 * block_size, head_dim] layout, with ONE scale per cache: code c of the key
 * cache stands for value(c) * k_scale, of the value cache for
 * value(c) * v_scale.  Storing x gives E4M3(fp32(x) * fp32(1 / scale)):
 * nearest value, ties to the even code, saturating to +-448, NaN kept.
 * ([KV-principles] §3.3 and its tuning Q&A: a quantised, e.g. FP8, KV cache
 * when KV memory binds; [vLLM-paging] "Kernel metadata": the KV dtype and
 * quantisation scales are passed explicitly.  The pages fix neither format
 * nor scale granularity; per-cache scales are the reading taken here.)
 * Halving the KV bytes nearly doubles decode throughput at the same
 * bandwidth.
 *
 * pa_paged_attention_decode_fp8 -- pa_paged_attention_decode over E4M3
 *   caches: the attention of each query over the dequantised history.  Same
 *   arguments, plus k_scale and v_scale (finite, > 0); dtype is that of query
 *   and out (bf16 or f16).  Supported: the shapes of the matrix-core kernel
 *   (head_dim 64/128/256, block_size 8/16/32/64, any gqa_group_size; a group
 *   of more than 16 heads, or 32 at head_dim 64/128, in several passes as
 *   for pa_paged_attention_decode -- except pa_decode_append_fp8/_i8, which
 *   take one pass only); other shapes return PA_ERR_UNSUPPORTED.  The
 *   workspace is sized by pa_decode_workspace_size with the query dtype.
 * pa_decode_append_fp8 -- pa_decode_append over E4M3 caches: each newest
 *   token's key/value (query dtype) is quantised as it is stored.
 * pa_reshape_and_cache_fp8 -- pa_reshape_and_cache into E4M3 caches: key and
 *   value [num_tokens, num_kv_heads, head_dim] of dtype f32, f16 or bf16 are
 *   quantised with k_scale / v_scale; head_dim a multiple of 16; slot rules
 *   as for pa_reshape_and_cache.
 * Cache pointers must be 16-byte aligned.
 */
int pa_paged_attention_decode_fp8(void* out, const void* query, const void* key_cache,
                                  const void* value_cache, const int32_t* block_tables,
                                  const int32_t* context_lens, int num_seqs, int num_heads,
                                  int num_kv_heads, int gqa_group_size, int head_dim,
                                  int block_size, int num_blocks, int max_blocks_per_seq,
                                  int max_context_len, float scale, pa_dtype dtype, float k_scale,
                                  float v_scale, int partition_size, void* workspace,
                                  size_t workspace_bytes, void* hip_stream);
int pa_decode_append_fp8(void* out, const void* query, const void* key, const void* value,
                         void* key_cache, void* value_cache, const int32_t* block_tables,
                         const int32_t* context_lens, int num_seqs, int num_heads,
                         int num_kv_heads, int gqa_group_size, int head_dim, int block_size,
                         int num_blocks, int max_blocks_per_seq, int max_context_len, float scale,
                         pa_dtype dtype, float k_scale, float v_scale, int partition_size,
                         void* workspace, size_t workspace_bytes, void* hip_stream);
int pa_reshape_and_cache_fp8(const void* key, const void* value, void* key_cache,
                             void* value_cache, const int64_t* slot_mapping, int num_tokens,
                             int num_kv_heads, int head_dim, int block_size, int num_blocks,
                             pa_dtype dtype, float k_scale, float v_scale, void* hip_stream);

/*
 * INT8 KV cache.  The caches hold signed 8-bit integer codes (two's
 * complement, -127 .. 127; the code -128 is never written and reads as
 * -128), in the same [num_blocks, num_kv_heads, block_size, head_dim]
 * layout, with ONE scale per cache: code c of the key cache stands for
 * c * k_scale, of the value cache for c * v_scale (symmetric, no zero
 * point).  Storing x gives the integer nearest fp32(x) * fp32(1 / scale),
 * ties to even, clamped to [-127, 127]; NaN is stored as 0, the one code
 * an integer cache has for it.  ([KV-principles] §3.3 "量化压缩 KV Cache":
 * 16-bit K and V quantised to INT8 to halve their memory, with a small
 * accuracy cost.  The pages fix neither the scale granularity nor the
 * rounding; a per-cache symmetric scale and round-half-even are the
 * readings taken here.)
 *
 * pa_paged_attention_decode_i8 -- pa_paged_attention_decode over INT8
 *   caches: the attention of each query over the dequantised history.  Same
 *   arguments, rules, supported shapes and workspace as
 *   pa_paged_attention_decode_fp8.
 * pa_decode_append_i8 -- pa_decode_append over INT8 caches: each newest
 *   token's key/value (query dtype) is quantised as it is stored.
 * pa_reshape_and_cache_i8 -- pa_reshape_and_cache into INT8 caches, with the
 *   arguments and rules of pa_reshape_and_cache_fp8.
 * Cache pointers must be 16-byte aligned.
 */
int pa_paged_attention_decode_i8(void* out, const void* query, const void* key_cache,
                                 const void* value_cache, const int32_t* block_tables,
                                 const int32_t* context_lens, int num_seqs, int num_heads,
                                 int num_kv_heads, int gqa_group_size, int head_dim,
                                 int block_size, int num_blocks, int max_blocks_per_seq,
                                 int max_context_len, float scale, pa_dtype dtype, float k_scale,
                                 float v_scale, int partition_size, void* workspace,
                                 size_t workspace_bytes, void* hip_stream);
int pa_decode_append_i8(void* out, const void* query, const void* key, const void* value,
                        void* key_cache, void* value_cache, const int32_t* block_tables,
                        const int32_t* context_lens, int num_seqs, int num_heads,
                        int num_kv_heads, int gqa_group_size, int head_dim, int block_size,
                        int num_blocks, int max_blocks_per_seq, int max_context_len, float scale,
                        pa_dtype dtype, float k_scale, float v_scale, int partition_size,
                        void* workspace, size_t workspace_bytes, void* hip_stream);
int pa_reshape_and_cache_i8(const void* key, const void* value, void* key_cache,
                            void* value_cache, const int64_t* slot_mapping, int num_tokens,
                            int num_kv_heads, int head_dim, int block_size, int num_blocks,
                            pa_dtype dtype, float k_scale, float v_scale, void* hip_stream);

/*
 * pa_copy_blocks -- copy whole physical blocks of both caches:
 *     key_cache  [dst_i, :, :, :] = key_cache  [src_i, :, :, :]
 *     value_cache[dst_i, :, :, :] = value_cache[src_i, :, :, :]
 * for every pair i (all KV heads and slots of the block): the copy behind
 * copy-on-write, when a sequence must write into a partially filled block
 * that other sequences still share ([vLLM-paging] "Copy-on-write 是共享的正确
 * 性边界": the branch copies the block and writes its new token into the
 * private copy).  A pure copy: bit-exact.
 *
 *   key_cache,
 *   value_cache    [num_blocks, num_kv_heads, block_size, head_dim] dtype
 *   block_pairs    DEVICE [num_pairs][2] int32 (src, dst), as pa_pool_append
 *                  returns them
 *
 * Supported: dtype f32, f16, bf16; head_dim * element size a multiple of 16
 * bytes; any block_size >= 1.  num_pairs = 0 is a no-op.
 *
 * Device-data preconditions: no dst is also a src or another pair's dst in
 * the same call (a copy-on-write destination is a freshly taken block), so
 * the pairs are independent.  A pair with an index outside [0, num_blocks),
 * or with src == dst, is skipped.
 */
int pa_copy_blocks(void* key_cache, void* value_cache, const int32_t* block_pairs,
                   int num_pairs, int num_kv_heads, int head_dim, int block_size,
                   int num_blocks, pa_dtype dtype, void* hip_stream);

/*
 * Block pool -- host-side ownership of the physical blocks of a paged cache,
 * with sharing ([vLLM-paging] "Copy-on-write 是共享的正确性边界" and its
 * "最小分页与 COW 模拟"; [MiniPaged-Qwen] §9 "差异 3", §10.1: shared
 * prefixes, branch sharing, reference counting, copy-on-write).  The pool
 * keeps no device memory: it hands out block tables, slots and copy pairs
 * for the cache write, the decode call and pa_copy_blocks.
 *
 *   - A block is taken from the END of the free list (blocks start as the
 *     list 0, 1, ..., num_blocks - 1) and starts with one reference.
 *   - A sequence is a block table; its tokens fill the blocks in order,
 *     block_size per block, the last block possibly partial.
 *   - pa_pool_fork: a new sequence naming the same blocks; each gains one
 *     reference.
 *   - pa_pool_append: one new token for each listed sequence, in list order.
 *     Empty table or full last block: a fresh block is taken.  Partial last
 *     block shared with another sequence: the sequence drops that reference,
 *     takes a fresh block and a copy pair (shared, fresh) is reported; the
 *     token goes into the copy.  Otherwise the token goes into the last block.
 *     slots[i] = block * block_size + position of the new token, the linear
 *     slot of pa_reshape_and_cache.  Before storing the new tokens, the caller
 *     runs pa_copy_blocks on the copy pairs (in the same stream order).
 *   - pa_pool_release: the sequence's blocks each lose one reference; blocks
 *     with none left return to the free list; the sequence id is retired.
 *
 * A pool is not thread-safe: calls on one pool must not overlap.  Distinct
 * pools are independent.
 */
typedef struct pa_block_pool pa_block_pool;

/* New pool of num_blocks blocks of block_size tokens; NULL for non-positive
 * sizes or when host memory runs out (pa_last_error says which).  Destroyed
 * by pa_pool_destroy (NULL is ignored). */
pa_block_pool* pa_pool_create(int num_blocks, int block_size);
void pa_pool_destroy(pa_block_pool* pool);

/* New empty sequence; returns its id (>= 0) or a negative status. */
int pa_pool_add_sequence(pa_block_pool* pool);

/* New sequence sharing every block of `seq`; returns its id or a negative
 * status (PA_ERR_INVALID_ARG for an unknown or retired id). */
int pa_pool_fork(pa_block_pool* pool, int seq);

/*
 * One new token for each of seqs[0..n) (distinct, live ids), as described
 * above.  HOST arrays: slots [n] int64 receives each token's slot;
 * copy_pairs [n][2] int32 receives the copy pairs (at most one per token),
 * *num_copies their count.  All or nothing: if the free blocks do not
 * suffice, returns PA_ERR_POOL_EXHAUSTED ("KV pool exhausted") and changes
 * nothing; PA_ERR_INVALID_ARG for a bad id, a repeated id or null arrays.
 */
int pa_pool_append(pa_block_pool* pool, const int* seqs, int n, int64_t* slots,
                   int32_t* copy_pairs, int* num_copies);

/* Drop a sequence (see above); PA_OK or PA_ERR_INVALID_ARG. */
int pa_pool_release(pa_block_pool* pool, int seq);

/* Tokens in a sequence, or a negative status. */
int pa_pool_length(const pa_block_pool* pool, int seq);

/* Number of blocks in the sequence's table (or a negative status); the first
 * min(capacity, that number) entries are written to the HOST array table. */
int pa_pool_table(const pa_block_pool* pool, int seq, int32_t* table, int capacity);

/* References to a block (0 = free), or a negative status. */
int pa_pool_refcount(const pa_block_pool* pool, int block);

/* Blocks on the free list. */
int pa_pool_free_blocks(const pa_block_pool* pool);

/*
 * pa_debug_gather_kv -- copy one sequence's history into contiguous form,
 * using the same address translation device code as the decode kernels
 * ([MiniPaged-Qwen] §6.2; §5: K = [K^(0), ..., K^(T-1)]).  For testing the
 * index math bit-exactly.
 *
 *   k_out, v_out   [num_kv_heads, max_context_len, head_dim] dtype; rows
 *                  j < L_seq are written, the rest untouched
 *   seq            sequence index in [0, num_seqs)
 *
 * Same device-data preconditions as the decode call; rows of a table entry
 * outside [0, num_blocks) are filled with 0xFF bytes.
 */
int pa_debug_gather_kv(void* k_out, void* v_out,
                       const void* key_cache, const void* value_cache,
                       const int32_t* block_tables, const int32_t* context_lens,
                       int seq, int num_seqs, int num_kv_heads, int head_dim,
                       int block_size, int num_blocks, int max_blocks_per_seq,
                       int max_context_len, pa_dtype dtype, void* hip_stream);

/*
 * pa_debug_select_kernel -- choose the decode kernel family for later calls in
 * this process: 0 = automatic (matrix-core kernel where supported, else the
 * vector-ALU kernel), 1 = vector-ALU kernel for every shape, 2 = matrix-core
 * kernel only (calls it does not support return PA_ERR_UNSUPPORTED).  Returns
 * the previous setting, or PA_ERR_INVALID_ARG for another value.  For tests
 * that compare the two device paths; process-wide, not synchronised with
 * calls running on other threads.
 */
int pa_debug_select_kernel(int kind);

/*
 * pa_decode_kernel -- the decode kernel family a decode call of this shape
 * runs under the current pa_debug_select_kernel setting: 1 = vector-ALU
 * kernel, 2 = matrix-core kernel.  PA_ERR_UNSUPPORTED when no kernel serves
 * the shape (or the matrix-core kernel is forced and does not),
 * PA_ERR_INVALID_ARG for an unknown dtype or gqa_group_size < 1.  Host only.
 * (Under the automatic setting a float32 call small enough for one
 * partition -- pa_decode_partition_size covering max_context_len -- runs on
 * the vector-ALU kernel, whatever this returns for its shape.)
 */
int pa_decode_kernel(int head_dim, int block_size, int gqa_group_size, pa_dtype dtype);

/*
 * Measurement helpers (not part of the decode path).
 *
 * pa_bench_stream_read -- read `bytes` (multiple of 16) from `src` once, one
 *   workgroup per compute unit streaming a contiguous region with 16-byte
 *   coalesced nontemporal loads, and write the XOR of the 16-byte words each
 *   workgroup read to sink[workgroup] (sink: at least 16 * 65536 bytes; the
 *   entries past the workgroup count are not written).  Gives the practical
 *   HBM read ceiling.
 * pa_bench_copy -- copy `bytes` (multiple of 16) from src to dst; a kernel of
 *   known traffic, used to calibrate hardware byte counters.
 */
int pa_bench_stream_read(const void* src, size_t bytes, void* sink, void* hip_stream);
int pa_bench_copy(void* dst, const void* src, size_t bytes, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
