// Internal declarations shared by the host API and the kernel launchers of
// libpagedattn.so.  Not part of the public ABI (that is include/pagedattn.h).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "pagedattn.h"

namespace pa {

// Everything a decode launch needs; passed to the kernels by value.
struct DecodeArgs {
    void* out;                 // [S, H, D] dtype
    const void* query;         // [S, H, D] dtype
    const void* key_cache;     // [N, H_kv, BS, D] dtype
    const void* value_cache;   // [N, H_kv, BS, D] dtype
    const int32_t* block_tables;   // [S, W]
    const int32_t* context_lens;   // [S]
    const int32_t* table_rows;     // [S]: block-table row of decode row b, or null (row b)
    // [S]: query rows carried by decode row b, or null (1 each).  Decode row
    // b with n_b > 0 query rows serves rows b .. b + n_b - 1 of one sequence
    // as n_b * group "columns": column n is query row b + n / group, head
    // kvh * group + n % group, and attends the context_lens[b] - (n_b - 1 -
    // n / group) oldest positions.  n_b = 0: the rows are carried by an
    // earlier decode row (its context_lens entry is 0 and nothing is written).
    const int32_t* row_tokens;
    // Verify rows on the balanced schedule: the kernels compute the row map
    // (verify_row) themselves from query_start [num_src_seqs + 1] and
    // src_lens [num_src_seqs] (the sequences' context lengths), with
    // table_rows, row_tokens and context_lens unused; null otherwise.
    const int32_t* query_start;
    const int32_t* src_lens;
    int num_src_seqs, max_query_len;
    int row_group;             // u: query rows a decode row carries at most
    const void* new_key;       // [S, H_kv, D] appended token per sequence, or null
    const void* new_value;     // [S, H_kv, D]
    float* ws_lse;             // [S, H, num_parts] float32 (log2 units)
    float* ws_out;             // [S, H, num_parts, D] float32
    int* ws_meta;              // balanced schedule: [num_wg][4] tail-segment records
    // num_kv_heads and group are the kernel's (virtual) KV heads and the
    // query heads each serves at most: a group of group_mem heads too large
    // for one pass of the matrix-core kernel is served as kv_split passes,
    // KV head h standing for kv_split virtual heads h kv_split + j, pass j
    // holding query heads h group_mem + j group + n for n < group (fewer in
    // the last pass when group_mem is not a multiple of group: pass_cols);
    // the caches are addressed with KV head virtual / kv_split of
    // kv_heads_mem.  Without a split kv_split = 1, group = group_mem.
    int num_seqs, num_heads, num_kv_heads, group, head_dim, block_size;
    int kv_split, kv_heads_mem, group_mem;
    int num_blocks, max_blocks_per_seq, max_context_len;
    int part_len;              // tokens per context partition (fixed schedule)
    int num_parts;             // ceil(max_context_len / part_len)
    int schedule;              // kFixed or kBalanced
    int num_wg;                // workgroups of the balanced schedule
    int col_tiles;             // 16-column tiles per decode row (2 only for verify rows
                               //   of the matrix-core kernel); slots hold 16 * col_tiles
    float scale_log2;          // scale * log2(e) (* k_scale): scores in log2 units
    int kv_format;             // KvFormat
    float out_scale;           // v_scale for 8-bit caches, else 1: output = out_scale * o
    float k_inv_scale;         // fp32(1 / k_scale), fp32(1 / v_scale): the appended
    float v_inv_scale;         //   token's quantisation (8-bit caches)
};

// Storage of the caches: the query's 16-bit type, or OCP FP8 E4M3 or signed
// INT8 codes with one scale per cache.
enum KvFormat { kKvSame = 0, kKvE4M3 = 1, kKvI8 = 2 };

// Work schedules of the decode kernels.
//   kFixed: workgroup (kv head, sequence, p) takes tokens [p P, (p+1) P);
//     partition states are indexed [S, H, num_parts].
//   kBalanced: the (sequence, kv head, work unit) list (kChunkUnits per
//     32-token chunk plus a start cost per history), in that order, is cut
//     into num_wg equal contiguous ranges, one per workgroup;
//     a (sequence, kv head) cut by a range boundary leaves one state per
//     piece in slot [w][0] (the piece that continues from workgroup w-1) or
//     [w][1] (the piece that continues into w+1), each slot holding up to
//     kMaxGroup heads.  Record ws_meta[w] = {key, w1 + 65536 n, T lo, T hi}
//     names the segment whose first piece is slot [w][1] (key = sequence *
//     H_kv + KV head, -1 if none), the last range w1 holding it, the query
//     rows n its decode row carries, and the work-list size T; the decode
//     kernel writes every record on every launch, and also the output rows
//     of decode rows with an empty (zeros) or invalid (NaN) history.
enum Schedule { kFixed = 0, kBalanced = 1 };
constexpr int kMaxGroup = 16;          // heads per column tile (matrix-core kernel)
constexpr int kMaxColTiles = 2;        // column tiles per decode row (verify)
constexpr int kMaxBalancedWg = 1024;   // workspace is sized for this many
constexpr int kMaxBalancedSeqs = 2048; // prefix table of the balanced schedule (dynamic LDS)
// Verify rows on the balanced schedule compute their row map in the decode
// kernel's prologue from the sequences' query starts and lengths, staged in
// its edge LDS (at least 8704 floats): up to this many sequences.
constexpr int kMaxVerifyFoldSeqs = 4096;

constexpr int kDecodeThreads = 256;   // 4 wavefronts per workgroup
constexpr int kChunk = 32;            // tokens a wavefront handles per step
// Work units of the balanced schedule.  A (decode row, KV head) history of
// nb chunks counts s + kChunkUnits nb units: its chunk c starts at unit
// s + kChunkUnits c, and the s units before its first chunk stand for the
// fixed cost of starting a history (loading its table row and first chunk
// with nothing else in flight, and writing its state).  s depends on the
// cache format, whose chunks take different times to stream; both values
// are tuned by measurement (16-bit: 1.5 chunks, timed wavefronts show about
// 2.3 us per history start against 2.9 us per chunk when a wavefront's
// range holds many short histories; 8-bit codes, half the bytes per chunk:
// 3 chunks).  A range of units holds the chunks that start inside it.
constexpr int kChunkUnits = 2;
constexpr int kStartUnits16 = 3;
constexpr int kStartUnits8 = 6;
constexpr int kMaxStartUnits = 6;

// Kernel families.
enum KernelKind { kAuto = 0, kGeneric = 1, kMfma = 2 };

bool mfma_supported(pa_dtype dt, int head_dim, int block_size, int group);
// Passes the matrix-core kernel serves a group of `group` query heads per KV
// head in (1: directly; otherwise the fewest passes of at most 16 heads, 32
// at head_dim 64/128), or 0 if it cannot (dtype or shape).
int mfma_split(pa_dtype dt, int head_dim, int block_size, int group);
// Query heads per pass of a group served in `split` passes: ceil(group /
// split); the last pass holds the remainder, at least one head.
inline int mfma_pass_group(int group, int split) { return (group + split - 1) / split; }
// Workgroups of the matrix-core kernel resident per compute unit.
int mfma_workgroups_per_cu(int head_dim);
hipError_t launch_decode_mfma(const DecodeArgs& a, pa_dtype dt, hipStream_t s);
hipError_t launch_decode_mfma_d64(const DecodeArgs& a, pa_dtype dt, hipStream_t s);
hipError_t launch_decode_mfma_d128(const DecodeArgs& a, pa_dtype dt, hipStream_t s);
hipError_t launch_decode_mfma_d256(const DecodeArgs& a, pa_dtype dt, hipStream_t s);
hipError_t launch_decode_generic(const DecodeArgs& a, pa_dtype dt, hipStream_t s);
hipError_t launch_lse_merge(const DecodeArgs& a, pa_dtype dt, hipStream_t s);

hipError_t launch_reshape_and_cache(const void* key, const void* value,
                                    void* key_cache, void* value_cache,
                                    const int64_t* slots, int num_tokens,
                                    int num_kv_heads, int row_bytes,
                                    int block_size, int num_blocks,
                                    hipStream_t s);

// Store the newest token of every sequence (history position L_b - 1) into
// its cache slot, read from the sequence's block table.
hipError_t launch_append_tokens(const void* key, const void* value, void* key_cache,
                                void* value_cache, const int32_t* block_tables,
                                const int32_t* context_lens, int num_seqs, int num_kv_heads,
                                int row_bytes, int block_size, int num_blocks,
                                int max_blocks_per_seq, int max_context_len, hipStream_t s);

// Cache write into 8-bit caches: each value x of key/value (dtype src_dtype)
// is stored as Q(fp32(x) * inv_scale), Q = INT8 (int8) or E4M3 (otherwise).
hipError_t launch_reshape_and_cache_q8(const void* key, const void* value, void* key_cache,
                                       void* value_cache, const int64_t* slots, int num_tokens,
                                       int num_kv_heads, int head_dim, int block_size,
                                       int num_blocks, pa_dtype src_dtype, bool int8,
                                       float k_inv_scale, float v_inv_scale, hipStream_t s);

// Verify mode: for every query row r < total_q, the decode row that starts
// at r -- the block-table row of its sequence, the effective history length
// of its last query row (-1 for an invalid row) and the number of query rows
// it carries (up to tokens_per_row consecutive rows of one sequence, 0 for a
// row carried by an earlier one; an invalid row carries itself alone).
hipError_t launch_verify_rows(const int32_t* query_start, const int32_t* context_lens,
                              int num_seqs, int total_queries, int max_query_len,
                              int max_context_len, int tokens_per_row, int32_t* table_rows,
                              int32_t* lens, int32_t* row_tokens, hipStream_t s);

// Copy whole blocks of both caches: pair i = (src, dst) in device memory.
hipError_t launch_copy_blocks(void* key_cache, void* value_cache, const int32_t* pairs,
                              int num_pairs, int block_bytes, int num_blocks, hipStream_t s);

// Record `msg` as the calling thread's pa_last_error text and return status.
int report_error(int status, const char* msg);

hipError_t launch_gather(void* k_out, void* v_out, const void* key_cache,
                         const void* value_cache, const int32_t* block_tables,
                         const int32_t* context_lens, int seq,
                         int num_kv_heads, int row_bytes, int block_size,
                         int num_blocks, int max_blocks_per_seq,
                         int max_context_len, hipStream_t s);

hipError_t launch_stream_read(const void* src, size_t bytes, void* sink, hipStream_t s);
hipError_t launch_copy(void* dst, const void* src, size_t bytes, hipStream_t s);

}  // namespace pa
