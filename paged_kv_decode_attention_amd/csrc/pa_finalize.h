// Shared tail of the decode kernels: merge the per-wavefront online-softmax
// states staged in LDS into one state per head and write it either as the
// final output row or as a float32 partial state (lse, o) for the merge
// kernel; the log-sum-exp merge of such partial states; and the arithmetic
// of the balanced work schedule.
#pragma once

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// Query rows carried by decode row b: 1 without a row map; in verify mode
// the count the row map gives (0: the rows are carried by an earlier decode
// row).  kRows = 1: the launch carries a row map; 0: it does not; -1: test
// a.row_tokens at run time.
// b is the same in every lane of the wavefront (a scalar load).
template <int kRows = -1>
__device__ __forceinline__ int row_tokens(const DecodeArgs& a, int b) {
    typedef __attribute__((address_space(4))) const int32_t ConstRow;
    if (kRows == 0 || (kRows < 0 && a.row_tokens == nullptr)) return 1;
    return __builtin_amdgcn_readfirstlane(((const ConstRow*)a.row_tokens)[b]);
}

// Columns (query heads) of KV head kvh: the group, or with a group split
// into passes of a.group heads (kv_split virtual heads per cache head) the
// heads its pass holds -- a.group, fewer in the last pass of a group that
// does not split evenly.
__device__ __forceinline__ int pass_cols(const DecodeArgs& a, int kvh) {
    if (a.kv_split == 1) return a.group;
    return min(a.group, a.group_mem - (kvh % a.kv_split) * a.group);
}

// Query head of column n < pass_cols(a, kvh) of KV head kvh: kvh G + n, or
// with a split group, head j G' + n of cache head kvh / kv_split's group
// (j = kvh % kv_split, G' = a.group heads per pass).
__device__ __forceinline__ int col_head(const DecodeArgs& a, int kvh, int n) {
    if (a.kv_split == 1) return kvh * a.group + n;
    const int h = kvh / a.kv_split;
    return h * a.group_mem + (kvh - h * a.kv_split) * a.group + n;
}

// [S, H] row index (of out, query and the fixed schedule's partition states)
// of column n of decode row b, KV head kvh: query row b + n / G, head
// col_head(kvh, n % G).  Without a row map n < G, so this is
// b H + col_head(kvh, n).  (Row maps come without a split: G = a.group.)
__device__ __forceinline__ uint64_t col_row(const DecodeArgs& a, int b, int kvh, int n) {
    const int t = n / a.group;
    return (uint64_t)(b + t) * a.num_heads + col_head(a, kvh, n - t * a.group);
}

// Columns n0 .. n0 + ncols - 1 of decode row b, KV head kvh, set to one value
// (0 for an empty history, NaN for an invalid context length).
template <typename Tag>
__device__ __forceinline__ void fill_cols(const DecodeArgs& a, int b, int kvh, int n0,
                                          int ncols, float v) {
    const int D = a.head_dim;
    for (int idx = threadIdx.x; idx < ncols * D; idx += blockDim.x) {
        const int n = idx / D;
        store_elem(Tag(), a.out, col_row(a, b, kvh, n0 + n) * D + (idx - n * D), v);
    }
}

// sm_m/sm_l: [nw][m_stride] reference max (log2 units) and denominator per
// wavefront and column slot; sm_o: un-normalised accumulators, element
// (w, g, d) at w * wave_stride + g * head_stride + d.  Merges the nw states
// of each column n0 + g, g < ncols (the update of [MiniPaged-Qwen] §5.2
// applied to whole states) and writes, for decode row b, KV head kvh:
//   part < 0 : the output row, o~ / l rounded once to the output type;
//   else     : partition state `part` of the fixed schedule: o~ / l and
//              m + log2 l at row col_row * num_parts + part.
// A column with no token in the partition (a verify column whose causal end
// lies before it) leaves the empty state: lse -inf, o 0.
template <typename Tag>
__device__ __forceinline__ void finalize_state(
    const DecodeArgs& a, const float* sm_m, const float* sm_l, const float* sm_o, int nw,
    int m_stride, int wave_stride, int head_stride, int b, int kvh, int n0, int ncols, bool bad,
    int part) {
    const int D = a.head_dim;
    for (int idx = threadIdx.x; idx < ncols * D; idx += blockDim.x) {
        const int g = idx / D;
        const int d = idx - g * D;
        float M = -INFINITY;
        for (int w = 0; w < nw; ++w) M = fmaxf(M, sm_m[w * m_stride + g]);
        float den = 0.0f, num = 0.0f;
        for (int w = 0; w < nw; ++w) {
            const float e = rescale_weight(sm_m[w * m_stride + g], M);
            den += e * sm_l[w * m_stride + g];
            num += e * sm_o[w * wave_stride + g * head_stride + d];
        }
        float o = den == 0.0f ? 0.0f : num / den;
        if (bad) o = __builtin_nanf("");
        const uint64_t r = col_row(a, b, kvh, n0 + g);
        if (part < 0) {
            store_elem(Tag(), a.out, r * D + d, a.out_scale * o);
        } else {
            const uint64_t row = r * a.num_parts + part;
            a.ws_out[row * D + d] = o;
            if (d == 0) a.ws_lse[row] = bad ? __builtin_nanf("") : M + __log2f(den);
        }
    }
}

// Log-sum-exp merge of the npieces partition states of columns 0 .. ncols-1
// of decode row b, KV head kvh ("reduce locally, then merge globally",
// [MiniPaged-Qwen] §10.2 (2)):
//   o = sum_p 2^(lse_p - M) o_p / sum_p 2^(lse_p - M),  M = max_p lse_p,
// the online update of §5.2 applied to whole pieces: batches of kBatch
// pieces are loaded together (one memory round trip per batch) and folded
// into a running (max, denominator, numerator).  Always in piece (token)
// order, so the result is deterministic.
template <typename Tag>
__device__ __forceinline__ void merge_pieces(const DecodeArgs& a, int b, int kvh, int ncols,
                                             int npieces) {
    constexpr int kBatch = 8;
    const int D = a.head_dim;
    const int D4 = D / 4;
    for (int it = threadIdx.x; it < ncols * D4; it += blockDim.x) {
        const int g = it / D4;
        const int d4 = it - g * D4;
        const uint64_t r = col_row(a, b, kvh, g);
        const float* lse_r = a.ws_lse + r * a.num_parts;
        const f32x4* o_r = reinterpret_cast<const f32x4*>(a.ws_out + r * a.num_parts * D) + d4;
        float M = -INFINITY, den = 0.0f;
        f32x4 num = {0.f, 0.f, 0.f, 0.f};
        int has_nan = 0;
        for (int p0 = 0; p0 < npieces; p0 += kBatch) {
            f32x4 o[kBatch];
            float lse[kBatch];
#pragma unroll
            for (int k = 0; k < kBatch; ++k) {
                const int p = min(p0 + k, npieces - 1);
                o[k] = o_r[(uint64_t)p * D4];
                lse[k] = p0 + k < npieces ? lse_r[p] : -INFINITY;
            }
            float mb = M;
#pragma unroll
            for (int k = 0; k < kBatch; ++k) {
                has_nan |= (lse[k] != lse[k]);
                mb = fmaxf(mb, lse[k]);
            }
            const float keep = rescale_weight(M, mb);
            den *= keep;
            num *= keep;
#pragma unroll
            for (int k = 0; k < kBatch; ++k) {
                const float w = rescale_weight(lse[k], mb);
                den += w;
                num += w * o[k];
            }
            M = mb;
        }
        const uint64_t out0 = r * D + 4 * d4;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            store_elem(Tag(), a.out, out0 + e,
                       has_nan ? __builtin_nanf("") : a.out_scale * (num[e] / den));
    }
}

// Offset of decode row b's block-table row (rows of several decode rows may
// be one sequence's in verify mode).
// b is the same in every lane of the wavefront (read through the constant
// address space, so the read is a scalar load and the row stays uniform).
// kRows = 1: the launch carries a row map (verify mode); 0: it does not;
// -1: test a.table_rows at run time.
template <int kRows = -1>
__device__ __forceinline__ uint64_t table_row_offset(const DecodeArgs& a, int b) {
    typedef __attribute__((address_space(4))) const int32_t ConstRow;
    int r = b;
    if (kRows == 1 || (kRows < 0 && a.table_rows != nullptr))
        r = __builtin_amdgcn_readfirstlane(((const ConstRow*)a.table_rows)[b]);
    return (uint64_t)r * a.max_blocks_per_seq;
}

// ---- arithmetic of the balanced schedule (shared by decode and merge) ----

// 32-token chunks of a history of L tokens; 0 for an empty or invalid length.
__device__ __forceinline__ int seq_chunks(int L, int max_context_len) {
    return (L <= 0 || L > max_context_len) ? 0 : (L + kChunk - 1) / kChunk;
}

// Work units of a history of L tokens whose start counts su units (the
// balanced schedule's cost model, kChunkUnits per chunk).
__device__ __forceinline__ int seq_units(int L, int max_context_len, int su) {
    const int nb = seq_chunks(L, max_context_len);
    return nb == 0 ? 0 : su + kChunkUnits * nb;
}

// Chunks of a history of nb chunks (start: su units) that start before unit
// u (0 <= u <= its units): the first chunk a range beginning at u holds.
__device__ __forceinline__ int chunks_before_unit(int u, int nb, int su) {
    return u <= su ? 0 : min(nb, (u - su + kChunkUnits - 1) / kChunkUnits);
}

// First work item of workgroup w when T items are cut into nwg equal ranges,
// and the workgroup whose range holds item x (T > 0).
// (32-bit division when the operands allow: the 64-bit one is a long
// scalar routine, and these sit on the path to a workgroup's first load.)
__device__ __forceinline__ int64_t range_start(int w, int64_t T, int nwg) {
    if ((T >> 21) == 0) return (uint32_t)w * (uint32_t)T / (uint32_t)nwg;   // w <= nwg <= 2^11
    return (int64_t)w * T / nwg;
}
__device__ __forceinline__ int range_owner(int64_t x, int64_t T, int nwg) {
    const int64_t num = (x + 1) * nwg + T - 1;
    if ((num >> 32) == 0) return (int)((uint32_t)num / (uint32_t)T) - 1;
    return (int)(num / T - 1);
}

// Inclusive prefix sums of seq_units (start: su units) over the decode rows
// into LDS, pref[0] = 0, pref[1 + i] = units of rows 0..i (per KV head),
// and the rows' context lengths len_of(i) into lens[0 .. num_seqs).  wsum:
// LDS scratch of one int per wavefront.  Called by every thread of the
// workgroup (kDecodeThreads of them, num_seqs <= kMaxBalancedSeqs).  Thread
// t takes the E = ceil(num_seqs / kDecodeThreads) consecutive rows from
// unit_prefix_row(t, num_seqs): its lengths share one cache line (after the
// first read the rest are cache hits), its own sums run in registers, and
// one scan over the threads' totals (two barriers) places them.  A pass per 256 rows waited on each pass's reads
// and barriers in turn: with 2048 rows the table took 5.8 us from the
// workgroup's start (2048 x U[32, 255] tokens: 116.7 -> 113.5 us per call).
// Up to 256 rows keep the one-row-a-thread pass (the same instructions as
// before, which the register allocation of the streaming loop after it
// turned out to depend on).
__device__ __forceinline__ int unit_prefix_rows(int num_seqs) {
    return (num_seqs + kDecodeThreads - 1) / kDecodeThreads;
}
__device__ __forceinline__ int unit_prefix_row(int t, int num_seqs) {
    return t * unit_prefix_rows(num_seqs);
}
template <typename LenOf>
__device__ __forceinline__ void unit_prefix(const DecodeArgs& a, int su, LenOf len_of, int* pref,
                                            int* lens, int* wsum) {
    constexpr int kE = (kMaxBalancedSeqs + kDecodeThreads - 1) / kDecodeThreads;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int S = a.num_seqs;
    if (threadIdx.x == 0) pref[0] = 0;
    if (S <= kDecodeThreads) {
        // one row a thread
        const int i = threadIdx.x;
        const int L = i < S ? len_of(i) : 0;
        if (i < S) lens[i] = L;
        int x = i < S ? seq_units(L, a.max_context_len, su) : 0;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(x, off);
            if (lane >= off) x += y;
        }
        if (lane == 63) wsum[wave] = x;
        __syncthreads();
        int add = 0;
        for (int w = 0; w < wave; ++w) add += wsum[w];
        if (i < S) pref[1 + i] = x + add;
        __syncthreads();
        return;
    }
    const int E = unit_prefix_rows(S);
    const int i0 = unit_prefix_row(threadIdx.x, S);
    int L[kE], run[kE];
#pragma unroll
    for (int j = 0; j < kE; ++j) L[j] = j < E && i0 + j < S ? len_of(i0 + j) : 0;
    int x = 0;
#pragma unroll
    for (int j = 0; j < kE; ++j) {
        x += j < E && i0 + j < S ? seq_units(L[j], a.max_context_len, su) : 0;
        run[j] = x;
    }
    int y = x;     // inclusive scan of the threads' totals over the wavefront
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int z = __shfl_up(y, off);
        if (lane >= off) y += z;
    }
    if (lane == 63) wsum[wave] = y;
    __syncthreads();
    int add = y - x;   // units of the rows before i0
    for (int w = 0; w < wave; ++w) add += wsum[w];
#pragma unroll
    for (int j = 0; j < kE; ++j) {
        if (j < E && i0 + j < S) {
            lens[i0 + j] = L[j];
            pref[1 + i0 + j] = run[j] + add;
        }
    }
    __syncthreads();
}

// Sequence whose units (counted per kv head) contain flattened work item x:
// the largest b with num_kv_heads * pref[b] <= x and a non-empty history.
// Wavefront-parallel: each round tests 64 evenly spaced candidates with one
// LDS read per lane and keeps the span after the last that passes (one
// round up to 64 sequences, two up to 4096).  Called with the whole
// wavefront active; the result is the same in every lane.
__device__ __forceinline__ int find_seq(const int* pref, int num_seqs, int num_kv_heads,
                                        int64_t x) {
    const int lane = threadIdx.x & 63;
    int lo = 0, n = num_seqs;      // answer in [lo, lo + n)
    while (n > 1) {
        const int stride = (n + 63) >> 6;
        const int i = lo + lane * stride;
        const bool ok = lane * stride < n && (int64_t)num_kv_heads * pref[i] <= x;
        const uint64_t m = __ballot(ok);        // lanes 0 .. j pass (pref is nondecreasing)
        const int j = 63 - __builtin_clzll(m);  // lane 0 passes: pref[lo] <= x
        lo += j * stride;
        n = min(stride, n - j * stride);
    }
    return __builtin_amdgcn_readfirstlane(lo);
}

}  // namespace pa
