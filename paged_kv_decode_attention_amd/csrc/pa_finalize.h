// Shared tail of the decode kernels: merge the per-wavefront online-softmax
// states staged in LDS into one state per head and write it either as the
// final output row or as a float32 partial state (lse, o) for the merge
// kernel; the log-sum-exp merge of such partial states; and the arithmetic
// of the balanced work schedule.
#pragma once

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// Rows of sequence b, heads head0 .. head0+nheads-1, set to one value
// (0 for an empty history, NaN for an invalid context length).
template <typename Tag>
__device__ __forceinline__ void fill_rows(const DecodeArgs& a, int b, int head0,
                                          int nheads, float v) {
    const int D = a.head_dim;
    for (int idx = threadIdx.x; idx < nheads * D; idx += blockDim.x) {
        const int g = idx / D;
        store_elem(Tag(), a.out, ((uint64_t)b * a.num_heads + head0 + g) * D + (idx - g * D), v);
    }
}

// sm_m/sm_l: [nw][16] reference max (log2 units) and denominator per
// wavefront and head slot; sm_o: un-normalised accumulators, element
// (w, g, d) at w * wave_stride + g * head_stride + d.  Merges the nw states
// of each head g < nheads (the update of [MiniPaged-Qwen] §5.2 applied to
// whole states) and writes, for heads head0 + g of sequence b:
//   plse == nullptr : out row = o~ / l (rounded once to the output type);
//   otherwise       : po[g * po_hs + d] = o~ / l, plse[g * plse_hs] = m + log2 l.
template <typename Tag>
__device__ __forceinline__ void finalize_state(
    const DecodeArgs& a, const float* sm_m, const float* sm_l, const float* sm_o, int nw,
    int wave_stride, int head_stride, int head0, int nheads, int b, bool bad, float* plse,
    int plse_hs, float* po, int po_hs) {
    const int D = a.head_dim;
    for (int idx = threadIdx.x; idx < nheads * D; idx += blockDim.x) {
        const int g = idx / D;
        const int d = idx - g * D;
        float M = -INFINITY;
        for (int w = 0; w < nw; ++w) M = fmaxf(M, sm_m[w * 16 + g]);
        float den = 0.0f, num = 0.0f;
        for (int w = 0; w < nw; ++w) {
            const float e = rescale_weight(sm_m[w * 16 + g], M);
            den += e * sm_l[w * 16 + g];
            num += e * sm_o[w * wave_stride + g * head_stride + d];
        }
        float o = num / den;
        if (bad) o = __builtin_nanf("");
        if (plse == nullptr) {
            store_elem(Tag(), a.out, ((uint64_t)b * a.num_heads + head0 + g) * D + d,
                       a.out_scale * o);
        } else {
            po[(uint64_t)g * po_hs + d] = o;
            if (d == 0) plse[(uint64_t)g * plse_hs] = bad ? __builtin_nanf("") : M + __log2f(den);
        }
    }
}

// Partial states of the fixed schedule: partition p of head head0 + g.
struct FixedPieces {
    const float* lse;    // a.ws_lse
    const float* o;      // a.ws_out
    uint64_t row0;       // (b * H + head0) * num_parts
    int num_parts;
    int D;
    __device__ __forceinline__ float lse_at(int p, int g) const {
        return lse[row0 + (uint64_t)g * num_parts + p];
    }
    __device__ __forceinline__ const f32x4* o_at(int p, int g) const {
        return reinterpret_cast<const f32x4*>(o + (row0 + (uint64_t)g * num_parts + p) * D);
    }
};

// Log-sum-exp merge of npieces partial states of heads head0 .. head0 +
// nheads - 1 of sequence b ("reduce locally, then merge globally",
// [MiniPaged-Qwen] §10.2 (2)):
//   o = sum_p 2^(lse_p - M) o_p / sum_p 2^(lse_p - M),  M = max_p lse_p,
// the online update of §5.2 applied to whole pieces: batches of kBatch
// pieces are loaded together (one memory round trip per batch) and folded
// into a running (max, denominator, numerator).  Always in piece (token)
// order, so the result is deterministic.
template <typename Tag, typename Pieces>
__device__ __forceinline__ void merge_pieces(const DecodeArgs& a, const Pieces& pc, int b,
                                             int head0, int nheads, int npieces) {
    constexpr int kBatch = 8;
    const int D = a.head_dim;
    const int D4 = D / 4;
    for (int it = threadIdx.x; it < nheads * D4; it += blockDim.x) {
        const int g = it / D4;
        const int d4 = it - g * D4;
        float M = -INFINITY, den = 0.0f;
        f32x4 num = {0.f, 0.f, 0.f, 0.f};
        int has_nan = 0;
        for (int p0 = 0; p0 < npieces; p0 += kBatch) {
            f32x4 o[kBatch];
            float lse[kBatch];
#pragma unroll
            for (int k = 0; k < kBatch; ++k) {
                const int p = min(p0 + k, npieces - 1);
                o[k] = pc.o_at(p, g)[d4];
                lse[k] = p0 + k < npieces ? pc.lse_at(p, g) : -INFINITY;
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
        const uint64_t out0 = ((uint64_t)b * a.num_heads + head0 + g) * D + 4 * d4;
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

// First work item of workgroup w when T items are cut into nwg equal ranges,
// and the workgroup whose range holds item x (T > 0).
__device__ __forceinline__ int64_t range_start(int w, int64_t T, int nwg) {
    return (int64_t)w * T / nwg;
}
__device__ __forceinline__ int range_owner(int64_t x, int64_t T, int nwg) {
    return (int)(((x + 1) * nwg + T - 1) / T - 1);
}

// Inclusive prefix sums of seq_chunks over the sequences into LDS:
// pref[0] = 0, pref[1 + i] = chunks of sequences 0..i.  wsum: LDS scratch of
// one int per wavefront.  Called by every thread of the workgroup.
__device__ __forceinline__ void chunk_prefix(const DecodeArgs& a, int* pref, int* wsum) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;
    if (threadIdx.x == 0) pref[0] = 0;
    for (int base = 0; base < a.num_seqs; base += blockDim.x) {
        const int i = base + threadIdx.x;
        int x = i < a.num_seqs ? seq_chunks(a.context_lens[i], a.max_context_len) : 0;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(x, off);
            if (lane >= off) x += y;
        }
        if (lane == 63) wsum[wave] = x;
        __syncthreads();
        int add = pref[base];
        for (int w = 0; w < wave && w < nw; ++w) add += wsum[w];
        if (i < a.num_seqs) pref[1 + i] = x + add;
        __syncthreads();
    }
}

// Sequence whose chunks (counted per kv head) contain flattened work item x:
// the largest b with num_kv_heads * pref[b] <= x and a non-empty history.
__device__ __forceinline__ int find_seq(const int* pref, int num_seqs, int num_kv_heads,
                                        int64_t x) {
    int lo = 0, hi = num_seqs - 1;     // answer in [lo, hi]
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((int64_t)num_kv_heads * pref[mid] <= x) lo = mid; else hi = mid - 1;
    }
    return lo;
}

}  // namespace pa
