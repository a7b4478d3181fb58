// Log-sum-exp merge of partial decode states: the "merge globally" half of
// the partitioned reduction ([MiniPaged-Qwen] §10.2 (2)).  One workgroup per
// (sequence, KV head) combines, in token order, the float32 states (lse, o)
// the decode workgroups left for the G query heads of that group
// (merge_pieces in pa_finalize.h).
#include "pa_finalize.h"

namespace pa {
namespace {

constexpr int kMergeThreads = 256;

// Fixed schedule: partitions [p P, p P + P); histories of one partition were
// written directly by the decode kernel.
template <typename Tag>
__global__ __launch_bounds__(kMergeThreads) void merge_fixed(DecodeArgs a) {
    const int kvh = blockIdx.x;
    const int b = blockIdx.y;
    const int L = a.context_lens[b];
    if (L <= a.part_len || L > a.max_context_len) return;
    const int nparts = (L + a.part_len - 1) / a.part_len;
    const int head0 = kvh * a.group;
    const FixedPieces pc{a.ws_lse, a.ws_out,
                         ((uint64_t)b * a.num_heads + head0) * a.num_parts, a.num_parts,
                         a.head_dim};
    merge_pieces<Tag>(a, pc, b, head0, a.group, nparts);
}

// Balanced schedule: the pieces of (b, kvh) are the slots of the workgroup
// ranges its chunks fall in.  Also writes the rows the decode kernel skips:
// zeros for an empty history, NaN for an invalid context length.  Only two
// sums over the context lengths are needed (chunks before sequence b, and in
// total), so they are a single workgroup reduction rather than a prefix table.
template <typename Tag>
__global__ __launch_bounds__(kMergeThreads) void merge_balanced(DecodeArgs a) {
    constexpr int NW = kMergeThreads / 64;
    __shared__ int red_before[NW], red_total[NW];
    __shared__ int slots[kMaxBalancedWg + 1];
    __shared__ int live[kMaxBalancedWg + 1];
    const int kvh = blockIdx.x;
    const int b = blockIdx.y;
    const int head0 = kvh * a.group;
    // The first batch of lengths is loaded together with L_b: one memory
    // round trip before the checks below.
    const int L = a.context_lens[b];
    const int i0 = threadIdx.x;
    const int len0 = i0 < a.num_seqs ? a.context_lens[i0] : 0;
    if (L < 0 || L > a.max_context_len) {
        fill_rows<Tag>(a, b, head0, a.group, __builtin_nanf(""));
        return;
    }
    if (L == 0) {
        fill_rows<Tag>(a, b, head0, a.group, 0.0f);
        return;
    }
    int total = seq_chunks(len0, a.max_context_len);
    int before = i0 < b ? total : 0;
    for (int i = i0 + kMergeThreads; i < a.num_seqs; i += kMergeThreads) {
        const int c = seq_chunks(a.context_lens[i], a.max_context_len);
        total += c;
        if (i < b) before += c;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        before += __shfl_xor(before, off);
        total += __shfl_xor(total, off);
    }
    if ((threadIdx.x & 63) == 0) {
        red_before[threadIdx.x >> 6] = before;
        red_total[threadIdx.x >> 6] = total;
    }
    __syncthreads();
    before = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        before += red_before[w];
        total += red_total[w];
    }
    const int H_kv = a.num_kv_heads;
    const int64_t T = (int64_t)H_kv * total;
    const int nb = seq_chunks(L, a.max_context_len);
    const int64_t x0 = (int64_t)H_kv * before + (int64_t)kvh * nb;
    const int w0 = range_owner(x0, T, a.num_wg);
    const int w1 = range_owner(x0 + nb - 1, T, a.num_wg);
    if (w0 == w1) return;   // one range held the whole history
    // piece k is slot [w0][1] for k = 0, then [w][0] for each non-empty
    // range w in (w0, w1]
    const int span = w1 - w0;
    for (int k = threadIdx.x; k < span; k += kMergeThreads) {
        const int w = w0 + 1 + k;
        live[k] = range_start(w, T, a.num_wg) < range_start(w + 1, T, a.num_wg);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int n = 0;
        slots[n++] = 2 * w0 + 1;
        for (int k = 0; k < span; ++k)
            if (live[k]) slots[n++] = 2 * (w0 + 1 + k);
        live[kMaxBalancedWg] = n;
    }
    __syncthreads();
    const BalancedPieces pc{a.ws_lse, a.ws_out, slots, a.head_dim};
    merge_pieces<Tag>(a, pc, b, head0, a.group, live[kMaxBalancedWg]);
}

template <typename Tag>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t s) {
    dim3 grid(a.num_kv_heads, a.num_seqs);
    if (a.schedule == kBalanced)
        hipLaunchKernelGGL((merge_balanced<Tag>), grid, dim3(kMergeThreads), 0, s, a);
    else
        hipLaunchKernelGGL((merge_fixed<Tag>), grid, dim3(kMergeThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_lse_merge(const DecodeArgs& a, pa_dtype dt, hipStream_t s) {
    switch (dt) {
        case PA_F32: return launch_typed<F32>(a, s);
        case PA_F16: return launch_typed<F16>(a, s);
        default: return launch_typed<BF16>(a, s);
    }
}

}  // namespace pa
