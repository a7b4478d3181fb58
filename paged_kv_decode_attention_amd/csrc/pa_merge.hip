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
// zeros for an empty history, NaN for an invalid context length.
template <typename Tag>
__global__ __launch_bounds__(kMergeThreads) void merge_balanced(DecodeArgs a) {
    __shared__ int pref[kMaxBalancedSeqs + 1];
    __shared__ int wsum[kMergeThreads / 64];
    __shared__ int slots[kMaxBalancedWg + 1];
    __shared__ int npieces;
    const int kvh = blockIdx.x;
    const int b = blockIdx.y;
    const int head0 = kvh * a.group;
    const int L = a.context_lens[b];
    if (L < 0 || L > a.max_context_len) {
        fill_rows<Tag>(a, b, head0, a.group, __builtin_nanf(""));
        return;
    }
    if (L == 0) {
        fill_rows<Tag>(a, b, head0, a.group, 0.0f);
        return;
    }
    chunk_prefix(a, pref, wsum);
    const int H_kv = a.num_kv_heads;
    const int64_t T = (int64_t)H_kv * pref[a.num_seqs];
    const int nb = pref[b + 1] - pref[b];
    const int64_t x0 = (int64_t)H_kv * pref[b] + (int64_t)kvh * nb;
    const int w0 = range_owner(x0, T, a.num_wg);
    const int w1 = range_owner(x0 + nb - 1, T, a.num_wg);
    if (w0 == w1) return;   // one range held the whole history
    if (threadIdx.x == 0) {
        int k = 0;
        slots[k++] = 2 * w0 + 1;
        for (int w = w0 + 1; w <= w1; ++w)
            if (range_start(w, T, a.num_wg) < range_start(w + 1, T, a.num_wg)) slots[k++] = 2 * w;
        npieces = k;
    }
    __syncthreads();
    const BalancedPieces pc{a.ws_lse, a.ws_out, slots, a.head_dim};
    merge_pieces<Tag>(a, pc, b, head0, a.group, npieces);
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
