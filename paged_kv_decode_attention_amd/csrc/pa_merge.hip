// Log-sum-exp merge of context partitions ("reduce locally, then merge
// globally", [MiniPaged-Qwen] §10.2 (2)).  Partition p of (b, h) left
// lse_p = m_p + log2 l_p and o_p = o~_p / l_p (float32, log2 units); the
// online update of [MiniPaged-Qwen] §5.2 applied to whole partitions gives
//   o = sum_p 2^(lse_p - M) o_p / sum_p 2^(lse_p - M),  M = max_p lse_p,
// summed in partition order (deterministic).
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kMergeThreads = 128;

template <typename Tag>
__global__ __launch_bounds__(kMergeThreads) void lse_merge_kernel(DecodeArgs a) {
    __shared__ float sm_w[kMergeThreads];
    __shared__ float sm_red[kMergeThreads / 64];
    __shared__ int sm_nan[kMergeThreads / 64];

    const int h = blockIdx.x;
    const int b = blockIdx.y;
    const int L = a.context_lens[b];
    // One partition (or an invalid length): the partition kernel wrote out.
    if (L <= a.part_len || L > a.max_context_len) return;
    const int np = (L + a.part_len - 1) / a.part_len;
    const uint64_t row0 = ((uint64_t)b * a.num_heads + h) * a.num_parts;
    const float* lse = a.ws_lse + row0;
    const int tid = threadIdx.x;

    float M = -INFINITY;
    int has_nan = 0;
    for (int p = tid; p < np; p += kMergeThreads) {
        const float x = lse[p];
        has_nan |= (x != x);
        M = fmaxf(M, x);
    }
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) {
        M = fmaxf(M, __shfl_xor(M, s));
        has_nan |= __shfl_xor(has_nan, s);
    }
    if ((tid & 63) == 0) {
        sm_red[tid >> 6] = M;
        sm_nan[tid >> 6] = has_nan;
    }
    __syncthreads();
    M = sm_red[0];
    has_nan = sm_nan[0];
#pragma unroll
    for (int w = 1; w < kMergeThreads / 64; ++w) {
        M = fmaxf(M, sm_red[w]);
        has_nan |= sm_nan[w];
    }

    const int D = a.head_dim;
    float num = 0.0f, den = 0.0f;
    for (int p0 = 0; p0 < np; p0 += kMergeThreads) {
        __syncthreads();
        if (p0 + tid < np) sm_w[tid] = fast_exp2(lse[p0 + tid] - M);
        __syncthreads();
        const int cnt = min(kMergeThreads, np - p0);
        for (int k = 0; k < cnt; ++k) {
            const float w = sm_w[k];
            den += w;
            if (tid < D) num += w * a.ws_out[(row0 + p0 + k) * D + tid];
        }
    }
    if (tid < D) {
        const float o = has_nan ? __builtin_nanf("") : num / den;
        store_elem(Tag(), a.out, ((uint64_t)b * a.num_heads + h) * D + tid, o);
    }
}

template <typename Tag>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t s) {
    dim3 grid(a.num_heads, a.num_seqs);
    hipLaunchKernelGGL((lse_merge_kernel<Tag>), grid, dim3(kMergeThreads), 0, s, a);
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
