// Last step of a decode partition workgroup, shared by both decode kernels:
// merge the per-wavefront online-softmax states staged in LDS and write either
// the final output row (history fits one partition) or the partition's
// float32 state for the log-sum-exp merge.
#pragma once

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// sm_m/sm_l: [nw][16] running max (log2 units) and denominator per wavefront
// and head slot; sm_o: un-normalised accumulators, element (w, g, d) at
// w * wave_stride + g * head_stride + d.  Heads head0 .. head0 + nheads - 1
// of sequence b are written.
template <typename Tag>
__device__ __forceinline__ void finalize_partition(
    const DecodeArgs& a, const float* sm_m, const float* sm_l, const float* sm_o,
    int nw, int wave_stride, int head_stride, int head0, int nheads, int b,
    int part, int nparts_b, bool bad) {
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
        const int h = head0 + g;
        if (nparts_b == 1) {
            store_elem(Tag(), a.out, ((uint64_t)b * a.num_heads + h) * D + d, o);
        } else {
            const uint64_t row = ((uint64_t)b * a.num_heads + h) * a.num_parts + part;
            a.ws_out[row * D + d] = o;
            if (d == 0) a.ws_lse[row] = bad ? __builtin_nanf("") : M + __log2f(den);
        }
    }
}

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

}  // namespace pa
