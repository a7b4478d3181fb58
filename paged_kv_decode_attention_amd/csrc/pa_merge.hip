// Log-sum-exp merge of partial decode states: the "merge globally" half of
// the partitioned reduction ([MiniPaged-Qwen] §10.2 (2)).  The float32
// states (lse, o) the decode workgroups left for the columns of a (decode
// row, KV head) -- its G query heads, or in verify mode the (query row, head)
// pairs it carries -- are combined in token order.
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
    merge_pieces<Tag>(a, b, kvh, row_tokens(a, b) * pass_cols(a, kvh), nparts);
}

// Balanced schedule.  Workgroup w merges the segment whose first piece
// range w left in slot [w][1], as named by record ws_meta[w]: the pieces
// are [w][1] and [w'][0] for every non-empty range w' in (w, w1], in token
// order, for the n G columns of its decode row (n query rows carried, from
// the record).  The record and the first kSpec candidate pieces are loaded
// together (one memory round trip for the common case of a segment spread
// over at most kSpec ranges).  (The rows of decode rows with no history are
// written by the decode kernel.)  A thread takes 4 consecutive d of one
// column (NC columns per slot, 16 or 32): NC * D / 4 threads.
// The first arguments repeat what the first loads need (records, slots, the
// range count and the columns a decode row can have: G, or u G for verify
// rows), so that the compiler preloads them into scalar registers and the
// loads leave without a round trip for the kernel arguments.
// A history of more than kSpec pieces (long histories on few sequences:
// 64 pieces each for one sequence of 131072 tokens) is folded by nsub
// subsets of the workgroup's threads at once -- the threads past the
// columns' would otherwise idle -- subset j taking pieces j, j + nsub, ...,
// kSubBatch per memory round trip; the subsets' states are then combined in
// LDS, in subset order (the same order on every call).
constexpr int kMaxSub = 8;
constexpr int kSubBatch = 16;

template <typename Tag, int D, int NC>
__global__ __launch_bounds__(NC * D / 4) void merge_balanced(
    const int4* __restrict__ ws_meta, const float* __restrict__ ws_out,
    const float* __restrict__ ws_lse, int nwg, int max_cols, DecodeArgs a) {
    constexpr int kSpec = 3;
    constexpr int D4 = D / 4;
    __shared__ float sub_m[NC * D4], sub_den[NC * D4];
    __shared__ f32x4 sub_num[NC * D4];
    __shared__ int sub_nan[NC * D4];
    const int w = blockIdx.x;
    const int items = max_cols * D4;                // one thread per (column, 4 d)
    const int nsub = max(1, min((int)(NC * D4) / items, kMaxSub));
    const int j = threadIdx.x / items;              // this thread's piece subset
    const int it = threadIdx.x - j * items;
    const int g = it / D4;
    const int d = (it % D4) * 4;
    if (j >= nsub) return;                          // no subset: load nothing
    auto slot_row = [&](int slot) { return (uint64_t)slot * NC + g; };
    const int4 meta = ws_meta[w];
    f32x4 o[kSpec];
    float lse[kSpec];
#pragma unroll
    for (int k = 0; k < kSpec; ++k) {
        const int slot = k == 0 ? 2 * w + 1 : 2 * min(w + k, nwg - 1);
        o[k] = *reinterpret_cast<const f32x4*>(ws_out + slot_row(slot) * D + d);
        lse[k] = ws_lse[slot_row(slot)];
    }
    // The pieces' loads, and those of the kernel arguments used below, go
    // out with the record's: without these uses the compiler sinks them
    // below the record's checks, a second round trip.
    const int H_kv = a.num_kv_heads;
    const int nkeys = a.num_seqs * H_kv;
    const int G = a.group;
#pragma unroll
    for (int k = 0; k < kSpec; ++k) asm volatile("" ::"v"(o[k]), "v"(lse[k]));
    asm volatile("" ::"s"(nkeys), "s"(G), "s"(a.num_heads), "s"(a.out), "s"(a.out_scale));
    const int key = meta.x;
    const int w1 = meta.y & 0xffff;
    const int ntok = meta.y >> 16;
    // (a record outside these bounds cannot come from the decode kernel)
    if (key < 0 || key >= nkeys || w1 <= w || w1 >= nwg) return;
    const int64_t T = (int64_t)(uint32_t)meta.z | ((int64_t)meta.w << 32);
    const int b = key / H_kv;
    const int kvh = key - b * H_kv;
    // every range is non-empty when T >= num_wg: pieces are then [w][1],
    // [w+1][0], ..., [w1][0]
    const int npieces = w1 - w + 1;
    // g: column of the decode row (G columns per query row, fewer in the
    // last pass of a split group)
    const bool active = g < ntok * (a.kv_split == 1 ? G : pass_cols(a, kvh));
    if (T >= nwg && npieces > kSpec && nsub > 1) {
        float M = -INFINITY, den = 0.0f;
        f32x4 num = {0.f, 0.f, 0.f, 0.f};
        bool has_nan = false;
        if (active) {
            for (int p0 = j; p0 < npieces; p0 += nsub * kSubBatch) {
                f32x4 ob[kSubBatch];
                float lb[kSubBatch];
#pragma unroll
                for (int k = 0; k < kSubBatch; ++k) {
                    const int p = min(p0 + k * nsub, npieces - 1);
                    const int slot = p == 0 ? 2 * w + 1 : 2 * (w + p);
                    ob[k] = *reinterpret_cast<const f32x4*>(ws_out + slot_row(slot) * D + d);
                    lb[k] = p0 + k * nsub < npieces ? ws_lse[slot_row(slot)] : -INFINITY;
                }
                float mb = M;
#pragma unroll
                for (int k = 0; k < kSubBatch; ++k) {
                    has_nan |= (lb[k] != lb[k]);
                    mb = fmaxf(mb, lb[k]);
                }
                const float keep = rescale_weight(M, mb);
                den *= keep;
                num *= keep;
#pragma unroll
                for (int k = 0; k < kSubBatch; ++k) {
                    const float wgt = rescale_weight(lb[k], mb);
                    den += wgt;
                    num += wgt * ob[k];
                }
                M = mb;
            }
        }
        sub_m[threadIdx.x] = M;
        sub_den[threadIdx.x] = den;
        sub_num[threadIdx.x] = num;
        sub_nan[threadIdx.x] = has_nan;
        __syncthreads();
        if (!active || j != 0) return;
        float Mt = -INFINITY;
        for (int q = 0; q < nsub; ++q) Mt = fmaxf(Mt, sub_m[q * items + it]);
        float dt = 0.0f;
        f32x4 nt = {0.f, 0.f, 0.f, 0.f};
        bool nan_any = false;
        for (int q = 0; q < nsub; ++q) {
            const float wgt = rescale_weight(sub_m[q * items + it], Mt);
            dt += wgt * sub_den[q * items + it];
            nt += wgt * sub_num[q * items + it];
            nan_any |= sub_nan[q * items + it] != 0;
        }
        const uint64_t out0 = col_row(a, b, kvh, g) * D + d;
        store4(Tag(), a.out, out0,
               nan_any ? (f32x4){__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""),
                                 __builtin_nanf("")}
                       : a.out_scale * (nt / dt));
        return;
    }
    if (!active || j != 0) return;
    float M = -INFINITY, den = 0.0f;
    f32x4 num = {0.f, 0.f, 0.f, 0.f};
    bool has_nan = false;
    auto fold = [&](float l, f32x4 v) {     // the update of [MiniPaged-Qwen] §5.2
        has_nan |= (l != l);
        const float m = fmaxf(M, l);
        const float keep = rescale_weight(M, m);
        const float wgt = rescale_weight(l, m);
        den = den * keep + wgt;
        num = num * keep + wgt * v;
        M = m;
    };
    if (T >= nwg && npieces <= kSpec) {
        float m = -INFINITY;
#pragma unroll
        for (int k = 0; k < kSpec; ++k) m = fmaxf(m, k < npieces ? lse[k] : -INFINITY);
#pragma unroll
        for (int k = 0; k < kSpec; ++k) {
            if (k >= npieces) continue;
            has_nan |= (lse[k] != lse[k]);
            const float wgt = rescale_weight(lse[k], m);
            den += wgt;
            num += wgt * o[k];
        }
        M = m;
    } else if (T >= nwg) {
        // contiguous pieces beyond the first kSpec: batches of kBatch loaded
        // together, folded in order
        constexpr int kBatch = 8;
#pragma unroll
        for (int k = 0; k < kSpec; ++k) fold(lse[k], o[k]);
        for (int k0 = kSpec; k0 < npieces; k0 += kBatch) {
            f32x4 ob[kBatch];
            float lb[kBatch];
#pragma unroll
            for (int k = 0; k < kBatch; ++k) {
                const int slot = 2 * (w + min(k0 + k, npieces - 1));
                ob[k] = *reinterpret_cast<const f32x4*>(ws_out + slot_row(slot) * D + d);
                lb[k] = ws_lse[slot_row(slot)];
            }
#pragma unroll
            for (int k = 0; k < kBatch; ++k)
                if (k0 + k < npieces) fold(lb[k], ob[k]);
        }
    } else {
        // fewer work items than workgroups: skip the empty ranges
        fold(lse[0], o[0]);
        for (int w2 = w + 1; w2 <= w1; ++w2) {
            if (range_start(w2, T, nwg) >= range_start(w2 + 1, T, nwg)) continue;
            const int slot = 2 * w2;
            fold(ws_lse[slot_row(slot)],
                 *reinterpret_cast<const f32x4*>(ws_out + slot_row(slot) * D + d));
        }
    }
    const uint64_t out0 = col_row(a, b, kvh, g) * D + d;
    const f32x4 r = a.out_scale * (num / den);
    store4(Tag(), a.out, out0,
           has_nan ? (f32x4){__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""),
                             __builtin_nanf("")}
                   : r);
}

template <typename Tag>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t s) {
    if (a.schedule == kBalanced) {
        const dim3 grid(a.num_wg);
        const bool two = a.col_tiles == 2;
        const int max_cols = (a.row_group > 0 ? a.row_group : 1) * a.group;
        const int4* meta = reinterpret_cast<const int4*>(a.ws_meta);
#define PA_MERGE(D_, NC_)                                                                  \
    hipLaunchKernelGGL((merge_balanced<Tag, D_, NC_>), grid, dim3(NC_ * D_ / 4), 0, s, meta, \
                       a.ws_out, a.ws_lse, a.num_wg, max_cols, a)
        if (a.head_dim == 64 && two)
            PA_MERGE(64, 32);
        else if (a.head_dim == 64)
            PA_MERGE(64, 16);
        else if (a.head_dim == 128 && two)
            PA_MERGE(128, 32);
        else if (a.head_dim == 128)
            PA_MERGE(128, 16);
        else
            PA_MERGE(256, 16);
#undef PA_MERGE
    } else {
        hipLaunchKernelGGL((merge_fixed<Tag>), dim3(a.num_kv_heads, a.num_seqs),
                           dim3(kMergeThreads), 0, s, a);
    }
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
