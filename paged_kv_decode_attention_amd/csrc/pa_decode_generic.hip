// Decode paged attention on the vector ALUs: every supported dtype (f32,
// f16, bf16), head_dim 64, 128 or 256, block size 8, 16, 32 or 64, any GQA
// group size.
// The matrix-core kernel covers the bf16/fp16 head_dim-128 cases; this one
// covers the rest (and serves as a second, independent device path).
//
// One workgroup (4 wavefronts) per (sequence, KV head, head group of up to GT
// query heads, context partition).  A token row of head_dim elements is
// D*E/16 lanes wide (16 bytes per lane, one coalesced load); the workgroup
// holds 256/(D*E/16) such token groups, which walk the partition's tokens in
// an interleaved order.  Each token group keeps its own online-softmax state
// per head ([MiniPaged-Qwen] §5.2 applied to the U tokens a group loads at
// once):
//   m' = max(m, max_u s_u),  l' = l 2^(m-m') + sum_u 2^(s_u-m'),
//   o' = o 2^(m-m') + sum_u 2^(s_u-m') v_u
// and the groups' states are merged at the end (same update rule applied to
// whole states), first across lanes, then across wavefronts in LDS.
#include <type_traits>

#include "pa_finalize.h"

namespace pa {
namespace {

// Sum of x over the TG lanes of this lane's token group (TG a power of two
// up to 64, groups aligned to TG lanes), in every lane of the group.  The
// partners are those of a butterfly (lanes 1, 2, 4, ... apart), so the sum is
// the same in every lane and the same as pairwise xor exchanges give; within
// a row of 16 lanes they are DPP moves (quad permutes, then the half-row and
// row mirrors, which pair each quad with the next and each half-row with
// the other), across rows lane permutes.
template <int TG>
__device__ __forceinline__ float group_sum(float x) {
    auto dpp = [](float v, auto ctrl) {
        return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v),
                                                                  decltype(ctrl)::value, 0xF,
                                                                  0xF, false));
    };
    using Q1 = std::integral_constant<int, 0xB1>;     // quad_perm [1, 0, 3, 2]
    using Q2 = std::integral_constant<int, 0x4E>;     // quad_perm [2, 3, 0, 1]
    using HM = std::integral_constant<int, 0x141>;    // row_half_mirror
    using RM = std::integral_constant<int, 0x140>;    // row_mirror
    if constexpr (TG >= 2) x += dpp(x, Q1{});
    if constexpr (TG >= 4) x += dpp(x, Q2{});
    if constexpr (TG >= 8) x += dpp(x, HM{});
    if constexpr (TG >= 16) x += dpp(x, RM{});
    if constexpr (TG >= 32) x += __shfl_xor(x, 16);
    if constexpr (TG >= 64) x += __shfl_xor(x, 32);
    return x;
}

// float32 rows of a workgroup of 8 heads are folded a batch at a time
// (below) at head_dim 64 and 256.  Measured on the bench batch: 88.8 vs
// 100.4 us at 64 (7 heads), 299 vs 306 at 256.  At 128 the per-token update
// is faster (163.5 vs 170 us): the block fold's registers leave one
// wavefront per SIMD or need a scheduling barrier per head.  With 4 heads
// or fewer it is slower (76.5 vs 68.4 us at head_dim 64, 4 heads): too few
// independent heads to cover the latency of each head's chain of scores,
// maximum and exponentials.
template <typename Tag, int D, int GT>
constexpr bool block_fold() { return Tag::kBytes == 4 && GT >= 8 && D != 128; }

// Wavefronts per SIMD the register allocation must leave room for: with the
// block fold three at head_dim 64 (at most 168 registers), two at 256;
// otherwise no bound (0: the compiler's default).
template <typename Tag, int D, int GT>
constexpr int generic_waves() { return !block_fold<Tag, D, GT>() ? 0 : D == 64 ? 3 : 2; }

template <typename Tag, int D, int BS, int GT>
__global__ __launch_bounds__(kDecodeThreads)
__attribute__((amdgpu_waves_per_eu(generic_waves<Tag, D, GT>(), 0))) void decode_generic_kernel(
    DecodeArgs a) {
    constexpr int E = Tag::kBytes;
    // Each lane holds VEC elements of a token row: 16 bytes, or 32 of a
    // float32 row at head_dim 128 and up, so that a row is at most 16 lanes
    // wide up to head_dim 128 and a head's dot product is reduced with DPP
    // moves within a row of lanes.
    constexpr int VEC = (E == 4 && D >= 128) ? 8 : 16 / E;   // elements per lane
    constexpr int W = VEC * E / 16;              // 16-byte words per lane and row
    constexpr int TG = D / VEC;                  // lanes per token row
    constexpr int NG = kDecodeThreads / TG;      // token groups per workgroup
    constexpr int NW = kDecodeThreads / 64;
    constexpr int kMaxBlocks = 64;               // part_len <= 64 * BS
    static_assert(TG >= 1 && TG <= 64 && 64 % TG == 0, "row width");

    __shared__ int sm_pb[kMaxBlocks];
    __shared__ float sm_m[NW * 16];
    __shared__ float sm_l[NW * 16];
    __shared__ float sm_o[NW * GT * D];

    const int hgroups = (a.group + GT - 1) / GT;
    const int kvh = blockIdx.x / hgroups;
    const int hg = blockIdx.x - kvh * hgroups;
    const int b = blockIdx.y;
    const int part = blockIdx.z;     // slowest: full partitions dispatch first
    const int g0 = hg * GT;
    // This kernel serves decode rows of at most one query row (a verify row
    // map built for it groups none), so its columns are the group's heads.
    const int ncols = min(row_tokens(a, b), 1) * a.group;
    const int nh = min(GT, ncols - g0);
    if (nh <= 0) return;
    const int head0 = kvh * a.group + g0;
    const int L = a.context_lens[b];

    if (L < 0 || L > a.max_context_len) {
        if (part == 0) fill_cols<Tag>(a, b, kvh, g0, nh, __builtin_nanf(""));
        return;
    }
    if (L == 0) {
        if (part == 0) fill_cols<Tag>(a, b, kvh, g0, nh, 0.0f);
        return;
    }
    const int t_begin = part * a.part_len;
    if (t_begin >= L) return;
    const int t_end = min(t_begin + a.part_len, L);
    const int nparts_b = (L + a.part_len - 1) / a.part_len;

    // Physical blocks of the partition.
    const int nblk = (t_end - t_begin + BS - 1) / BS;
    int bad_t = 0;
    for (int i = threadIdx.x; i < nblk; i += kDecodeThreads) {
        int pb = a.block_tables[table_row_offset(a, b) + t_begin / BS + i];
        if ((unsigned)pb >= (unsigned)a.num_blocks) {
            bad_t = 1;
            pb = 0;
        }
        sm_pb[i] = pb;
    }
    const bool bad = __syncthreads_or(bad_t);

    const int lane = threadIdx.x & 63;
    const int c = lane % TG;                     // 16-byte column of the row
    const int grp = threadIdx.x / TG;            // token group
    const int wave = threadIdx.x >> 6;

    float qf[GT][VEC];
#pragma unroll
    for (int g = 0; g < GT; ++g) {
        if (g < nh) {
            const char* qp = reinterpret_cast<const char*>(a.query) +
                             (((uint64_t)b * a.num_heads + head0 + g) * D + c * VEC) * E;
#pragma unroll
            for (int w = 0; w < W; ++w) to_float(Tag(), load16(qp + 16 * w), qf[g] + (16 / E) * w);
#pragma unroll
            for (int e = 0; e < VEC; ++e) qf[g][e] *= a.scale_log2;
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) qf[g][e] = 0.0f;
        }
    }

    float m[GT], l[GT], o[GT][VEC];
#pragma unroll
    for (int g = 0; g < GT; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.0f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[g][e] = 0.0f;
    }

    // Each token group takes tokens t0, t0 + NG, ..., U at a time: their K and
    // V rows are loaded together (nontemporal: streamed once), then folded
    // in token order, so that U rows per lane are in flight instead of one
    // (64 to 128 bytes of K and V per lane).  Loads past the partition's end
    // re-read its last token and are not folded.
    typedef __attribute__((address_space(1))) const u32x4 GlobalRow;
    constexpr int U = W == 1 && E == 4 ? 8 : 4;   // rows per lane in flight
    const char* kbase = reinterpret_cast<const char*>(a.key_cache);
    const char* vbase = reinterpret_cast<const char*>(a.value_cache);
    for (int t0 = t_begin + grp; t0 < t_end; t0 += NG * U) {
        u32x4 kr[U][W], vr[U][W];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = min(t0 + u * NG, t_end - 1);
            const int pb = sm_pb[(t - t_begin) / BS];
            const uint64_t byte =
                (kv_row(pb, kvh, t % BS, a.num_kv_heads, BS) * D + c * VEC) * E;
#pragma unroll
            for (int w = 0; w < W; ++w) {
                kr[u][w] = __builtin_nontemporal_load((GlobalRow*)(kbase + byte + 16 * w));
                vr[u][w] = __builtin_nontemporal_load((GlobalRow*)(vbase + byte + 16 * w));
            }
        }
        // At head_dim 128 and 256 a scheduling barrier keeps the batch's
        // loads all issued before its fold, which the compiler would
        // otherwise interleave (float32 rows: 47 and 52 % of 8 TB/s against
        // 43 and 45); at 64 the registers it takes would cost a third
        // wavefront per SIMD.
        if constexpr (D >= 128) __builtin_amdgcn_sched_barrier(0);
        // float32 rows of a workgroup of 8 heads are folded a batch at a
        // time (see block_fold): the per-token rescale of every head's
        // accumulators is what their vector-ALU time goes to.  Otherwise
        // each token's update is applied on its own, which also skips a
        // short history's absent tokens (the latency case: a few tokens per
        // partition).
        if constexpr (block_fold<Tag, D, GT>()) {
            // float32 rows need no conversion (the batch's rows are the loaded
            // registers themselves); which of its tokens lie inside the
            // partition is the same in every lane of a token group.
            float kf[U][VEC], vf[U][VEC];
            bool live[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                live[u] = t0 + u * NG < t_end;
#pragma unroll
                for (int w = 0; w < W; ++w) {
                    to_float(Tag(), kr[u][w], kf[u] + (16 / E) * w);
                    to_float(Tag(), vr[u][w], vf[u] + (16 / E) * w);
                }
            }
            // Head by head, the batch's U scores first, then one update of
            // the head's state for all of them (the block update above):
            // one rescale per batch instead of one per token.  Tokens past
            // the partition (in a later token group of the wavefront) score
            // -inf and weigh 0; token u = 0 is always inside, so m' is
            // finite.
#pragma unroll
            for (int g = 0; g < GT; ++g) {
                float sc[U];
                float m_new = m[g];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    float dot = 0.0f;
#pragma unroll
                    for (int e = 0; e < VEC; ++e) dot += qf[g][e] * kf[u][e];
                    dot = group_sum<TG>(dot);
                    sc[u] = live[u] ? dot : -INFINITY;
                    m_new = fmaxf(m_new, sc[u]);
                }
                const float al = fast_exp2(m[g] - m_new);
                float ls = 0.0f;
#pragma unroll
                for (int e = 0; e < VEC; ++e) o[g][e] *= al;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const float pe = fast_exp2(sc[u] - m_new);
                    ls += pe;
#pragma unroll
                    for (int e = 0; e < VEC; ++e) o[g][e] += pe * vf[u][e];
                }
                l[g] = l[g] * al + ls;
                m[g] = m_new;
                // one head at a time: interleaving the next head's dot
                // products with this update takes registers head_dim 256
                // does not have
                if constexpr (D >= 128) __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            // (16-bit rows are converted one token at a time: converting the
            // whole batch first would hold U more rows of floats.)
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (t0 + u * NG >= t_end) break;   // the same for every lane of a token group
                float kf[VEC], vf[VEC];
#pragma unroll
                for (int w = 0; w < W; ++w) {
                    to_float(Tag(), kr[u][w], kf + (16 / E) * w);
                    to_float(Tag(), vr[u][w], vf + (16 / E) * w);
                }
#pragma unroll
                for (int g = 0; g < GT; ++g) {
                    float dot = 0.0f;
#pragma unroll
                    for (int e = 0; e < VEC; ++e) dot += qf[g][e] * kf[e];
                    dot = group_sum<TG>(dot);
                    const float m_new = fmaxf(m[g], dot);
                    const float al = fast_exp2(m[g] - m_new);
                    const float pe = fast_exp2(dot - m_new);
                    l[g] = l[g] * al + pe;
#pragma unroll
                    for (int e = 0; e < VEC; ++e) o[g][e] = o[g][e] * al + pe * vf[e];
                    m[g] = m_new;
                }
            }
        }
    }

    // Merge the token groups of each wavefront (lanes TG apart).
#pragma unroll
    for (int s = TG; s < 64; s <<= 1) {
#pragma unroll
        for (int g = 0; g < GT; ++g) {
            const float m2 = __shfl_xor(m[g], s);
            const float l2 = __shfl_xor(l[g], s);
            const float M = fmaxf(m[g], m2);
            const float e1 = rescale_weight(m[g], M);
            const float e2 = rescale_weight(m2, M);
            l[g] = e1 * l[g] + e2 * l2;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const float o2 = __shfl_xor(o[g][e], s);
                o[g][e] = e1 * o[g][e] + e2 * o2;
            }
            m[g] = M;
        }
    }
    if (lane < TG) {
#pragma unroll
        for (int g = 0; g < GT; ++g) {
            if (c == 0) {
                sm_m[wave * 16 + g] = m[g];
                sm_l[wave * 16 + g] = l[g];
            }
#pragma unroll
            for (int e = 0; e < VEC; ++e) sm_o[(wave * GT + g) * D + c * VEC + e] = o[g][e];
        }
    }
    __syncthreads();
    finalize_state<Tag>(a, sm_m, sm_l, sm_o, NW, 16, GT * D, D, b, kvh, g0, nh, bad,
                        nparts_b == 1 ? -1 : part);
}

template <typename Tag, int D, int BS, int GT>
hipError_t launch4(const DecodeArgs& a, hipStream_t s) {
    const int hgroups = (a.group + GT - 1) / GT;
    dim3 grid(a.num_kv_heads * hgroups, a.num_seqs, a.num_parts);
    hipLaunchKernelGGL((decode_generic_kernel<Tag, D, BS, GT>), grid, dim3(kDecodeThreads), 0, s, a);
    return hipGetLastError();
}

template <typename Tag, int D, int BS>
hipError_t launch3(const DecodeArgs& a, hipStream_t s) {
    if (a.group == 1) return launch4<Tag, D, BS, 1>(a, s);
    if (a.group == 2) return launch4<Tag, D, BS, 2>(a, s);
    if (a.group <= 4) return launch4<Tag, D, BS, 4>(a, s);
    return launch4<Tag, D, BS, 8>(a, s);
}

template <typename Tag, int D>
hipError_t launch2(const DecodeArgs& a, hipStream_t s) {
    switch (a.block_size) {
        case 8: return launch3<Tag, D, 8>(a, s);
        case 16: return launch3<Tag, D, 16>(a, s);
        case 32: return launch3<Tag, D, 32>(a, s);
        default: return launch3<Tag, D, 64>(a, s);
    }
}

template <typename Tag>
hipError_t launch1(const DecodeArgs& a, hipStream_t s) {
    switch (a.head_dim) {
        case 64: return launch2<Tag, 64>(a, s);
        case 128: return launch2<Tag, 128>(a, s);
        default: return launch2<Tag, 256>(a, s);
    }
}

}  // namespace

hipError_t launch_decode_generic(const DecodeArgs& a, pa_dtype dt, hipStream_t s) {
    switch (dt) {
        case PA_F32: return launch1<F32>(a, s);
        case PA_F16: return launch1<F16>(a, s);
        default: return launch1<BF16>(a, s);
    }
}

}  // namespace pa
