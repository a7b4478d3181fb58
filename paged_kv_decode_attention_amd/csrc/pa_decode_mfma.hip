// Decode paged attention on the gfx950 matrix cores, bf16/fp16 caches,
// head_dim 128, GQA groups of up to 16 query heads.
//
// Work decomposition: one workgroup of 4 wavefronts per (sequence b, KV head,
// context partition); the partition's tokens are split into 32-token chunks
// dealt round-robin to the wavefronts.  Every query head of the GQA group is
// served from the same K/V bytes, so each KV byte is fetched once.
//
// Per chunk a wavefront computes (the per-block online softmax of
// [MiniPaged-Qwen] §5.2, one 32-token chunk at a time):
//   S^T = K Q^T      (tokens x heads)   4 MFMA 16x16x32 per 16-token tile
//   m'  = max(m, max_t s),  p = 2^(s - m'),  l' = l 2^(m-m') + sum p
//   O^T = 2^(m-m') O^T + V^T P^T   (d x heads)  8 MFMA 16x16x32
// with scores in log2 units (scale * log2 e folded in), so exp is a single
// v_exp_f32.
//
// Lane layout (lane = 16 q + n): in every MFMA the column index (lane % 16)
// is the query head n of the group, so the running max / denominator of head
// n and the rescale of its accumulators stay inside the lanes that own them.
//   K operand: lane holds K[token n][d = 32 kk + 8 q .. +8], a 16-byte load;
//   Q operand: lane holds Q[head n][same d];
//   S^T tile : lane holds s[token 4 q + i][head n], i = 0..3;
//   P operand: lane holds p[head n][its own 8 tokens] -- no data movement;
//   V operand: lane loads V[token][d = 8 n .. 8 n + 8] for its 8 tokens
//              (four whole 256-byte rows per load instruction, fully
//              coalesced) and transposes them in registers so that MFMA j
//              consumes d = 8 m + j for row m = lane % 16;
//   O^T acc  : lane holds O[head n][d = 32 q + 8 i + j] for MFMA j, reg i.
// The address of every row is kv_row(): block_tables[b, t / BS] gives the
// physical block, t % BS the slot ([MiniPaged-Qwen] §6.2).
#include "pa_finalize.h"

namespace pa {
namespace {

__device__ __forceinline__ f32x4 mfma16x16x32(BF16, u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(F16, u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

template <typename Tag, int BS>
__global__ __launch_bounds__(kDecodeThreads) void decode_mfma_kernel(DecodeArgs a) {
    constexpr int D = 128;
    constexpr int E = 2;                         // bytes per element
    constexpr int NW = kDecodeThreads / 64;      // wavefronts per workgroup
    constexpr int OS = D + 4;                    // padded LDS row (floats)
    static_assert(BS == 16 || BS == 32, "block size");

    __shared__ float sm_m[NW * 16];
    __shared__ float sm_l[NW * 16];
    __shared__ __attribute__((aligned(16))) float sm_o[NW * 16 * OS];

    const int part = blockIdx.x;
    const int kvh = blockIdx.y;
    const int b = blockIdx.z;
    const int G = a.group;
    const int head0 = kvh * G;
    const int L = a.context_lens[b];

    if (L < 0 || L > a.max_context_len) {
        if (part == 0) fill_rows<Tag>(a, b, head0, G, __builtin_nanf(""));
        return;
    }
    if (L == 0) {
        if (part == 0) fill_rows<Tag>(a, b, head0, G, 0.0f);
        return;
    }
    const int t_begin = part * a.part_len;
    if (t_begin >= L) return;
    const int t_end = min(t_begin + a.part_len, L);
    const int nparts_b = (L + a.part_len - 1) / a.part_len;
    const int nchunks = (t_end - t_begin + kChunk - 1) / kChunk;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15;
    const int q = lane >> 4;

    // Physical blocks of this partition, one per lane (part_len <= 64 * BS).
    const int nblk = (t_end - t_begin + BS - 1) / BS;
    int my_pb = 0;
    int bad_lane = 0;
    if (lane < nblk) {
        my_pb = a.block_tables[(uint64_t)b * a.max_blocks_per_seq + t_begin / BS + lane];
        if ((unsigned)my_pb >= (unsigned)a.num_blocks) {
            bad_lane = 1;
            my_pb = 0;
        }
    }
    const bool bad = __any(bad_lane);

    // Query operand: Q[head n][32 kk + 8 q .. +8]; zero for padding heads.
    u32x4 qop[4];
    if (n < G) {
        const char* qp = reinterpret_cast<const char*>(a.query) +
                         (((uint64_t)b * a.num_heads + head0 + n) * D + 8 * q) * E;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) qop[kk] = load16(qp + kk * 64);
    } else {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) qop[kk] = (u32x4){0u, 0u, 0u, 0u};
    }

    const char* kbase = reinterpret_cast<const char*>(a.key_cache);
    const char* vbase = reinterpret_cast<const char*>(a.value_cache);
    const uint32_t koff = (uint32_t)(n * D + 8 * q) * E;        // K row n, d 8q
    const uint32_t voff = (uint32_t)(4 * q * D + 8 * n) * E;    // V row 4q, d 8n
    const float sl2 = a.scale_log2;

    float m_run = -INFINITY;
    float l_run = 0.0f;
    f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = (f32x4){0.f, 0.f, 0.f, 0.f};

    for (int c = wave; c < nchunks; c += NW) {
        const int tc = t_begin + c * kChunk;
        int pb0, pb1, off1;
        if constexpr (BS == 16) {
            pb0 = __builtin_amdgcn_readlane(my_pb, 2 * c);
            pb1 = __builtin_amdgcn_readlane(my_pb, 2 * c + 1);
            off1 = 0;
        } else {
            pb0 = __builtin_amdgcn_readlane(my_pb, c);
            pb1 = pb0;
            off1 = 16;
        }
        const uint64_t base0 = kv_row(pb0, kvh, 0, a.num_kv_heads, BS) * (D * E);
        const uint64_t base1 = kv_row(pb1, kvh, off1, a.num_kv_heads, BS) * (D * E);
        const bool tile1 = tc + 16 < t_end;

        u32x4 k0[4], k1[4], v[8];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) k0[kk] = load16(kbase + base0 + koff + kk * 64);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = load16(vbase + base0 + voff + i * (D * E));
        if (tile1) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) k1[kk] = load16(kbase + base1 + koff + kk * 64);
#pragma unroll
            for (int i = 0; i < 4; ++i) v[4 + i] = load16(vbase + base1 + voff + i * (D * E));
        } else {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) k1[kk] = (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
            for (int i = 0; i < 4; ++i) v[4 + i] = (u32x4){0u, 0u, 0u, 0u};
        }

        // Scores: S^T[token][head] for the two 16-token tiles.
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) s0 = mfma16x16x32(Tag(), k0[kk], qop[kk], s0);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) s1 = mfma16x16x32(Tag(), k1[kk], qop[kk], s1);

        float s[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s[i] = s0[i] * sl2;
            s[4 + i] = s1[i] * sl2;
        }
        if (tc + kChunk > t_end) {
            // Last chunk of the partition: tokens at or past the end of the
            // history are excluded (score -inf, V row zero so that stale
            // slot contents cannot reach the accumulator).
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (tc + 4 * q + i >= t_end) {
                    s[i] = -INFINITY;
                    v[i] = (u32x4){0u, 0u, 0u, 0u};
                }
                if (tc + 16 + 4 * q + i >= t_end) {
                    s[4 + i] = -INFINITY;
                    v[4 + i] = (u32x4){0u, 0u, 0u, 0u};
                }
            }
        }

        // Online softmax update for head n over this chunk.
        float cmax = s[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) cmax = fmaxf(cmax, s[i]);
        cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
        cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
        const float m_new = fmaxf(m_run, cmax);
        const float alpha = fast_exp2(m_run - m_new);
        u32x4 pop;
#pragma unroll
        for (int u = 0; u < 4; ++u)
            pop[u] = pack2(Tag(), fast_exp2(s[2 * u] - m_new), fast_exp2(s[2 * u + 1] - m_new));
        // The denominator sums the same rounded weights the MFMA consumes.
        float psum = 0.0f;
#pragma unroll
        for (int u = 0; u < 4; ++u) psum += unpack_lo(Tag(), pop[u]) + unpack_hi(Tag(), pop[u]);
        l_run = l_run * alpha + psum;
        m_run = m_new;

#pragma unroll
        for (int j = 0; j < 8; ++j) {
            acc[j] *= alpha;
            // V^T operand for d = 8 n + j: element j of each of the 8 rows.
            u32x4 w;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t r0 = v[2 * u][j >> 1];
                const uint32_t r1 = v[2 * u + 1][j >> 1];
                w[u] = (j & 1) ? ((r0 >> 16) | (r1 & 0xffff0000u))
                               : ((r0 & 0xffffu) | (r1 << 16));
            }
            acc[j] = mfma16x16x32(Tag(), w, pop, acc[j]);
        }
    }

    // Denominator of head n: sum the four lane groups' partial sums.
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    if (q == 0) {
        sm_m[wave * 16 + n] = m_run;
        sm_l[wave * 16 + n] = l_run;
    }
    float* ow = sm_o + (wave * 16 + n) * OS + 32 * q;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<f32x4*>(ow + 8 * i) = (f32x4){acc[0][i], acc[1][i], acc[2][i], acc[3][i]};
        *reinterpret_cast<f32x4*>(ow + 8 * i + 4) = (f32x4){acc[4][i], acc[5][i], acc[6][i], acc[7][i]};
    }
    __syncthreads();
    finalize_partition<Tag>(a, sm_m, sm_l, sm_o, NW, 16 * OS, OS, head0, G, b, part,
                            nparts_b, bad);
}

template <typename Tag, int BS>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t s) {
    dim3 grid(a.num_parts, a.num_kv_heads, a.num_seqs);
    hipLaunchKernelGGL((decode_mfma_kernel<Tag, BS>), grid, dim3(kDecodeThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

bool mfma_supported(pa_dtype dt, int head_dim, int block_size, int group) {
    return (dt == PA_BF16 || dt == PA_F16) && head_dim == 128 &&
           (block_size == 16 || block_size == 32) && group >= 1 && group <= 16;
}

hipError_t launch_decode_mfma(const DecodeArgs& a, pa_dtype dt, hipStream_t s) {
    if (dt == PA_BF16) {
        return a.block_size == 16 ? launch_typed<BF16, 16>(a, s) : launch_typed<BF16, 32>(a, s);
    }
    return a.block_size == 16 ? launch_typed<F16, 16>(a, s) : launch_typed<F16, 32>(a, s);
}

}  // namespace pa
