// Decode paged attention on the gfx950 matrix cores, bf16/fp16 queries,
// 16-bit, FP8 E4M3 or INT8 caches, head_dim 64, 128 or 256, GQA groups of up to 16
// query heads (32 at head_dim 64 and 128).  The kernel templates; each head
// dim is instantiated in a translation unit of its own
// (pa_decode_mfma_d64.hip, _d128.hip, _d256.hip) so that they compile in
// parallel, and pa_decode_mfma.hip dispatches to them.
//
// Work decomposition: one workgroup of 4 wavefronts per (sequence b, KV head,
// context partition), or per equal-work range of the whole batch (balanced
// schedule, below); tokens are taken in 32-token chunks.  Every query head of
// the GQA group is served from the same K/V bytes, so each KV byte is fetched
// once.
//
// Per chunk a wavefront computes (the per-block online softmax of
// [MiniPaged-Qwen] §5.2, one 32-token chunk at a time):
//   S^T = K Q^T      (tokens x heads)   D/32 MFMA 16x16x32 per 16-token tile
//   m'  = max(m, max_t s),  p = 2^(s - m'),  l' = l 2^(m-m') + sum p
//   O^T = 2^(m-m') O^T + V^T P^T   (d x heads)  D/16 MFMA 16x16x32
// with scores in log2 units (scale * log2 e folded in), so exp is a single
// v_exp_f32.  The reference max m is only moved (and O, l rescaled) when a
// chunk's max exceeds it by more than 2^8; in between, weights 2^(s - m) are
// at most 2^8, and the final o = O / l does not depend on the choice of m.
// l is summed on the matrix core (P times a ones operand).  While one
// chunk is computed, the next chunk's loads are in flight (two register
// buffers; one at head_dim 256).  Histories longer than one partition leave
// float32 partition states that the merge kernel (pa_merge.hip) combines.
// In verify mode the 16 columns (or 32, in two column tiles) are (query
// row, head) pairs of several query rows of one sequence, each column
// masked at its own causal end.
//
// Lane layout (lane = 16 q + n; VW = D / 16): in every MFMA the column index
// (lane % 16) is the query head n of the group, so the running max /
// denominator of head n and the rescale of its accumulators stay inside the
// lanes that own them.
//   K operand: lane holds K[token n][d = 32 kk + 8 q .. +8], a 16-byte load;
//   Q operand: lane holds Q[head n][same d];
//   S^T tile : lane holds s[token 4 q + i][head n], i = 0..3;
//   P operand: lane holds p[head n][its own 8 tokens] -- no data movement;
//   V operand: lane loads V[token][d = VW n .. VW n + VW] for its 8 tokens
//              (whole rows per load instruction, fully coalesced) and
//              transposes them in registers so that MFMA j consumes
//              d = VW m + j for row m = lane % 16;
//   O^T acc  : lane holds O[head n][d = VW (4 q + i) + j] for MFMA j, reg i.
// The address of every row is kv_row(): block_tables[b, t / BS] gives the
// physical block, t % BS the slot ([MiniPaged-Qwen] §6.2).
#pragma once

#include <type_traits>

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

// Float32 operands: A[m][k] and B[k][n] one value per lane (lane 16 k + m /
// 16 k + n), K = 4.
__device__ __forceinline__ f32x4 mfma16x16x4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Element e of four loaded dwords as a float.  The whole vector is cast: a
// bit cast of the element expression itself compiles to a read of element 0
// (seen in the generated code), whatever e is.
__device__ __forceinline__ float f32_at(u32x4 v, int e) { return __builtin_bit_cast(f32x4, v)[e]; }

// Two 16-bit 1.0 values packed in one dword.
template <typename Tag>
constexpr uint32_t kOnePair();
template <>
constexpr uint32_t kOnePair<BF16>() { return 0x3f803f80u; }
template <>
constexpr uint32_t kOnePair<F16>() { return 0x3c003c00u; }

// Tile geometry of one head dimension.
template <int D>
struct Dim {
    static_assert(D == 64 || D == 128 || D == 256, "matrix-core kernel: head_dim 64/128/256");
    static constexpr int KD = D / 32;   // K / Q MFMA steps per 16-token tile
    static constexpr int VW = D / 16;   // d values a lane holds per V row = PV MFMAs
    static constexpr int RB = D * 2;    // bytes per 16-bit token row
    static constexpr int OS = D + 4;    // padded LDS row of one column (floats)
    // 32-bit dwords of this lane's slice of a V row: 16-bit / 8-bit storage
    using VRow = typename std::conditional<
        D == 64, u32x2, typename std::conditional<D == 128, u32x4, u32x8>::type>::type;
    using VRow8 = typename std::conditional<
        D == 64, uint32_t, typename std::conditional<D == 128, u32x2, u32x4>::type>::type;
};

// One 32-token chunk's K and V operands, as loaded (two 16-token tiles).
template <int D>
struct ChunkRegs {
    u32x4 k0[Dim<D>::KD], k1[Dim<D>::KD];   // K tile 0 / 1: row n, d = 32 kk + 8 q .. +8
    typename Dim<D>::VRow v[8];              // V rows of this lane's 8 tokens, d = VW n ..
};

// Physical blocks of chunk c's two 16-token tiles, read from the sequence's
// table row (wave-uniform scalar loads).  A tile past the end of the history
// reuses tile 0's block; its table entry is not used.  Entries outside the
// pool set `bad` and are replaced by block 0 (never an out-of-bounds read).
// The block table is read-only for the whole launch: read it through the
// constant address space, which lets uniform reads become scalar loads.
typedef __attribute__((address_space(4))) const int32_t ConstI32;

// Row of chunk c's first tile inside its block: blocks of 16 or 32 tokens
// start a chunk at row 0; a 64-token block holds two chunks.
template <int BS>
__device__ __forceinline__ int tile_row(int c) {
    return BS == 64 ? (c & 1) * 32 : 0;
}

// Blocks of 8 tokens: a chunk spans four blocks (two per 16-token tile).
template <int BS>
using BlockIds = typename std::conditional<BS == 8, int4, int2>::type;

__device__ __forceinline__ int checked_block(int pb, int num_blocks, int& bad) {
    if ((unsigned)pb >= (unsigned)num_blocks) { bad = 1; return 0; }
    return pb;
}

// The table entries chunk c may need (block size 8: four, 16: two, 32 and
// 64: one), each index clamped to the history's last block, so inside the
// table row.  The reads are independent and go out together; their values
// are checked only where the chunk's loads are issued (chunk_blocks), so
// that the wait for them falls after whatever was issued in between -- at
// the start of a history, the next chunk's entries too.  Reading an entry
// only once its tile is known to be live would chain a memory round trip per
// entry.
template <int BS>
__device__ __forceinline__ BlockIds<BS> chunk_entries(const ConstI32* row, int c, int L) {
    const int j0 = c * kChunk / BS;
    const int jl = (L - 1) / BS;                 // the history's last block
    if constexpr (BS == 8)
        return make_int4(row[j0], row[min(j0 + 1, jl)], row[min(j0 + 2, jl)],
                         row[min(j0 + 3, jl)]);
    else if constexpr (BS == 16)
        return make_int2(row[j0], row[min(j0 + 1, jl)]);
    else
        return make_int2(row[j0], 0);
}

// The physical blocks of chunk c from its entries e: a block past the end of
// the history reuses the first (its entry is not used).
template <int BS>
__device__ __forceinline__ BlockIds<BS> chunk_blocks(BlockIds<BS> e, int c, int L,
                                                     int num_blocks, int& bad) {
    const int j0 = c * kChunk / BS;
    const int jl = (L - 1) / BS;
    const int pb0 = checked_block(e.x, num_blocks, bad);
    if constexpr (BS == 8) {
        const int pb1 = j0 + 1 <= jl ? checked_block(e.y, num_blocks, bad) : pb0;
        const int pb2 = j0 + 2 <= jl ? checked_block(e.z, num_blocks, bad) : pb0;
        const int pb3 = j0 + 3 <= jl ? checked_block(e.w, num_blocks, bad) : pb0;
        return make_int4(pb0, pb1, pb2, pb3);
    } else if constexpr (BS == 16) {
        return make_int2(pb0, j0 + 1 <= jl ? checked_block(e.y, num_blocks, bad) : pb0);
    } else {
        return make_int2(pb0, pb0);
    }
}

// Buffer descriptor of one 16-token tile (kTileBytes: 16 rows of K or V):
// base address, size.  A size of 0 makes every load from it return zero
// without touching memory.
template <int kTileBytes>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char* base, bool live) {
    constexpr int kRawBufferFlags = 0x00020000;   // 32-bit data format: raw loads return data
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, live ? kTileBytes : 0,
                                             kRawBufferFlags);
}

// Issue the loads of one chunk: always the same number, so the in-order load
// counter the compiler waits on is the same on every path and the next
// chunk's loads stay in flight while this one is computed.  KV is streamed
// once: loads are nontemporal.  A tile that is not live (past the end of the
// history, or a prefetch past the wave's last chunk) is read through an
// empty descriptor: the loads return zeros and move no bytes.
constexpr int kNonTemporal = 2;   // buffer cache-policy bit: nt

// V row slices: 8, 16 or 32 bytes (head_dim 64, 128, 256) of 16-bit values;
// 4, 8 or 16 bytes of 8-bit codes.
__device__ __forceinline__ void load_row(u32x8& x, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNonTemporal);
    const u32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, kNonTemporal);
    x = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ void load_row(u32x4& x, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNonTemporal);
}
__device__ __forceinline__ void load_row(u32x2& x, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    x = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kNonTemporal);
}
__device__ __forceinline__ void load_row(uint32_t& x, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    x = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kNonTemporal);
}

// Loads through per-lane 64-bit addresses instead of a tile descriptor.
// Blocks of 8 tokens need them: each 16-token tile spans two blocks, so one
// instruction's lanes read rows of two blocks (the K operand row of lane
// (q, n) is token n of the tile, block n / 8; its V rows are tokens
// 4 q .. 4 q + 3, block q / 2).  Larger blocks keep the descriptor path
// (measured equal or up to 1 % faster with the last-level cache defeated).
// A tile that is not live points every lane at the first bytes of the pool
// (one cache line per instruction, never out of bounds); such tiles are
// masked or never computed.  Loads are nontemporal.  kin / vin: this lane's
// byte offsets inside a K row / V row.
template <int BS, int D>
constexpr bool lane_addressed() { return BS == 8; }
typedef __attribute__((address_space(1))) const u32x4 GlobalU32x4;
typedef __attribute__((address_space(1))) const u32x2 GlobalU32x2;
typedef __attribute__((address_space(1))) const uint32_t GlobalU32;

__device__ __forceinline__ void load_row_at(u32x8& x, const char* p) {
    const u32x4 lo = __builtin_nontemporal_load((GlobalU32x4*)p);
    const u32x4 hi = __builtin_nontemporal_load((GlobalU32x4*)(p + 16));
    x = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ void load_row_at(u32x4& x, const char* p) {
    x = __builtin_nontemporal_load((GlobalU32x4*)p);
}
__device__ __forceinline__ void load_row_at(u32x2& x, const char* p) {
    x = __builtin_nontemporal_load((GlobalU32x2*)p);
}
__device__ __forceinline__ void load_row_at(uint32_t& x, const char* p) {
    x = __builtin_nontemporal_load((GlobalU32*)p);
}
// A float32 V row's slices (KvF32): D/64 16-byte slices, 256 bytes apart.
template <int H>
__device__ __forceinline__ void load_row(u32x4 (&x)[H], __amdgpu_buffer_rsrc_t r, uint32_t off) {
#pragma unroll
    for (int h = 0; h < H; ++h)
        x[h] = __builtin_amdgcn_raw_buffer_load_b128(r, off + 256 * h, 0, kNonTemporal);
}
template <int H>
__device__ __forceinline__ void load_row_at(u32x4 (&x)[H], const char* p) {
#pragma unroll
    for (int h = 0; h < H; ++h) x[h] = __builtin_nontemporal_load((GlobalU32x4*)(p + 256 * h));
}

// kRB: bytes per token row; kKLoads 16-byte K loads per tile, kKStep bytes
// apart; Regs: ChunkRegs or ChunkRegs8.  Blocks of 16 or more tokens: tile
// t lies in block pb[t] from row r0 (tile 0) or the row after tile 0's
// (tile 1), as in load_chunk.
template <int BS, int kRB, int kKLoads, int kKStep, typename Regs>
__device__ __forceinline__ void load_chunk_lanes(Regs& r, const char* kbase, const char* vbase,
                                                 BlockIds<BS> pb, int r0, bool live0, bool live1,
                                                 int kvh, int num_kv_heads, uint32_t kin,
                                                 uint32_t vin) {
    const int lane = threadIdx.x & 63;
    const int n = lane & 15;
    const int q = lane >> 4;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const bool live = t == 0 ? live0 : live1;
        int kblk, kslot, vblk, vslot;
        if constexpr (BS == 8) {
            const int blk_a = t == 0 ? pb.x : pb.z;
            const int blk_b = t == 0 ? pb.y : pb.w;
            kblk = n < 8 ? blk_a : blk_b;
            kslot = n & 7;
            vblk = q < 2 ? blk_a : blk_b;
            vslot = 4 * (q & 1);
        } else {
            const int row_t = t == 0 ? r0 : (BS == 16 ? 0 : r0 + 16);
            kblk = vblk = t == 0 ? pb.x : pb.y;
            kslot = row_t + n;
            vslot = row_t + 4 * q;
        }
        const uint64_t krow = live ? kv_row(kblk, kvh, kslot, num_kv_heads, BS) : 0;
        const uint64_t vrow = live ? kv_row(vblk, kvh, vslot, num_kv_heads, BS) : 0;
        const char* kp = kbase + krow * kRB + kin;
        const char* vp = vbase + vrow * kRB + vin;
#pragma unroll
        for (int kk = 0; kk < kKLoads; ++kk)
            load_row_at(t == 0 ? r.k0[kk] : r.k1[kk], kp + kk * kKStep);
#pragma unroll
        for (int i = 0; i < 4; ++i) load_row_at(r.v[4 * t + i], vp + i * kRB);
    }
}

template <int BS, int D>
__device__ __forceinline__ void load_chunk(ChunkRegs<D>& r, const char* kbase, const char* vbase,
                                           BlockIds<BS> pb, int r0, bool live0, bool live1,
                                           int kvh, int num_kv_heads, uint32_t koff,
                                           uint32_t voff) {
    constexpr int RB = Dim<D>::RB;   // bytes per token row
    constexpr int KD = Dim<D>::KD;
    if constexpr (lane_addressed<BS, D>()) {
        // koff = n RB + kin, voff = 4 q RB + vin
        const int lane = threadIdx.x & 63;
        load_chunk_lanes<BS, RB, KD, 64>(r, kbase, vbase, pb, r0, live0, live1, kvh,
                                         num_kv_heads, koff - (lane & 15) * RB,
                                         voff - 4 * (lane >> 4) * RB);
    } else {
    const uint64_t row0 = kv_row(pb.x, kvh, r0, num_kv_heads, BS) * RB;
    const uint64_t row1 = kv_row(pb.y, kvh, BS == 16 ? 0 : r0 + 16, num_kv_heads, BS) * RB;
    const __amdgpu_buffer_rsrc_t k0 = tile_rsrc<16 * RB>(kbase + row0, live0);
    const __amdgpu_buffer_rsrc_t k1 = tile_rsrc<16 * RB>(kbase + row1, live1);
    const __amdgpu_buffer_rsrc_t v0 = tile_rsrc<16 * RB>(vbase + row0, live0);
    const __amdgpu_buffer_rsrc_t v1 = tile_rsrc<16 * RB>(vbase + row1, live1);
#pragma unroll
    for (int kk = 0; kk < KD; ++kk)
        r.k0[kk] = __builtin_amdgcn_raw_buffer_load_b128(k0, koff + kk * 64, 0, kNonTemporal);
#pragma unroll
    for (int kk = 0; kk < KD; ++kk)
        r.k1[kk] = __builtin_amdgcn_raw_buffer_load_b128(k1, koff + kk * 64, 0, kNonTemporal);
#pragma unroll
    for (int i = 0; i < 4; ++i) load_row(r.v[i], v0, voff + i * RB);
#pragma unroll
    for (int i = 0; i < 4; ++i) load_row(r.v[4 + i], v1, voff + i * RB);
    }
}

// ---- KV storage formats -----------------------------------------------------
// KvSame: the caches hold the query's 16-bit type.  KvE4M3: they hold OCP FP8
// E4M3 codes; KvI8: signed 8-bit integer codes (one scale per cache; the
// value of a code is decode(code) * scale).  For 8-bit codes a lane takes a
// contiguous D/4-element slice of d for K: in MFMA step kk it supplies
// K[token n][d = (D/4) q + 8 kk .. +8] and Q uses the same d, so the
// contraction over d is the same sum in another order.
struct KvSame {
    static constexpr bool k8 = false;    // 8-bit codes
    static constexpr bool kI8 = false;   // integer codes
    static constexpr bool kF32 = false;  // float32 rows (and queries)
};
struct KvE4M3 {
    static constexpr bool k8 = true;
    static constexpr bool kI8 = false;
    static constexpr bool kF32 = false;
};
struct KvI8 {
    static constexpr bool k8 = true;
    static constexpr bool kI8 = true;
    static constexpr bool kF32 = false;
};
// KvF32: float32 caches and queries, on the float32 matrix instruction
// (16x16x4: one value per lane and step, K = 4).  A lane takes 16-byte
// slices: for K, lane (n, q) holds K[token n][d = 16 kk + 4 q .. +4] and MFMA
// step (kk, e) contracts d = 16 kk + 4 q + e (the query uses the same d); for
// V, lane (m, q) holds V[token 4 q + i][d = 64 h + 4 m .. +4], and the PV
// product's output tile (h, e) holds d = 64 h + 4 m + e in its row m, so
// no register moves are needed.
struct KvF32 {
    static constexpr bool k8 = false;
    static constexpr bool kI8 = false;
    static constexpr bool kF32 = true;
};

// One 32-token chunk of 8-bit codes, as loaded.
template <int D>
struct ChunkRegs8 {
    u32x4 k0[D / 64], k1[D / 64];            // K tile 0 / 1: row n, d = (D/4) q ..
    typename Dim<D>::VRow8 v[8];             // V rows of this lane's 8 tokens, d = VW n ..
};

// One 32-token chunk of float32 rows, as loaded (two 16-token tiles; see
// KvF32): K tile t slice kk, and V rows [4 t + i] slice h.
template <int D>
struct ChunkRegsF {
    u32x4 k0[D / 16], k1[D / 16];
    u32x4 v[8][D / 64];
};

// The loads of one float32 chunk (same rules as load_chunk).
template <int BS, int D>
__device__ __forceinline__ void load_chunk(ChunkRegsF<D>& r, const char* kbase, const char* vbase,
                                           BlockIds<BS> pb, int r0, bool live0, bool live1,
                                           int kvh, int num_kv_heads, uint32_t koff,
                                           uint32_t voff) {
    constexpr int RB = D * 4;     // bytes per token row
    if constexpr (lane_addressed<BS, D>()) {
        const int lane = threadIdx.x & 63;
        load_chunk_lanes<BS, RB, D / 16, 64>(r, kbase, vbase, pb, r0, live0, live1, kvh,
                                             num_kv_heads, koff - (lane & 15) * RB,
                                             voff - 4 * (lane >> 4) * RB);
    } else {
        const uint64_t row0 = kv_row(pb.x, kvh, r0, num_kv_heads, BS) * RB;
        const uint64_t row1 = kv_row(pb.y, kvh, BS == 16 ? 0 : r0 + 16, num_kv_heads, BS) * RB;
        const __amdgpu_buffer_rsrc_t k0 = tile_rsrc<16 * RB>(kbase + row0, live0);
        const __amdgpu_buffer_rsrc_t k1 = tile_rsrc<16 * RB>(kbase + row1, live1);
        const __amdgpu_buffer_rsrc_t v0 = tile_rsrc<16 * RB>(vbase + row0, live0);
        const __amdgpu_buffer_rsrc_t v1 = tile_rsrc<16 * RB>(vbase + row1, live1);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            r.k0[kk] = __builtin_amdgcn_raw_buffer_load_b128(k0, koff + kk * 64, 0, kNonTemporal);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            r.k1[kk] = __builtin_amdgcn_raw_buffer_load_b128(k1, koff + kk * 64, 0, kNonTemporal);
#pragma unroll
        for (int i = 0; i < 4; ++i) load_row(r.v[i], v0, voff + i * RB);
#pragma unroll
        for (int i = 0; i < 4; ++i) load_row(r.v[4 + i], v1, voff + i * RB);
    }
}

// The loads of one 8-bit chunk (same rules as load_chunk: always issued, dead
// tiles through an empty descriptor, nontemporal).
template <int BS, int D>
__device__ __forceinline__ void load_chunk(ChunkRegs8<D>& r, const char* kbase, const char* vbase,
                                           BlockIds<BS> pb, int r0, bool live0, bool live1,
                                           int kvh, int num_kv_heads, uint32_t koff,
                                           uint32_t voff) {
    constexpr int RB = D;         // bytes per token row
    constexpr int kTile = 16 * RB;
    if constexpr (lane_addressed<BS, D>()) {
        const int lane = threadIdx.x & 63;
        load_chunk_lanes<BS, RB, D / 64, 16>(r, kbase, vbase, pb, r0, live0, live1, kvh,
                                             num_kv_heads, koff - (lane & 15) * RB,
                                             voff - 4 * (lane >> 4) * RB);
    } else {
    const uint64_t row0 = kv_row(pb.x, kvh, r0, num_kv_heads, BS) * RB;
    const uint64_t row1 = kv_row(pb.y, kvh, BS == 16 ? 0 : r0 + 16, num_kv_heads, BS) * RB;
    const __amdgpu_buffer_rsrc_t k0 = tile_rsrc<kTile>(kbase + row0, live0);
    const __amdgpu_buffer_rsrc_t k1 = tile_rsrc<kTile>(kbase + row1, live1);
    const __amdgpu_buffer_rsrc_t v0 = tile_rsrc<kTile>(vbase + row0, live0);
    const __amdgpu_buffer_rsrc_t v1 = tile_rsrc<kTile>(vbase + row1, live1);
#pragma unroll
    for (int h = 0; h < D / 64; ++h)
        r.k0[h] = __builtin_amdgcn_raw_buffer_load_b128(k0, koff + h * 16, 0, kNonTemporal);
#pragma unroll
    for (int h = 0; h < D / 64; ++h)
        r.k1[h] = __builtin_amdgcn_raw_buffer_load_b128(k1, koff + h * 16, 0, kNonTemporal);
#pragma unroll
    for (int i = 0; i < 4; ++i) load_row(r.v[i], v0, voff + i * RB);
#pragma unroll
    for (int i = 0; i < 4; ++i) load_row(r.v[4 + i], v1, voff + i * RB);
    }
}

// Two E4M3 codes (the low or the high half of w) -> two 16-bit values,
// exactly (every E4M3 value is representable in bf16 and in fp16).
template <bool kHigh>
__device__ __forceinline__ uint32_t e4m3_pair(BF16, uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHigh));
}
template <bool kHigh>
__device__ __forceinline__ uint32_t e4m3_pair(F16, uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, kHigh));
}
// Two signed 8-bit codes (bytes 0, 1 or 2, 3 of w) -> two 16-bit values,
// exactly (every integer in [-128, 127] is representable in bf16 and fp16).
// The sign-extending field extract is typed unsigned: convert as int.
template <bool kHigh, typename Tag>
__device__ __forceinline__ uint32_t i8_pair(Tag t, uint32_t w) {
    const int s = kHigh ? 16 : 0;
    const float lo = (float)(int)__builtin_amdgcn_sbfe(w, s, 8);
    const float hi = (float)(int)__builtin_amdgcn_sbfe(w, s + 8, 8);
    return pack2(t, lo, hi);
}

// Two codes of format Kv (the low or the high half of w) -> two 16-bit values.
template <typename Kv, bool kHigh, typename Tag>
__device__ __forceinline__ uint32_t code_pair(Tag t, uint32_t w) {
    if constexpr (Kv::kI8)
        return i8_pair<kHigh>(t, w);
    else
        return e4m3_pair<kHigh>(t, w);
}
template <typename Tag, typename Kv>
__device__ __forceinline__ u32x4 codes_eight(uint32_t w0, uint32_t w1) {
    return (u32x4){code_pair<Kv, false>(Tag(), w0), code_pair<Kv, true>(Tag(), w0),
                   code_pair<Kv, false>(Tag(), w1), code_pair<Kv, true>(Tag(), w1)};
}
// One V row slice of 8-bit codes -> the 16-bit slice.
template <typename Tag, typename Kv>
__device__ __forceinline__ u32x8 codes_row(u32x4 w) {
    return __builtin_shufflevector(codes_eight<Tag, Kv>(w[0], w[1]),
                                   codes_eight<Tag, Kv>(w[2], w[3]), 0, 1, 2, 3, 4, 5, 6, 7);
}
template <typename Tag, typename Kv>
__device__ __forceinline__ u32x4 codes_row(u32x2 w) { return codes_eight<Tag, Kv>(w[0], w[1]); }
template <typename Tag, typename Kv>
__device__ __forceinline__ u32x2 codes_row(uint32_t w) {
    return (u32x2){code_pair<Kv, false>(Tag(), w), code_pair<Kv, true>(Tag(), w)};
}

// 8-bit chunk -> the 16-bit operands compute_chunk takes (K step kk holds
// d = (D/4) q + 8 kk .. +8: dwords 2 kk, 2 kk + 1 of the lane's slice; V
// rows as for the 16-bit format).
template <typename Tag, typename Kv, int D>
__device__ __forceinline__ ChunkRegs<D> expand(const ChunkRegs8<D>& r8) {
    ChunkRegs<D> r;
#pragma unroll
    for (int kk = 0; kk < Dim<D>::KD; ++kk) {
        const int w = 2 * kk;
        const u32x4 a = r8.k0[w >> 2], b = r8.k1[w >> 2];
        r.k0[kk] = codes_eight<Tag, Kv>(a[w & 3], a[(w & 3) + 1]);
        r.k1[kk] = codes_eight<Tag, Kv>(b[w & 3], b[(w & 3) + 1]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) r.v[i] = codes_row<Tag, Kv>(r8.v[i]);
    return r;
}

template <typename Kv, int D>
using KvRegs = typename std::conditional<
    Kv::kF32, ChunkRegsF<D>,
    typename std::conditional<Kv::k8, ChunkRegs8<D>, ChunkRegs<D>>::type>::type;

// Byte offsets of this lane's K and V data inside a tile.
template <typename Kv, int D>
__device__ __forceinline__ uint32_t lane_koff(int n, int q) {
    if constexpr (Kv::kF32) return (uint32_t)(n * D + 4 * q) * 4;
    return Kv::k8 ? (uint32_t)(n * D + (D / 4) * q) : (uint32_t)(n * D + 8 * q) * 2;
}
template <typename Kv, int D>
__device__ __forceinline__ uint32_t lane_voff(int n, int q) {
    constexpr int VW = Dim<D>::VW;
    if constexpr (Kv::kF32) return (uint32_t)(4 * q * D + 4 * n) * 4;
    return Kv::k8 ? (uint32_t)(4 * q * D + VW * n) : (uint32_t)(4 * q * D + VW * n) * 2;
}

// 16-byte query slices per column tile: D/32 (16-bit: 8 values per MFMA
// step), D/16 for float32 rows (4 values, 4 steps each).
template <typename Kv, int D>
constexpr int query_slices() { return Kv::kF32 ? D / 16 : Dim<D>::KD; }

// [S, H] row of column n of decode row b (KV head kvh): query head
// col_head(kvh, n) of row b, or with verify columns (kCols) the (query row,
// head) pair the column stands for.
template <bool kCols>
__device__ __forceinline__ uint64_t column_row(const DecodeArgs& a, int b, int kvh, int n) {
    return kCols ? col_row(a, b, kvh, n) : (uint64_t)b * a.num_heads + col_head(a, kvh, n);
}

// Query operand: Q[column n][d] for the d each MFMA step contracts (see the
// K layouts above); zero for padding columns n >= ncols.
template <typename Kv, bool kCols, int D>
__device__ __forceinline__ void load_query(const DecodeArgs& a, int b, int kvh, int n, int q,
                                           int ncols, u32x4* qop) {
    constexpr int KD = Dim<D>::KD;
    if constexpr (Kv::kF32) {
        // Q[column n][d = 16 kk + 4 q .. +4]
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            qop[kk] = n < ncols ? load16(reinterpret_cast<const char*>(a.query) +
                                         (column_row<kCols>(a, b, kvh, n) * D + 16 * kk + 4 * q) *
                                             4)
                                : (u32x4){0u, 0u, 0u, 0u};
        return;
    }
    if (n < ncols) {
        const char* qp = reinterpret_cast<const char*>(a.query) +
                         column_row<kCols>(a, b, kvh, n) * D * 2;
#pragma unroll
        for (int kk = 0; kk < KD; ++kk)
            qop[kk] = load16(qp + (Kv::k8 ? (D / 4) * q + 8 * kk : 32 * kk + 8 * q) * 2);
    } else {
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) qop[kk] = (u32x4){0u, 0u, 0u, 0u};
    }
}

// Append step: lanes 0 .. D/8-1 store the newest token's K row, the next D/8
// lanes its V row (8 values each), into slot pos of the sequence's tail
// block (row: its table row).  For 8-bit codes each value is quantised:
// Q(fp32(x) * fp32(1 / scale)), Q = E4M3 (nearest, ties to even, saturating
// at +-448) or INT8 (nearest integer, ties to even, saturating at +-127).
template <typename Tag, typename Kv, int BS, int D>
__device__ __forceinline__ void append_token(const DecodeArgs& a, const ConstI32* row, int b,
                                             int kvh, int pos, int lane) {
    constexpr int LP = D / 8;     // lanes per row
    const int pb = row[pos / BS];
    if ((unsigned)pb >= (unsigned)a.num_blocks || lane >= 2 * LP) return;
    const bool is_k = lane < LP;
    const int c = lane % LP;
    // (calls that split a group append in a kernel of their own: here the
    // virtual head is the caches' head)
    const char* from = reinterpret_cast<const char*>(is_k ? a.new_key : a.new_value) +
                       (((uint64_t)b * a.kv_heads_mem + kvh) * D + c * 8) * 2;
    char* to = reinterpret_cast<char*>(const_cast<void*>(is_k ? a.key_cache : a.value_cache));
    const uint64_t r = kv_row(pb, kvh, pos % BS, a.kv_heads_mem, BS);
    const u32x4 x = load16(from);
    if constexpr (Kv::k8) {
        // both scales as register values first: a per-lane choice between
        // two kernel-argument fields would otherwise become a per-lane load
        // from a private copy of the arguments
        const float ki = __builtin_bit_cast(
            float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, a.k_inv_scale)));
        const float vi = __builtin_bit_cast(
            float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, a.v_inv_scale)));
        const float inv = is_k ? ki : vi;
        uint32_t cd[8];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float y0 = unpack_lo(Tag(), x[u]) * inv, y1 = unpack_hi(Tag(), x[u]) * inv;
            cd[2 * u] = Kv::kI8 ? i8_encode(y0) : e4m3_encode(y0);
            cd[2 * u + 1] = Kv::kI8 ? i8_encode(y1) : e4m3_encode(y1);
        }
        const u32x2 w = {cd[0] | cd[1] << 8 | cd[2] << 16 | cd[3] << 24,
                         cd[4] | cd[5] << 8 | cd[6] << 16 | cd[7] << 24};
        *reinterpret_cast<u32x2*>(to + r * D + c * 8) = w;
    } else {
        *reinterpret_cast<u32x4*>(to + r * D * 2 + c * 16) = x;
    }
}

// Running state of one wavefront: for head n (lane % 16), the reference max
// m_ref (log2 units), the accumulators O^T and the denominator l (computed
// on the matrix core as P times a ones operand, so it sums exactly the
// rounded weights the PV product uses).
template <int D>
struct WaveState {
    float m_ref;
    f32x4 acc[Dim<D>::VW];
    f32x4 acc_l;
};

template <int D>
__device__ __forceinline__ void init_state(WaveState<D>& st) {
    st.m_ref = -INFINITY;
#pragma unroll
    for (int j = 0; j < Dim<D>::VW; ++j) st.acc[j] = (f32x4){0.f, 0.f, 0.f, 0.f};
    st.acc_l = (f32x4){0.f, 0.f, 0.f, 0.f};
}

// Scores may exceed the reference max by up to 2^kLazy before the
// accumulators are rescaled (weights stay <= 2^8; float32 accumulators and
// 16-bit weights hold that range with no loss of relative precision).
constexpr float kLazy = 8.0f;

// Tokens at or past t_end (the end of the history, or of the piece) are
// excluded.  With verify columns (kCols) column n's causal end t_col (this
// lane's column in tile t) may lie before t_end; t_lo is the smallest column
// end of the wavefront.  A column that has seen no token yet has m_ref =
// -inf: its weights are then 2^(-inf) = 0 and its rescale factor 0.  NT
// column tiles (16 columns each) share the chunk's K and V operands: st,
// qop (KD per tile) and t_col hold one entry per tile.
template <typename Tag, bool kCols, int D, int NT>
__device__ __forceinline__ void compute_chunk(WaveState<D>* st, ChunkRegs<D>& r, const u32x4* qop,
                                              float sl2, int tc, int t_end, const int* t_col,
                                              int t_lo, int q) {
    constexpr int KD = Dim<D>::KD;
    constexpr int VW = Dim<D>::VW;
    // Scores: S^T[token][column] for the two 16-token tiles.
    float s[NT][8];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) s0 = mfma16x16x32(Tag(), r.k0[kk], qop[t * KD + kk], s0);
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) s1 = mfma16x16x32(Tag(), r.k1[kk], qop[t * KD + kk], s1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s[t][i] = s0[i] * sl2;
            s[t][4 + i] = s1[i] * sl2;
        }
    }
    if (tc + kChunk > (kCols ? t_lo : t_end)) {
        // Tokens at or past the end of the history are excluded (the last
        // block is masked past the context length): score -inf, and the V
        // row zeroed so stale slot contents cannot reach the accumulator.
        // A verify column's tokens past its causal end only get score -inf
        // (their V rows hold data other columns use).
        using VRow = typename Dim<D>::VRow;
        const VRow zero = {};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int t_s = kCols ? t_col[t] : t_end;
                if (tc + 4 * q + i >= t_s) s[t][i] = -INFINITY;
                if (tc + 16 + 4 * q + i >= t_s) s[t][4 + i] = -INFINITY;
            }
            if (tc + 4 * q + i >= t_end) r.v[i] = zero;
            if (tc + 16 + 4 * q + i >= t_end) r.v[4 + i] = zero;
        }
    }
    const u32x4 ones = {kOnePair<Tag>(), kOnePair<Tag>(), kOnePair<Tag>(), kOnePair<Tag>()};
    u32x4 pop[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        float cmax = fmaxf(fmaxf(fmaxf(s[t][0], s[t][1]), fmaxf(s[t][2], s[t][3])),
                           fmaxf(fmaxf(s[t][4], s[t][5]), fmaxf(s[t][6], s[t][7])));
        cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
        cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
        // Online softmax update ([MiniPaged-Qwen] §5.2), with the rescale of
        // the accumulators deferred until the running max has grown by 2^kLazy.
        WaveState<D>& w = st[t];
        if (__any(cmax > w.m_ref + kLazy)) {
            const float m_new = fmaxf(w.m_ref, cmax);
            const float alpha = kCols ? rescale_weight(w.m_ref, m_new) : fast_exp2(w.m_ref - m_new);
#pragma unroll
            for (int j = 0; j < VW; ++j) w.acc[j] *= alpha;
            w.acc_l *= alpha;
            w.m_ref = m_new;
        }
        const float m_ref = (kCols && w.m_ref == -INFINITY) ? 0.0f : w.m_ref;
#pragma unroll
        for (int u = 0; u < 4; ++u)
            pop[t][u] = pack2(Tag(), fast_exp2(s[t][2 * u] - m_ref),
                              fast_exp2(s[t][2 * u + 1] - m_ref));
        w.acc_l = mfma16x16x32(Tag(), ones, pop[t], w.acc_l);
    }
#pragma unroll
    for (int j = 0; j < VW; ++j) {
        // V^T operand for d = VW n + j: 16-bit element j of each of the 8 rows.
        const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
        u32x4 w;
#pragma unroll
        for (int u = 0; u < 4; ++u)
            w[u] = __builtin_amdgcn_perm(r.v[2 * u + 1][j >> 1], r.v[2 * u][j >> 1], sel);
#pragma unroll
        for (int t = 0; t < NT; ++t) st[t].acc[j] = mfma16x16x32(Tag(), w, pop[t], st[t].acc[j]);
    }
}

// The same chunk math on float32 rows (KvF32; decode rows only, no verify
// columns): S^T = K Q^T in D/4 steps of the 16x16x4 instruction per tile,
// the scores in the same lane layout as above, P kept in float32 in the
// registers the scores came out in (step i of a tile contracts tokens
// 4 q + i), O^T = V^T P^T per output tile (h, e), and l = P summed on the
// matrix core as before.
template <int D, int NT>
__device__ __forceinline__ void compute_chunk_f32(WaveState<D>* st, ChunkRegsF<D>& r,
                                                  const u32x4* qop, float sl2, int tc, int t_end,
                                                  int q) {
    constexpr int KF = D / 16;      // K / query slices per tile
    constexpr int VH = D / 64;      // V slices per row
    float s[NT][8];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KF; ++kk)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float qv = f32_at(qop[t * KF + kk], e);
                s0 = mfma16x16x4(f32_at(r.k0[kk], e), qv, s0);
                s1 = mfma16x16x4(f32_at(r.k1[kk], e), qv, s1);
            }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s[t][i] = s0[i] * sl2;
            s[t][4 + i] = s1[i] * sl2;
        }
    }
    if (tc + kChunk > t_end) {
        // tokens at or past the end: score -inf, V row zeroed (as above)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                if (tc + 4 * q + i >= t_end) s[t][i] = -INFINITY;
                if (tc + 16 + 4 * q + i >= t_end) s[t][4 + i] = -INFINITY;
            }
#pragma unroll
            for (int h = 0; h < VH; ++h) {
                if (tc + 4 * q + i >= t_end) r.v[i][h] = (u32x4){0u, 0u, 0u, 0u};
                if (tc + 16 + 4 * q + i >= t_end) r.v[4 + i][h] = (u32x4){0u, 0u, 0u, 0u};
            }
        }
    }
    float p[NT][8];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        float cmax = fmaxf(fmaxf(fmaxf(s[t][0], s[t][1]), fmaxf(s[t][2], s[t][3])),
                           fmaxf(fmaxf(s[t][4], s[t][5]), fmaxf(s[t][6], s[t][7])));
        cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
        cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
        WaveState<D>& w = st[t];
        if (__any(cmax > w.m_ref + kLazy)) {
            const float m_new = fmaxf(w.m_ref, cmax);
            const float alpha = fast_exp2(w.m_ref - m_new);
#pragma unroll
            for (int j = 0; j < Dim<D>::VW; ++j) w.acc[j] *= alpha;
            w.acc_l *= alpha;
            w.m_ref = m_new;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            p[t][i] = fast_exp2(s[t][i] - w.m_ref);
            w.acc_l = mfma16x16x4(1.0f, p[t][i], w.acc_l);
        }
    }
#pragma unroll
    for (int h = 0; h < VH; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float v = f32_at(r.v[i][h], e);
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    st[t].acc[4 * h + e] = mfma16x16x4(v, p[t][i], st[t].acc[4 * h + e]);
            }
}

// One chunk's math on either storage format.
template <typename Tag, typename Kv, bool kCols, int D, int NT>
__device__ __forceinline__ void compute(WaveState<D>* st, KvRegs<Kv, D>& r, const u32x4* qop,
                                        float sl2, int tc, int t_end, const int* t_col, int t_lo,
                                        int q) {
    if constexpr (Kv::kF32) {
        static_assert(!kCols, "float32 rows: decode rows only");
        compute_chunk_f32<D, NT>(st, r, qop, sl2, tc, t_end, q);
    } else if constexpr (Kv::k8) {
        ChunkRegs<D> ops = expand<Tag, Kv, D>(r);
        compute_chunk<Tag, kCols, D, NT>(st, ops, qop, sl2, tc, t_end, t_col, t_lo, q);
    } else {
        compute_chunk<Tag, kCols, D, NT>(st, r, qop, sl2, tc, t_end, t_col, t_lo, q);
    }
}

// The wavefront's chunks chunk_of(0 .. K-1) (K >= 1) of one (decode row,
// KV head): loads and math.  Two register buffers (head_dim 64 and 128):
// while chunk k is computed, chunk k+1's loads are in flight and chunk
// k+2's block numbers are being fetched (scalar loads of the table).  At
// head_dim 256 (float32 rows: 128) a chunk's operands take 128 registers,
// so there is one buffer; only the next chunk's block numbers are fetched
// ahead, and the other wavefronts of the compute unit keep its loads in
// flight.
template <typename Tag, int BS, typename Kv, bool kCols, int D, int NT, typename ChunkOf>
__device__ __forceinline__ void stream_chunks(const DecodeArgs& a, WaveState<D>* st, int K,
                                              ChunkOf chunk_of, const ConstI32* row, int L,
                                              int kvh, uint32_t koff, uint32_t voff,
                                              const u32x4* qop, int t_end, const int* t_col,
                                              int t_lo, int q, int& bad) {
    const char* kbase = reinterpret_cast<const char*>(a.key_cache);
    const char* vbase = reinterpret_cast<const char*>(a.value_cache);
    const float sl2 = a.scale_log2;
    // the caches' KV head of (virtual) head kvh
    const int H_mem = a.kv_heads_mem;
    kvh = a.kv_split == 1 ? kvh : kvh / a.kv_split;
    // tile 1 of chunk c is live when it holds history tokens
    auto tile1_live = [&](int k) { return chunk_of(k) * kChunk + 16 < L; };
    const int nb = a.num_blocks;
    // one chunk buffer where a chunk's operands take 128 registers: 16-bit
    // rows at head_dim 256, float32 rows at 128
    constexpr bool kOneBuffer = D * (Kv::kF32 ? 4 : 2) >= 512;
    if constexpr (kOneBuffer) {
        BlockIds<BS> e = chunk_entries<BS>(row, chunk_of(0), L);
        for (int k = 0; k < K; ++k) {
            KvRegs<Kv, D> buf;
            load_chunk<BS, D>(buf, kbase, vbase, chunk_blocks<BS>(e, chunk_of(k), L, nb, bad),
                              tile_row<BS>(chunk_of(k)), true, tile1_live(k), kvh, H_mem, koff,
                              voff);
            e = chunk_entries<BS>(row, chunk_of(k + 1), L);
            compute<Tag, Kv, kCols, D, NT>(st, buf, qop, sl2, chunk_of(k) * kChunk, t_end, t_col,
                                       t_lo, q);
        }
    } else {
        KvRegs<Kv, D> bufA, bufB;
        BlockIds<BS> eA = chunk_entries<BS>(row, chunk_of(0), L);
        BlockIds<BS> eB = chunk_entries<BS>(row, chunk_of(1), L);
        load_chunk<BS, D>(bufA, kbase, vbase, chunk_blocks<BS>(eA, chunk_of(0), L, nb, bad),
                          tile_row<BS>(chunk_of(0)), true, tile1_live(0), kvh, H_mem, koff,
                          voff);
        int k = 0;
        // The scheduling barriers keep each phase's loads after the previous
        // chunk's math and before this chunk's: the load counter is in
        // order, so a load hoisted above the math would make it wait for
        // the prefetch too.  A prefetch past the wave's last chunk is issued
        // dead (no bytes move) so that every path has the same loads in
        // flight.
        for (;;) {
            __builtin_amdgcn_sched_barrier(0);
            load_chunk<BS, D>(bufB, kbase, vbase,
                              chunk_blocks<BS>(eB, chunk_of(k + 1), L, nb, bad),
                              tile_row<BS>(chunk_of(k + 1)), k + 1 < K,
                              k + 1 < K && tile1_live(k + 1), kvh, H_mem, koff, voff);
            eA = chunk_entries<BS>(row, chunk_of(k + 2), L);
            __builtin_amdgcn_sched_barrier(0);
            compute<Tag, Kv, kCols, D, NT>(st, bufA, qop, sl2, chunk_of(k) * kChunk, t_end, t_col,
                                       t_lo, q);
            if (++k >= K) break;
            __builtin_amdgcn_sched_barrier(0);
            load_chunk<BS, D>(bufA, kbase, vbase,
                              chunk_blocks<BS>(eA, chunk_of(k + 1), L, nb, bad),
                              tile_row<BS>(chunk_of(k + 1)), k + 1 < K,
                              k + 1 < K && tile1_live(k + 1), kvh, H_mem, koff, voff);
            eB = chunk_entries<BS>(row, chunk_of(k + 2), L);
            __builtin_amdgcn_sched_barrier(0);
            compute<Tag, Kv, kCols, D, NT>(st, bufB, qop, sl2, chunk_of(k) * kChunk, t_end, t_col,
                                       t_lo, q);
            if (++k >= K) break;
        }
    }
}

// This lane's accumulators (column n = lane % 16, d = VW (4 q + i) + j in
// acc[j][i]; float32 rows: d = 64 h + 16 q + 4 i + e in acc[4 h + e][i]) ->
// an LDS row of the column (float offset d).
template <int D, bool kF32 = false>
__device__ __forceinline__ void stage_acc(float* col_row_lds, int q, const WaveState<D>& st) {
    constexpr int VW = Dim<D>::VW;
    if constexpr (kF32) {
#pragma unroll
        for (int h = 0; h < D / 64; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<f32x4*>(col_row_lds + 64 * h + 16 * q + 4 * i) =
                    (f32x4){st.acc[4 * h][i], st.acc[4 * h + 1][i], st.acc[4 * h + 2][i],
                            st.acc[4 * h + 3][i]};
        return;
    }
    float* ow = col_row_lds + 4 * q * VW;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j0 = 0; j0 < VW; j0 += 4)
            *reinterpret_cast<f32x4*>(ow + VW * i + j0) =
                (f32x4){st.acc[j0][i], st.acc[j0 + 1][i], st.acc[j0 + 2][i], st.acc[j0 + 3][i]};
}

constexpr int kNW = kDecodeThreads / 64;   // wavefronts per workgroup

template <int D, int NT>
struct SegmentLds {
    float m[kNW * 16 * NT];
    float l[kNW * 16 * NT];
    __attribute__((aligned(16))) float o[kNW * 16 * NT * Dim<D>::OS];
};

// Query operands and causal ends of the NT column tiles of this lane
// (column t 16 + n of tile t): see load_query and compute_chunk.
template <typename Kv, bool kCols, int D, int NT>
__device__ __forceinline__ void tile_columns(const DecodeArgs& a, int b, int kvh, int n, int q,
                                             int ntok, int L, int t_end, u32x4* qop,
                                             int* t_col) {
    const int G = a.group;
    const int ncols = ntok * pass_cols(a, kvh);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int col = t * 16 + n;
        load_query<Kv, kCols, D>(a, b, kvh, col, q, ncols, qop + t * query_slices<Kv, D>());
        // verify columns: column col attends the L - (ntok - 1 - col / G)
        // oldest tokens
        t_col[t] = kCols ? min(t_end, L - (ntok - 1 - col / G)) : t_end;
    }
}

// All wavefronts of the workgroup attend chunks [c0, c1) of (decode row b,
// KV head kvh) -- chunk c covers history tokens [32 c, 32 c + 32) -- with
// the chunks dealt round-robin to the wavefronts, then merge their states
// and write the result: the final output rows when the segment is the whole
// history (part < 0), else partition state `part`.
template <typename Tag, int BS, typename Kv, int kRows, int D, int NT>
__device__ __forceinline__ void attend_segment(const DecodeArgs& a, SegmentLds<D, NT>& sm, int b,
                                               int kvh, int L, int c0, int c1, int part) {
    constexpr bool kCols = kRows == 1;
    constexpr int OS = Dim<D>::OS;
    // The segment is the same for every lane; say so, so that block numbers
    // are fetched with scalar loads (which do not share the vector loads'
    // in-order counter) and addresses are computed once per wavefront.
    b = __builtin_amdgcn_readfirstlane(b);
    kvh = __builtin_amdgcn_readfirstlane(kvh);
    L = __builtin_amdgcn_readfirstlane(L);
    c0 = __builtin_amdgcn_readfirstlane(c0);
    c1 = __builtin_amdgcn_readfirstlane(c1);
    const int ntok = kCols ? row_tokens<kRows>(a, b) : 1;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15;
    const int q = lane >> 4;
    const int t_end = min(c1 * kChunk, L);
    const int t_lo = kCols ? min(t_end, L - (ntok - 1)) : t_end;
    u32x4 qop[NT * query_slices<Kv, D>()];
    int t_col[NT];
    tile_columns<Kv, kCols, D, NT>(a, b, kvh, n, q, ntok, L, t_end, qop, t_col);

    const ConstI32* row =
        (const ConstI32*)(a.block_tables) + table_row_offset<kRows>(a, b);
    const uint32_t koff = lane_koff<Kv, D>(n, q);
    const uint32_t voff = lane_voff<Kv, D>(n, q);

    // Append step: the wave that will read the chunk holding the newest
    // history position (L - 1) first stores that token's K/V row there.  Its
    // own later load of the row follows in program order; no other
    // wavefront reads the slot in this launch (the tail block of a sequence
    // being appended to is private to it).
    // (float32 rows are appended by a kernel of their own first)
    if constexpr (!Kv::kF32) {
        if (a.new_key != nullptr) {
            const int c_last = (L - 1) / kChunk;
            if (c_last >= c0 && c_last < c1 && (c_last - c0) % kNW == wave)
                append_token<Tag, Kv, BS, D>(a, row, b, kvh, L - 1, lane);
        }
    }

    WaveState<D> st[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) init_state(st[t]);
    int bad = 0;

    // This wave's chunks are c0 + wave + kNW k, k < K.
    const int first = c0 + wave;
    const int K = first < c1 ? (c1 - first + kNW - 1) / kNW : 0;
    if (K > 0) {
        auto chunk_of = [=](int k) { return first + kNW * min(k, K - 1); };
        stream_chunks<Tag, BS, Kv, kCols, D, NT>(a, st, K, chunk_of, row, L, kvh, koff, voff,
                                                 qop, t_end, t_col, t_lo, q, bad);
    }

    constexpr int NC = 16 * NT;   // columns per wavefront state
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int col = wave * NC + t * 16 + n;
        if (q == 0) {
            sm.m[col] = st[t].m_ref;
            sm.l[col] = st[t].acc_l[0];
        }
        stage_acc<D, Kv::kF32>(sm.o + col * OS, q, st[t]);
    }
    const bool any_bad = __syncthreads_or(bad);
    finalize_state<Tag>(a, sm.m, sm.l, sm.o, kNW, NC, NC * OS, OS, b, kvh, 0,
                        ntok * pass_cols(a, kvh), any_bad, part);
    __syncthreads();   // LDS is reused by the next segment
}

// Fixed schedule: workgroup (kvh, b, part) takes tokens [part P, part P + P).
// The partition index varies slowest, so every sequence's first (full)
// partition is dispatched before any shorter trailing one.
template <typename Tag, int BS, typename Kv, int kRows, int D, int NT>
__global__ __launch_bounds__(kDecodeThreads) void decode_mfma_fixed(DecodeArgs a) {
    __shared__ SegmentLds<D, NT> sm;
    const int kvh = blockIdx.x;
    const int b = blockIdx.y;
    const int part = blockIdx.z;
    const int ncols = row_tokens<kRows>(a, b) * pass_cols(a, kvh);
    const int L = a.context_lens[b];
    if (L < 0 || L > a.max_context_len) {
        if (part == 0) fill_cols<Tag>(a, b, kvh, 0, ncols, __builtin_nanf(""));
        return;
    }
    if (L == 0) {
        if (part == 0) fill_cols<Tag>(a, b, kvh, 0, ncols, 0.0f);
        return;
    }
    const int t_begin = part * a.part_len;
    if (t_begin >= L) return;
    const int nparts_b = (L + a.part_len - 1) / a.part_len;
    const int c0 = t_begin / kChunk;
    const int c1 = min(L, t_begin + a.part_len);
    const int c1c = (c1 + kChunk - 1) / kChunk;
    attend_segment<Tag, BS, Kv, kRows, D, NT>(a, sm, b, kvh, L, c0, c1c,
                                              nparts_b == 1 ? -1 : part);
}

// ---- balanced schedule ----------------------------------------------------
//
// The flattened (sequence, KV head, chunk) work list is cut into gridDim.x
// equal ranges, one per workgroup (all resident at once), and each range
// into kNW contiguous wavefront ranges.  A wavefront walks its own range
// with no barrier: a (sequence, KV head) segment lying wholly inside it is
// finished there and its output rows written; the segment the wavefront
// starts inside and the one it ends inside ("edge pieces", at most two) are
// staged in LDS.  After one barrier the workgroup merges the edge pieces of
// each segment and writes either its output rows (the segment lies inside
// the workgroup's range) or a partial state in slot [w][0] (continues from
// the previous range) or [w][1] (continues into the next) for the merge
// kernel.

// Output rows a wavefront stages in LDS before writing them (balanced
// schedule, 16-bit decode rows at head_dim 64 and 128): what the compute
// unit's 160 KB leave beside the edge pieces and the largest prefix table
// (2 * 2048 + 1 ints) -- 200 rows at head_dim 64 (26 KB a wavefront), 75 at
// 128 (19.5 KB), checked where the stage is declared.
template <int D>
constexpr int stage_rows() { return D == 64 ? 200 : 75; }

// write_rows into LDS: the same packed 16-bit values, row n of the history
// (n < ncols) at stage_o + n * D / 8 (16-byte words), its [S, H] row index
// at stage_r[n]; written to the output later by flush_stage.
template <typename Tag, int D>
__device__ __forceinline__ void stage_rows_of(const DecodeArgs& a, int b, int kvh, int ncols,
                                              const WaveState<D>& st, bool bad, u32x4* stage_o,
                                              uint32_t* stage_r) {
    constexpr int VW = Dim<D>::VW;
    const int lane = threadIdx.x & 63;
    const int n = lane & 15;
    const int q = lane >> 4;
    if (n >= ncols) return;
    const float scale = a.out_scale / st.acc_l[0];
    // this lane's 4 VW values of row n, d = 4 q VW .. +4 VW: VW / 2 words
    uint32_t w[2 * VW];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < VW; j += 2)
            w[(VW * i + j) / 2] =
                pack2(Tag(), bad ? __builtin_nanf("") : st.acc[j][i] * scale,
                      bad ? __builtin_nanf("") : st.acc[j + 1][i] * scale);
    u32x4* dst = stage_o + n * (D / 8) + q * (VW / 2);
#pragma unroll
    for (int k = 0; k < VW / 2; ++k)
        dst[k] = (u32x4){w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]};
    if (q == 0) stage_r[n] = (uint32_t)((uint64_t)b * a.num_heads + col_head(a, kvh, n));
}

// The staged rows (count rows) to the output, 16 bytes a lane.  Rows are a
// wavefront's own: its LDS writes above come first in its instruction order.
template <int D>
__device__ __forceinline__ void flush_stage(const DecodeArgs& a, const u32x4* stage_o,
                                            const uint32_t* stage_r, int count) {
    constexpr int W = D / 8;    // 16-byte words a row
    const int lane = threadIdx.x & 63;
    for (int u = lane; u < count * W; u += 64) {
        const int r = u / W;
        *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(a.out) +
                                  ((uint64_t)stage_r[r] * D) * 2 + (u - r * W) * 16) =
            stage_o[u];
    }
}

// Edge pieces of the workgroup's wavefronts, in work-list order: piece
// 2 v + 0 is the segment wavefront v starts inside (or its only piece),
// 2 v + 1 the one it ends inside.  key: sequence * num_kv_heads + KV head of
// the piece's segment, -1 when the piece is absent.
template <int D, int NT>
struct EdgeLds {
    float m[2 * kNW][16 * NT];
    float l[2 * kNW][16 * NT];
    __attribute__((aligned(16))) float o[2 * kNW][16 * NT * Dim<D>::OS];
    int key[2 * kNW];
    int bad[2 * kNW];
};

// Wavefront state over chunks [cs, ce) of (decode row b, KV head kvh) with
// a history of L tokens in block-table row trow (ntok query rows carried:
// verify columns): the two-buffer pipeline of attend_segment with the chunks
// taken in order.  Includes the append step when the newest history position
// lies in [cs, ce): this wavefront alone reads that chunk.
template <typename Tag, int BS, typename Kv, int kRows, int D, int NT>
__device__ __forceinline__ void attend_piece(const DecodeArgs& a, int b, int trow, int kvh, int L,
                                             int ntok, int cs, int ce, WaveState<D>* st,
                                             int& bad) {
    constexpr bool kCols = kRows == 1;
    const int lane = threadIdx.x & 63;
    const int n = lane & 15;
    const int q = lane >> 4;
    const int t_end = min(ce * kChunk, L);
    const int t_lo = kCols ? min(t_end, L - (ntok - 1)) : t_end;
    u32x4 qop[NT * query_slices<Kv, D>()];
    int t_col[NT];
    tile_columns<Kv, kCols, D, NT>(a, b, kvh, n, q, ntok, L, t_end, qop, t_col);

    const ConstI32* row =
        (const ConstI32*)(a.block_tables) + (uint64_t)trow * a.max_blocks_per_seq;
    const uint32_t koff = lane_koff<Kv, D>(n, q);
    const uint32_t voff = lane_voff<Kv, D>(n, q);

    // (float32 rows are appended by a kernel of their own first)
    if constexpr (!Kv::kF32) {
        if (a.new_key != nullptr) {
            const int c_last = (L - 1) / kChunk;
            if (c_last >= cs && c_last < ce)
                append_token<Tag, Kv, BS, D>(a, row, b, kvh, L - 1, lane);
        }
    }

    const int K = ce - cs;
    auto chunk_of = [=](int k) { return cs + min(k, K - 1); };
    stream_chunks<Tag, BS, Kv, kCols, D, NT>(a, st, K, chunk_of, row, L, kvh, koff, voff, qop,
                                             t_end, t_col, t_lo, q, bad);
}

// Output rows of a whole history held by one wavefront: o = õ / l for the
// ncols columns (the G heads of the group; verify: its (query row, head)
// pairs) -- lane 16 q + n holds column n, d = VW (4 q + i) + j in acc[j][i]
// -- rounded once to the storage type; NaN when a table entry was out of the
// pool.
template <typename Tag, bool kCols, int D>
__device__ __forceinline__ void write_rows(const DecodeArgs& a, int b, int kvh, int ncols,
                                           int col0, const WaveState<D>& st, bool bad) {
    constexpr int VW = Dim<D>::VW;
    const int lane = threadIdx.x & 63;
    const int n = col0 + (lane & 15);
    const int q = lane >> 4;
    if (n >= ncols) return;
    // one division per column, then products (an IEEE division per element
    // costs about ten instructions, and short histories write rows often)
    const float scale = a.out_scale / st.acc_l[0];
    if constexpr (std::is_same<Tag, F32>::value) {
        // float32 rows (layout of stage_acc): d = 64 h + 16 q + 4 i + e
        float* orow = reinterpret_cast<float*>(a.out) + column_row<kCols>(a, b, kvh, n) * D;
#pragma unroll
        for (int h = 0; h < D / 64; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                f32x4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    o[e] = bad ? __builtin_nanf("") : st.acc[4 * h + e][i] * scale;
                *reinterpret_cast<f32x4*>(orow + 64 * h + 16 * q + 4 * i) = o;
            }
    } else {
        char* orow = reinterpret_cast<char*>(a.out) +
                     (column_row<kCols>(a, b, kvh, n) * D + 4 * q * VW) * 2;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float o[VW];
#pragma unroll
            for (int j = 0; j < VW; ++j) o[j] = bad ? __builtin_nanf("") : st.acc[j][i] * scale;
            if constexpr (VW >= 8) {
#pragma unroll
                for (int j0 = 0; j0 < VW; j0 += 8) {
                    const u32x4 v = {pack2(Tag(), o[j0], o[j0 + 1]),
                                     pack2(Tag(), o[j0 + 2], o[j0 + 3]),
                                     pack2(Tag(), o[j0 + 4], o[j0 + 5]),
                                     pack2(Tag(), o[j0 + 6], o[j0 + 7])};
                    *reinterpret_cast<u32x4*>(orow + 2 * VW * i + 2 * j0) = v;
                }
            } else {
                const u32x2 v = {pack2(Tag(), o[0], o[1]), pack2(Tag(), o[2], o[3])};
                *reinterpret_cast<u32x2*>(orow + 2 * VW * i) = v;
            }
        }
    }
}

// Merge of the edge pieces in `mask` (bit p: piece p) of one segment (the
// update of [MiniPaged-Qwen] §5.2 applied to whole states, in piece order)
// and its write for its ncols columns: output rows when plse == nullptr,
// else the partial state (o~/l, m + log2 l) at (plse, po) -- the empty state
// (o 0, lse -inf) for a verify column none of whose tokens lie in the
// pieces.  Called by every thread of the workgroup; a thread takes 4
// consecutive d of one column.  The pieces are listed by position in NP
// slots, NP >= the number of pieces (absent slots repeat the last piece with
// weight 0), so that all of a thread's LDS reads are issued together.
template <typename Tag, bool kCols, int D, int NT, int NP>
__device__ __forceinline__ void finalize_edges_n(const DecodeArgs& a, const EdgeLds<D, NT>& e,
                                                 unsigned mask, int b, int kvh, int ncols,
                                                 bool bad, float* plse, float* po) {
    constexpr int OS = Dim<D>::OS;
    constexpr int D4 = D / 4;
    int idx[NP];
    bool on[NP];
    unsigned mm = mask;
    int last = 0;
#pragma unroll
    for (int k = 0; k < NP; ++k) {
        on[k] = mm != 0;
        idx[k] = on[k] ? __builtin_ctz(mm) : last;
        last = idx[k];
        mm &= mm - 1;
    }
    for (int it = threadIdx.x; it < ncols * D4; it += blockDim.x) {
        const int g = it / D4;
        const int d = (it % D4) * 4;
        float mv[NP], lv[NP];
        f32x4 ov[NP];
#pragma unroll
        for (int k = 0; k < NP; ++k) {
            mv[k] = e.m[idx[k]][g];
            lv[k] = e.l[idx[k]][g];
            ov[k] = *reinterpret_cast<const f32x4*>(&e.o[idx[k]][g * OS + d]);
        }
        float M = -INFINITY;
#pragma unroll
        for (int k = 0; k < NP; ++k) M = fmaxf(M, on[k] ? mv[k] : -INFINITY);
        float den = 0.0f;
        f32x4 num = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < NP; ++k) {
            const float w = on[k] ? rescale_weight(mv[k], M) : 0.0f;
            den += w * lv[k];
            num += w * ov[k];
        }
        f32x4 o = num * (den == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(den));
        if (bad) o = (f32x4){__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""),
                             __builtin_nanf("")};
        if (plse == nullptr) {
            store4(Tag(), a.out, column_row<kCols>(a, b, kvh, g) * D + d, a.out_scale * o);
        } else {
            *reinterpret_cast<f32x4*>(po + g * D + d) = o;
            if (d == 0) plse[g] = bad ? __builtin_nanf("") : M + __log2f(den);
        }
    }
}

// The merge above with as few slots as the segment has pieces (1, 2, 4 or
// all 2 kNW): at one wavefront per SIMD this loop runs on the critical path
// at the end of the workgroup, and its length is set by its instruction count.
template <typename Tag, bool kCols, int D, int NT>
__device__ __forceinline__ void finalize_edges(const DecodeArgs& a, const EdgeLds<D, NT>& e,
                                               unsigned mask, int b, int kvh, int ncols, bool bad,
                                               float* plse, float* po) {
    const int np = __builtin_popcount(mask);
    if (np == 1)
        finalize_edges_n<Tag, kCols, D, NT, 1>(a, e, mask, b, kvh, ncols, bad, plse, po);
    else if (np == 2)
        finalize_edges_n<Tag, kCols, D, NT, 2>(a, e, mask, b, kvh, ncols, bad, plse, po);
    else if (np <= 4)
        finalize_edges_n<Tag, kCols, D, NT, 4>(a, e, mask, b, kvh, ncols, bad, plse, po);
    else
        finalize_edges_n<Tag, kCols, D, NT, 2 * kNW>(a, e, mask, b, kvh, ncols, bad, plse, po);
}

// The prefix table of the balanced schedule (num_seqs + 1 ints), the decode
// rows' context lengths (num_seqs ints) and, for verify rows, their row map
// (num_seqs ints: block-table row * 64 + query rows carried) are dynamic
// LDS, sized at launch.
extern __shared__ int balanced_pref[];

template <int kRows>
constexpr int balanced_lds_ints(int num_seqs) {
    return (kRows == 1 ? 3 : 2) * num_seqs + 1;
}

// The first arguments (p0, p1, n0) are the arrays the prologue reads first:
// the context lengths (p1 unused, n0 = num_seqs), or for verify rows the
// query starts and the sequences' lengths (n0 = num_src_seqs).  They come
// first so that the compiler preloads them into scalar registers
// (-amdgpu-kernarg-preload-count): the first loads then leave at once,
// without a round trip for the kernel arguments before them.
template <typename Tag, int BS, typename Kv, int kRows, int D, int NT>
__global__ __launch_bounds__(kDecodeThreads) void decode_mfma_balanced(
    const int32_t* __restrict__ p0, const int32_t* __restrict__ p1, int n0, DecodeArgs a) {
    constexpr bool kCols = kRows == 1;
    constexpr int OS = Dim<D>::OS;
    constexpr int NC = 16 * NT;   // columns per slot
    __shared__ EdgeLds<D, NT> edge;
    __shared__ int wsum[kNW];
    // Whole histories' output rows are staged and written after the
    // wavefront's last piece: output writes that reach memory while the
    // K/V stream is being read slow it far beyond their size (2048 x
    // U[32, 255] tokens: 137 us with the rows stored as each history ends,
    // 114 us with the same stores all aimed at a few cached lines).  16-bit
    // decode rows at head_dim 64 and 128, one column tile; a stage that is
    // full, or another case, stores directly.
    constexpr bool kStage = D <= 128 && NT == 1 && kRows == 0 && !Kv::kF32;
    constexpr int SR = kStage ? stage_rows<D>() : 1;
    __shared__ u32x4 stage_o[kStage ? kNW * SR * (D / 8) : 1];
    __shared__ uint32_t stage_r[kStage ? kNW * SR : 1];
    static_assert(!kStage || sizeof(edge) + sizeof(wsum) + sizeof(stage_o) + sizeof(stage_r) +
                                     (2 * kMaxBalancedSeqs + 1) * sizeof(int) <=
                                 160 * 1024,
                  "staged rows, edge pieces and prefix table exceed the compute unit's LDS");
    // this thread's first entries, loaded before anything waits
    const int t0 = threadIdx.x;
    // (decode rows: the first row of this thread's block in unit_prefix)
    const int i00 = kRows == 1 ? t0 : unit_prefix_row(t0, n0);
    const int v0 = i00 < n0 + (kRows == 1 ? 1 : 0) ? p0[i00] : 0;
    const int v1 = kRows == 1 && t0 < n0 ? p1[t0] : 0;
    constexpr int kSU = Kv::k8 ? kStartUnits8 : kStartUnits16;
    int* pref = balanced_pref;
    int* lens = pref + a.num_seqs + 1;
    int* rmap = lens + a.num_seqs;     // verify rows only
    if constexpr (kRows == 1) {
        // Verify rows: the row map of every decode row, from the sequences'
        // query starts and lengths staged in the edge LDS (untouched until
        // the first piece ends; unit_prefix's barriers come first).
        static_assert(sizeof(edge.o) >= (2 * kMaxVerifyFoldSeqs + 1) * sizeof(int),
                      "edge LDS too small to stage the sequences");
        int* qs = reinterpret_cast<int*>(&edge.o);
        int* sl = qs + n0 + 1;
        for (int i = t0; i <= n0; i += blockDim.x) {
            qs[i] = i == t0 ? v0 : p0[i];
            if (i < n0) sl[i] = i == t0 ? v1 : p1[i];
        }
        __syncthreads();
        unit_prefix(a, kSU, [&](int r) {
            const VerifyRow v = verify_row([=](int i) { return qs[i]; },
                                           [=](int i) { return sl[i]; }, n0,
                                           a.max_query_len, a.max_context_len, a.row_group, r);
            rmap[r] = v.table_row * 64 + v.ntok;
            return v.len;
        }, pref, lens, wsum);
    } else {
        unit_prefix(a, kSU, [&](int r) { return r == i00 ? v0 : p0[r]; }, pref, lens, wsum);
    }
    // query rows decode row b carries, and its block-table row (b is uniform)
    auto ntok_of = [&](int b) {
        return kRows == 1 ? __builtin_amdgcn_readfirstlane(rmap[b] & 63) : 1;
    };
    auto trow_of = [&](int b) {
        return kRows == 1 ? __builtin_amdgcn_readfirstlane(rmap[b] >> 6) : b;
    };
    const int H_kv = a.num_kv_heads;
    const int64_t T = (int64_t)H_kv * pref[a.num_seqs];
    const int w = blockIdx.x;

    // Output rows of decode rows with no history to attend: zeros for an
    // empty one, NaN for an invalid length (rows w, w + num_wg, ...: every
    // wavefront tests 64 of them at once, and the workgroup writes those
    // found).
    const int nmine = a.num_seqs > w ? (a.num_seqs - w + a.num_wg - 1) / a.num_wg : 0;
    for (int k0 = 0; k0 < nmine; k0 += 64) {
        const int k = k0 + (threadIdx.x & 63);
        const int Lk = k < nmine ? lens[w + k * a.num_wg] : 1;
        uint64_t todo = __ballot(!(Lk > 0 && Lk <= a.max_context_len));
        while (todo != 0) {
            const int r = w + (k0 + __builtin_ctzll(todo)) * a.num_wg;
            todo &= todo - 1;
            const float v = lens[r] == 0 ? 0.0f : __builtin_nanf("");
            const int64_t count = (int64_t)ntok_of(r) * a.num_heads * D;
            const uint64_t base = (uint64_t)r * a.num_heads * D;
            for (int64_t i = threadIdx.x; i < count; i += blockDim.x)
                store_elem(Tag(), a.out, base + i, v);
        }
    }

    // record of the segment whose first piece this range leaves in [w][1]
    int4 meta = make_int4(-1, 0, (int)(uint32_t)T, (int)(T >> 32));
    const int64_t xb = T > 0 ? range_start(w, T, a.num_wg) : 0;
    const int64_t xe = T > 0 ? range_start(w + 1, T, a.num_wg) : 0;
    if (xb >= xe) {
        if (threadIdx.x == 0) reinterpret_cast<int4*>(a.ws_meta)[w] = meta;
        return;
    }

    const int lane = threadIdx.x & 63;
    const int n = lane & 15;
    const int q = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t ws = xb + wave * (xe - xb) / kNW;       // this wavefront's range
    const int64_t we = xb + (wave + 1) * (xe - xb) / kNW;
    if (lane < 2) edge.key[2 * wave + lane] = -1;
    int staged = 0;     // rows in this wavefront's stage

    for (int64_t x = ws; x < we;) {
        const int b = find_seq(pref, a.num_seqs, H_kv, x);
        const int nu = __builtin_amdgcn_readfirstlane(pref[b + 1] - pref[b]);
        const int nb = (nu - kSU) / kChunkUnits;
        const int64_t off = x - (int64_t)H_kv * pref[b];
        const int kvh = __builtin_amdgcn_readfirstlane(
            (off >> 31) == 0 ? (int)((uint32_t)off / (uint32_t)nu) : (int)(off / nu));
        const int u0 = __builtin_amdgcn_readfirstlane((int)(off - (int64_t)kvh * nu));
        const int u1 = __builtin_amdgcn_readfirstlane((int)min((int64_t)nu, u0 + (we - x)));
        const int c0 = chunks_before_unit(u0, nb, kSU);
        const int c1 = chunks_before_unit(u1, nb, kSU);
        x += u1 - u0;
        // no chunk starts here: nothing to do before the history's first
        // chunk or after its last; inside it, an empty piece keeps the
        // pieces of every range the history crosses in place
        if (c0 == c1 && (c0 == 0 || c0 == nb)) continue;
        const int L = __builtin_amdgcn_readfirstlane(lens[b]);
        const int ntok = ntok_of(b);

        WaveState<D> st[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) init_state(st[t]);
        int bad = 0;
        if (c0 < c1)
            attend_piece<Tag, BS, Kv, kRows, D, NT>(a, b, trow_of(b), kvh, L, ntok, c0, c1, st,
                                                    bad);

        const bool starts_before = c0 > 0;    // the segment began before this range
        const bool ends_after = c1 < nb;      // it continues past this range
        if (!starts_before && !ends_after) {
            const int ncols = ntok * pass_cols(a, kvh);
            bool kept = false;
            if constexpr (kStage) {
                if (staged + ncols <= SR) {
                    stage_rows_of<Tag, D>(a, b, kvh, ncols, st[0], bad != 0,
                                          &stage_o[(wave * SR + staged) * (D / 8)],
                                          &stage_r[wave * SR + staged]);
                    staged += ncols;
                    kept = true;
                }
            }
            if (!kept) {
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    write_rows<Tag, kCols, D>(a, b, kvh, ncols, t * 16, st[t], bad != 0);
            }
        } else {
            const int p = 2 * wave + (starts_before ? 0 : 1);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int col = t * 16 + n;
                if (q == 0) {
                    edge.m[p][col] = st[t].m_ref;
                    edge.l[p][col] = st[t].acc_l[0];
                }
                stage_acc<D, Kv::kF32>(&edge.o[p][col * OS], q, st[t]);
            }
            if (lane == 0) {
                edge.key[p] = b * H_kv + kvh;
                edge.bad[p] = bad;
            }
        }
    }
    if constexpr (kStage) {
        if (staged > 0) {
            // (the wavefront's own LDS writes, read back by other lanes)
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            flush_stage<D>(a, &stage_o[wave * SR * (D / 8)], &stage_r[wave * SR], staged);
        }
    }
    __syncthreads();

    // The edge pieces of one segment are consecutive in work-list order
    // (absent pieces aside): gather each segment's as a bit mask and go on
    // after its last piece.
    for (int p = 0; p < 2 * kNW;) {
        const int k = edge.key[p];
        if (k < 0) { ++p; continue; }
        unsigned mask = 0;
        int bad = 0;
#pragma unroll
        for (int p1 = 0; p1 < 2 * kNW; ++p1) {
            if (edge.key[p1] == k) {
                mask |= 1u << p1;
                bad |= edge.bad[p1];
            }
        }
        const int p1 = 32 - __builtin_clz(mask);
        const int b = k / H_kv;
        const int kvh = k - b * H_kv;
        const int nu = pref[b + 1] - pref[b];
        const int nb = (nu - kSU) / kChunkUnits;
        // units where the history's first and last chunks start
        const int64_t xf = (int64_t)H_kv * pref[b] + (int64_t)kvh * nu + kSU;
        const int64_t xl = xf + (int64_t)kChunkUnits * (nb - 1);
        const bool head = xf < xb;            // continues from the previous range
        const bool tail = xl >= xe;           // continues into the next range
        const int ntok = ntok_of(b);
        const int ncols = ntok * pass_cols(a, kvh);
        if (!head && !tail) {
            finalize_edges<Tag, kCols, D, NT>(a, edge, mask, b, kvh, ncols, bad != 0, nullptr,
                                              nullptr);
        } else {
            const uint64_t slot = (uint64_t)w * 2 + (head ? 0 : 1);
            finalize_edges<Tag, kCols, D, NT>(a, edge, mask, b, kvh, ncols, bad != 0,
                                              a.ws_lse + slot * NC, a.ws_out + slot * NC * D);
            if (!head) meta.x = k, meta.y = range_owner(xl, T, a.num_wg) | ntok << 16;
        }
        p = p1;
    }
    if (threadIdx.x == 0) reinterpret_cast<int4*>(a.ws_meta)[w] = meta;
}

template <typename Tag, int BS, typename Kv, int kRows, int D, int NT>
hipError_t launch_rows(const DecodeArgs& a, hipStream_t s) {
    if (a.schedule == kBalanced) {
        const size_t pref_bytes = (size_t)balanced_lds_ints<kRows>(a.num_seqs) * sizeof(int);
        const bool rows = kRows == 1;
        hipLaunchKernelGGL((decode_mfma_balanced<Tag, BS, Kv, kRows, D, NT>), dim3(a.num_wg),
                           dim3(kDecodeThreads), pref_bytes, s,
                           rows ? a.query_start : a.context_lens,
                           rows ? a.src_lens : (const int32_t*)nullptr,
                           rows ? a.num_src_seqs : a.num_seqs, a);
    } else {
        dim3 grid(a.num_kv_heads, a.num_seqs, a.num_parts);
        hipLaunchKernelGGL((decode_mfma_fixed<Tag, BS, Kv, kRows, D, NT>), grid,
                           dim3(kDecodeThreads), 0, s, a);
    }
    return hipGetLastError();
}

// One column tile, or two (up to 32 columns: GQA groups of 17 to 32 heads, or
// verify rows carrying more than 16 (row, head) pairs; head_dim 64 and 128,
// whose edge LDS then still fits a compute unit).  Decode rows with a row map
// (verify mode, 16-bit caches only) run their own instantiations.
template <typename Tag, int BS, typename Kv, int kRows, int D>
hipError_t launch_tiles(const DecodeArgs& a, hipStream_t s) {
    if constexpr (D <= 128) {
        if (a.col_tiles == 2) return launch_rows<Tag, BS, Kv, kRows, D, 2>(a, s);
    }
    return launch_rows<Tag, BS, Kv, kRows, D, 1>(a, s);
}

template <typename Tag, int BS, int D>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t s) {
    if constexpr (std::is_same<Tag, F32>::value) {
        // float32 rows: decode rows of one column tile (at most 16 heads a pass)
        return launch_rows<F32, BS, KvF32, 0, D, 1>(a, s);
    } else {
        if (a.kv_format == kKvE4M3) return launch_tiles<Tag, BS, KvE4M3, 0, D>(a, s);
        if (a.kv_format == kKvI8) return launch_tiles<Tag, BS, KvI8, 0, D>(a, s);
        if (a.table_rows == nullptr && a.query_start == nullptr)
            return launch_tiles<Tag, BS, KvSame, 0, D>(a, s);
        return launch_tiles<Tag, BS, KvSame, 1, D>(a, s);
    }
}

template <typename Tag, int D>
hipError_t launch_bs(const DecodeArgs& a, hipStream_t s) {
    switch (a.block_size) {
        case 8: return launch_typed<Tag, 8, D>(a, s);
        case 16: return launch_typed<Tag, 16, D>(a, s);
        case 32: return launch_typed<Tag, 32, D>(a, s);
        default: return launch_typed<Tag, 64, D>(a, s);
    }
}

}  // namespace
}  // namespace pa
