// Matrix-core decode: which shapes it serves, its launch geometry, and the
// dispatch to the per-head-dim translation units (pa_decode_mfma_d*.hip).
#include "pa_internal.h"

namespace pa {

// Groups of up to 16 heads fill one column tile; up to 32 take two (head_dim
// 64 and 128, whose edge LDS then still fits a compute unit).
bool mfma_supported(pa_dtype dt, int head_dim, int block_size, int group) {
    return (dt == PA_BF16 || dt == PA_F16) &&
           (head_dim == 64 || head_dim == 128 || head_dim == 256) &&
           (block_size == 8 || block_size == 16 || block_size == 32 || block_size == 64) &&
           group >= 1 && (group <= kMaxGroup || (group <= 2 * kMaxGroup && head_dim <= 128));
}

// A larger group is split into the fewest passes of equal groups that one
// pass serves, at most kMaxSplit: each pass reads the KV head's history once
// more, still cheaper than the vector-ALU kernel, which re-reads it for
// every 8 heads.  (A group with no such split -- a prime above 32 -- stays
// on the vector-ALU kernel.)
constexpr int kMaxSplit = 4;

int mfma_split(pa_dtype dt, int head_dim, int block_size, int group) {
    if (group < 1) return 0;
    for (int sp = 1; sp <= kMaxSplit && sp <= group; ++sp)
        if (group % sp == 0 && mfma_supported(dt, head_dim, block_size, group / sp)) return sp;
    return 0;
}

// Workgroups of the balanced schedule per compute unit: one (4 wavefronts,
// one per SIMD).  One wavefront's two chunk buffers per SIMD already keep the
// compute unit at its share of the HBM bandwidth; more, smaller ranges only
// add split segments, partial states and merge work (measured: two per
// compute unit is 2.5 % slower at head_dim 128, four 4 % slower at 64).
int mfma_workgroups_per_cu(int) { return 1; }

hipError_t launch_decode_mfma(const DecodeArgs& a, pa_dtype dt, hipStream_t s) {
    switch (a.head_dim) {
        case 64: return launch_decode_mfma_d64(a, dt, s);
        case 128: return launch_decode_mfma_d128(a, dt, s);
        default: return launch_decode_mfma_d256(a, dt, s);
    }
}

}  // namespace pa
