// Matrix-core decode: which shapes it serves, its launch geometry, and the
// dispatch to the per-head-dim translation units (pa_decode_mfma_d*.hip).
#include "pa_internal.h"

namespace pa {

// Groups of up to 16 heads fill one column tile; up to 32 take two (head_dim
// 64 and 128, whose edge LDS then still fits a compute unit).  float32 rows
// (the float32 matrix instruction) at head_dim 64 and 128, one column tile:
// at 256 a 32-token chunk of float32 rows would take 256 registers.
bool mfma_supported(pa_dtype dt, int head_dim, int block_size, int group) {
    const bool bs_ok =
        block_size == 8 || block_size == 16 || block_size == 32 || block_size == 64;
    if (dt == PA_F32)
        return (head_dim == 64 || head_dim == 128) && bs_ok && group >= 1 && group <= kMaxGroup;
    return (dt == PA_BF16 || dt == PA_F16) &&
           (head_dim == 64 || head_dim == 128 || head_dim == 256) && bs_ok && group >= 1 &&
           (group <= kMaxGroup || (group <= 2 * kMaxGroup && head_dim <= 128));
}

// A larger group is split into passes over the KV head's history, each
// serving at most the columns one pass holds (16, or 32 at head_dim 64/128):
// the fewest such passes, with heads dealt as evenly as ceil() allows (the
// last pass may hold fewer).  Each pass reads the history once more, still
// less often than the vector-ALU kernel, which re-reads it for every 8 heads.
int mfma_split(pa_dtype dt, int head_dim, int block_size, int group) {
    if (group < 1 || !mfma_supported(dt, head_dim, block_size, 1)) return 0;
    if (mfma_supported(dt, head_dim, block_size, group)) return 1;
    const int cap = head_dim <= 128 && dt != PA_F32 ? 2 * kMaxGroup : kMaxGroup;
    const int pg = mfma_pass_group(group, (group + cap - 1) / cap);
    return (group + pg - 1) / pg;   // every pass, the last included, holds a head
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
