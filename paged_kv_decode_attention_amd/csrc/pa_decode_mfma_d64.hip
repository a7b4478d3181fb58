// Matrix-core decode kernels at head_dim 64 (one translation unit per head
// dim; the templates are in pa_decode_mfma.h).
#include "pa_decode_mfma.h"

namespace pa {

hipError_t launch_decode_mfma_d64(const DecodeArgs& a, pa_dtype dt, hipStream_t s) {
    if (dt == PA_F32) return launch_bs<F32, 64>(a, s);
    return dt == PA_BF16 ? launch_bs<BF16, 64>(a, s) : launch_bs<F16, 64>(a, s);
}

}  // namespace pa
