// Matrix-core decode kernels at head_dim 128 (one translation unit per head
// dim; the templates are in pa_decode_mfma.h).
#include "pa_decode_mfma.h"

namespace pa {

hipError_t launch_decode_mfma_d128(const DecodeArgs& a, pa_dtype dt, hipStream_t s) {
    if (dt == PA_F32) return launch_bs<F32, 128>(a, s);
    return dt == PA_BF16 ? launch_bs<BF16, 128>(a, s) : launch_bs<F16, 128>(a, s);
}

}  // namespace pa
