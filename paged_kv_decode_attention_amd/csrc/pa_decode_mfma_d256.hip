// Matrix-core decode kernels at head_dim 256 (one translation unit per head
// dim; the templates are in pa_decode_mfma.h).
#include "pa_decode_mfma.h"

namespace pa {

hipError_t launch_decode_mfma_d256(const DecodeArgs& a, pa_dtype dt, hipStream_t s) {
    return dt == PA_BF16 ? launch_bs<BF16, 256>(a, s) : launch_bs<F16, 256>(a, s);
}

}  // namespace pa
