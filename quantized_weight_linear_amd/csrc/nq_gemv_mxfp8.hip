// Decode GEMV kernels instantiated for one weight format (W_MXFP8).
#include "nq_gemv_kernels.h"

namespace nq {

NQ_GEMV_FMT_ENTRY(gemv_launch_mxfp8) {
    launch_fmt<W_MXFP8>(p, packed, w, scales, x, Tc, N, K, bf16_out, y, partial, counters, stream);
}

}  // namespace nq
