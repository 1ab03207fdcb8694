// Decode GEMV kernels instantiated for one weight format (W_FP8ROW).
#include "nq_gemv_kernels.h"

namespace nq {

NQ_GEMV_FMT_ENTRY(gemv_launch_fp8row) {
    launch_fmt<W_FP8ROW>(p, packed, w, scales, x, Tc, N, K, bf16_out, y, partial, counters, stream);
}

}  // namespace nq
