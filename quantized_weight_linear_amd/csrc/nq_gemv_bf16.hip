// Decode GEMV kernels instantiated for one weight format (W_BF16).
#include "nq_gemv_kernels.h"

namespace nq {

NQ_GEMV_FMT_ENTRY(gemv_launch_bf16) {
    launch_fmt<W_BF16>(p, packed, w, scales, x, Tc, N, K, bf16_out, y, partial, counters, stream);
}

}  // namespace nq
