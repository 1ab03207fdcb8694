// Decode GEMV kernels instantiated for one weight format (W_Q8G32).
#include "nq_gemv_kernels.h"

namespace nq {

NQ_GEMV_FMT_ENTRY(gemv_launch_q8g32) {
    launch_fmt<W_Q8G32>(p, packed, w, scales, x, Tc, N, K, bf16_out, y, partial, counters, stream);
}

}  // namespace nq
