// A plain streaming read of device memory: the measured HBM read ceiling that
// the weight-streaming kernels are compared against.  Every thread reads
// 16-byte pieces i = tid + j * stride (stride = all threads of the grid),
// READ_UNROLL of them issued back to back before any is used, with
// non-temporal global loads (the form the decode GEMVs load their weights
// with); piece indices past the end are clamped to the last piece, so every
// group keeps READ_UNROLL loads in flight without a branch.  The pieces are
// folded into one word per workgroup so the loads cannot be dropped; the sink
// receives one word per workgroup.
#include "nq_device.h"
#include "nq_launch.h"

namespace nq {

// Measured on 89 MB and 1 GiB: 2 workgroups per CU with 4 loads in flight per
// thread read fastest; more in flight (4 or 8 per CU, 8 or 16 loads per
// thread) and per-workgroup contiguous ranges were slower.  Load forms, same
// shape (89 MB / 1 GiB, us): non-temporal global 14.6 / 156, plain global
// 15.4 / 170, buffer loads 16.0 / 176 (non-temporal buffer loads 15.5 / 170,
// with the device-scope bit as well 15.5 / 161).
constexpr int READ_UNROLL = 4;
constexpr int READ_WGS_PER_CU = 2;

__global__ __launch_bounds__(256) void stream_read_kernel(const uint8_t* __restrict__ src, int64_t pieces, int groups,
                                                          uint32_t* __restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * 256;          // pieces between a thread's loads
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    uint32_t acc = 0;
    for (int g = 0; g < groups; ++g) {
        uint4 v[READ_UNROLL];
#pragma unroll
        for (int u = 0; u < READ_UNROLL; ++u) {
            const int64_t j = i + u * stride;
            v[u] = ld_nt16(src + 16 * (j < pieces ? j : pieces - 1));
        }
#pragma unroll
        for (int u = 0; u < READ_UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
        i += READ_UNROLL * stride;
    }
    for (int o = 32; o >= 1; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
    __shared__ uint32_t red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

int stream_read_blocks() { return READ_WGS_PER_CU * device_cu_count(); }

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream) {
    if (bytes == 0) return hipSuccess;
    if (bytes >= ((int64_t)1 << 31) - 16) return hipErrorInvalidValue;     // the documented limit
    const int64_t blocks = stream_read_blocks();
    const int64_t per_group = blocks * 256 * 16 * READ_UNROLL;
    const int groups = (int)((bytes + per_group - 1) / per_group);
    stream_read_kernel<<<(unsigned)blocks, 256, 0, stream>>>(reinterpret_cast<const uint8_t*>(src), bytes / 16,
                                                             groups, sink);
    return hipGetLastError();
}

}  // namespace nq
