// A plain streaming read of device memory: the measured HBM read ceiling that
// the weight-streaming kernels are compared against.  Every thread reads
// 16-byte pieces with non-temporal loads, UNROLL of them in flight, the
// whole grid sweeping the buffer in step (consecutive threads, consecutive
// pieces); the pieces are folded into one word per workgroup so the loads
// cannot be dropped.  The sink receives one word per workgroup.
#include "nq_device.h"
#include "nq_launch.h"

namespace nq {

constexpr int READ_UNROLL = 8;

__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ src, int64_t n_pieces,
                                                          uint32_t* __restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    uint32_t acc = 0;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + (READ_UNROLL - 1) * stride < n_pieces; i += READ_UNROLL * stride) {
        uint4 v[READ_UNROLL];
#pragma unroll
        for (int u = 0; u < READ_UNROLL; ++u) v[u] = ld_nt16(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < READ_UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n_pieces; i += stride) {
        const uint4 v = ld_nt16(src + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    for (int off = 32; off >= 1; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off, 64);
    __shared__ uint32_t red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

int stream_read_blocks() { return 8 * device_cu_count(); }

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream) {
    const int64_t n_pieces = bytes / 16;
    if (n_pieces == 0) return hipSuccess;
    stream_read_kernel<<<(unsigned)stream_read_blocks(), 256, 0, stream>>>(reinterpret_cast<const uint4*>(src),
                                                                          n_pieces, sink);
    return hipGetLastError();
}

}  // namespace nq
