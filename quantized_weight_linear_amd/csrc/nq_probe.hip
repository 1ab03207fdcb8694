// A plain streaming read of device memory: the measured HBM read ceiling that
// the weight-streaming kernels are compared against.  Every thread reads
// 16-byte pieces i = tid + j * stride (stride = all threads of the grid),
// READ_UNROLL of them issued back to back before any is used, with buffer
// loads whose offsets past the end read zero (so the last group needs no
// branch and every group keeps READ_UNROLL loads in flight).  The pieces are
// folded into one word per workgroup so the loads cannot be dropped; the
// sink receives one word per workgroup.
#include "nq_device.h"
#include "nq_launch.h"

namespace nq {

// Measured on 89 MB and 1 GiB: 2 workgroups per CU with 4 loads in flight per
// thread read fastest (14.96 us, 6.45 TB/s); more in flight (4 or 8 per CU,
// 8 or 16 loads per thread) and per-workgroup contiguous ranges were slower.
constexpr int READ_UNROLL = 4;
constexpr int READ_WGS_PER_CU = 2;

__global__ __launch_bounds__(256) void stream_read_kernel(const uint8_t* __restrict__ src, int bytes, int groups,
                                                          uint32_t* __restrict__ sink) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, bytes, 0x00020000u);
    const int stride = (int)gridDim.x * 256 * 16;            // bytes between a thread's pieces
    int off = ((int)blockIdx.x * 256 + (int)threadIdx.x) * 16;
    uint32_t acc = 0;
    for (int g = 0; g < groups; ++g) {
        v4u v[READ_UNROLL];
#pragma unroll
        for (int u = 0; u < READ_UNROLL; ++u) {
            const int o = off + u * stride;
            // past the end (or past the int range, for the last group) the offset reads zero
            v[u] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(r, o < bytes && o >= 0 ? o : bytes,
                                                                                 0, 0));
        }
#pragma unroll
        for (int u = 0; u < READ_UNROLL; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
        off += READ_UNROLL * stride;
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
    if (bytes >= ((int64_t)1 << 31) - 16) return hipErrorInvalidValue;     // 32-bit buffer offsets
    const int64_t blocks = stream_read_blocks();
    const int64_t per_group = blocks * 256 * 16 * READ_UNROLL;
    const int groups = (int)((bytes + per_group - 1) / per_group);
    stream_read_kernel<<<(unsigned)blocks, 256, 0, stream>>>(reinterpret_cast<const uint8_t*>(src), (int)bytes, groups,
                                                             sink);
    return hipGetLastError();
}

}  // namespace nq
