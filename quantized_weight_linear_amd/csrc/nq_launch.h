// Host-side launchers for the HIP kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nq {

// Weight formats, same values as nq_wfmt plus the row-scaled FP8 format.
enum WFmt { W_Q4G64 = 0, W_Q8G32 = 1, W_Q8G64 = 2, W_MXFP8 = 3, W_BF16 = 4, W_Q3G64 = 5, W_Q5G64 = 6, W_Q6G64 = 7,
            W_FP8ROW = 8 };

hipError_t launch_decode_mxfp8(const uint32_t* words, const uint8_t* e8, int64_t N, int64_t K, bool bf16_out,
                               void* out, hipStream_t stream);
hipError_t launch_decode_mlx_affine_int8(const uint8_t* codes, const uint16_t* scales, const uint16_t* biases,
                                         int64_t N, int64_t K, bool bf16_out, void* out, hipStream_t stream);
hipError_t launch_unpack_q4_to_int8(const uint8_t* codes, int64_t N, int64_t K, int8_t* out, hipStream_t stream);
hipError_t launch_reencode_block128(const uint8_t* codes, const float* wsi, int64_t N, int64_t K, int64_t gc,
                                    int64_t r0, int64_t r1, uint8_t* out_codes, uint16_t* out_scale,
                                    hipStream_t stream);
hipError_t launch_encode_fp8row_bf16(const uint16_t* w, int64_t N, int64_t K, uint8_t* out_codes,
                                     uint16_t* out_scale, hipStream_t stream);
hipError_t launch_quantize_int8_g64(const uint16_t* x, int64_t T, int64_t K, int8_t* q, float* scale,
                                    hipStream_t stream);
hipError_t launch_quantize_fp8_row(const uint16_t* x, int64_t M, int64_t K, uint8_t* codes, float* scale,
                                   hipStream_t stream);

// Decode GEMV for every weight format.  `scales` is the per-format scale
// array (row scales for W_FP8ROW).  `workspace` (may be NULL) enables split-K
// across workgroups when it is large enough (gemv_workspace_bytes).
int64_t gemv_workspace_bytes(int fmt, int64_t T, int64_t N, int64_t K);
// `packed`: weights in the layout written by launch_pack_weights (requires K % 128 == 0).
hipError_t launch_gemv(int fmt, const void* w, const void* scales, const uint16_t* x, int64_t T, int64_t N,
                       int64_t K, bool bf16_out, void* y, void* workspace, int64_t workspace_bytes,
                       hipStream_t stream, bool packed);
int64_t packed_weight_bytes(int fmt, int64_t N, int64_t K);
// launch_gemv with the library's own per-device scratch array instead of a
// caller workspace (no allocation); the caller checks gemv_workspace_bytes
// against GEMV_STATIC_SCRATCH_BYTES first.
constexpr int64_t GEMV_STATIC_SCRATCH_BYTES = (int64_t)8 << 20;
hipError_t launch_gemv_noalloc(int fmt, const void* w, const void* scales, const uint16_t* x, int64_t T, int64_t N,
                               int64_t K, bool bf16_out, void* y, hipStream_t stream, bool packed);
hipError_t launch_pack_weights(int fmt, const void* src, int64_t N, int64_t K, void* dst, hipStream_t stream);

// A8 decode GEMV (int8 activation codes and scales from launch_quantize_int8_g64,
// Q8 or Q4 group-64 weights, row-major or packed as for launch_gemv).
int64_t gemv_a8_workspace_bytes(int64_t T, int64_t N, int64_t K);
hipError_t launch_gemv_a8(int fmt, const void* w, const uint16_t* w_scale, const int8_t* aq, const float* asc,
                          int64_t T, int64_t N, int64_t K, bool bf16_out, void* y, void* workspace,
                          int64_t workspace_bytes, hipStream_t stream, bool packed);

// Q3 / Q5 / Q6 group-64 (dense little-endian bit streams): the BF16-activation
// GEMV (row-major or packed), the packing, and the widening to int8.
int qbits_of(int fmt);   // 3, 5, 6, or 0 for other formats
int64_t gemv_qbits_workspace_bytes(int64_t T, int64_t N, int64_t K);
hipError_t launch_gemv_qbits(int fmt, const void* w, const uint16_t* w_scale, const uint16_t* x, int64_t T, int64_t N,
                             int64_t K, bool bf16_out, void* y, void* workspace, int64_t workspace_bytes,
                             hipStream_t stream, bool packed);
hipError_t launch_pack_qbits(int fmt, const void* src, int64_t N, int64_t K, void* dst, hipStream_t stream);
hipError_t launch_unpack_qbits_to_int8(int fmt, const uint8_t* codes, int64_t N, int64_t K, int8_t* out,
                                       hipStream_t stream);

hipError_t launch_gemm_w8a8(const int8_t* a_q, const float* a_scale, const int8_t* w_q, const uint16_t* w_scale,
                            int64_t M, int64_t N, int64_t K, bool bf16_out, void* y, int32_t* group_sums,
                            hipStream_t stream);
hipError_t launch_gemm_fp8(const uint8_t* a_codes, const float* a_scale, const uint8_t* w, const uint16_t* w_scale,
                           int64_t M, int64_t N, int64_t K, bool bf16_out, void* y, hipStream_t stream);

int device_cu_count();

// Plain streaming read of `bytes` (a multiple of 16) from src; one word per
// workgroup (stream_read_blocks() of them) goes to sink.
int stream_read_blocks();
hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream);

}  // namespace nq
