// C ABI: argument validation, then dispatch to the HIP launchers on the
// caller's stream.  Every check runs before anything is enqueued, so an
// invalid call writes nothing and makes no HIP call at all.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "nq.h"
#include "nq_launch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A pointer is required when the buffer it points to is non-empty.
nq_status need(const void* p, int64_t elems) {
    if (elems == 0) return NQ_OK;
    if (p == nullptr) return NQ_ERR_NULL;
    return NQ_OK;
}

nq_status align_ok(const void* p) { return (p == nullptr || aligned16(p)) ? NQ_OK : NQ_ERR_ALIGN; }

#define NQ_TRY(expr)                     \
    do {                                 \
        nq_status _s = (expr);           \
        if (_s != NQ_OK) return _s;      \
    } while (0)

nq_status from_hip(hipError_t e) { return e == hipSuccess ? NQ_OK : NQ_ERR_HIP; }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

bool out_ok(int out_dt) { return out_dt == NQ_OUT_F32 || out_dt == NQ_OUT_BF16; }

int group_of(int fmt) {
    switch (fmt) {
        case NQ_W_Q4G64_F16S: return 64;
        case NQ_W_Q8G32_F16S: return 32;
        case NQ_W_Q8G64_F16S: return 64;
        case NQ_W_MXFP8_G32: return 32;
        case NQ_W_BF16: return 1;
        case NQ_W_Q3G64_F16S: return 64;
        case NQ_W_Q5G64_F16S: return 64;
        case NQ_W_Q6G64_F16S: return 64;
        default: return 0;
    }
}

}  // namespace

namespace nq {

int device_cu_count() {
    static std::mutex mu;
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    std::lock_guard<std::mutex> g(mu);
    if (cached[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        cached[dev] = cus;
    }
    return cached[dev];
}

}  // namespace nq

extern "C" {

int nq_abi_version(void) { return NQ_ABI_VERSION; }

const char* nq_status_string(int status) {
    switch (status) {
        case NQ_OK: return "ok";
        case NQ_ERR_NULL: return "a required pointer is NULL";
        case NQ_ERR_SHAPE: return "invalid shape";
        case NQ_ERR_ALIGN: return "pointer not 16-byte aligned";
        case NQ_ERR_FORMAT: return "unknown format or output type";
        case NQ_ERR_RANGE: return "row range out of bounds";
        case NQ_ERR_HIP: return "HIP runtime error";
        case NQ_ERR_SCRATCH: return "the call needs more scratch than the library's static array holds";
        default: return "unknown status";
    }
}

nq_status nq_decode_mxfp8(const uint32_t* words, const uint8_t* e8m0, int64_t N, int64_t K, int out_dt,
                          void* w_out, void* stream) {
    if (N < 0 || K < 0 || K % 32 != 0) return NQ_ERR_SHAPE;
    if (!out_ok(out_dt)) return NQ_ERR_FORMAT;
    NQ_TRY(need(words, N * K));
    NQ_TRY(need(e8m0, N * K));
    NQ_TRY(need(w_out, N * K));
    NQ_TRY(align_ok(words));
    NQ_TRY(align_ok(e8m0));
    NQ_TRY(align_ok(w_out));
    if (N == 0 || K == 0) return NQ_OK;
    return from_hip(nq::launch_decode_mxfp8(words, e8m0, N, K, out_dt == NQ_OUT_BF16, w_out, as_stream(stream)));
}

nq_status nq_decode_mlx_affine_int8(const uint8_t* codes, const uint16_t* scales, const uint16_t* biases, int64_t N,
                                    int64_t K, int out_dt, void* w_out, void* stream) {
    if (N < 0 || K < 0 || K % 128 != 0) return NQ_ERR_SHAPE;
    if (!out_ok(out_dt)) return NQ_ERR_FORMAT;
    NQ_TRY(need(codes, N * K));
    NQ_TRY(need(scales, N * K));
    NQ_TRY(need(biases, N * K));
    NQ_TRY(need(w_out, N * K));
    NQ_TRY(align_ok(codes));
    NQ_TRY(align_ok(w_out));
    if (N == 0 || K == 0) return NQ_OK;
    return from_hip(nq::launch_decode_mlx_affine_int8(codes, scales, biases, N, K, out_dt == NQ_OUT_BF16, w_out,
                                                      as_stream(stream)));
}

nq_status nq_unpack_q4_to_int8(const uint8_t* codes, int64_t N, int64_t K, int8_t* out, void* stream) {
    if (N < 0 || K < 0 || K % 64 != 0) return NQ_ERR_SHAPE;
    NQ_TRY(need(codes, N * K));
    NQ_TRY(need(out, N * K));
    NQ_TRY(align_ok(codes));
    NQ_TRY(align_ok(out));
    if (N == 0 || K == 0) return NQ_OK;
    return from_hip(nq::launch_unpack_q4_to_int8(codes, N, K, out, as_stream(stream)));
}

nq_status nq_reencode_block128_to_row(const uint8_t* codes, const float* wsi, int64_t N, int64_t K, int64_t gr,
                                      int64_t gc, int64_t row_begin, int64_t row_end, uint8_t* out_codes,
                                      uint16_t* out_scale, void* stream) {
    if (N < 0 || K < 0) return NQ_ERR_SHAPE;
    if (gr != (N + 127) / 128 || gc != (K + 127) / 128) return NQ_ERR_SHAPE;
    if (!(row_begin >= 0 && row_begin < row_end && row_end <= N)) return NQ_ERR_RANGE;
    const int64_t rows = row_end - row_begin;
    NQ_TRY(need(codes, N * K));
    NQ_TRY(need(wsi, gr * gc));
    NQ_TRY(need(out_codes, rows * K));
    NQ_TRY(need(out_scale, rows));
    NQ_TRY(align_ok(codes));
    NQ_TRY(align_ok(wsi));
    NQ_TRY(align_ok(out_codes));
    NQ_TRY(align_ok(out_scale));
    return from_hip(nq::launch_reencode_block128(codes, wsi, N, K, gc, row_begin, row_end, out_codes, out_scale,
                                                 as_stream(stream)));
}

nq_status nq_encode_fp8row_bf16(const uint16_t* w, int64_t N, int64_t K, uint8_t* out_codes, uint16_t* out_scale,
                                void* stream) {
    if (N < 0 || K < 0) return NQ_ERR_SHAPE;
    NQ_TRY(need(w, N * K));
    NQ_TRY(need(out_codes, N * K));
    NQ_TRY(need(out_scale, N));
    NQ_TRY(align_ok(w));
    NQ_TRY(align_ok(out_codes));
    NQ_TRY(align_ok(out_scale));
    if (N == 0) return NQ_OK;
    return from_hip(nq::launch_encode_fp8row_bf16(w, N, K, out_codes, out_scale, as_stream(stream)));
}

nq_status nq_quantize_act_int8_g64(const uint16_t* x, int64_t T, int64_t K, int8_t* q, float* scale, void* stream) {
    if (T < 0 || K < 0 || K % 64 != 0) return NQ_ERR_SHAPE;
    NQ_TRY(need(x, T * K));
    NQ_TRY(need(q, T * K));
    NQ_TRY(need(scale, T * K));
    NQ_TRY(align_ok(x));
    NQ_TRY(align_ok(q));
    NQ_TRY(align_ok(scale));
    if (T == 0 || K == 0) return NQ_OK;
    return from_hip(nq::launch_quantize_int8_g64(x, T, K, q, scale, as_stream(stream)));
}

nq_status nq_quantize_act_fp8_row(const uint16_t* x, int64_t M, int64_t K, uint8_t* codes, float* scale,
                                  void* stream) {
    if (M < 0 || K < 0) return NQ_ERR_SHAPE;
    NQ_TRY(need(x, M * K));
    NQ_TRY(need(codes, M * K));
    NQ_TRY(need(scale, M));
    NQ_TRY(align_ok(x));
    NQ_TRY(align_ok(codes));
    NQ_TRY(align_ok(scale));
    if (M == 0) return NQ_OK;
    return from_hip(nq::launch_quantize_fp8_row(x, M, K, codes, scale, as_stream(stream)));
}

int64_t nq_gemv_workspace_bytes(int fmt, int64_t T, int64_t N, int64_t K) {
    if (T < 0 || N < 0 || K < 0) return 0;
    if (nq::qbits_of(fmt)) return nq::gemv_qbits_workspace_bytes(T, N, K);
    return nq::gemv_workspace_bytes(fmt, T, N, K);
}

}  // extern "C"

namespace {

// Token rows a pass of the decode kernels addresses: a pass takes at most 64
// tokens, padded to whole blocks of 16 (the padding rows read as zero through
// out-of-range buffer offsets, which must not wrap around 32 bits).
static int64_t padded_pass_rows(int64_t T) {
    const int64_t t = T < 64 ? T : 64;
    return (t + 15) / 16 * 16;
}

// Q3 / Q5 / Q6: whole 256-column chunks and 32-bit buffer offsets for the
// codes (rows padded to 16), activations and scales.
bool qbits_shape_ok(int fmt, int64_t T, int64_t N, int64_t K) {
    const int64_t b = nq::qbits_of(fmt);
    return K % 256 == 0 && (N + 15) / 16 * 16 * (K * b / 8) < ((int64_t)1 << 31) &&
           padded_pass_rows(T) * K * 2 < ((int64_t)1 << 31) && N * (K / 64) * 2 < ((int64_t)1 << 31);
}

// The packed layout needs whole 128-column chunks and 32-bit buffer offsets.
bool packed_shape_ok(int64_t N, int64_t K) {
    return K % 256 == 0 && K > 0 && 64 * K * 2 < ((int64_t)1 << 31) && N * (K / 32) * 2 < ((int64_t)1 << 31);
}

nq_status gemv_fp8row_impl(const uint8_t* w, const uint16_t* w_scale, const uint16_t* x, int64_t T, int64_t N,
                           int64_t K, int out_dt, void* y, void* workspace, int64_t workspace_bytes, void* stream,
                           bool packed) {
    if (T < 0 || N < 0 || K < 0 || workspace_bytes < 0) return NQ_ERR_SHAPE;
    if (packed && !packed_shape_ok(N, K)) return NQ_ERR_SHAPE;
    if (!out_ok(out_dt)) return NQ_ERR_FORMAT;
    NQ_TRY(need(w, N * K));
    NQ_TRY(need(w_scale, N));
    NQ_TRY(need(x, T * K));
    NQ_TRY(need(y, T * N));
    NQ_TRY(align_ok(w));
    NQ_TRY(align_ok(w_scale));
    NQ_TRY(align_ok(x));
    NQ_TRY(align_ok(y));
    NQ_TRY(align_ok(workspace));
    if (T == 0 || N == 0) return NQ_OK;
    return from_hip(nq::launch_gemv(nq::W_FP8ROW, w, w_scale, x, T, N, K, out_dt == NQ_OUT_BF16, y, workspace,
                                    workspace ? workspace_bytes : 0, as_stream(stream), packed));
}

nq_status gemv_qgroup_impl(int fmt, const void* w_codes, const void* w_scales, const uint16_t* x, int64_t T,
                           int64_t N, int64_t K, int out_dt, void* y, void* workspace, int64_t workspace_bytes,
                           void* stream, bool packed) {
    const int gs = group_of(fmt);
    if (gs == 0) return NQ_ERR_FORMAT;
    if (!out_ok(out_dt)) return NQ_ERR_FORMAT;
    if (T < 0 || N < 0 || K < 0 || workspace_bytes < 0 || K % gs != 0) return NQ_ERR_SHAPE;
    if (packed && !packed_shape_ok(N, K)) return NQ_ERR_SHAPE;
    if (nq::qbits_of(fmt) && !qbits_shape_ok(fmt, T, N, K)) return NQ_ERR_SHAPE;
    NQ_TRY(need(w_codes, N * K));
    if (fmt != NQ_W_BF16) NQ_TRY(need(w_scales, N * K));
    NQ_TRY(need(x, T * K));
    NQ_TRY(need(y, T * N));
    NQ_TRY(align_ok(w_codes));
    if (fmt != NQ_W_BF16) NQ_TRY(align_ok(w_scales));
    NQ_TRY(align_ok(x));
    NQ_TRY(align_ok(y));
    NQ_TRY(align_ok(workspace));
    if (T == 0 || N == 0) return NQ_OK;
    if (nq::qbits_of(fmt))
        return from_hip(nq::launch_gemv_qbits(fmt, w_codes, reinterpret_cast<const uint16_t*>(w_scales), x, T, N, K,
                                              out_dt == NQ_OUT_BF16, y, workspace, workspace ? workspace_bytes : 0,
                                              as_stream(stream), packed));
    return from_hip(nq::launch_gemv(fmt, w_codes, fmt == NQ_W_BF16 ? nullptr : w_scales, x, T, N, K,
                                    out_dt == NQ_OUT_BF16, y, workspace, workspace ? workspace_bytes : 0,
                                    as_stream(stream), packed));
}

// nq_wfmt, or -1 for row-scaled FP8, to the internal format code
int internal_fmt(int fmt) { return fmt == -1 ? nq::W_FP8ROW : fmt; }

}  // namespace

extern "C" {

nq_status nq_gemv_fp8row(const uint8_t* w, const uint16_t* w_scale, const uint16_t* x, int64_t T, int64_t N,
                         int64_t K, int out_dt, void* y, void* workspace, int64_t workspace_bytes, void* stream) {
    return gemv_fp8row_impl(w, w_scale, x, T, N, K, out_dt, y, workspace, workspace_bytes, stream, false);
}

nq_status nq_gemv_fp8row_packed(const uint8_t* w_packed, const uint16_t* w_scale, const uint16_t* x, int64_t T,
                                int64_t N, int64_t K, int out_dt, void* y, void* workspace, int64_t workspace_bytes,
                                void* stream) {
    return gemv_fp8row_impl(w_packed, w_scale, x, T, N, K, out_dt, y, workspace, workspace_bytes, stream, true);
}

nq_status nq_gemv_qgroup(int fmt, const void* w_codes, const void* w_scales, const uint16_t* x, int64_t T,
                         int64_t N, int64_t K, int out_dt, void* y, void* workspace, int64_t workspace_bytes,
                         void* stream) {
    return gemv_qgroup_impl(fmt, w_codes, w_scales, x, T, N, K, out_dt, y, workspace, workspace_bytes, stream,
                            false);
}

nq_status nq_gemv_qgroup_packed(int fmt, const void* w_packed, const void* w_scales, const uint16_t* x, int64_t T,
                                int64_t N, int64_t K, int out_dt, void* y, void* workspace, int64_t workspace_bytes,
                                void* stream) {
    return gemv_qgroup_impl(fmt, w_packed, w_scales, x, T, N, K, out_dt, y, workspace, workspace_bytes, stream,
                            true);
}

nq_status nq_gemv_fp8row_packed_noalloc(const uint8_t* w_packed, const uint16_t* w_scale, const uint16_t* x,
                                        int64_t T, int64_t N, int64_t K, int out_dt, void* y, void* stream) {
    if (T < 0 || N < 0 || K < 0) return NQ_ERR_SHAPE;
    if (!packed_shape_ok(N, K)) return NQ_ERR_SHAPE;
    if (!out_ok(out_dt)) return NQ_ERR_FORMAT;
    NQ_TRY(need(w_packed, N * K));
    NQ_TRY(need(w_scale, N));
    NQ_TRY(need(x, T * K));
    NQ_TRY(need(y, T * N));
    NQ_TRY(align_ok(w_packed));
    NQ_TRY(align_ok(w_scale));
    NQ_TRY(align_ok(x));
    NQ_TRY(align_ok(y));
    if (T == 0 || N == 0) return NQ_OK;
    if (nq::gemv_workspace_bytes(nq::W_FP8ROW, T, N, K) > nq::GEMV_STATIC_SCRATCH_BYTES) return NQ_ERR_SCRATCH;
    return from_hip(nq::launch_gemv_noalloc(nq::W_FP8ROW, w_packed, w_scale, x, T, N, K, out_dt == NQ_OUT_BF16, y,
                                            as_stream(stream), true));
}

int64_t nq_packed_weight_bytes(int fmt, int64_t N, int64_t K) {
    if (N < 0 || K < 0 || (fmt != -1 && group_of(fmt) == 0)) return 0;
    if (nq::qbits_of(fmt)) return (N + 15) / 16 * 16 * (K * nq::qbits_of(fmt) / 8);
    return nq::packed_weight_bytes(internal_fmt(fmt), N, K);
}

nq_status nq_pack_weights(int fmt, const void* w, int64_t N, int64_t K, void* w_packed, void* stream) {
    if (fmt != -1 && group_of(fmt) == 0) return NQ_ERR_FORMAT;
    if (N < 0 || K < 0) return NQ_ERR_SHAPE;
    if (N > 0 && !packed_shape_ok(N, K)) return NQ_ERR_SHAPE;
    NQ_TRY(need(w, N * K));
    NQ_TRY(need(w_packed, N * K));
    NQ_TRY(align_ok(w));
    NQ_TRY(align_ok(w_packed));
    if (N == 0) return NQ_OK;
    if (nq::qbits_of(fmt)) {
        if (!qbits_shape_ok(fmt, 0, N, K)) return NQ_ERR_SHAPE;
        return from_hip(nq::launch_pack_qbits(fmt, w, N, K, w_packed, as_stream(stream)));
    }
    return from_hip(nq::launch_pack_weights(internal_fmt(fmt), w, N, K, w_packed, as_stream(stream)));
}

nq_status nq_gemm_w8a8_g64(const int8_t* a_q, const float* a_scale, const int8_t* w_q, const uint16_t* w_scale,
                           int64_t M, int64_t N, int64_t K, int out_dt, void* y, int32_t* group_sums,
                           void* stream) {
    if (M < 0 || N < 0 || K < 0 || K % 64 != 0) return NQ_ERR_SHAPE;
    if (!out_ok(out_dt)) return NQ_ERR_FORMAT;
    NQ_TRY(need(a_q, M * K));
    NQ_TRY(need(a_scale, M * K));
    NQ_TRY(need(w_q, N * K));
    NQ_TRY(need(w_scale, N * K));
    NQ_TRY(need(y, M * N));
    NQ_TRY(align_ok(a_q));
    NQ_TRY(align_ok(a_scale));
    NQ_TRY(align_ok(w_q));
    NQ_TRY(align_ok(w_scale));
    NQ_TRY(align_ok(y));
    NQ_TRY(align_ok(group_sums));
    if (M == 0 || N == 0) return NQ_OK;
    return from_hip(nq::launch_gemm_w8a8(a_q, a_scale, w_q, w_scale, M, N, K, out_dt == NQ_OUT_BF16, y, group_sums,
                                         as_stream(stream)));
}

nq_status nq_gemm_fp8row(const uint16_t* x, const uint8_t* w, const uint16_t* w_scale, int64_t M, int64_t N,
                         int64_t K, uint8_t* a_codes, float* a_scale, int out_dt, void* y, void* stream) {
    if (M < 0 || N < 0 || K < 0 || K % 16 != 0) return NQ_ERR_SHAPE;
    if (!out_ok(out_dt)) return NQ_ERR_FORMAT;
    NQ_TRY(need(x, M * K));
    NQ_TRY(need(w, N * K));
    NQ_TRY(need(w_scale, N));
    NQ_TRY(need(a_codes, M * K));
    NQ_TRY(need(a_scale, M));
    NQ_TRY(need(y, M * N));
    NQ_TRY(align_ok(x));
    NQ_TRY(align_ok(w));
    NQ_TRY(align_ok(w_scale));
    NQ_TRY(align_ok(a_codes));
    NQ_TRY(align_ok(a_scale));
    NQ_TRY(align_ok(y));
    if (M == 0 || N == 0) return NQ_OK;
    hipStream_t s = as_stream(stream);
    hipError_t e = nq::launch_quantize_fp8_row(x, M, K, a_codes, a_scale, s);
    if (e != hipSuccess) return NQ_ERR_HIP;
    return from_hip(nq::launch_gemm_fp8(a_codes, a_scale, w, w_scale, M, N, K, out_dt == NQ_OUT_BF16, y, s));
}

}  // extern "C"

namespace {

nq_status gemv_a8_impl(int fmt, const void* w, const uint16_t* w_scale, const int8_t* a_q, const float* a_scale,
                       int64_t T, int64_t N, int64_t K, int out_dt, void* y, void* workspace, int64_t workspace_bytes,
                       void* stream, bool packed) {
    if (fmt != NQ_W_Q8G64_F16S && fmt != NQ_W_Q4G64_F16S) return NQ_ERR_FORMAT;
    if (!out_ok(out_dt)) return NQ_ERR_FORMAT;
    if (T < 0 || N < 0 || K < 0 || workspace_bytes < 0 || K % 256 != 0) return NQ_ERR_SHAPE;
    if (T * K >= ((int64_t)1 << 31) || padded_pass_rows(T) * K >= ((int64_t)1 << 31) ||
        N * (K / 64) * 2 >= ((int64_t)1 << 31))
        return NQ_ERR_SHAPE;
    if (packed && !packed_shape_ok(N, K)) return NQ_ERR_SHAPE;
    NQ_TRY(need(w, N * K));
    NQ_TRY(need(w_scale, N * K));
    NQ_TRY(need(a_q, T * K));
    NQ_TRY(need(a_scale, T * K));
    NQ_TRY(need(y, T * N));
    NQ_TRY(align_ok(w));
    NQ_TRY(align_ok(w_scale));
    NQ_TRY(align_ok(a_q));
    NQ_TRY(align_ok(a_scale));
    NQ_TRY(align_ok(y));
    NQ_TRY(align_ok(workspace));
    if (T == 0 || N == 0) return NQ_OK;
    return from_hip(nq::launch_gemv_a8(fmt == NQ_W_Q8G64_F16S ? nq::W_Q8G64 : nq::W_Q4G64, w, w_scale, a_q, a_scale,
                                       T, N, K, out_dt == NQ_OUT_BF16, y, workspace, workspace ? workspace_bytes : 0,
                                       as_stream(stream), packed));
}

}  // namespace

extern "C" {

nq_status nq_gemv_a8_g64(int fmt, const void* w_codes, const uint16_t* w_scale, const int8_t* a_q,
                         const float* a_scale, int64_t T, int64_t N, int64_t K, int out_dt, void* y, void* workspace,
                         int64_t workspace_bytes, void* stream) {
    return gemv_a8_impl(fmt, w_codes, w_scale, a_q, a_scale, T, N, K, out_dt, y, workspace, workspace_bytes, stream,
                        false);
}

nq_status nq_gemv_a8_g64_packed(int fmt, const void* w_packed, const uint16_t* w_scale, const int8_t* a_q,
                                const float* a_scale, int64_t T, int64_t N, int64_t K, int out_dt, void* y,
                                void* workspace, int64_t workspace_bytes, void* stream) {
    return gemv_a8_impl(fmt, w_packed, w_scale, a_q, a_scale, T, N, K, out_dt, y, workspace, workspace_bytes, stream,
                        true);
}

int64_t nq_stream_read_sink_words(void) { return nq::stream_read_blocks(); }

nq_status nq_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
    if (bytes < 0 || bytes % 16 != 0 || bytes >= ((int64_t)1 << 31) - 16) return NQ_ERR_SHAPE;
    NQ_TRY(need(src, bytes));
    NQ_TRY(need(sink, bytes));
    NQ_TRY(align_ok(src));
    NQ_TRY(align_ok(sink));
    if (bytes == 0) return NQ_OK;
    return from_hip(nq::launch_stream_read(src, bytes, sink, as_stream(stream)));
}

int nq_route(int64_t T, int a8_flags) {
    if ((a8_flags & NQ_A8_PREFILL) && T >= 129) return NQ_ROUTE_A8;
    if ((a8_flags & NQ_A8_DECODE) && T <= 128) return NQ_ROUTE_A8_DECODE;
    return NQ_ROUTE_BF16;
}

int64_t nq_gemv_a8_workspace_bytes(int64_t T, int64_t N, int64_t K) {
    if (T < 0 || N < 0 || K < 0) return 0;
    return nq::gemv_a8_workspace_bytes(T, N, K);
}

nq_status nq_linear_q8g64(const uint16_t* x, int64_t T, const int8_t* w_q, const uint16_t* w_scale, int64_t N,
                          int64_t K, int allow_a8, int8_t* a_q_ws, float* a_scale_ws, int out_dt, void* y,
                          void* workspace, int64_t workspace_bytes, void* stream) {
    if (T < 0 || N < 0 || K < 0 || K % 64 != 0 || workspace_bytes < 0) return NQ_ERR_SHAPE;
    if (!out_ok(out_dt)) return NQ_ERR_FORMAT;
    const int route = nq_route(T, allow_a8);
    const bool a8 = route == NQ_ROUTE_A8;
    const bool a8d = route == NQ_ROUTE_A8_DECODE;
    if (a8d && K % 256 != 0) return NQ_ERR_SHAPE;
    NQ_TRY(need(x, T * K));
    NQ_TRY(need(w_q, N * K));
    NQ_TRY(need(w_scale, N * K));
    NQ_TRY(need(y, T * N));
    if (a8 || a8d) {
        NQ_TRY(need(a_q_ws, T * K));
        NQ_TRY(need(a_scale_ws, T * K));
        NQ_TRY(align_ok(a_q_ws));
        NQ_TRY(align_ok(a_scale_ws));
    }
    NQ_TRY(align_ok(x));
    NQ_TRY(align_ok(w_q));
    NQ_TRY(align_ok(w_scale));
    NQ_TRY(align_ok(y));
    NQ_TRY(align_ok(workspace));
    if (T == 0 || N == 0) return NQ_OK;
    hipStream_t s = as_stream(stream);
    if (!a8 && !a8d)
        return from_hip(nq::launch_gemv(nq::W_Q8G64, w_q, w_scale, x, T, N, K, out_dt == NQ_OUT_BF16, y, workspace,
                                        workspace ? workspace_bytes : 0, s, false));
    hipError_t e = nq::launch_quantize_int8_g64(x, T, K, a_q_ws, a_scale_ws, s);
    if (e != hipSuccess) return NQ_ERR_HIP;
    if (a8d)
        return from_hip(nq::launch_gemv_a8(nq::W_Q8G64, w_q, w_scale, a_q_ws, a_scale_ws, T, N, K,
                                           out_dt == NQ_OUT_BF16, y, workspace, workspace ? workspace_bytes : 0, s,
                                           false));
    return from_hip(nq::launch_gemm_w8a8(a_q_ws, a_scale_ws, w_q, w_scale, T, N, K, out_dt == NQ_OUT_BF16, y,
                                         nullptr, s));
}

nq_status nq_linear_q4g64(const uint16_t* x, int64_t T, const uint8_t* w_codes, const uint16_t* w_scale, int64_t N,
                          int64_t K, int allow_a8, int8_t* a_q_ws, float* a_scale_ws, int8_t* w_i8_ws, int out_dt,
                          void* y, void* workspace, int64_t workspace_bytes, void* stream) {
    if (T < 0 || N < 0 || K < 0 || K % 64 != 0 || workspace_bytes < 0) return NQ_ERR_SHAPE;
    if (!out_ok(out_dt)) return NQ_ERR_FORMAT;
    const int route = nq_route(T, allow_a8);
    const bool a8 = route == NQ_ROUTE_A8;
    const bool a8d = route == NQ_ROUTE_A8_DECODE;
    if (a8d && K % 256 != 0) return NQ_ERR_SHAPE;
    NQ_TRY(need(x, T * K));
    NQ_TRY(need(w_codes, N * K));
    NQ_TRY(need(w_scale, N * K));
    NQ_TRY(need(y, T * N));
    if (a8 || a8d) {
        NQ_TRY(need(a_q_ws, T * K));
        NQ_TRY(need(a_scale_ws, T * K));
        NQ_TRY(align_ok(a_q_ws));
        NQ_TRY(align_ok(a_scale_ws));
    }
    if (a8) {
        NQ_TRY(need(w_i8_ws, N * K));
        NQ_TRY(align_ok(w_i8_ws));
    }
    NQ_TRY(align_ok(x));
    NQ_TRY(align_ok(w_codes));
    NQ_TRY(align_ok(w_scale));
    NQ_TRY(align_ok(y));
    NQ_TRY(align_ok(workspace));
    if (T == 0 || N == 0) return NQ_OK;
    hipStream_t s = as_stream(stream);
    if (!a8 && !a8d)
        return from_hip(nq::launch_gemv(nq::W_Q4G64, w_codes, w_scale, x, T, N, K, out_dt == NQ_OUT_BF16, y,
                                        workspace, workspace ? workspace_bytes : 0, s, false));
    hipError_t e = nq::launch_quantize_int8_g64(x, T, K, a_q_ws, a_scale_ws, s);
    if (e != hipSuccess) return NQ_ERR_HIP;
    if (a8d)
        return from_hip(nq::launch_gemv_a8(nq::W_Q4G64, w_codes, w_scale, a_q_ws, a_scale_ws, T, N, K,
                                           out_dt == NQ_OUT_BF16, y, workspace, workspace ? workspace_bytes : 0, s,
                                           false));
    e = nq::launch_unpack_q4_to_int8(w_codes, N, K, w_i8_ws, s);
    if (e != hipSuccess) return NQ_ERR_HIP;
    return from_hip(nq::launch_gemm_w8a8(a_q_ws, a_scale_ws, w_i8_ws, w_scale, T, N, K, out_dt == NQ_OUT_BF16, y,
                                         nullptr, s));
}

nq_status nq_unpack_qbits_to_int8(int fmt, const uint8_t* codes, int64_t N, int64_t K, int8_t* out, void* stream) {
    if (!nq::qbits_of(fmt)) return NQ_ERR_FORMAT;
    if (N < 0 || K < 0 || K % 64 != 0) return NQ_ERR_SHAPE;
    NQ_TRY(need(codes, N * K));
    NQ_TRY(need(out, N * K));
    NQ_TRY(align_ok(codes));
    NQ_TRY(align_ok(out));
    if (N == 0 || K == 0) return NQ_OK;
    return from_hip(nq::launch_unpack_qbits_to_int8(fmt, codes, N, K, out, as_stream(stream)));
}

nq_status nq_linear_qbits_g64(int fmt, const uint16_t* x, int64_t T, const uint8_t* w_codes, const uint16_t* w_scale,
                              int64_t N, int64_t K, int a8_flags, int8_t* a_q_ws, float* a_scale_ws, int8_t* w_i8_ws,
                              int out_dt, void* y, void* workspace, int64_t workspace_bytes, void* stream) {
    if (!nq::qbits_of(fmt)) return NQ_ERR_FORMAT;
    if (!out_ok(out_dt)) return NQ_ERR_FORMAT;
    if (T < 0 || N < 0 || K < 0 || workspace_bytes < 0 || K % 256 != 0) return NQ_ERR_SHAPE;
    if (!qbits_shape_ok(fmt, T, N, K)) return NQ_ERR_SHAPE;
    const int route = nq_route(T, a8_flags);
    NQ_TRY(need(x, T * K));
    NQ_TRY(need(w_codes, N * K));
    NQ_TRY(need(w_scale, N * K));
    NQ_TRY(need(y, T * N));
    if (route != NQ_ROUTE_BF16) {
        NQ_TRY(need(a_q_ws, T * K));
        NQ_TRY(need(a_scale_ws, T * K));
        NQ_TRY(need(w_i8_ws, N * K));
        NQ_TRY(align_ok(a_q_ws));
        NQ_TRY(align_ok(a_scale_ws));
        NQ_TRY(align_ok(w_i8_ws));
    }
    NQ_TRY(align_ok(x));
    NQ_TRY(align_ok(w_codes));
    NQ_TRY(align_ok(w_scale));
    NQ_TRY(align_ok(y));
    NQ_TRY(align_ok(workspace));
    if (T == 0 || N == 0) return NQ_OK;
    hipStream_t s = as_stream(stream);
    const bool bf16 = out_dt == NQ_OUT_BF16;
    if (route == NQ_ROUTE_BF16)
        return from_hip(nq::launch_gemv_qbits(fmt, w_codes, w_scale, x, T, N, K, bf16, y, workspace,
                                              workspace ? workspace_bytes : 0, s, false));
    hipError_t e = nq::launch_quantize_int8_g64(x, T, K, a_q_ws, a_scale_ws, s);
    if (e != hipSuccess) return NQ_ERR_HIP;
    e = nq::launch_unpack_qbits_to_int8(fmt, w_codes, N, K, w_i8_ws, s);
    if (e != hipSuccess) return NQ_ERR_HIP;
    if (route == NQ_ROUTE_A8_DECODE)
        return from_hip(nq::launch_gemv_a8(nq::W_Q8G64, w_i8_ws, w_scale, a_q_ws, a_scale_ws, T, N, K, bf16, y,
                                           workspace, workspace ? workspace_bytes : 0, s, false));
    return from_hip(nq::launch_gemm_w8a8(a_q_ws, a_scale_ws, w_i8_ws, w_scale, T, N, K, bf16, y, nullptr, s));
}

}  // extern "C"
