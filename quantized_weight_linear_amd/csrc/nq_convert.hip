// Format conversion kernels: MXFP8 decode, MLX affine int8 decode, per-row FP8 encode (from
// block-128 E4M3 or from BF16), per-token-per-64 int8 activation quantization
// and per-token E4M3 activation quantization.
#include "nq_device.h"
#include "nq_launch.h"

namespace nq {

// ---------------------------------------------------------------------------
// MXFP8 -> FP32 / BF16.  One thread per u32 word (four codes).  The value is
// e4m3(code) * 2^(b-127): an exact FP32 product (4 significant bits times a
// power of two; subnormal results are kept), rounded once to BF16 if asked.
// ---------------------------------------------------------------------------
template <bool BF16_OUT>
__global__ __launch_bounds__(256) void decode_mxfp8_kernel(const uint32_t* __restrict__ words,
                                                           const uint8_t* __restrict__ e8, int64_t n_words,
                                                           int64_t words_per_row, int64_t groups_per_row,
                                                           void* __restrict__ out) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_words;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = i / words_per_row;
        const int64_t j = i - row * words_per_row;
        const uint32_t b = e8[row * groups_per_row + (j >> 3)];
        const float sc = ue8m0_to_f32(b);
        const uint32_t w = words[i];
        float v[4];
        e4m3x4_to_f32(w, v);
        uint32_t bits[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float p = v[e] * sc;
            const bool nan = !(p == p);
            if (BF16_OUT) bits[e] = nan ? 0x7FC0u : f32_to_bf16_rne(p);
            else bits[e] = nan ? 0x7FC00000u : __float_as_uint(p);
        }
        if (BF16_OUT) {
            uint2 o = make_uint2(bits[0] | (bits[1] << 16), bits[2] | (bits[3] << 16));
            reinterpret_cast<uint2*>(out)[i] = o;
        } else {
            reinterpret_cast<uint4*>(out)[i] = make_uint4(bits[0], bits[1], bits[2], bits[3]);
        }
    }
}

hipError_t launch_decode_mxfp8(const uint32_t* words, const uint8_t* e8, int64_t N, int64_t K, bool bf16_out,
                               void* out, hipStream_t stream) {
    const int64_t n_words = N * (K / 4);
    if (n_words == 0) return hipSuccess;
    int64_t blocks = (n_words + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (bf16_out)
        decode_mxfp8_kernel<true><<<(unsigned)blocks, 256, 0, stream>>>(words, e8, n_words, K / 4, K / 32, out);
    else
        decode_mxfp8_kernel<false><<<(unsigned)blocks, 256, 0, stream>>>(words, e8, n_words, K / 4, K / 32, out);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// MLX affine int8 -> BF16 / FP32: w = q * scale + bias, one FP16 scale and one
// FP16 bias per 128 codes along K.  One thread per 16 codes (one 16-byte load;
// 8 threads per group).  The value is formed in FP64, where it is exact (q *
// scale has at most 19 significant bits and every FP16 value is a multiple of
// 2^-24 below 2^16), and rounded once: to FP32 by the hardware convert, to
// BF16 by rounding the FP64 significand to 8 bits, nearest-even.  Every such
// value lies far inside BF16's normal range (nonzero |w| in [2^-24, 2^25)), so
// no subnormal or overflow case arises; an infinite bias stays infinite and
// NaN gives the canonical quiet NaN.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double v) {
    if (!(v == v)) return 0x7FC0u;
    uint64_t b = (uint64_t)__double_as_longlong(v);
    b += ((uint64_t)1 << 44) - 1 + ((b >> 45) & 1);   // round the 52-bit fraction to 7 bits
    b &= ~(((uint64_t)1 << 45) - 1);
    return __float_as_uint((float)__longlong_as_double((long long)b)) >> 16;   // exact
}

template <bool BF16_OUT>
__global__ __launch_bounds__(256) void decode_mlx_affine_int8_kernel(const uint8_t* __restrict__ codes,
                                                                     const uint16_t* __restrict__ scales,
                                                                     const uint16_t* __restrict__ biases,
                                                                     int64_t n_pieces, int64_t pieces_per_row,
                                                                     int64_t groups_per_row, void* __restrict__ out) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_pieces;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = i / pieces_per_row;
        const int64_t g = row * groups_per_row + ((i - row * pieces_per_row) >> 3);
        const double s = (double)f16_bits_to_f32(scales[g]);
        const double b = (double)f16_bits_to_f32(biases[g]);
        const uint4 c = reinterpret_cast<const uint4*>(codes)[i];
        const uint32_t w[4] = {c.x, c.y, c.z, c.w};
        uint32_t bits[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const double v = fma((double)((w[e >> 2] >> (8 * (e & 3))) & 0xFFu), s, b);
            if (BF16_OUT) bits[e] = f64_to_bf16_rne(v);
            else bits[e] = (v == v) ? __float_as_uint((float)v) : 0x7FC00000u;
        }
        if (BF16_OUT) {
            uint4* o = reinterpret_cast<uint4*>(out) + 2 * i;
            o[0] = make_uint4(bits[0] | (bits[1] << 16), bits[2] | (bits[3] << 16), bits[4] | (bits[5] << 16),
                              bits[6] | (bits[7] << 16));
            o[1] = make_uint4(bits[8] | (bits[9] << 16), bits[10] | (bits[11] << 16), bits[12] | (bits[13] << 16),
                              bits[14] | (bits[15] << 16));
        } else {
            uint4* o = reinterpret_cast<uint4*>(out) + 4 * i;
#pragma unroll
            for (int q = 0; q < 4; ++q) o[q] = make_uint4(bits[4 * q], bits[4 * q + 1], bits[4 * q + 2], bits[4 * q + 3]);
        }
    }
}

hipError_t launch_decode_mlx_affine_int8(const uint8_t* codes, const uint16_t* scales, const uint16_t* biases,
                                         int64_t N, int64_t K, bool bf16_out, void* out, hipStream_t stream) {
    const int64_t n_pieces = N * (K / 16);
    if (n_pieces == 0) return hipSuccess;
    int64_t blocks = (n_pieces + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (bf16_out)
        decode_mlx_affine_int8_kernel<true><<<(unsigned)blocks, 256, 0, stream>>>(codes, scales, biases, n_pieces,
                                                                                 K / 16, K / 128, out);
    else
        decode_mlx_affine_int8_kernel<false><<<(unsigned)blocks, 256, 0, stream>>>(codes, scales, biases, n_pieces,
                                                                                  K / 16, K / 128, out);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Q4 codes -> int8 (the A8 route's weights): two's complement nibbles, low
// nibble first, each sign-extended to one byte.  One thread per 8 bytes (16
// codes, a 16-byte store).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t q4x4_to_i8x4(uint32_t b2) {   // 2 bytes -> 4 int8 codes
    uint32_t o = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int v = (int)(b2 >> (4 * j)) & 15;
        o |= ((uint32_t)((v ^ 8) - 8) & 0xFFu) << (8 * j);
    }
    return o;
}

__global__ __launch_bounds__(256) void unpack_q4_to_int8_kernel(const uint2* __restrict__ codes, int64_t n_pieces,
                                                                uint4* __restrict__ out) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_pieces;
         i += (int64_t)gridDim.x * blockDim.x) {
        const uint2 c = codes[i];
        out[i] = make_uint4(q4x4_to_i8x4(c.x & 0xFFFFu), q4x4_to_i8x4(c.x >> 16), q4x4_to_i8x4(c.y & 0xFFFFu),
                            q4x4_to_i8x4(c.y >> 16));
    }
}

hipError_t launch_unpack_q4_to_int8(const uint8_t* codes, int64_t N, int64_t K, int8_t* out, hipStream_t stream) {
    const int64_t n_pieces = N * (K / 16);
    if (n_pieces == 0) return hipSuccess;
    int64_t blocks = (n_pieces + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    unpack_q4_to_int8_kernel<<<(unsigned)blocks, 256, 0, stream>>>(reinterpret_cast<const uint2*>(codes), n_pieces,
                                                                  reinterpret_cast<uint4*>(out));
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Per-row FP8 encode ("fp8_row_maxabs").  One workgroup per output row, two
// passes over the row: (1) decode every element to FP32 and take the largest
// magnitude (NaN tracked separately so that it propagates), (2) s = bf16(m /
// 448) and code = e4m3_sat(v / s), both IEEE divisions.  Each thread keeps
// the decoded values of its first ROW_CACHE 16-element steps in registers
// (rows of up to 20480 elements), so pass 2 reads the row again only beyond
// that (the unrolled loads of pass 1 are also all in flight at once).
//
// Source SRC_BLOCK: E4M3 codes times the FP32 scale of their 128x128 block
// (one FP32 multiply, rounded once).  Source SRC_BF16: BF16 values (exact).
// ---------------------------------------------------------------------------
enum { SRC_BLOCK = 0, SRC_BF16 = 1 };

template <int SRC>
struct RowSource;

template <>
struct RowSource<SRC_BLOCK> {
    const uint8_t* codes;
    const float* wsi;
    int64_t K, gc;
    // decode 16 consecutive elements starting at k (k % 16 == 0, inside one block)
    __device__ __forceinline__ void load16(int64_t row, int64_t k, float* v) const {
        const uint4 c = *reinterpret_cast<const uint4*>(codes + row * K + k);
        const float s = wsi[(row >> 7) * gc + (k >> 7)];
        uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float f[4];
            e4m3x4_to_f32(w[q], f);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[4 * q + e] = f[e] * s;
        }
    }
    __device__ __forceinline__ float load1(int64_t row, int64_t k) const {
        return e4m3_to_f32(codes[row * K + k]) * wsi[(row >> 7) * gc + (k >> 7)];
    }
    __device__ __forceinline__ bool vec_ok() const { return (K & 15) == 0; }
};

template <>
struct RowSource<SRC_BF16> {
    const uint16_t* w;
    int64_t K;
    __device__ __forceinline__ void load16(int64_t row, int64_t k, float* v) const {
        const uint4* p = reinterpret_cast<const uint4*>(w + row * K + k);
        const uint4 a = p[0], b = p[1];
        uint32_t d[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            v[2 * q] = __uint_as_float(d[q] << 16);
            v[2 * q + 1] = __uint_as_float(d[q] & 0xFFFF0000u);
        }
    }
    __device__ __forceinline__ float load1(int64_t row, int64_t k) const {
        return bf16_bits_to_f32(w[row * K + k]);
    }
    __device__ __forceinline__ bool vec_ok() const { return (K & 15) == 0; }
};

__device__ __forceinline__ uint32_t encode_one(float v, float s) {
    // 0 / 0 (a zero element of an all-zero row) keeps the element's signed zero
    if (v == 0.0f && s == 0.0f) return (__float_as_uint(v) >> 24) & 0x80u;
    return f32_to_e4m3_sat(v / s);
}

template <int SRC>
__global__ __launch_bounds__(256) void encode_rows_kernel(RowSource<SRC> src, int64_t K, int64_t row_begin,
                                                          uint8_t* __restrict__ out_codes,
                                                          uint16_t* __restrict__ out_scale) {
    __shared__ float red_max[4];
    __shared__ int red_nan[4];
    const int64_t row = row_begin + blockIdx.x;
    const int64_t orow = blockIdx.x;
    const int tid = threadIdx.x;
    const bool vec = src.vec_ok();

    constexpr int ROW_CACHE = 5;
    float cache[ROW_CACHE][16];
    float m = 0.0f;
    int nan = 0;
    if (vec) {
#pragma unroll
        for (int it = 0; it < ROW_CACHE; ++it) {
            const int64_t k = (int64_t)tid * 16 + (int64_t)it * (256 * 16);
            if (k < K) src.load16(row, k, cache[it]);
        }
#pragma unroll
        for (int it = 0; it < ROW_CACHE; ++it) {
            const int64_t k = (int64_t)tid * 16 + (int64_t)it * (256 * 16);
            if (k < K) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    m = fmaxf(m, fabsf(cache[it][e]));
                    nan |= !(cache[it][e] == cache[it][e]);
                }
            }
        }
        for (int64_t k = (int64_t)tid * 16 + ROW_CACHE * (256 * 16); k < K; k += 256 * 16) {
            float v[16];
            src.load16(row, k, v);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                m = fmaxf(m, fabsf(v[e]));
                nan |= !(v[e] == v[e]);
            }
        }
    } else {
        for (int64_t k = tid; k < K; k += 256) {
            const float v = src.load1(row, k);
            m = fmaxf(m, fabsf(v));
            nan |= !(v == v);
        }
    }
    m = wave_max(m);
    nan = __any(nan) ? 1 : 0;
    const int wave = tid >> 6;
    if ((tid & 63) == 0) {
        red_max[wave] = m;
        red_nan[wave] = nan;
    }
    __syncthreads();
    m = fmaxf(fmaxf(red_max[0], red_max[1]), fmaxf(red_max[2], red_max[3]));
    nan = red_nan[0] | red_nan[1] | red_nan[2] | red_nan[3];

    uint32_t s_bits;
    if (nan) s_bits = 0x7FC0u;
    else s_bits = f32_to_bf16_rne(m / 448.0f);
    const float s = bf16_bits_to_f32(s_bits);
    if (tid == 0) out_scale[orow] = (uint16_t)s_bits;

    uint8_t* orow_ptr = out_codes + orow * K;
    // A finite scale in BF16's normal range (s >= 2^-126) carries m / 448 to
    // within 2^-9 relative, so every quotient stays below 448 (1 + 2^-8) < 464,
    // the range where the hardware convert equals the saturating encoder.  A
    // subnormal scale has fewer significant bits (m near 1e-37 gives quotients
    // up to ~670, which must saturate to +-448), so such rows, like the zero,
    // NaN and infinite ones, take the per-element path.
    const bool fast = s >= __uint_as_float(0x00800000u) && s < __uint_as_float(0x7F800000u);
    const double r = 1.0 / (double)s;
    if (vec && fast) {
        auto encode16 = [&](const float* v, int64_t k) {
            uint32_t d[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                d[q] = f32x4_to_e4m3_hw(div_via_recip64(v[4 * q], r), div_via_recip64(v[4 * q + 1], r),
                                        div_via_recip64(v[4 * q + 2], r), div_via_recip64(v[4 * q + 3], r));
            *reinterpret_cast<uint4*>(orow_ptr + k) = make_uint4(d[0], d[1], d[2], d[3]);
        };
#pragma unroll
        for (int it = 0; it < ROW_CACHE; ++it) {
            const int64_t k = (int64_t)tid * 16 + (int64_t)it * (256 * 16);
            if (k < K) encode16(cache[it], k);
        }
        for (int64_t k = (int64_t)tid * 16 + ROW_CACHE * (256 * 16); k < K; k += 256 * 16) {
            float v[16];
            src.load16(row, k, v);
            encode16(v, k);
        }
    } else if (vec) {
        for (int64_t k = (int64_t)tid * 16; k < K; k += 256 * 16) {
            float v[16];
            src.load16(row, k, v);
            uint32_t d[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                d[q] = encode_one(v[4 * q], s) | (encode_one(v[4 * q + 1], s) << 8) |
                       (encode_one(v[4 * q + 2], s) << 16) | (encode_one(v[4 * q + 3], s) << 24);
            }
            *reinterpret_cast<uint4*>(orow_ptr + k) = make_uint4(d[0], d[1], d[2], d[3]);
        }
    } else {
        for (int64_t k = tid; k < K; k += 256) orow_ptr[k] = (uint8_t)encode_one(src.load1(row, k), s);
    }
}

hipError_t launch_reencode_block128(const uint8_t* codes, const float* wsi, int64_t N, int64_t K, int64_t gc,
                                    int64_t r0, int64_t r1, uint8_t* out_codes, uint16_t* out_scale,
                                    hipStream_t stream) {
    (void)N;
    RowSource<SRC_BLOCK> src{codes, wsi, K, gc};
    const int64_t rows = r1 - r0;
    if (rows <= 0) return hipSuccess;
    encode_rows_kernel<SRC_BLOCK><<<(unsigned)rows, 256, 0, stream>>>(src, K, r0, out_codes, out_scale);
    return hipGetLastError();
}

hipError_t launch_encode_fp8row_bf16(const uint16_t* w, int64_t N, int64_t K, uint8_t* out_codes,
                                     uint16_t* out_scale, hipStream_t stream) {
    RowSource<SRC_BF16> src{w, K};
    if (N <= 0) return hipSuccess;
    encode_rows_kernel<SRC_BF16><<<(unsigned)N, 256, 0, stream>>>(src, K, 0, out_codes, out_scale);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Int8 activation quantization, per token and per 64 channels.  Eight threads
// per group, eight BF16 values (16 bytes) per thread; the group's largest
// magnitude is combined across the eight lanes with shuffles (NaN propagated
// by a flag), s = amax / 127 and q = clamp(rne(x / s)) by IEEE division.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quantize_int8_g64_kernel(const uint16_t* __restrict__ x, int64_t n_threads,
                                                                int8_t* __restrict__ q,
                                                                float* __restrict__ scale) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const bool live = i < n_threads;
    uint4 a = make_uint4(0, 0, 0, 0);
    if (live) a = reinterpret_cast<const uint4*>(x)[i];
    const uint32_t d[4] = {a.x, a.y, a.z, a.w};
    float v[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        v[2 * e] = __uint_as_float(d[e] << 16);
        v[2 * e + 1] = __uint_as_float(d[e] & 0xFFFF0000u);
    }
    float m = 0.0f;
    int nan = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        m = fmaxf(m, fabsf(v[e]));
        nan |= !(v[e] == v[e]);
    }
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) {
        m = fmaxf(m, __shfl_xor(m, off, 64));
        nan |= __shfl_xor(nan, off, 64);
    }
    const float s = nan ? __uint_as_float(0x7FC00000u) : m / 127.0f;
    const double r = 1.0 / (double)s;          // x / s below: BF16 over FP32, exact (div_via_recip64)
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) lo |= ((uint32_t)f32_to_i8_sat(div_via_recip64(v[e], r)) & 0xFFu) << (8 * e);
#pragma unroll
    for (int e = 0; e < 4; ++e) hi |= ((uint32_t)f32_to_i8_sat(div_via_recip64(v[4 + e], r)) & 0xFFu) << (8 * e);
    if (live) {
        reinterpret_cast<uint2*>(q)[i] = make_uint2(lo, hi);
        if ((i & 7) == 0) scale[i >> 3] = s;
    }
}

hipError_t launch_quantize_int8_g64(const uint16_t* x, int64_t T, int64_t K, int8_t* q, float* scale,
                                    hipStream_t stream) {
    const int64_t n_threads = T * K / 8;
    if (n_threads == 0) return hipSuccess;
    const int64_t blocks = (n_threads + 255) / 256;
    quantize_int8_g64_kernel<<<(unsigned)blocks, 256, 0, stream>>>(x, n_threads, q, scale);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Per-token E4M3 activation quantization.  One workgroup per token row.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quantize_fp8_row_kernel(const uint16_t* __restrict__ x, int64_t K,
                                                               uint8_t* __restrict__ codes,
                                                               float* __restrict__ scale) {
    __shared__ float red_max[4];
    __shared__ int red_nan[4];
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x;
    const uint16_t* xr = x + row * K;
    const bool vec = (K & 7) == 0;
    float m = 0.0f;
    int nan = 0;
    if (vec) {
        for (int64_t k = (int64_t)tid * 8; k < K; k += 256 * 8) {
            const uint4 a = *reinterpret_cast<const uint4*>(xr + k);
            const uint32_t d[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float f0 = __uint_as_float(d[e] << 16), f1 = __uint_as_float(d[e] & 0xFFFF0000u);
                m = fmaxf(m, fmaxf(fabsf(f0), fabsf(f1)));
                nan |= !(f0 == f0) | !(f1 == f1);
            }
        }
    } else {
        for (int64_t k = tid; k < K; k += 256) {
            const float f = bf16_bits_to_f32(xr[k]);
            m = fmaxf(m, fabsf(f));
            nan |= !(f == f);
        }
    }
    m = wave_max(m);
    nan = __any(nan) ? 1 : 0;
    if ((tid & 63) == 0) {
        red_max[tid >> 6] = m;
        red_nan[tid >> 6] = nan;
    }
    __syncthreads();
    m = fmaxf(fmaxf(red_max[0], red_max[1]), fmaxf(red_max[2], red_max[3]));
    nan = red_nan[0] | red_nan[1] | red_nan[2] | red_nan[3];
    const float s = nan ? __uint_as_float(0x7FC00000u) : m / 448.0f;
    if (tid == 0) scale[row] = s;
    uint8_t* cr = codes + row * K;
    // Every quotient is below 450 < 464 (the hardware convert's exact range):
    // s = fp32(m / 448) is within 2^-24 of m / 448 when normal, and an FP32
    // subnormal s still holds at least 146 quanta of 2^-149 (m is at least
    // 2^-133, the smallest BF16 magnitude), within 1/292 of it.
    const bool fast = s > 0.0f && s < __uint_as_float(0x7F800000u);
    const double r = 1.0 / (double)s;
    if (vec && fast) {
        for (int64_t k = (int64_t)tid * 8; k < K; k += 256 * 8) {
            const uint4 a = *reinterpret_cast<const uint4*>(xr + k);
            const uint32_t d[4] = {a.x, a.y, a.z, a.w};
            float f[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                f[2 * e] = div_via_recip64(__uint_as_float(d[e] << 16), r);
                f[2 * e + 1] = div_via_recip64(__uint_as_float(d[e] & 0xFFFF0000u), r);
            }
            *reinterpret_cast<uint2*>(cr + k) =
                make_uint2(f32x4_to_e4m3_hw(f[0], f[1], f[2], f[3]), f32x4_to_e4m3_hw(f[4], f[5], f[6], f[7]));
        }
    } else if (vec) {
        for (int64_t k = (int64_t)tid * 8; k < K; k += 256 * 8) {
            const uint4 a = *reinterpret_cast<const uint4*>(xr + k);
            const uint32_t d[4] = {a.x, a.y, a.z, a.w};
            uint32_t o[2] = {0, 0};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float f0 = __uint_as_float(d[e] << 16), f1 = __uint_as_float(d[e] & 0xFFFF0000u);
                const uint32_t pair = encode_one(f0, s) | (encode_one(f1, s) << 8);
                o[e >> 1] |= pair << (16 * (e & 1));
            }
            *reinterpret_cast<uint2*>(cr + k) = make_uint2(o[0], o[1]);
        }
    } else {
        for (int64_t k = tid; k < K; k += 256) cr[k] = (uint8_t)encode_one(bf16_bits_to_f32(xr[k]), s);
    }
}

hipError_t launch_quantize_fp8_row(const uint16_t* x, int64_t M, int64_t K, uint8_t* codes, float* scale,
                                   hipStream_t stream) {
    if (M <= 0) return hipSuccess;
    quantize_fp8_row_kernel<<<(unsigned)M, 256, 0, stream>>>(x, K, codes, scale);
    return hipGetLastError();
}

}  // namespace nq
