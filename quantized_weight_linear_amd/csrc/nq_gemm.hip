// Prefill GEMMs on CDNA4 MFMA: y[m][n] = sum_k A[m][k] * W[n][k] with
// int8 x int8 (W8A8, per-64-group FP32 rescale) or E4M3 x E4M3 (row scales).
//
// Tiling: a workgroup of 4 waves computes a 128 (tokens) x 128 (weight rows)
// block; each wave a 64 x 64 quadrant as 2 x 2 tiles of 32 x 32 MFMA output.
// A and W panels of one K step are staged in LDS (rows padded by 16 bytes),
// the next step's panels are prefetched into registers while the current
// step computes.
//
// W8A8 (one K step = one 64-channel scale group): two v_mfma_i32_32x32x32_i8
// per tile sum the group exactly in int32.  The MFMA's C operand is the
// constant 0x4B400000 (the float 1.5 * 2^23), so the int32 result D = C + P
// read as a float is exactly 12582912 + P for |P| < 2^22 (here |P| <= 64 *
// 127^2).  The rescale is then two FP32 FMAs per element:
//     X   = fma(float(D), ws, -12582912 * ws)   -> P * ws rounded once
//     acc = fma(X, as, acc)
// (-12582912 * ws is exact: ws is FP16, 11 significant bits).
//
// FP8 (one K step = 128 channels): v_mfma_f32_32x32x64_f8f6f4 on E4M3 codes,
// FP32 accumulation over all K; y = acc * a_scale[m] * w_scale[n] at the end.
#include "nq_device.h"
#include "nq_launch.h"

namespace nq {

constexpr int GM_BM = 128;
constexpr int GM_BN = 128;

template <int BK>
struct GemmSmem {
    static constexpr int PITCH = BK + 16;   // bytes per LDS row
    uint8_t a[GM_BM * PITCH];
    uint8_t b[GM_BN * PITCH];
};

// 32x32 MFMA output layout: lane l holds column (l % 32) and rows
// 8 j + 4 (l / 32) + r for j, r in 0..3 (element 4 j + r).
__device__ __forceinline__ int d_row(int lane, int e) { return 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3); }

template <bool W8A8>
__global__ __launch_bounds__(256) void gemm_kernel(const uint8_t* __restrict__ A, const float* __restrict__ a_scale,
                                                   const uint8_t* __restrict__ W,
                                                   const uint16_t* __restrict__ w_scale, int M, int N, int64_t K,
                                                   int bf16_out, void* __restrict__ y,
                                                   int32_t* __restrict__ group_sums) {
    constexpr int BK = W8A8 ? 64 : 128;
    constexpr int PITCH = GemmSmem<BK>::PITCH;
    constexpr int CHUNKS = BK / 16;                    // 16-byte pieces per panel row
    constexpr int LOADS = GM_BM * CHUNKS / 256;        // 16-byte loads per thread per panel
    __shared__ __attribute__((aligned(16))) GemmSmem<BK> sm;
    __shared__ __attribute__((aligned(16))) float s_as[W8A8 ? GM_BM : 1];
    __shared__ __attribute__((aligned(16))) float s_ws[W8A8 ? 2 * GM_BN : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int wm = wv & 1, wn = wv >> 1;
    const int64_t m0 = (int64_t)blockIdx.y * GM_BM;
    const int64_t n0 = (int64_t)blockIdx.x * GM_BN;
    const int64_t nsteps = (K + BK - 1) / BK;
    const int64_t G = K / 64;

    // register prefetch of one K step
    uint4 ra[LOADS], rb[LOADS];
    float r_as = 0.f, r_ws = 0.f;
    auto load_step = [&](int64_t s) {
        const int64_t k0 = s * BK;
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            const int idx = tid + 256 * j;
            const int r = idx / CHUNKS, c = idx % CHUNKS;
            const int64_t k = k0 + 16 * c;
            int64_t am = m0 + r; if (am >= M) am = M - 1;
            int64_t bn = n0 + r; if (bn >= N) bn = N - 1;
            if (k < K) {
                ra[j] = *reinterpret_cast<const uint4*>(A + am * K + k);
                rb[j] = ld_nt16(W + bn * K + k);
            } else {
                ra[j] = make_uint4(0, 0, 0, 0);
                rb[j] = make_uint4(0, 0, 0, 0);
            }
        }
        if constexpr (W8A8) {
            if (tid < GM_BM) {
                int64_t am = m0 + tid; if (am >= M) am = M - 1;
                r_as = a_scale[am * G + s];
            } else {
                int64_t bn = n0 + (tid - GM_BM); if (bn >= N) bn = N - 1;
                r_ws = f16_bits_to_f32(w_scale[bn * G + s]);
            }
        }
    };
    auto store_step = [&]() {
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            const int idx = tid + 256 * j;
            const int r = idx / CHUNKS, c = idx % CHUNKS;
            *reinterpret_cast<uint4*>(&sm.a[r * PITCH + 16 * c]) = ra[j];
            *reinterpret_cast<uint4*>(&sm.b[r * PITCH + 16 * c]) = rb[j];
        }
        if constexpr (W8A8) {
            if (tid < GM_BM) s_as[tid] = r_as;
            else {
                s_ws[2 * (tid - GM_BM)] = r_ws;
                s_ws[2 * (tid - GM_BM) + 1] = -12582912.0f * r_ws;
            }
        }
    };

    v16f acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int fr = lane & 31;       // fragment row (A) / column (B) within a 32 tile
    const int fk = lane >> 5;       // k half of the fragment

    if (nsteps > 0) load_step(0);
    for (int64_t s = 0; s < nsteps; ++s) {
        __syncthreads();
        store_step();
        __syncthreads();
        if (s + 1 < nsteps) load_step(s + 1);
        if constexpr (W8A8) {
            const v16i bias = {0x4B400000, 0x4B400000, 0x4B400000, 0x4B400000, 0x4B400000, 0x4B400000,
                               0x4B400000, 0x4B400000, 0x4B400000, 0x4B400000, 0x4B400000, 0x4B400000,
                               0x4B400000, 0x4B400000, 0x4B400000, 0x4B400000};
            v16i d[2][2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                v4i af[2], bf[2];
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    af[i] = *reinterpret_cast<const v4i*>(&sm.a[(wm * 64 + 32 * i + fr) * PITCH + 32 * h + 16 * fk]);
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    bf[j] = *reinterpret_cast<const v4i*>(&sm.b[(wn * 64 + 32 * j + fr) * PITCH + 32 * h + 16 * fk]);
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        d[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], h == 0 ? bias : d[i][j], 0, 0, 0);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const float2 wsp = *reinterpret_cast<const float2*>(&s_ws[2 * (wn * 64 + 32 * j + fr)]);
#pragma unroll
                for (int i = 0; i < 2; ++i) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const v4f as4 = *reinterpret_cast<const v4f*>(&s_as[wm * 64 + 32 * i + 8 * q + 4 * fk]);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int e = 4 * q + r;
                            const float X = fmaf(__int_as_float(d[i][j][e]), wsp.x, wsp.y);
                            acc[i][j][e] = fmaf(X, as4[r], acc[i][j][e]);
                        }
                    }
                    if (group_sums != nullptr) {
                        const int64_t n = n0 + wn * 64 + 32 * j + fr;
#pragma unroll
                        for (int e = 0; e < 16; ++e) {
                            const int64_t m = m0 + wm * 64 + 32 * i + d_row(lane, e);
                            if (m < M && n < N) group_sums[(m * N + n) * G + s] = d[i][j][e] - 0x4B400000;
                        }
                    }
                }
            }
        } else {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                v8i af[2], bf[2];
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    af[i] = *reinterpret_cast<const v8i*>(&sm.a[(wm * 64 + 32 * i + fr) * PITCH + 64 * h + 32 * fk]);
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    bf[j] = *reinterpret_cast<const v8i*>(&sm.b[(wn * 64 + 32 * j + fr) * PITCH + 64 * h + 32 * fk]);
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], acc[i][j], 0, 0,
                                                                                   0, 0, 0, 0);
            }
        }
    }

    // epilogue: write y
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t n = n0 + wn * 64 + 32 * j + fr;
            if (n >= N) continue;
            float sw = 1.0f;
            if constexpr (!W8A8) sw = bf16_bits_to_f32(w_scale[n]);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t m = m0 + wm * 64 + 32 * i + d_row(lane, e);
                if (m >= M) continue;
                float v = acc[i][j][e];
                if constexpr (!W8A8) v = (v * a_scale[m]) * sw;
                if (bf16_out) reinterpret_cast<uint16_t*>(y)[m * N + n] = (uint16_t)f32_to_bf16_rne(v);
                else reinterpret_cast<float*>(y)[m * N + n] = v;
            }
        }
}

hipError_t launch_gemm_w8a8(const int8_t* a_q, const float* a_scale, const int8_t* w_q, const uint16_t* w_scale,
                            int64_t M, int64_t N, int64_t K, bool bf16_out, void* y, int32_t* group_sums,
                            hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    dim3 grid((unsigned)((N + GM_BN - 1) / GM_BN), (unsigned)((M + GM_BM - 1) / GM_BM));
    gemm_kernel<true><<<grid, 256, 0, stream>>>(reinterpret_cast<const uint8_t*>(a_q), a_scale,
                                                reinterpret_cast<const uint8_t*>(w_q), w_scale, (int)M, (int)N, K,
                                                bf16_out ? 1 : 0, y, group_sums);
    return hipGetLastError();
}

hipError_t launch_gemm_fp8(const uint8_t* a_codes, const float* a_scale, const uint8_t* w, const uint16_t* w_scale,
                           int64_t M, int64_t N, int64_t K, bool bf16_out, void* y, hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    dim3 grid((unsigned)((N + GM_BN - 1) / GM_BN), (unsigned)((M + GM_BM - 1) / GM_BM));
    gemm_kernel<false><<<grid, 256, 0, stream>>>(a_codes, a_scale, w, w_scale, (int)M, (int)N, K,
                                                 bf16_out ? 1 : 0, y, nullptr);
    return hipGetLastError();
}

}  // namespace nq
