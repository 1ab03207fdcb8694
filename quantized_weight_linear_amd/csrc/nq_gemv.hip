// Decode GEMV / skinny GEMM: y[t][n] = sum_k x[t][k] * W[n][k] for a few
// tokens (T <= 64 per pass), weights decoded on the fly in registers.
//
// Main path (K % 128 == 0): BF16 MFMA 16x16x32 on exactly decoded weights.
//   - A workgroup (4 waves) owns 64 weight rows and a K range; waves are
//     2 row-pairs (32 rows each) x 2 K-halves of every 256-wide K chunk.
//   - Weights stream from HBM with 16-byte loads straight into registers (one
//     chunk ahead) and are decoded there: E4M3 -> BF16 with the hardware
//     scaled convert (exact), int8/int4 -> FP32 -> BF16 (exact for |q| <= 128).
//   - The activation chunk [T_pad][256] is staged in LDS (zero-padded to a
//     multiple of 16 tokens) and read as the MFMA B operand; each B fragment
//     feeds two 16-row weight blocks.
//   - Grouped formats run one MFMA chain per scale group and fold the group
//     scale in FP32 (acc += sc * D); row-scaled FP8 applies its row scale once
//     at the end; MXFP8 folds its power-of-two group scale into the exact
//     convert.
//   - The two K-halves are summed through LDS in a fixed order.  With a
//     workspace, the K range is also split across workgroups; each split
//     writes an FP32 partial and the last workgroup of a row tile (atomic
//     counter) sums the partials in split order, so results are deterministic.
// Fallback (any K): one wave per (row, 8 tokens), scalar decode, FP32 sums.
#include "nq_device.h"
#include "nq_launch.h"

namespace nq {

constexpr int GV_ROWS = 64;
constexpr int GV_KC = 256;
constexpr int GV_XPITCH = GV_KC + 8;   // bf16 elements per LDS row (528 bytes: rows shift by 4 banks)

template <int FMT>
__device__ __forceinline__ int64_t row_bytes(int64_t K) {
    if (FMT == W_Q4G64) return K >> 1;
    if (FMT == W_BF16) return K << 1;
    return K;
}

template <int FMT>
constexpr int group_size() {
    return FMT == W_Q8G32 ? 32 : ((FMT == W_Q4G64 || FMT == W_Q8G64) ? 64 : 0);
}

// Per-lane raw weight bytes for one 16-row block and one 128-wide K half.
template <int FMT>
struct WRegs {
    uint4 q[FMT == W_BF16 ? 4 : 2];
    uint32_t e8;  // MXFP8 scale byte of the lane's 32-element group
};
template <>
struct WRegs<W_Q4G64> {
    uint2 q[2];
    uint32_t e8;
};
template <>
struct WRegs<W_Q8G32> {
    uint2 q[4];
    uint32_t e8;
};

// Lane (i = row in block, g = lane group) loads its part of a K half starting
// at absolute column kh0.  Layouts per format:
//   FP8ROW / MXFP8 / BF16: g covers 32 contiguous columns kh0 + 32g ..
//   Q8G64 / Q4G64:         g covers 16 columns in each 64-span: kh0 + 64s + 16g ..
//   Q8G32:                 g covers 8 columns in each 32-span:  kh0 + 32s + 8g ..
template <int FMT>
__device__ __forceinline__ void load_wregs(WRegs<FMT>& r, const uint8_t* __restrict__ w,
                                           const uint8_t* __restrict__ e8, int64_t row, int64_t K, int64_t kh0,
                                           int g) {
    const uint8_t* base = w + row * row_bytes<FMT>(K);
    if constexpr (FMT == W_FP8ROW || FMT == W_MXFP8) {
        const uint8_t* p = base + kh0 + 32 * g;
        r.q[0] = ld_nt16(p);
        r.q[1] = ld_nt16(p + 16);
        if constexpr (FMT == W_MXFP8) r.e8 = e8[row * (K >> 5) + ((kh0 + 32 * g) >> 5)];
    } else if constexpr (FMT == W_BF16) {
        const uint8_t* p = base + 2 * (kh0 + 32 * g);
#pragma unroll
        for (int j = 0; j < 4; ++j) r.q[j] = ld_nt16(p + 16 * j);
    } else if constexpr (FMT == W_Q8G64) {
#pragma unroll
        for (int s = 0; s < 2; ++s) r.q[s] = ld_nt16(base + kh0 + 64 * s + 16 * g);
    } else if constexpr (FMT == W_Q4G64) {
#pragma unroll
        for (int s = 0; s < 2; ++s) r.q[s] = ld_nt8(base + ((kh0 + 64 * s + 16 * g) >> 1));
    } else {  // W_Q8G32
#pragma unroll
        for (int s = 0; s < 4; ++s) r.q[s] = ld_nt8(base + kh0 + 32 * s + 8 * g);
    }
}

// LDS column offset (within the 256-wide chunk) of k-step ks for lane group g.
template <int FMT>
__device__ __forceinline__ int kstep_col(int kh, int ks, int g) {
    if constexpr (FMT == W_Q8G64 || FMT == W_Q4G64) return kh * 128 + (ks >> 1) * 64 + 16 * g + (ks & 1) * 8;
    else if constexpr (FMT == W_Q8G32) return kh * 128 + ks * 32 + 8 * g;
    else return kh * 128 + 32 * g + ks * 8;
}

__device__ __forceinline__ uint32_t i8x2_to_bf16x2(uint32_t d, int sh) {
    const float a = (float)(int8_t)(d >> sh);
    const float b = (float)(int8_t)(d >> (sh + 8));
    return f32x2_to_bf16x2(a, b);
}

__device__ __forceinline__ uint32_t i4x2_to_bf16x2(uint32_t d, int sh) {
    const float a = (float)((int32_t)(d << (28 - sh)) >> 28);
    const float b = (float)((int32_t)(d << (24 - sh)) >> 28);
    return f32x2_to_bf16x2(a, b);
}

// Decode the A fragment (8 BF16 weights) of k-step ks.
template <int FMT>
__device__ __forceinline__ v8bf decode_afrag(const WRegs<FMT>& r, int ks) {
    uint32_t o[4];
    if constexpr (FMT == W_FP8ROW || FMT == W_MXFP8) {
        const uint32_t* d = reinterpret_cast<const uint32_t*>(&r.q[0]);
        const uint32_t d0 = d[2 * ks], d1 = d[2 * ks + 1];
        const float sc = (FMT == W_MXFP8) ? ue8m0_to_f32(r.e8) : 1.0f;
        o[0] = e4m3x2_to_bf16x2<false>(d0, sc);
        o[1] = e4m3x2_to_bf16x2<true>(d0, sc);
        o[2] = e4m3x2_to_bf16x2<false>(d1, sc);
        o[3] = e4m3x2_to_bf16x2<true>(d1, sc);
    } else if constexpr (FMT == W_BF16) {
        const uint4 q = r.q[ks];
        o[0] = q.x; o[1] = q.y; o[2] = q.z; o[3] = q.w;
    } else if constexpr (FMT == W_Q8G64) {
        const uint32_t* d = reinterpret_cast<const uint32_t*>(&r.q[ks >> 1]);
        const uint32_t d0 = d[(ks & 1) * 2], d1 = d[(ks & 1) * 2 + 1];
        o[0] = i8x2_to_bf16x2(d0, 0);
        o[1] = i8x2_to_bf16x2(d0, 16);
        o[2] = i8x2_to_bf16x2(d1, 0);
        o[3] = i8x2_to_bf16x2(d1, 16);
    } else if constexpr (FMT == W_Q4G64) {
        const uint32_t* d = reinterpret_cast<const uint32_t*>(&r.q[ks >> 1]);
        const uint32_t d0 = d[ks & 1];
        o[0] = i4x2_to_bf16x2(d0, 0);
        o[1] = i4x2_to_bf16x2(d0, 8);
        o[2] = i4x2_to_bf16x2(d0, 16);
        o[3] = i4x2_to_bf16x2(d0, 24);
    } else {  // W_Q8G32
        const uint2 q = r.q[ks];
        o[0] = i8x2_to_bf16x2(q.x, 0);
        o[1] = i8x2_to_bf16x2(q.x, 16);
        o[2] = i8x2_to_bf16x2(q.y, 0);
        o[3] = i8x2_to_bf16x2(q.y, 16);
    }
    return __builtin_bit_cast(v8bf, make_uint4(o[0], o[1], o[2], o[3]));
}

template <int FMT, int NCB>
__global__ __launch_bounds__(256) void gemv_mfma_kernel(const uint8_t* __restrict__ w,
                                                        const void* __restrict__ scales,
                                                        const uint16_t* __restrict__ x, int T, int N, int64_t K,
                                                        int64_t k_per_split, int splits,
                                                        float* __restrict__ partial,
                                                        unsigned* __restrict__ counters, int bf16_out,
                                                        void* __restrict__ y) {
    constexpr int TP = 16 * NCB;
    constexpr int GS = group_size<FMT>();
    constexpr int NG = GS ? GV_KC / (GS ? GS : 1) : 1;  // scale groups per chunk
    __shared__ __attribute__((aligned(16))) uint16_t xs[TP * GV_XPITCH];
    __shared__ __attribute__((aligned(16))) uint16_t scs[GS ? NG * GV_ROWS : 1];
    __shared__ int s_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int rp = wv & 1;       // row pair: rows [32 rp, 32 rp + 32) of the tile
    const int kh = wv >> 1;      // K half of each chunk
    const int li = lane & 15;
    const int lg = lane >> 4;
    const int tile = blockIdx.x;
    const int split = blockIdx.y;
    const int64_t row0 = (int64_t)tile * GV_ROWS;
    const int64_t k_begin = (int64_t)split * k_per_split;
    int64_t k_end = k_begin + k_per_split;
    if (k_end > K) k_end = K;
    const int nch = (int)((k_end - k_begin + GV_KC - 1) / GV_KC);

    const uint8_t* e8 = reinterpret_cast<const uint8_t*>(scales);
    const uint16_t* sc16 = reinterpret_cast<const uint16_t*>(scales);

    int64_t wrow[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        int64_t r = row0 + rp * 32 + rb * 16 + li;
        wrow[rb] = r < N ? r : (int64_t)N - 1;
    }

    v4f acc[2][NCB];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) acc[rb][cb] = v4f{0.f, 0.f, 0.f, 0.f};

    // activation chunk staging: thread covers 16 bytes of 2*NCB token rows
    const int xc = tid & 31;
    const int xr = tid >> 5;
    uint4 xreg[2 * NCB];
    uint16_t sreg[GS ? (NG * GV_ROWS + 255) / 256 : 1];

    auto load_x = [&](int64_t kc0) {
#pragma unroll
        for (int j = 0; j < 2 * NCB; ++j) {
            const int t = xr + 8 * j;
            const int64_t k = kc0 + 8 * xc;
            if (t < T && k < k_end) xreg[j] = *reinterpret_cast<const uint4*>(x + (int64_t)t * K + k);
            else xreg[j] = make_uint4(0, 0, 0, 0);
        }
        if constexpr (GS != 0) {
#pragma unroll
            for (int j = 0; j < (NG * GV_ROWS + 255) / 256; ++j) {
                const int idx = tid + 256 * j;       // idx = row * NG + grp
                const int r = idx / NG, gi = idx % NG;
                int64_t row = row0 + r;
                if (row >= N) row = N - 1;
                const int64_t grp = kc0 / GS + gi;
                sreg[j] = (idx < NG * GV_ROWS && kc0 + (int64_t)gi * GS < k_end)
                              ? sc16[row * (K / GS) + grp] : (uint16_t)0;
            }
        }
    };
    auto store_x = [&]() {
#pragma unroll
        for (int j = 0; j < 2 * NCB; ++j)
            *reinterpret_cast<uint4*>(&xs[(xr + 8 * j) * GV_XPITCH + 8 * xc]) = xreg[j];
        if constexpr (GS != 0) {
#pragma unroll
            for (int j = 0; j < (NG * GV_ROWS + 255) / 256; ++j) {
                const int idx = tid + 256 * j;
                if (idx < NG * GV_ROWS) scs[(idx % NG) * GV_ROWS + idx / NG] = sreg[j];
            }
        }
    };

    WRegs<FMT> wc[2], wn[2];
    auto load_w = [&](WRegs<FMT>* dst, int64_t kc0) {
        const int64_t kh0 = kc0 + 128 * kh;
        if (kh0 < k_end) {
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) load_wregs<FMT>(dst[rb], w, e8, wrow[rb], K, kh0, lg);
        }
    };

    if (nch > 0) {
        load_w(wc, k_begin);
        load_x(k_begin);
    }
    for (int c = 0; c < nch; ++c) {
        const int64_t kc0 = k_begin + (int64_t)c * GV_KC;
        __syncthreads();
        store_x();
        __syncthreads();
        if (c + 1 < nch) {
            load_w(wn, kc0 + GV_KC);
            load_x(kc0 + GV_KC);
        }
        if (kc0 + 128 * kh < k_end) {
            if constexpr (GS == 0) {
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const int col = kstep_col<FMT>(kh, ks, lg);
                    v8bf b[NCB];
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb)
                        b[cb] = *reinterpret_cast<const v8bf*>(&xs[(cb * 16 + li) * GV_XPITCH + col]);
#pragma unroll
                    for (int rb = 0; rb < 2; ++rb) {
                        const v8bf a = decode_afrag<FMT>(wc[rb], ks);
#pragma unroll
                        for (int cb = 0; cb < NCB; ++cb)
                            acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[cb], acc[rb][cb], 0, 0, 0);
                    }
                }
            } else {
                constexpr int KPG = GS / 32;             // k-steps per scale group
#pragma unroll
                for (int gq = 0; gq < 4 / KPG; ++gq) {
                    v4f d[2][NCB];
#pragma unroll
                    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                        for (int cb = 0; cb < NCB; ++cb) d[rb][cb] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < KPG; ++kk) {
                        const int ks = gq * KPG + kk;
                        const int col = kstep_col<FMT>(kh, ks, lg);
                        v8bf b[NCB];
#pragma unroll
                        for (int cb = 0; cb < NCB; ++cb)
                            b[cb] = *reinterpret_cast<const v8bf*>(&xs[(cb * 16 + li) * GV_XPITCH + col]);
#pragma unroll
                        for (int rb = 0; rb < 2; ++rb) {
                            const v8bf a = decode_afrag<FMT>(wc[rb], ks);
#pragma unroll
                            for (int cb = 0; cb < NCB; ++cb)
                                d[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[cb], d[rb][cb], 0, 0, 0);
                        }
                    }
                    // group index within the chunk of this k-step group
                    const int gi = (kh * 128) / GS + gq;
#pragma unroll
                    for (int rb = 0; rb < 2; ++rb) {
                        const uint2 s4 = *reinterpret_cast<const uint2*>(
                            &scs[gi * GV_ROWS + rp * 32 + rb * 16 + 4 * lg]);
                        const float s0 = f16_bits_to_f32(s4.x & 0xFFFFu), s1 = f16_bits_to_f32(s4.x >> 16);
                        const float s2 = f16_bits_to_f32(s4.y & 0xFFFFu), s3 = f16_bits_to_f32(s4.y >> 16);
#pragma unroll
                        for (int cb = 0; cb < NCB; ++cb) {
                            acc[rb][cb][0] = fmaf(d[rb][cb][0], s0, acc[rb][cb][0]);
                            acc[rb][cb][1] = fmaf(d[rb][cb][1], s1, acc[rb][cb][1]);
                            acc[rb][cb][2] = fmaf(d[rb][cb][2], s2, acc[rb][cb][2]);
                            acc[rb][cb][3] = fmaf(d[rb][cb][3], s3, acc[rb][cb][3]);
                        }
                    }
                }
            }
        }
        if (c + 1 < nch) {
            wc[0] = wn[0];
            wc[1] = wn[1];
        }
    }

    // Sum the two K halves through LDS (fixed order: half 0 + half 1).
    __syncthreads();
    float* red = reinterpret_cast<float*>(xs);
    if (kh == 1) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
                *reinterpret_cast<v4f*>(&red[(((rp * 2 + rb) * NCB + cb) * 64 + lane) * 4]) = acc[rb][cb];
    }
    __syncthreads();
    if (kh == 0) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                const v4f o = *reinterpret_cast<const v4f*>(&red[(((rp * 2 + rb) * NCB + cb) * 64 + lane) * 4]);
                acc[rb][cb] += o;
            }
    }

    const int64_t npad = (int64_t)gridDim.x * GV_ROWS;
    auto write_out = [&](int rb, int cb, v4f v) {
        const int t = cb * 16 + li;
        const int64_t n0 = row0 + rp * 32 + rb * 16 + 4 * lg;
        if (t >= T) return;
        if constexpr (FMT == W_FP8ROW) {
            const uint16_t* rs = reinterpret_cast<const uint16_t*>(scales);
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = (n0 + r < N) ? v[r] * bf16_bits_to_f32(rs[n0 + r]) : 0.f;
        }
        if (bf16_out) {
            uint16_t* yo = reinterpret_cast<uint16_t*>(y) + (int64_t)t * N;
            if (n0 + 3 < N && (N & 3) == 0) {
                *reinterpret_cast<uint2*>(yo + n0) =
                    make_uint2(f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16),
                               f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16));
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (n0 + r < N) yo[n0 + r] = (uint16_t)f32_to_bf16_rne(v[r]);
            }
        } else {
            float* yo = reinterpret_cast<float*>(y) + (int64_t)t * N;
            if (n0 + 3 < N && (N & 3) == 0) {
                *reinterpret_cast<v4f*>(yo + n0) = v;
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (n0 + r < N) yo[n0 + r] = v[r];
            }
        }
    };

    if (splits == 1) {
        if (kh == 0) {
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) write_out(rb, cb, acc[rb][cb]);
        }
        return;
    }

    // Split-K: publish this split's partial, the last workgroup of the tile sums.
    if (kh == 0) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                const int t = cb * 16 + li;
                if (t < T) {
                    const int64_t n0 = row0 + rp * 32 + rb * 16 + 4 * lg;
                    *reinterpret_cast<v4f*>(&partial[((int64_t)split * T + t) * npad + n0]) = acc[rb][cb];
                }
            }
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const unsigned prev = atomicAdd(&counters[tile], 1u);
        s_last = (prev == (unsigned)(splits - 1));
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    if (kh == 0) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                const int t = cb * 16 + li;
                if (t >= T) continue;
                const int64_t n0 = row0 + rp * 32 + rb * 16 + 4 * lg;
                v4f sum = v4f{0.f, 0.f, 0.f, 0.f};
                for (int s = 0; s < splits; ++s) {
                    const uint32_t* p =
                        reinterpret_cast<const uint32_t*>(&partial[((int64_t)s * T + t) * npad + n0]);
                    v4f part;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        part[r] = __uint_as_float(__hip_atomic_load(p + r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
                    sum += part;
                }
                write_out(rb, cb, sum);
            }
    }
    if (tid == 0) __hip_atomic_store(&counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Fallback: any K.  One wave per (row, up to 8 tokens).
// ---------------------------------------------------------------------------
template <int FMT>
__device__ __forceinline__ float decode_scalar(const uint8_t* __restrict__ w, const void* __restrict__ scales,
                                               int64_t row, int64_t k, int64_t K) {
    if constexpr (FMT == W_FP8ROW) {
        return e4m3_to_f32(w[row * K + k]);
    } else if constexpr (FMT == W_MXFP8) {
        const uint8_t* e8 = reinterpret_cast<const uint8_t*>(scales);
        return e4m3_to_f32(w[row * K + k]) * ue8m0_to_f32(e8[row * (K >> 5) + (k >> 5)]);
    } else if constexpr (FMT == W_BF16) {
        return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(w)[row * K + k]);
    } else {
        constexpr int GS = group_size<FMT>();
        const uint16_t* sc = reinterpret_cast<const uint16_t*>(scales);
        float q;
        if constexpr (FMT == W_Q4G64) {
            const uint32_t b = w[row * (K >> 1) + (k >> 1)];
            const uint32_t nib = (k & 1) ? (b >> 4) : (b & 15u);
            q = (float)((int32_t)(nib << 28) >> 28);
        } else {
            q = (float)(int8_t)w[row * K + k];
        }
        return q * f16_bits_to_f32(sc[row * (K / GS) + k / GS]);    // exact product
    }
}

template <int FMT>
__global__ __launch_bounds__(64) void gemv_generic_kernel(const uint8_t* __restrict__ w,
                                                          const void* __restrict__ scales,
                                                          const uint16_t* __restrict__ x, int T, int N, int64_t K,
                                                          int bf16_out, void* __restrict__ y) {
    const int64_t row = blockIdx.x;
    const int t0 = blockIdx.y * 8;
    const int lane = threadIdx.x;
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.f;
    for (int64_t k = lane; k < K; k += 64) {
        const float wv = decode_scalar<FMT>(w, scales, row, k, K);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (t0 + j < T) acc[j] = fmaf(bf16_bits_to_f32(x[(int64_t)(t0 + j) * K + k]), wv, acc[j]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = wave_sum(acc[j]);
    if (lane < 8 && t0 + lane < T) {
        float v = acc[0];
#pragma unroll
        for (int j = 1; j < 8; ++j)
            if (lane == j) v = acc[j];
        if constexpr (FMT == W_FP8ROW) v *= bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(scales)[row]);
        const int64_t o = (int64_t)(t0 + lane) * N + row;
        if (bf16_out) reinterpret_cast<uint16_t*>(y)[o] = (uint16_t)f32_to_bf16_rne(v);
        else reinterpret_cast<float*>(y)[o] = v;
    }
}

// ---------------------------------------------------------------------------
// Host side: schedule selection and launch.
// ---------------------------------------------------------------------------
struct GemvPlan {
    bool mfma;
    int64_t tiles;
    int splits;
    int64_t k_per_split;
};

static GemvPlan plan_gemv(int64_t Tc, int64_t N, int64_t K) {
    (void)Tc;
    GemvPlan p{};
    p.mfma = (K > 0) && (K % 128 == 0);
    p.tiles = (N + GV_ROWS - 1) / GV_ROWS;
    p.splits = 1;
    p.k_per_split = K;
    if (!p.mfma) return p;
    const int64_t chunks = (K + GV_KC - 1) / GV_KC;
    const int64_t target = 2 * (int64_t)device_cu_count();
    int64_t s = (target + p.tiles - 1) / p.tiles;
    if (s > chunks / 2) s = chunks / 2;
    if (s > 16) s = 16;
    if (s < 1) s = 1;
    const int64_t cps = (chunks + s - 1) / s;
    p.k_per_split = cps * GV_KC;
    p.splits = (int)((chunks + cps - 1) / cps);
    return p;
}

static int64_t align256(int64_t v) { return (v + 255) & ~(int64_t)255; }

int64_t gemv_workspace_bytes(int fmt, int64_t T, int64_t N, int64_t K) {
    (void)fmt;
    const int64_t Tc = T < 64 ? T : 64;
    const GemvPlan p = plan_gemv(Tc, N, K);
    if (!p.mfma || p.splits == 1) return 0;
    return align256(p.tiles * 4) + (int64_t)p.splits * Tc * p.tiles * GV_ROWS * 4;
}

template <int FMT, int NCB>
static void launch_mfma(const GemvPlan& p, const void* w, const void* scales, const uint16_t* x, int Tc, int64_t N,
                        int64_t K, bool bf16_out, void* y, float* partial, unsigned* counters,
                        hipStream_t stream) {
    dim3 grid((unsigned)p.tiles, (unsigned)p.splits);
    gemv_mfma_kernel<FMT, NCB><<<grid, 256, 0, stream>>>(reinterpret_cast<const uint8_t*>(w), scales, x, Tc,
                                                         (int)N, K, p.k_per_split, p.splits, partial, counters,
                                                         bf16_out ? 1 : 0, y);
}

template <int FMT>
static void launch_fmt(const GemvPlan& p, const void* w, const void* scales, const uint16_t* x, int Tc, int64_t N,
                       int64_t K, bool bf16_out, void* y, float* partial, unsigned* counters,
                       hipStream_t stream) {
    if (p.mfma) {
        const int ncb = (Tc + 15) / 16;
        switch (ncb) {
            case 1: launch_mfma<FMT, 1>(p, w, scales, x, Tc, N, K, bf16_out, y, partial, counters, stream); break;
            case 2: launch_mfma<FMT, 2>(p, w, scales, x, Tc, N, K, bf16_out, y, partial, counters, stream); break;
            case 3: launch_mfma<FMT, 3>(p, w, scales, x, Tc, N, K, bf16_out, y, partial, counters, stream); break;
            default: launch_mfma<FMT, 4>(p, w, scales, x, Tc, N, K, bf16_out, y, partial, counters, stream); break;
        }
    } else {
        dim3 grid((unsigned)N, (unsigned)((Tc + 7) / 8));
        gemv_generic_kernel<FMT><<<grid, 64, 0, stream>>>(reinterpret_cast<const uint8_t*>(w), scales, x, Tc,
                                                          (int)N, K, bf16_out ? 1 : 0, y);
    }
}

hipError_t launch_gemv(int fmt, const void* w, const void* scales, const uint16_t* x, int64_t T, int64_t N,
                       int64_t K, bool bf16_out, void* y, void* workspace, int64_t workspace_bytes,
                       hipStream_t stream) {
    if (T == 0 || N == 0) return hipSuccess;
    const size_t ybytes = bf16_out ? 2 : 4;
    for (int64_t t0 = 0; t0 < T; t0 += 64) {
        const int Tc = (int)((T - t0) < 64 ? (T - t0) : 64);
        GemvPlan p = plan_gemv(Tc, N, K);
        float* partial = nullptr;
        unsigned* counters = nullptr;
        if (p.splits > 1) {
            const int64_t need = align256(p.tiles * 4) + (int64_t)p.splits * Tc * p.tiles * GV_ROWS * 4;
            if (workspace != nullptr && workspace_bytes >= need) {
                counters = reinterpret_cast<unsigned*>(workspace);
                partial = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + align256(p.tiles * 4));
            } else {
                p.splits = 1;
                p.k_per_split = K;
            }
        }
        const uint16_t* xc = x + t0 * K;
        void* yc = reinterpret_cast<char*>(y) + t0 * N * ybytes;
        switch (fmt) {
            case W_FP8ROW: launch_fmt<W_FP8ROW>(p, w, scales, xc, Tc, N, K, bf16_out, yc, partial, counters, stream); break;
            case W_MXFP8: launch_fmt<W_MXFP8>(p, w, scales, xc, Tc, N, K, bf16_out, yc, partial, counters, stream); break;
            case W_BF16: launch_fmt<W_BF16>(p, w, scales, xc, Tc, N, K, bf16_out, yc, partial, counters, stream); break;
            case W_Q8G64: launch_fmt<W_Q8G64>(p, w, scales, xc, Tc, N, K, bf16_out, yc, partial, counters, stream); break;
            case W_Q4G64: launch_fmt<W_Q4G64>(p, w, scales, xc, Tc, N, K, bf16_out, yc, partial, counters, stream); break;
            case W_Q8G32: launch_fmt<W_Q8G32>(p, w, scales, xc, Tc, N, K, bf16_out, yc, partial, counters, stream); break;
            default: return hipErrorInvalidValue;
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace nq
