// A8 decode GEMV: the W8A8 arithmetic at decode sizes (T <= 64 per pass).
//   y[t][n] = sum_g P[t][n][g] * (ws[n][g] * as[t][g]),
//   P[t][n][g] = sum_{k in g} aq[t][k] * wq[n][k]   (int32, exact),
// with int8 activation codes aq and FP32 scales as from the per-token-per-64
// quantizer, and Q8 group-64 (or Q4 group-64) weights with FP16 scales.
//
// One wave per 16-row block: the wave owns its rows over its K range
// outright (no cross-wave sum).  At one token block each wave is a 64-thread
// workgroup of its own and no barrier runs; from two token blocks on, four
// waves share each chunk's activation codes through LDS (one barrier per
// chunk).  A chunk is 256 columns = 4 groups of 64.  For group q of chunk c,
// lane 16 g + i holds the 16 codes k = 256 c + 64 q + 16 g + [0, 16) of row i
// (the A fragment of one v_mfma_i32_16x16x64_i8) and the same 16 activation
// codes of token i of the token block (the B fragment): A and B use the same
// lane -> k assignment, so each MFMA forms one group's exact dot products.
// Q8 codes feed the MFMA as stored (no decode).  Q4 codes are widened to
// bytes in registers as biased values u = q + 8 (0..15, two masks and two
// byte permutes per 8 codes), and the bias is removed inside the matrix unit:
// a first MFMA of a fragment of -8s against the activations starts the
// accumulator at C - 8 sum(aq), so the second one ends at C + P exactly.
// C is the bit pattern of 1.5 * 2^23 (0x4B400000): read as a float, the
// int32 result is 12582912 + P exactly (|P| <= 64 * 127 * 127 < 2^22), and
// the rescale is two FP32 FMAs per element and group:
//     X = fma(D, ws, -12582912 ws)  (= P ws, rounded once),
//     acc = fma(X, as, acc).
// Weights stream from HBM into a register ring, 3 chunks deep (2 with three or
// four token blocks); activation codes and scales come through buffer loads
// whose out-of-range offsets read zero (tokens t >= T).  Row-major weights
// are loaded four lanes to a row and moved into fragment order by ds_bpermute.  With a workspace the
// K range is split over workgroups and the partial sums are exchanged as in
// the BF16-activation GEMV (device-coherent stores and loads, a counter per
// row block, the last arriver sums the splits in order: deterministic).
#include "nq_wave_gemv.h"

namespace nq {

constexpr int A8_KC = WG_KC;
constexpr unsigned A8_BUF_FLAGS = WG_BUF_FLAGS;

template <int FMT>
struct A8Piece {
    static constexpr int PB = FMT == W_Q4G64 ? 8 : 16;                  // bytes per lane and group
    static constexpr int64_t BLOCK_CHUNK = (int64_t)4 * 64 * PB;          // packed bytes per (chunk, row block)
    using T = typename std::conditional<FMT == W_Q4G64, uint2, uint4>::type;
};

template <int NCB>
constexpr int a8_depth() {
    return NCB >= 3 ? 2 : 3;
}

template <int FMT, int NCB, bool SH, int XS = 0>
struct A8Chunk {
    typename A8Piece<FMT>::T w[4];      // group q's weight piece
    // SH: this thread's share of the chunk's activation codes (staged to LDS);
    // XS > 0: the wave's own share of its first 4 XS token rows (staged to
    // its LDS rows); otherwise the lane's B fragments [q * NCB + cb]
    uint4 x[SH ? NCB : (XS > 0 ? XS : 4 * NCB)];
    uint4 as[NCB];                      // the token's activation scales of the chunk's 4 groups
    uint2 ws[4];                        // row 4 lg + e: FP16 weight scales of the 4 groups
};

// 16 Q4 codes (row-major: two's complement nibbles, element 2j low in byte j;
// packed: biased nibbles, code 2i at bits 4i and 2i + 1 at bits 16 + 4i of
// each word) -> 16 bytes u = q + 8 in element order.
template <bool PK>
__device__ __forceinline__ v4i q4_to_biased_bytes(uint2 p) {
    uint32_t d[2] = {p.x, p.y};
    uint32_t o[4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t u = PK ? d[h] : (d[h] ^ 0x88888888u);
        const uint32_t m = u & 0x0F0F0F0Fu, n = (u >> 4) & 0x0F0F0F0Fu;
        if (PK) {   // m = [u0 u4 u1 u5], n = [u2 u6 u3 u7]
            o[2 * h] = __builtin_amdgcn_perm(n, m, 0x06040200u);
            o[2 * h + 1] = __builtin_amdgcn_perm(n, m, 0x07050301u);
        } else {    // m = [u0 u2 u4 u6], n = [u1 u3 u5 u7]
            o[2 * h] = __builtin_amdgcn_perm(n, m, 0x05010400u);
            o[2 * h + 1] = __builtin_amdgcn_perm(n, m, 0x07030602u);
        }
    }
    return v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
}

// SH: the workgroup's WG_WAVES waves (row blocks) share each chunk's
// activation codes, staged in LDS (two or more token blocks: 17408x5120
// Q8G64 T = 33 46.8 -> 40.9 us, 5120x17408 44.8 -> 34.9); otherwise each
// 64-thread workgroup works alone, and the single-wave workgroups spread
// evenly over the SIMDs (one token block: 17408x5120 21.7 against 25.8 us
// with four row blocks per workgroup).  A single wave either loads its B
// fragments straight into registers (XS = 0: 4 loads of 16 bytes per lane
// and chunk, rows t >= T read as zero) or (XS > 0, few tokens) loads only the
// first 4 XS token rows of the chunk, XS contiguous 1 KiB loads, and stages
// them in its own LDS rows; the fragment reads of the lanes past those rows
// hit one zero row (zero-reading loads of absent rows cost as much address
// work as real ones).
template <int FMT, int NCB, bool PK, bool SH, int XS = 0>
__global__ __launch_bounds__(SH ? 64 * WG_WAVES : 64, SH ? 2 : 1) void gemv_a8_kernel(const uint8_t* __restrict__ w, const uint16_t* __restrict__ wsc,
                                                     const int8_t* __restrict__ aq, const float* __restrict__ asc,
                                                     int T, int N, int64_t K, int chunks_per_split, int splits,
                                                     float* __restrict__ partial, unsigned* __restrict__ counters,
                                                     int bf16_out, void* __restrict__ y) {
    using P = A8Piece<FMT>;
    constexpr int D = a8_depth<NCB>();
    constexpr int TP = 16 * NCB;                 // token rows of the staged activation codes
    constexpr int XPITCH = A8_KC + 16;           // bytes per LDS row: rows shift by 4 banks
    constexpr bool CS = !SH && XS > 0;           // the wave stages its own first 4 XS token rows
    static_assert(!CS || NCB == 1, "compact staging: one token block");
    constexpr int SROWS = 4 * XS;                // CS: token rows staged; row SROWS stays zero
    __shared__ __attribute__((aligned(16))) uint8_t xs[2][SH ? TP * XPITCH : (CS ? (SROWS + 1) * XPITCH : 16)];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int li = lane & 15, lg = lane >> 4;
    const int64_t nrb = ((int64_t)N + 15) / 16;
    const int rb_own = (SH ? WG_WAVES : 1) * (int)blockIdx.x + (tid >> 6);   // this wave's row block
    const bool rb_valid = rb_own < nrb;
    const int rb = rb_valid ? rb_own : (int)nrb - 1;           // past the last: loads clamped, nothing written
    const int split = blockIdx.y;
    const int64_t G = K / 64;
    const int64_t total_chunks = K / A8_KC;
    const int64_t c_begin = (int64_t)split * chunks_per_split;
    int nch = (int)(total_chunks - c_begin);
    if (nch > chunks_per_split) nch = chunks_per_split;

    // weights: the lane's piece of the row block (packed), or (row-major) a
    // row with four neighbouring lanes on it, lane l on row l / 4 of the
    // block at lane group l % 4, so that each quad reads one contiguous run;
    // the pieces are moved into fragment order (lane 16 g + i on row i) by
    // ds_bpermute before use.  Rows past N are clamped (never written).
    int64_t rowc = (int64_t)rb * 16 + (lane >> 2);
    if (rowc > N - 1) rowc = N - 1;
    const uint8_t* wrow = PK ? w + (int64_t)rb * P::BLOCK_CHUNK + (int64_t)lane * P::PB
                             : w + rowc * (FMT == W_Q4G64 ? K / 2 : K) + (int64_t)(lane & 3) * P::PB;
    const int64_t wcstride = PK ? nrb * P::BLOCK_CHUNK : A8_KC * P::PB / 16;
    const int64_t wqstride = PK ? 64 * P::PB : 4 * P::PB;
    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc((void*)aq, (short)0, (int)((int64_t)T * K), A8_BUF_FLAGS);
    const __amdgpu_buffer_rsrc_t ar =
        __builtin_amdgcn_make_buffer_rsrc((void*)asc, (short)0, (int)((int64_t)T * G * 4), A8_BUF_FLAGS);
    const __amdgpu_buffer_rsrc_t sr =
        __builtin_amdgcn_make_buffer_rsrc((void*)wsc, (short)0, (int)((int64_t)N * G * 2), A8_BUF_FLAGS);
    int xoff[NCB], aoff[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        const int t = cb * 16 + li;
        xoff[cb] = (int)((int64_t)t * K + 16 * lg);        // !SH: the lane's B fragment row
        aoff[cb] = (int)((int64_t)t * G * 4);
    }
    int soff[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) soff[e] = (int)(((int64_t)rb * 16 + 4 * lg + e) * G * 2);

    A8Chunk<FMT, NCB, SH, XS> ring[D];
    auto load = [&](int slot, int64_t c) {
        A8Chunk<FMT, NCB, SH, XS>& r = ring[slot];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            // packed: non-temporal (1-7 % faster at T = 1, 8 in the same run, level
            // at 33); row-major rows are read in quarters of a line by four waves,
            // which non-temporal loads made 12-55 % slower
            if constexpr (PK) ld_nt(r.w[q], wrow + c * wcstride + q * wqstride);
            else r.w[q] = *reinterpret_cast<const typename P::T*>(wrow + c * wcstride + q * wqstride);
        if constexpr (SH || CS) {
            // piece j of thread tid is row (tid + 256 j) / 16, 16 bytes
            // (tid + 256 j) % 16 (CS: lane + 64 j; rows >= T read zero)
#pragma unroll
            for (int j = 0; j < (SH ? NCB : XS); ++j) {
                const int idx = tid + (SH ? 256 : 64) * j;
                r.x[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                       xr, (int)((int64_t)(idx >> 4) * K + c * A8_KC + 16 * (idx & 15)),
                                                       0, 0));
            }
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
                    r.x[q * NCB + cb] = __builtin_bit_cast(
                        uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, xoff[cb] + (int)(c * A8_KC) + 64 * q, 0, 0));
        }
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
            r.as[cb] = __builtin_bit_cast(uint4,
                                          __builtin_amdgcn_raw_buffer_load_b128(ar, aoff[cb] + (int)(c * 16), 0, 0));
#pragma unroll
        for (int e = 0; e < 4; ++e)
            r.ws[e] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(sr, soff[e] + (int)(c * 8), 0, 0));
    };

    v4f acc[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[cb] = v4f{0.f, 0.f, 0.f, 0.f};
    const v4i bias = {0x4B400000, 0x4B400000, 0x4B400000, 0x4B400000};
    const v4i neg8 = {(int)0xF8F8F8F8u, (int)0xF8F8F8F8u, (int)0xF8F8F8F8u, (int)0xF8F8F8F8u};

    auto store_x = [&](int buf, int slot) {
        if constexpr (SH || CS)
#pragma unroll
        for (int j = 0; j < (SH ? NCB : XS); ++j) {
            const int idx = tid + (SH ? 256 : 64) * j;
            *reinterpret_cast<uint4*>(&xs[buf][(idx >> 4) * XPITCH + 16 * (idx & 15)]) = ring[slot].x[j];
        }
    };

    // CS: the zero row of both buffers (lanes 0..15 buffer 0, 16..31 buffer
    // 1) and the lane's fragment row (its token, or the zero row).  One wave:
    // its LDS accesses take effect in program order, no barrier.
    int xrow1 = 0;
    if constexpr (CS) {
        if (lane < 32)
            *reinterpret_cast<uint4*>(&xs[lane >> 4][SROWS * XPITCH + 16 * (lane & 15)]) = make_uint4(0u, 0u, 0u, 0u);
        xrow1 = (li < SROWS ? li : SROWS) * XPITCH;
    }

    auto compute = [&](int slot, const uint8_t* xb) {
        A8Chunk<FMT, NCB, SH, XS>& r = ring[slot];
        if constexpr (!PK) {
            const int addr = 4 * (4 * li + lg);       // fragment lane 16 g + i takes lane 4 i + g's words
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint32_t v[P::PB / 4];
                __builtin_memcpy(v, &r.w[q], P::PB);
#pragma unroll
                for (int d = 0; d < P::PB / 4; ++d) v[d] = (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)v[d]);
                __builtin_memcpy(&r.w[q], v, P::PB);
            }
        }
        float wsf[4][4], nb[4][4];     // [e][q]
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t s01 = r.ws[e].x, s23 = r.ws[e].y;
            wsf[e][0] = f16_bits_to_f32(s01 & 0xFFFFu);
            wsf[e][1] = f16_bits_to_f32(s01 >> 16);
            wsf[e][2] = f16_bits_to_f32(s23 & 0xFFFFu);
            wsf[e][3] = f16_bits_to_f32(s23 >> 16);
#pragma unroll
            for (int q = 0; q < 4; ++q) nb[e][q] = -12582912.0f * wsf[e][q];   // exact: FP16 times 1.5 2^23
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            v4i a;
            if constexpr (FMT == W_Q4G64) a = q4_to_biased_bytes<PK>(r.w[q]);
            else a = __builtin_bit_cast(v4i, r.w[q]);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                // B fragment: token cb * 16 + i, codes 64 q + 16 g .. + 16 of the chunk
                const v4i b = SH   ? *reinterpret_cast<const v4i*>(&xb[(cb * 16 + li) * XPITCH + 64 * q + 16 * lg])
                              : CS ? *reinterpret_cast<const v4i*>(&xb[xrow1 + 64 * q + 16 * lg])
                                   : __builtin_bit_cast(v4i, r.x[q * NCB + cb]);
                v4i d;
                if constexpr (FMT == W_Q4G64) {
                    d = __builtin_amdgcn_mfma_i32_16x16x64_i8(neg8, b, bias, 0, 0, 0);
                    d = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, d, 0, 0, 0);
                } else {
                    d = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, bias, 0, 0, 0);
                }
                const float sa = __uint_as_float(q == 0 ? r.as[cb].x : q == 1 ? r.as[cb].y : q == 2 ? r.as[cb].z
                                                                                                  : r.as[cb].w);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float x = fmaf(__int_as_float(d[e]), wsf[e][q], nb[e][q]);
                    acc[cb][e] = fmaf(x, sa, acc[cb][e]);
                }
            }
        }
    };

    // One chunk c (ring slot u = c mod D): compute from LDS buffer c & 1,
    // stage the activation codes of chunk c + 1, request chunk c + D into
    // slot u (indices clamped to the last chunk, so the body has no branch),
    // barrier.  The four waves (four row blocks) share the staged codes.
    // CS: the same staging within one wave, no barrier.  Otherwise: compute
    // from the registers, refill the slot, no barrier.
    auto body = [&](int c, int u) {
        compute(u, xs[c & 1]);
        if constexpr (SH || CS) store_x((c + 1) & 1, (u + 1) % D);
        load(u, c_begin + min(c + D, nch - 1));
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (SH) __syncthreads();
    };
    if (nch > 0) {
#pragma unroll
        for (int d = 0; d < D; ++d) load(d, c_begin + min(d, nch - 1));
        if constexpr (SH || CS) store_x(0, 0);
        if constexpr (SH) __syncthreads();
        int c = 0;
        for (; c + D <= nch; c += D) {
#pragma unroll
            for (int u = 0; u < D; ++u) body(c + u, u);
        }
#pragma unroll
        for (int u = 0; u < D - 1; ++u) {
            if (c + u < nch) {
                if constexpr (SH || CS) body(c + u, u);     // the next chunk's codes are staged here
                else compute(u, xs[0]);
            }
        }
    }

    if (rb_valid) wave_finish<NCB>(acc, T, N, rb, split, splits, partial, counters, bf16_out, y);
}

// ---------------------------------------------------------------------------
// Host side (plan: plan_wave).
// ---------------------------------------------------------------------------
int64_t gemv_a8_workspace_bytes(int64_t T, int64_t N, int64_t K) {
    if (T <= 0 || N <= 0 || K <= 0 || K % A8_KC != 0) return 0;
    int64_t need = 0;
    for (int64_t tc = 1; tc <= (T < 64 ? T : 64); tc += 15) {     // the largest over the passes' plans
        const int64_t w = wave_workspace(plan_wave(N, K, tc, 0), tc);
        if (w > need) need = w;
    }
    const int64_t tl = T < 64 ? T : 64;
    const int64_t wl = wave_workspace(plan_wave(N, K, tl, 0), tl);
    if (wl > need) need = wl;
    if (T > 64 && T % 64) {                                       // the remainder pass
        const int64_t wr = wave_workspace(plan_wave(N, K, T % 64, 0), T % 64);
        if (wr > need) need = wr;
    }
    return need;
}

template <int FMT, int NCB, bool PK, int XS = 0>
static void launch_a8_ncb(const WavePlan& p, const void* w, const uint16_t* wsc, const int8_t* aq, const float* asc,
                          int Tc, int64_t N, int64_t K, bool bf16_out, void* y, float* partial, unsigned* counters,
                          hipStream_t stream) {
    constexpr bool SH = NCB >= 2;
    constexpr int NW = SH ? WG_WAVES : 1;
    gemv_a8_kernel<FMT, NCB, PK, SH, XS><<<dim3((unsigned)((p.rbs + NW - 1) / NW), (unsigned)p.splits), 64 * NW, 0,
                                           stream>>>(
        reinterpret_cast<const uint8_t*>(w), wsc, aq, asc, Tc, (int)N, K, p.chunks_per_split, p.splits, partial,
        counters, bf16_out ? 1 : 0, y);
}

template <int FMT, bool PK>
static void launch_a8_fmt(const WavePlan& p, const void* w, const uint16_t* wsc, const int8_t* aq, const float* asc,
                          int Tc, int64_t N, int64_t K, bool bf16_out, void* y, float* partial, unsigned* counters,
                          hipStream_t stream) {
    // one token block: the wave stages its first 4 or 8 token rows itself (T <= 8)
    switch (Tc <= 4 ? 1 : Tc <= 8 ? 2 : (Tc + 15) / 16 + 8) {
        case 1: launch_a8_ncb<FMT, 1, PK, 1>(p, w, wsc, aq, asc, Tc, N, K, bf16_out, y, partial, counters, stream); break;
        case 2: launch_a8_ncb<FMT, 1, PK, 2>(p, w, wsc, aq, asc, Tc, N, K, bf16_out, y, partial, counters, stream); break;
        case 9: launch_a8_ncb<FMT, 1, PK>(p, w, wsc, aq, asc, Tc, N, K, bf16_out, y, partial, counters, stream); break;
        case 10: launch_a8_ncb<FMT, 2, PK>(p, w, wsc, aq, asc, Tc, N, K, bf16_out, y, partial, counters, stream); break;
        case 11: launch_a8_ncb<FMT, 3, PK>(p, w, wsc, aq, asc, Tc, N, K, bf16_out, y, partial, counters, stream); break;
        default: launch_a8_ncb<FMT, 4, PK>(p, w, wsc, aq, asc, Tc, N, K, bf16_out, y, partial, counters, stream); break;
    }
}

hipError_t launch_gemv_a8(int fmt, const void* w, const uint16_t* w_scale, const int8_t* aq, const float* asc,
                          int64_t T, int64_t N, int64_t K, bool bf16_out, void* y, void* workspace,
                          int64_t workspace_bytes, hipStream_t stream, bool packed) {
    if (T == 0 || N == 0) return hipSuccess;
    if (K % A8_KC != 0 || (fmt != W_Q8G64 && fmt != W_Q4G64)) return hipErrorInvalidValue;
    const int64_t G = K / 64;
    const size_t ybytes = bf16_out ? 2 : 4;
    for (int64_t t0 = 0; t0 < T; t0 += 64) {
        const int Tc = (int)((T - t0) < 64 ? (T - t0) : 64);
        float* partial;
        unsigned* counters;
        const WavePlan p = plan_wave_with(N, K, Tc, 0, workspace, workspace_bytes, &partial, &counters);
        const int8_t* aqc = aq + t0 * K;
        const float* ac = asc + t0 * G;
        void* yc = reinterpret_cast<char*>(y) + t0 * N * ybytes;
        if (fmt == W_Q8G64) {
            if (packed) launch_a8_fmt<W_Q8G64, true>(p, w, w_scale, aqc, ac, Tc, N, K, bf16_out, yc, partial, counters, stream);
            else launch_a8_fmt<W_Q8G64, false>(p, w, w_scale, aqc, ac, Tc, N, K, bf16_out, yc, partial, counters, stream);
        } else {
            if (packed) launch_a8_fmt<W_Q4G64, true>(p, w, w_scale, aqc, ac, Tc, N, K, bf16_out, yc, partial, counters, stream);
            else launch_a8_fmt<W_Q4G64, false>(p, w, w_scale, aqc, ac, Tc, N, K, bf16_out, yc, partial, counters, stream);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace nq
