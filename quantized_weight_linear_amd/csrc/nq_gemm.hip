// Prefill GEMMs on CDNA4 MFMA: y[m][n] = sum_k A[m][k] * W[n][k] with
// int8 x int8 codes (W8A8, FP32 rescale per 64-channel group) or E4M3 x E4M3
// codes (one scale per token and one per weight row).
//
// Tiling.  A workgroup of WM x WN waves computes a BM (tokens) x BN (weight
// rows) tile; each wave 32 TM x 32 TN of it as TM x TN MFMA tiles of 32 x 32.
// W8A8: 8 waves, 256 x 128, 64 x 64 per wave (the wave also holds a second
// set of int32 group sums for its software pipeline, which bounds its tile).
// FP8: 8 waves, 256 x 256, 64 x 128 per wave.  Larger tiles mean fewer bytes
// staged per output: (BM + BN) x K bytes per tile.
//
// Staging.  Codes go from memory straight into LDS with buffer loads in LDS
// mode (no VGPR round trip, no VALU work): one load instruction of a wave
// writes 1 KB of LDS in lane order, four lanes per row reading the row's 64
// contiguous bytes of the stage; the 16-byte pieces of a row are XOR-swizzled
// so that the MFMA fragment reads (16 bytes per lane) are conflict-free.  One
// stage holds 64 K-columns of both panels (plus, for W8A8, the group's
// activation and weight scales); a ring of S stages keeps S - 1 in flight
// while one is consumed, with one barrier per stage.  Rows past M / N and
// columns past K are out of the buffer range and read as zero.
//
// W8A8 (one stage = one 64-channel group): two v_mfma_i32_32x32x32_i8 per
// tile sum the group exactly in int32.  The first MFMA's C operand is the
// constant 0x4B400000 (the float 1.5 * 2^23), so the int32 result D = C + P
// read as a float is exactly 12582912 + P for |P| < 2^22 (here |P| <= 64 *
// 128^2).  The rescale is then two FP32 FMAs per element:
//     X   = fma(float(D), ws, -12582912 * ws)   -> P * ws rounded once
//     acc = fma(X, as, acc)
// (-12582912 * ws is exact: ws is FP16, 11 significant bits).  Those two
// FMAs per output element and group are the kernel's floor on this part:
// 2 * M * N * K / 64 FP32 FMAs on the vector ALUs, about twice the int8 MFMA
// time, so the MFMAs of one group are issued before the rescale of the
// previous one and the two overlap.
//
// FP8: E4M3 codes are decoded exactly to BF16 (the hardware convert, scale 1)
// after the fragment read and multiplied with v_mfma_f32_32x32x16_bf16: every
// product of two E4M3 values is exact and the sums are FP32.  The native FP8
// MFMA is not used: its dot products are not FP32-accurate (relative errors of
// a few 1e-5 were measured on one instruction), outside this path's 1e-5
// bound.  y = (acc * a_scale[m]) * w_scale[n] at the end.
#include "nq_device.h"
#include "nq_launch.h"

// m0 is written by the LDS-mode loads below; nothing else in this file uses it.
#pragma clang diagnostic ignored "-Winline-asm"

namespace nq {

constexpr int GB_K = 64;     // K columns (bytes) per stage
constexpr unsigned GB_FLAGS = 0x00020000u;
constexpr int GB_OOB = 0x40000000;   // a buffer offset past every range used here

template <bool W8A8>
struct GemmCfg {
    static constexpr int WM = W8A8 ? 4 : 4, WN = W8A8 ? 2 : 2;   // wave grid
    static constexpr int TM = W8A8 ? 2 : 2, TN = W8A8 ? 2 : 4;   // 32 x 32 tiles per wave
    static constexpr int S = W8A8 ? 4 : 4;                       // stages in the LDS ring
    static constexpr int NW = WM * WN;
    static constexpr int BM = 32 * TM * WM, BN = 32 * TN * WN;
    static constexpr int LOADS = (BM + BN) / 16 / NW;   // panel loads per wave and stage (16 rows each)
    static_assert((BM + BN) % (16 * NW) == 0, "panel loads must divide evenly over the waves");
};

// 16-byte aligned size: every stage of the ring starts on a 16-byte boundary,
// so fragment reads stay single 16-byte LDS reads.
template <bool W8A8>
struct alignas(16) GemmStage {
    static constexpr int BM = GemmCfg<W8A8>::BM, BN = GemmCfg<W8A8>::BN;
    uint8_t a[BM * GB_K];
    uint8_t b[BN * GB_K];
    float as[W8A8 ? BM : 1];       // W8A8: activation scales of the stage's group
    uint32_t ws[W8A8 ? BN : 1];    // W8A8: weight scales of the stage's group (FP16 bits, zero-extended:
                                   // a 2-byte load in LDS mode still writes 4 bytes per lane)
    uint32_t sink[W8A8 ? 64 : 1];  // W8A8: target of the empty scale loads (they write zeros)
};

// 32x32 MFMA output layout: lane l holds column (l % 32) and rows
// 8 j + 4 (l / 32) + r for j, r in 0..3 (element 4 j + r).
__device__ __forceinline__ int d_row(int lane, int e) { return 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3); }

// Buffer descriptor (base, no stride, num_records bytes): offsets at or past
// num_records read as zero.
__device__ __forceinline__ v4u buffer_desc(const void* base, uint32_t bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    v4u d;
    d.x = (uint32_t)b;
    d.y = (uint32_t)(b >> 32) & 0xFFFFu;
    d.z = bytes;
    d.w = GB_FLAGS;
    return d;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// One buffer load in LDS mode: lane i's SIZE bytes from desc + voff land at
// LDS address m0 + max(SIZE, 4) * i (sub-dword loads write a zero-extended
// dword per lane).  Written as inline assembly so that the compiler
// does not pair these loads with the LDS reads that follow them (it would
// wait for every one still in flight); the ring below waits for exactly the
// stage it consumes.  The instruction has no register result.
template <int SIZE>
__device__ __forceinline__ void lds_dma(v4u desc, uint32_t lds, int voff) {
    if constexpr (SIZE == 16)
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                     :: "v"(voff), "s"(desc), "s"(lds) : "memory", "m0");
    else if constexpr (SIZE == 4)
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
                     :: "v"(voff), "s"(desc), "s"(lds) : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_ushort %0, %1, 0 offen lds"
                     :: "v"(voff), "s"(desc), "s"(lds) : "memory", "m0");
}

template <bool W8A8, bool SUMS, bool KTAIL>
__global__ __launch_bounds__(64 * GemmCfg<W8A8>::NW) void gemm_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ a_scale, const uint8_t* __restrict__ W,
    const uint16_t* __restrict__ w_scale, int M, int N, int K, int bf16_out, void* __restrict__ y,
    int32_t* __restrict__ group_sums) {
    using C = GemmCfg<W8A8>;
    constexpr int BM = C::BM, BN = C::BN, TM = C::TM, TN = C::TN, S = C::S;
    constexpr int DMA_PER_STAGE = C::LOADS + (W8A8 ? 1 : 0);   // load instructions per wave and stage
    __shared__ __attribute__((aligned(16))) GemmStage<W8A8> st[S];
    __shared__ float s_rs[W8A8 ? 1 : BM + BN];                 // FP8: token scales, then weight-row scales

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar branches, SGPR resources
    const int wm = wv % C::WM, wn = wv / C::WM;
    const int m0 = blockIdx.y * BM;
    const int n0 = blockIdx.x * BN;
    const int G = K >> 6;
    const int nsteps = (K + GB_K - 1) / GB_K;
    const int rows_a = min(M - m0, BM);
    const int rows_b = min(N - n0, BN);

    // Buffer ranges start at the tile: rows past M / N fall outside them.
    const v4u ra = buffer_desc(A + (int64_t)m0 * K, (uint32_t)(rows_a * K));
    const v4u rb = buffer_desc(W + (int64_t)n0 * K, (uint32_t)(rows_b * K));

    // Panel layout in LDS: row r of a panel at byte 64 r, its 16-byte piece c
    // (columns k0 + 16 c + [0, 16)) in slot c ^ ((r >> 2) & 3).  Panel loads
    // cover 16 rows each: A rows first, then B rows; wave wv issues loads
    // wv * LOADS + [0, LOADS).  Lane L writes slot L % 4 of row L / 4 of its
    // load, so four lanes read one row's 64 contiguous bytes (one full memory
    // request).  The XOR keeps fragment reads conflict-free (see frag_off).
    const int lr = lane >> 2;
    const int lk = 16 * ((lane & 3) ^ ((lr >> 2) & 3));   // (r >> 2) & 3 is the same for r = 16 q + lr
    int voff_ld[C::LOADS];
    uint32_t lds_ld_a[C::LOADS];   // LDS byte offset within the stage
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
        const int q = wv * C::LOADS + i;                  // wave-uniform
        const int row = 16 * (q < BM / 16 ? q : q - BM / 16) + lr;
        voff_ld[i] = row * K + lk;
        lds_ld_a[i] = (q < BM / 16) ? (uint32_t)(1024 * q) : (uint32_t)(BM * GB_K + 1024 * (q - BM / 16));
    }
    // W8A8 scale loads: as rows in loads of 64 (BM / 64 of them), then ws rows
    // (BN / 64); a wave without one issues an empty load so that every wave
    // issues the same number per stage.
    constexpr int NSL = W8A8 ? (BM + BN) / 64 : 0;
    static_assert(NSL <= C::NW, "one scale load per wave at most");
    v4u rs = ra;
    int voff_s = GB_OOB, sz_s = 0;
    uint32_t lds_s = 0;
    if constexpr (W8A8) {
        if (wv < BM / 64) {
            rs = buffer_desc(a_scale + (int64_t)m0 * G, (uint32_t)(rows_a * G * 4));
            voff_s = (64 * wv + lane) * G * 4;
            sz_s = 4;
            lds_s = (uint32_t)(offsetof(GemmStage<W8A8>, as) + 256 * wv);
        } else {
            const int j = wv - BM / 64;                    // past the ws loads: an empty load into sink
            rs = buffer_desc(w_scale + (int64_t)n0 * G, (uint32_t)(rows_b * G * 2));
            voff_s = j < BN / 64 ? (64 * j + lane) * G * 2 : GB_OOB;
            sz_s = 2;
            lds_s = j < BN / 64 ? (uint32_t)(offsetof(GemmStage<W8A8>, ws) + 256 * j)
                                : (uint32_t)offsetof(GemmStage<W8A8>, sink);
        }
    }

    auto issue = [&](GemmStage<W8A8>& Sg, int s) {
        const uint32_t base = lds_addr(&Sg);
        const int k0 = s < nsteps ? s * GB_K : GB_OOB;   // stages past the end load nothing
#pragma unroll
        for (int i = 0; i < C::LOADS; ++i) {
            const int q = wv * C::LOADS + i;
            int vo = voff_ld[i] + k0;
            if constexpr (KTAIL) {
                if (k0 + lk >= K) vo = GB_OOB;                // K % 16 == 0: pieces are whole
            }
            lds_dma<16>(q < BM / 16 ? ra : rb, base + lds_ld_a[i], vo);
        }
        if constexpr (W8A8) {
            const int g = s < nsteps ? s : GB_OOB / 8;
            if (sz_s == 4) lds_dma<4>(rs, base + lds_s, voff_s + 4 * g);
            else lds_dma<2>(rs, base + lds_s, voff_s >= GB_OOB ? GB_OOB : voff_s + 2 * g);
        }
    };

    v16f acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    // Byte offset of this lane's 16-byte fragment piece in a panel: row
    // rt + lane % 32 of the panel, piece c0 + lane / 32.  Within a quarter
    // wave (16 lanes, 16 rows, one piece) the XOR spreads the rows over all 16
    // four-bank groups.
    auto frag_off = [&](int rt, int c0) {
        const int r = rt + (lane & 31);
        return 64 * r + 16 * ((c0 + (lane >> 5)) ^ ((r >> 2) & 3));
    };
    const int wr0 = 32 * TM * wm;       // first panel row of the wave, A
    const int wc0 = 32 * TN * wn;       // ... and B

    // W8A8, MFMA part of one stage: d = 12582912 + P (as float bits) for the
    // wave's tiles.
    auto mfma_i8 = [&](const GemmStage<W8A8>& Sg, v16i (&d)[TM][TN]) {
        const v16i bias = {0x4B400000, 0x4B400000, 0x4B400000, 0x4B400000, 0x4B400000, 0x4B400000,
                           0x4B400000, 0x4B400000, 0x4B400000, 0x4B400000, 0x4B400000, 0x4B400000,
                           0x4B400000, 0x4B400000, 0x4B400000, 0x4B400000};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            v4i af[TM], bf[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) af[i] = *reinterpret_cast<const v4i*>(&Sg.a[frag_off(wr0 + 32 * i, 2 * h)]);
#pragma unroll
            for (int j = 0; j < TN; ++j) bf[j] = *reinterpret_cast<const v4i*>(&Sg.b[frag_off(wc0 + 32 * j, 2 * h)]);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    d[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], h == 0 ? bias : d[i][j], 0, 0, 0);
        }
    };

    // W8A8, rescale part: acc += (P * ws) * as with the group's scales.
    auto rescale = [&](const GemmStage<W8A8>& Sg, const v16i (&d)[TM][TN], int s) {
        float wsf[TN], wsc[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            wsf[j] = f16_bits_to_f32(Sg.ws[wc0 + 32 * j + (lane & 31)] & 0xFFFFu);
            wsc[j] = -12582912.0f * wsf[j];
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const v4f as4 = *reinterpret_cast<const v4f*>(&Sg.as[wr0 + 32 * i + 8 * q + 4 * (lane >> 5)]);
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int e = 4 * q + r;
                        const float X = fmaf(__int_as_float(d[i][j][e]), wsf[j], wsc[j]);
                        acc[i][j][e] = fmaf(X, as4[r], acc[i][j][e]);
                    }
            }
        }
        if constexpr (SUMS) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int n = n0 + wc0 + 32 * j + (lane & 31);
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int m = m0 + wr0 + 32 * i + d_row(lane, e);
                        if (m < M && n < N) group_sums[((int64_t)m * N + n) * G + s] = d[i][j][e] - 0x4B400000;
                    }
                }
            // the ring's wait counts only loads: drain these stores here
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
    };

    // FP8, one stage.  For column pair p each lane reads 16 consecutive codes
    // of its row (k = 32 p + 16 (lane / 32) + [0, 16)) in one conflict-free
    // read and feeds bytes [0, 8) to one 32x32x16 MFMA and bytes [8, 16) to a
    // second.  The first MFMA thus sums k in {32p + [0,8), 32p + 16 + [0,8)},
    // the second the other 16: the A and B fragments use the same lane -> k
    // assignment, so the two MFMAs together form the exact dot product over
    // the 32 columns.
    auto compute_fp8 = [&](const GemmStage<W8A8>& Sg) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            uint4 ca[TM], cb[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) ca[i] = *reinterpret_cast<const uint4*>(&Sg.a[frag_off(wr0 + 32 * i, 2 * p)]);
#pragma unroll
            for (int j = 0; j < TN; ++j) cb[j] = *reinterpret_cast<const uint4*>(&Sg.b[frag_off(wc0 + 32 * j, 2 * p)]);
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                v8bf af[TM], bf[TN];
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    const uint32_t w0 = hh ? ca[i].z : ca[i].x, w1 = hh ? ca[i].w : ca[i].y;
                    af[i] = __builtin_bit_cast(v8bf, make_uint4(e4m3x2_to_bf16x2<false>(w0, 1.0f),
                                                                e4m3x2_to_bf16x2<true>(w0, 1.0f),
                                                                e4m3x2_to_bf16x2<false>(w1, 1.0f),
                                                                e4m3x2_to_bf16x2<true>(w1, 1.0f)));
                }
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const uint32_t w0 = hh ? cb[j].z : cb[j].x, w1 = hh ? cb[j].w : cb[j].y;
                    bf[j] = __builtin_bit_cast(v8bf, make_uint4(e4m3x2_to_bf16x2<false>(w0, 1.0f),
                                                                e4m3x2_to_bf16x2<true>(w0, 1.0f),
                                                                e4m3x2_to_bf16x2<false>(w1, 1.0f),
                                                                e4m3x2_to_bf16x2<true>(w1, 1.0f)));
                }
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
            }
        }
    };

    auto sync_stage = [&]() {
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

#pragma unroll
    for (int s = 0; s < S - 1; ++s) issue(st[s], s);
    if constexpr (!W8A8) {
        for (int i = tid; i < BM + BN; i += 64 * C::NW) {
            s_rs[i] = i < BM ? (i < rows_a ? a_scale[m0 + i] : 0.f)
                             : (i - BM < rows_b ? bf16_bits_to_f32(w_scale[n0 + i - BM]) : 0.f);
        }
        __syncthreads();
    }

    if constexpr (W8A8) {
        // Software pipeline: iteration s issues stage s + 1's MFMAs and then
        // rescales stage s, whose MFMAs were issued one iteration earlier, so
        // the matrix unit and the vector ALU of a wave work side by side.
        // Buffers: MFMA(s + 1) reads stage s + 1, the rescale reads stage s's
        // scales, and the refill of iteration s (stage s + S - 1) goes into
        // the buffer of stage s - 1, which the barrier shows nobody reads any
        // more.  Stage s + 1 must have landed: stages s + 2 .. s + S - 2 may
        // still be in flight.
        static_assert(S >= 3, "pipelined ring");
        v16i d0[TM][TN], d1[TM][TN];
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(DMA_PER_STAGE * (S - 2)) : "memory");
        sync_stage();
        if (nsteps > 0) mfma_i8(st[0], d0);
        for (int s = 0; s < nsteps; s += 2) {
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(DMA_PER_STAGE * (S - 3)) : "memory");
            sync_stage();
            issue(st[(s + S - 1) % S], s + S - 1);
            if (s + 1 < nsteps) mfma_i8(st[(s + 1) % S], d1);
            rescale(st[s % S], d0, s);
            if (s + 1 < nsteps) {
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(DMA_PER_STAGE * (S - 3)) : "memory");
                sync_stage();
                issue(st[(s + S) % S], s + S);
                if (s + 2 < nsteps) mfma_i8(st[(s + 2) % S], d0);
                rescale(st[(s + 1) % S], d1, s + 1);
            }
        }
    } else {
        // Ring: before consuming stage s this wave waits for its own loads of
        // stage s (the S - 2 later stages may stay in flight); the barrier
        // makes every wave's loads visible and shows that buffer (s - 1) % S,
        // refilled next, is no longer read.
        for (int s = 0; s < nsteps; ++s) {
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(DMA_PER_STAGE * (S - 2)) : "memory");
            sync_stage();
            issue(st[(s + S - 1) % S], s + S - 1);
            compute_fp8(st[s % S]);
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // drain the empty tail loads

#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int nl = wc0 + 32 * j + (lane & 31);
            const int n = n0 + nl;
            if (n >= N) continue;
            float sw = 1.0f;
            if constexpr (!W8A8) sw = s_rs[BM + nl];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int ml = wr0 + 32 * i + d_row(lane, e);
                const int m = m0 + ml;
                if (m >= M) continue;
                float v = acc[i][j][e];
                if constexpr (!W8A8) v = (v * s_rs[ml]) * sw;
                if (bf16_out) reinterpret_cast<uint16_t*>(y)[(int64_t)m * N + n] = (uint16_t)f32_to_bf16_rne(v);
                else reinterpret_cast<float*>(y)[(int64_t)m * N + n] = v;
            }
        }
}

template <bool W8A8, bool SUMS, bool KTAIL>
static hipError_t launch_gemm_t(const uint8_t* A, const float* a_scale, const uint8_t* W, const uint16_t* w_scale,
                                int64_t M, int64_t N, int64_t K, bool bf16_out, void* y, int32_t* sums,
                                hipStream_t stream) {
    using C = GemmCfg<W8A8>;
    dim3 grid((unsigned)((N + C::BN - 1) / C::BN), (unsigned)((M + C::BM - 1) / C::BM));
    gemm_kernel<W8A8, SUMS, KTAIL><<<grid, 64 * C::NW, 0, stream>>>(A, a_scale, W, w_scale, (int)M, (int)N, (int)K,
                                                                     bf16_out ? 1 : 0, y, sums);
    return hipGetLastError();
}

// Offsets inside a tile are 32-bit: 256 rows x K bytes, and the scale rows.
static bool gemm_shape_ok(int64_t M, int64_t N, int64_t K) {
    return M < ((int64_t)1 << 31) && N < ((int64_t)1 << 31) && (int64_t)256 * K * 4 < ((int64_t)1 << 30);
}

hipError_t launch_gemm_w8a8(const int8_t* a_q, const float* a_scale, const int8_t* w_q, const uint16_t* w_scale,
                            int64_t M, int64_t N, int64_t K, bool bf16_out, void* y, int32_t* group_sums,
                            hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    if (!gemm_shape_ok(M, N, K) || K % 64 != 0) return hipErrorInvalidValue;
    const uint8_t* A = reinterpret_cast<const uint8_t*>(a_q);
    const uint8_t* W = reinterpret_cast<const uint8_t*>(w_q);
    if (group_sums != nullptr)
        return launch_gemm_t<true, true, false>(A, a_scale, W, w_scale, M, N, K, bf16_out, y, group_sums, stream);
    return launch_gemm_t<true, false, false>(A, a_scale, W, w_scale, M, N, K, bf16_out, y, nullptr, stream);
}

hipError_t launch_gemm_fp8(const uint8_t* a_codes, const float* a_scale, const uint8_t* w, const uint16_t* w_scale,
                           int64_t M, int64_t N, int64_t K, bool bf16_out, void* y, hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    if (!gemm_shape_ok(M, N, K) || K % 16 != 0) return hipErrorInvalidValue;
    if (K % GB_K == 0)
        return launch_gemm_t<false, false, false>(a_codes, a_scale, w, w_scale, M, N, K, bf16_out, y, nullptr, stream);
    return launch_gemm_t<false, false, true>(a_codes, a_scale, w, w_scale, M, N, K, bf16_out, y, nullptr, stream);
}

}  // namespace nq
