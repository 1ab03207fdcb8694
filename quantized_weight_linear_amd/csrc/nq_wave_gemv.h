// Shared parts of the wave-per-row-block GEMVs (the A8 decode GEMV and the
// Q3 / Q5 / Q6 GEMV): one wave owns 16 weight rows over its K range, so a
// wave's sums need no cross-wave reduction.  At one token block each wave is
// a workgroup of its own; with more, WG_WAVES waves (consecutive row blocks)
// form a workgroup and share each chunk's activations through LDS.  Output layout of a
// 16x16 MFMA result: lane 16 g + i holds rows 4 g + e (e = 0..3) of token i of
// the token block.  With a K split the partial sums go to a workspace
// [splits][T][rows padded to 16] through device-coherent stores (the cache
// policy of an agent-scope atomic access, sc1), the wave waits for them, a
// counter per row block is bumped, and the last arriver loads every split's
// partial the same way and sums them in split order (deterministic); it then
// resets the counter.
#pragma once

#include "nq_device.h"
#include "nq_launch.h"

namespace nq {

constexpr int WG_KC = 256;                  // columns per chunk: 4 groups of 64
constexpr int WG_WAVES = 4;                 // waves (row blocks) per workgroup, sharing each chunk's activations
constexpr unsigned WG_BUF_FLAGS = 0x00020000u;
constexpr int WG_CPOL_DEVICE = 16;          // sc1
constexpr int64_t WG_OOB = 0x7FFFFFF0 / 4;  // an element index whose load reads zero

// Rows n0 .. n0 + 3 of token t (t < T checked here).
__device__ __forceinline__ void wave_write_rows(v4f v, int t, int64_t n0, int T, int N, int bf16_out,
                                                void* __restrict__ y) {
    if (t >= T) return;
    if (bf16_out) {
        uint16_t* yo = reinterpret_cast<uint16_t*>(y) + (int64_t)t * N;
        if (n0 + 3 < N && (N & 3) == 0) {
            *reinterpret_cast<uint2*>(yo + n0) = make_uint2(f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16),
                                                            f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16));
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (n0 + e < N) yo[n0 + e] = (uint16_t)f32_to_bf16_rne(v[e]);
        }
    } else {
        float* yo = reinterpret_cast<float*>(y) + (int64_t)t * N;
        if (n0 + 3 < N && (N & 3) == 0) {
            *reinterpret_cast<v4f*>(yo + n0) = v;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (n0 + e < N) yo[n0 + e] = v[e];
        }
    }
}

// The wave's finished sums acc[cb] (token cb * 16 + i) for row block rb:
// written, or exchanged across the K splits as described above.
template <int NCB>
__device__ __forceinline__ void wave_finish(v4f (&acc)[NCB], int T, int N, int rb, int split, int splits,
                                            float* __restrict__ partial, unsigned* __restrict__ counters,
                                            int bf16_out, void* __restrict__ y) {
    const int lane = threadIdx.x & 63;
    const int li = lane & 15, lg = lane >> 4;
    const int64_t n0 = (int64_t)rb * 16 + 4 * lg;
    if (splits == 1) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) wave_write_rows(acc[cb], cb * 16 + li, n0, T, N, bf16_out, y);
        return;
    }
    const int64_t npad = ((int64_t)N + 15) / 16 * 16;
    const __amdgpu_buffer_rsrc_t pr =
        __builtin_amdgcn_make_buffer_rsrc((void*)partial, (short)0, 0x7FFFFFF0, WG_BUF_FLAGS);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        const int t = cb * 16 + li;
        if (t < T)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, acc[cb]), pr,
                                                   (int)((((int64_t)split * T + t) * npad + n0) * 4), 0,
                                                   WG_CPOL_DEVICE);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    unsigned prev = 0;
    if (lane == 0) prev = __hip_atomic_fetch_add(&counters[rb], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    prev = (unsigned)__shfl((int)prev, 0, 64);
    if (prev != (unsigned)(splits - 1)) return;
    constexpr int SB = 8;
    v4f sum[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) sum[cb] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int sb = 0; sb < splits; sb += SB) {
        v4f part[NCB][SB];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const int t = cb * 16 + li;
#pragma unroll
            for (int j = 0; j < SB; ++j) {
                const int64_t idx = (t < T && sb + j < splits) ? (((int64_t)(sb + j) * T + t) * npad + n0) : WG_OOB;
                part[cb][j] = __builtin_bit_cast(
                    v4f, __builtin_amdgcn_raw_buffer_load_b128(pr, (int)(idx * 4), 0, WG_CPOL_DEVICE));
            }
        }
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int j = 0; j < SB; ++j)
                if (sb + j < splits) sum[cb] += part[cb][j];
    }
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) wave_write_rows(sum[cb], cb * 16 + li, n0, T, N, bf16_out, y);
    if (lane == 0) __hip_atomic_store(&counters[rb], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Row blocks of 16; with fewer row blocks than the SIMDs (4 per CU), K is
// split so that there are about as many waves as SIMDs, at least 4 chunks per
// split (only with a workspace).  Twice as many waves (two per SIMD, K split
// twice as often) where that measured faster: two or more token blocks with
// fewer row blocks than SIMDs (5120 x 17408 T = 33: Q3 / Q5 -8 %, A8 Q8G64 /
// Q4G64 -9 / -15 %), and the Q3 / Q5 / Q6 kernel at T <= 2 (17408 x 5120 and
// 5120 x 17408 T = 1: -6..10 %), for Q3 up to T = 4 (T = 3, 4: -6..9 %; Q5
// +5..7 %).  Elsewhere two waves per SIMD were slower (T = 6, 8: Q3 / Q5
// +1..11 %; the A8 kernel at one token block +5..16 %).  qbits: the code
// width of the Q3 / Q5 / Q6 kernel, 0 for the A8 kernel.
struct WavePlan {
    int64_t rbs;
    int splits;
    int chunks_per_split;
};

inline WavePlan plan_wave(int64_t N, int64_t K, int64_t Tc, int qbits) {
    WavePlan p{};
    p.rbs = (N + 15) / 16;
    const int64_t chunks = K / WG_KC;
    const int64_t simds = 4 * (int64_t)device_cu_count();
    const bool two_per_simd = (qbits && Tc <= (qbits == 3 ? 4 : 2)) || (Tc > 16 && p.rbs < simds);
    const int64_t waves = (two_per_simd ? 2 : 1) * simds;
    int64_t s = p.rbs >= waves ? 1 : (waves + p.rbs / 2) / p.rbs;
    int64_t smax = chunks / 4;
    if (smax < 1) smax = 1;
    if (s > smax) s = smax;
    if (s > 32) s = 32;
    if (s < 1) s = 1;
    const int64_t cps = (chunks + s - 1) / s;
    p.chunks_per_split = (int)cps;
    p.splits = (int)((chunks + cps - 1) / cps);
    return p;
}

inline int64_t wave_align256(int64_t v) { return (v + 255) & ~(int64_t)255; }

inline int64_t wave_workspace(const WavePlan& p, int64_t Tc) {
    if (p.splits == 1) return 0;
    return wave_align256(p.rbs * 4) + (int64_t)p.splits * Tc * p.rbs * 16 * 4;
}

// The plan for one pass of Tc tokens, given the caller's workspace: the
// counters and partials, or no split when the workspace is missing or small.
inline WavePlan plan_wave_with(int64_t N, int64_t K, int64_t Tc, int qbits, void* workspace,
                               int64_t workspace_bytes, float** partial, unsigned** counters) {
    WavePlan p = plan_wave(N, K, Tc, qbits);
    *partial = nullptr;
    *counters = nullptr;
    if (p.splits > 1) {
        if (workspace != nullptr && workspace_bytes >= wave_workspace(p, Tc)) {
            *counters = reinterpret_cast<unsigned*>(workspace);
            *partial = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + wave_align256(p.rbs * 4));
        } else {
            p.splits = 1;
            p.chunks_per_split = (int)(K / WG_KC);
        }
    }
    return p;
}

}  // namespace nq
