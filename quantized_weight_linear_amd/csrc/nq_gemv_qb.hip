// Q3 / Q5 / Q6 group-64 weights: b-bit two's-complement codes stored as a
// dense little-endian bit stream along each row (element j at bits
// [b j, b j + b)), one FP16 scale per 64 codes.
//   - gemv_qbits_kernel: the decode GEMV on BF16 activations,
//     y[t][n] = sum_g sc[n][g] * sum_{k in g} x[t][k] * q[n][k], FP32 sums;
//   - pack_qbits_kernel: the one-time packed layout that kernel streams;
//   - unpack_qbits_to_int8_kernel: the codes widened to int8 for the A8
//     routes (exact).
//
// GEMV: one wave per 16-row block (nq_wave_gemv.h); a chunk is 256 columns =
// 4 groups of 64.  For group q of chunk c, lane 16 g + i takes the 16 codes k
// = 256 c + 64 q + 16 g + [0, 16) of row i: 2 b bytes of the row, starting on
// a byte boundary (b (32 c + 8 q + 2 g) bytes into the row).  The lane moves
// them into a window whose bit 0 is the first code's bit 0, decodes each pair
// of codes to a biased BF16 pair (qb_pair; positions known at compile time),
// and runs two 16x16x32 BF16 MFMAs against the matching activations (rows
// t >= T read zero) after the two that remove the bias; the group's FP32 sum
// is then scaled by its FP16 scale.
//   Row-major: the 2 b bytes are loaded as 32-bit words from the 4-byte
//   boundary at or below them (for odd b and odd g they start 2 bytes past
//   it) and shifted down.  Packed: per (chunk, row block) the 64 lanes' 8 b
//   bytes (their 4 groups' codes back to back, the same bit stream) are
//   stored as 16-byte pieces (and an 8-byte tail for b = 3, 5), piece-major,
//   lane after lane, so that each load instruction reads a contiguous 1 KiB
//   (or 512 B); the groups' windows are then taken from the lane's words.
#include "nq_wave_gemv.h"

namespace nq {

template <int B>
struct QbLayout {
    static constexpr int LANE_BYTES = 8 * B;                   // 4 groups x 16 codes x B bits
    static constexpr int NP16 = LANE_BYTES / 16;               // 16-byte pieces
    static constexpr bool TAIL8 = (LANE_BYTES % 16) != 0;      // an 8-byte tail piece
    static constexpr int WORDS = LANE_BYTES / 4;               // 32-bit words per lane and chunk
    static constexpr int GWORDS = (2 * B + 2 + 3) / 4;         // words covering one group's 2 B bytes (+2 B shift)
    static constexpr int64_t BLOCK_CHUNK = (int64_t)64 * LANE_BYTES;
};

// Bits [pos, pos + B) of the little-endian words w, sign-extended.
template <int B, int N>
__device__ __forceinline__ int extract_code(const uint32_t (&w)[N], int pos) {
    const int wi = pos >> 5, r = pos & 31;
    if (r + B <= 32) return __builtin_amdgcn_sbfe((int)w[wi], r, B);
    return __builtin_amdgcn_sbfe((int)__builtin_amdgcn_alignbit(w[wi + 1], w[wi], r), 0, B);
}

// Biased decode.  With every code's top bit flipped, the B-bit field holds
// u = q + 2^(B-1) in [0, 2^B); placed in mantissa bits [7 - B, 7) of BF16 1.0
// it is the BF16 value 1 + u / 2^B = 1.5 + q / 2^B, exactly.  The MFMA chain
// of a group starts at -1.5 * sum x (two MFMAs of a fragment of -1.5s
// against the activations), so it ends at sum x q / 2^B, scaled by 2^B once
// per wave.  Two codes take one unsigned extract of their 2 B adjacent bits,
// one multiply that lays the field down twice (at bit 7 - B and 16 bits
// higher, carry-free for B <= 5; two shifted ORs for B = 6) and one and-or,
// instead of two signed extracts, two integer converts and a pack.
constexpr uint32_t QB_ONE = 0x3F803F80u;     // two BF16 1.0
constexpr uint32_t QB_NEG15 = 0xBFC0BFC0u;   // two BF16 -1.5

// Word i of the top-bit flip of the 16 B-bit fields of a group window.
template <int B>
constexpr uint32_t qb_flip_word(int i) {
    uint32_t m = 0;
    for (int j = 0; j < 16; ++j) {
        const int bit = B * j + B - 1 - 32 * i;
        if (bit >= 0 && bit < 32) m |= 1u << bit;
    }
    return m;
}

// The BF16 pair (1.5 + q_j / 2^B, 1.5 + q_{j+1} / 2^B) of codes j, j + 1 of a
// flipped window (pos = B j); mask and one as in decode_afrag's Q4 pairs
// (the mask uniform, the 1.0 pair in a vector register, so that the last
// step is a single and-or).
template <int B, int N>
__device__ __forceinline__ uint32_t qb_pair(const uint32_t (&w)[N], int pos, uint32_t mask, uint32_t one) {
    const int wi = pos >> 5, r = pos & 31;
    const uint32_t t = (r + 2 * B <= 32) ? __builtin_amdgcn_ubfe(w[wi], r, 2 * B)
                                         : __builtin_amdgcn_ubfe(__builtin_amdgcn_alignbit(w[wi + 1], w[wi], r), 0, 2 * B);
    uint32_t a;
    if constexpr (B <= 5) a = __umul24(t, (1u << (7 - B)) | (1u << (23 - 2 * B)));
    else a = (t << (7 - B)) | (t << (23 - 2 * B));
    return (a & mask) | one;
}

// SH: the workgroup's WG_WAVES waves (row blocks) share each chunk's
// activations, staged in LDS (two or more token blocks, where the activation
// loads outweigh the weights: 17408x5120 Q5 T = 33 75.9 -> 44.4 us);
// otherwise each 64-thread workgroup works alone, and the single-wave
// workgroups spread evenly over the SIMDs (with four row blocks per
// workgroup, 1088 row blocks are 272 workgroups on 256 CUs: T = 1 23.6 ->
// 28.6 us).  A single wave either loads its B fragments straight into
// registers (XS = 0: 8 loads of 16 bytes per lane and chunk, every lane's
// token row, rows t >= T read as zero), or (XS > 0, few tokens) loads only
// the first 2 XS token rows of the chunk, XS contiguous 1 KiB loads, and
// stages them in its own LDS rows, where the fragment reads of the lanes
// past those rows hit one zero row.  The zero-reading loads of absent token
// rows cost as much address work as real ones: at T <= 8 they were most of
// a wave's memory instructions.
template <int B, int NCB, bool PK, bool SH, int XS = 0>
__global__ __launch_bounds__(SH ? 64 * WG_WAVES : 64, SH ? 2 : 1) void gemv_qbits_kernel(const uint8_t* __restrict__ w,
                                                        const uint16_t* __restrict__ wsc,
                                                        const uint16_t* __restrict__ x, int T, int N, int64_t K,
                                                        int chunks_per_split, int splits,
                                                        float* __restrict__ partial, unsigned* __restrict__ counters,
                                                        int bf16_out, void* __restrict__ y) {
    using L = QbLayout<B>;
    constexpr int TP = 16 * NCB;                 // token rows of the staged activations
    constexpr int XPITCH = WG_KC + 8;            // bf16 per LDS row: rows shift by 4 banks
    constexpr int XP = TP * (WG_KC / 8) / 256;   // 16-byte activation pieces per thread and chunk
    constexpr bool CS = !SH && XS > 0;           // the wave stages its own first 2 XS token rows
    static_assert(!CS || NCB == 1, "compact staging: one token block");
    constexpr bool SK = SH && XS > 0;            // SH: only the first XS 8-row staging rounds hold tokens
    static_assert(!SK || XS < XP, "skipped staging rounds");
    constexpr int SROWS = CS ? 2 * XS : 8 * XS;  // CS / SK: token rows staged; row SROWS stays zero
    constexpr int XR = SH ? (SK ? XS : XP) : (CS ? XS : 8 * NCB);   // activation registers per ring slot
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][SH ? TP * XPITCH : (CS ? (SROWS + 1) * XPITCH : 8)];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int li = lane & 15, lg = lane >> 4;
    const int64_t nrb = ((int64_t)N + 15) / 16;
    const int rb_own = (SH ? WG_WAVES : 1) * (int)blockIdx.x + (tid >> 6);   // this wave's row block
    const bool rb_valid = rb_own < nrb;
    const int rb = rb_valid ? rb_own : (int)nrb - 1;           // past the last: loads clamped, nothing written
    const int split = blockIdx.y;
    const int64_t G = K / 64;
    const int64_t total_chunks = K / WG_KC;
    const int64_t c_begin = (int64_t)split * chunks_per_split;
    int nch = (int)(total_chunks - c_begin);
    if (nch > chunks_per_split) nch = chunks_per_split;

    int64_t row = (int64_t)rb * 16 + li;
    if (row > N - 1) row = N - 1;
    const int64_t row_bytes = K * B / 8;
    // row-major: byte offset of the lane's group-0 codes in chunk 0, and the
    // shift that takes them down to bit 0 of the first loaded word
    const int64_t rm_off = row * row_bytes + 2 * B * lg;
    const int rm_shift = (rm_off & 3) * 8;
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)w, (short)0, (int)(PK ? nrb * 16 * row_bytes : (int64_t)N * row_bytes), WG_BUF_FLAGS);
    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, (int)((int64_t)T * K * 2), WG_BUF_FLAGS);
    const __amdgpu_buffer_rsrc_t sr =
        __builtin_amdgcn_make_buffer_rsrc((void*)wsc, (short)0, (int)((int64_t)N * G * 2), WG_BUF_FLAGS);
    int xoff[NCB];        // !SH: the lane's B fragment rows (token cb * 16 + i, columns 16 g ..)
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) xoff[cb] = (int)(((int64_t)(cb * 16 + li) * K + 16 * lg) * 2);
    int soff[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) soff[e] = (int)(((int64_t)rb * 16 + 4 * lg + e) * G * 2);

    struct Chunk {
        uint32_t wd[PK ? L::WORDS : 4 * L::GWORDS];
        // SH: this thread's share of the chunk's activations, staged to LDS one
        // chunk ahead; otherwise the lane's B fragments [(q * 2 + h) * NCB + cb]
        uint4 xa[XR];
        uint2 ws[4];
    };
    // ring depth: two at three or more token blocks, and for Q6 in the shared
    // form (its wider code windows would spill at three within two workgroups per CU)
    constexpr int D = (NCB >= 3 || (SH && B == 6)) ? 2 : 3;
    Chunk ring[D];
    auto load = [&](int slot, int64_t c) {
        Chunk& r = ring[slot];
        if constexpr (PK) {
            const int64_t base = (c * nrb + rb) * L::BLOCK_CHUNK;
#pragma unroll
            for (int p = 0; p < L::NP16; ++p) {
                const uint4 v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                              wr, (int)(base + (int64_t)p * 1024 + lane * 16), 0, 0));
                r.wd[4 * p] = v.x; r.wd[4 * p + 1] = v.y; r.wd[4 * p + 2] = v.z; r.wd[4 * p + 3] = v.w;
            }
            if constexpr (L::TAIL8) {
                const uint2 v = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
                                                              wr, (int)(base + L::NP16 * 1024 + lane * 8), 0, 0));
                r.wd[4 * L::NP16] = v.x; r.wd[4 * L::NP16 + 1] = v.y;
            }
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int off = (int)((rm_off + c * (32 * B) + q * (8 * B)) & ~(int64_t)3);
#pragma unroll
                for (int i = 0; i < L::GWORDS; ++i)
                    r.wd[q * L::GWORDS + i] = __builtin_amdgcn_raw_buffer_load_b32(wr, off + 4 * i, 0, 0);
            }
        }
        if constexpr (SH || CS) {
            // piece idx = tid + 256 j (CS: lane + 64 j) is row idx / 32, 16 bytes idx % 32 (rows >= T read zero)
#pragma unroll
            for (int j = 0; j < XR; ++j) {
                const int idx = tid + (SH ? 256 : 64) * j;
                const int t = idx >> 5, pc = idx & 31;
                r.xa[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                        xr, (int)(((int64_t)t * K + c * WG_KC + 8 * pc) * 2), 0, 0));
            }
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb)
                        r.xa[(q * 2 + h) * NCB + cb] = __builtin_bit_cast(
                            uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, xoff[cb] + (int)(c * WG_KC * 2) + 128 * q + 16 * h,
                                                                         0, 0));
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
            r.ws[e] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(sr, soff[e] + (int)(c * 8), 0, 0));
    };
    auto store_x = [&](int buf, int slot) {
        if constexpr (SH || CS)
#pragma unroll
        for (int j = 0; j < XR; ++j) {
            const int idx = tid + (SH ? 256 : 64) * j;
            *reinterpret_cast<uint4*>(&xs[buf][(idx >> 5) * XPITCH + 8 * (idx & 31)]) = ring[slot].xa[j];
        }
    };

    v4f acc[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[cb] = v4f{0.f, 0.f, 0.f, 0.f};
    // CS: the zero row of both buffers (columns [0, 256): lanes 0..31 buffer 0,
    // 32..63 buffer 1), and the lane's fragment row (its token, or the zero row).
    // One wave: its LDS accesses take effect in program order, no barrier.
    int xrow1 = 0;
    if constexpr (CS) {
        *reinterpret_cast<uint4*>(&xs[lane >> 5][SROWS * XPITCH + 8 * (lane & 31)]) = make_uint4(0u, 0u, 0u, 0u);
        xrow1 = (li < SROWS ? li : SROWS) * XPITCH;
    }
    // SK: the zero row of both buffers (threads 0..63), before the first barrier
    if constexpr (SK) {
        if (tid < 64)
            *reinterpret_cast<uint4*>(&xs[tid >> 5][SROWS * XPITCH + 8 * (tid & 31)]) = make_uint4(0u, 0u, 0u, 0u);
    }

    const uint32_t mask = __builtin_amdgcn_readfirstlane(((1u << B) - 1u) * 0x00010001u << (7 - B));
    uint32_t one;
    asm("v_mov_b32 %0, %1" : "=v"(one) : "s"(__builtin_amdgcn_readfirstlane(QB_ONE)));
    auto compute = [&](int slot, const uint16_t* xb) {
        const Chunk& r = ring[slot];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            // the group's window: its 2 B bytes from bit 0
            uint32_t gw[L::GWORDS];
            if constexpr (PK) {
                const int bit0 = 16 * B * q;        // compile-time after unrolling
                const int w0 = bit0 >> 5, sh = bit0 & 31;
#pragma unroll
                for (int i = 0; i < L::GWORDS; ++i) {
                    const uint32_t lo = (w0 + i < L::WORDS) ? r.wd[w0 + i] : 0u;
                    const uint32_t hi = (w0 + i + 1 < L::WORDS) ? r.wd[w0 + i + 1] : 0u;
                    gw[i] = sh ? __builtin_amdgcn_alignbit(hi, lo, sh) : lo;
                }
            } else {
#pragma unroll
                for (int i = 0; i < L::GWORDS; ++i) {
                    const uint32_t lo = r.wd[q * L::GWORDS + i];
                    const uint32_t hi = (i + 1 < L::GWORDS) ? r.wd[q * L::GWORDS + i + 1] : 0u;
                    gw[i] = __builtin_amdgcn_alignbit(hi, lo, rm_shift);
                }
            }
#pragma unroll
            for (int i = 0; i < L::GWORDS; ++i) gw[i] ^= qb_flip_word<B>(i);
            // B fragments: token cb * 16 + i, columns 64 q + 16 g + 8 h .. + 8 of the chunk
            v8bf bx[2][NCB];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
                    bx[h][cb] = SH   ? *reinterpret_cast<const v8bf*>(&xb[(SK && cb * 16 + li > SROWS ? SROWS : cb * 16 + li) * XPITCH + 64 * q + 16 * lg + 8 * h])
                                : CS ? *reinterpret_cast<const v8bf*>(&xb[xrow1 + 64 * q + 16 * lg + 8 * h])
                                     : __builtin_bit_cast(v8bf, r.xa[(q * 2 + h) * NCB + cb]);
            const v8bf neg = __builtin_bit_cast(v8bf, make_uint4(QB_NEG15, QB_NEG15, QB_NEG15, QB_NEG15));
            v4f d[NCB];
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                d[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(neg, bx[0][cb], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                d[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(neg, bx[1][cb], d[cb], 0, 0, 0);
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint32_t o[4];
#pragma unroll
                for (int p = 0; p < 4; ++p) o[p] = qb_pair<B>(gw, B * (8 * h + 2 * p), mask, one);
                const v8bf af = __builtin_bit_cast(v8bf, make_uint4(o[0], o[1], o[2], o[3]));
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
                    d[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bx[h][cb], d[cb], 0, 0, 0);
            }
            float sc[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t pair = (q < 2) ? r.ws[e].x : r.ws[e].y;
                sc[e] = f16_bits_to_f32((q & 1) ? (pair >> 16) : (pair & 0xFFFFu));
            }
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[cb][e] = fmaf(d[cb][e], sc[e], acc[cb][e]);
        }
    };

    // One chunk c (ring slot u = c mod D): compute from LDS buffer c & 1,
    // stage the activations of chunk c + 1 (slot (u + 1) mod D), request the
    // weights, scales and activations of chunk c + D into slot u (indices
    // clamped to the last chunk, so the body has no branch), barrier.  The
    // four waves of the workgroup (four row blocks) share the staged chunk.
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
                if constexpr (SH || CS) body(c + u, u);     // the next chunk's activations are staged here
                else compute(u, xs[0]);
            }
        }
    }
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[cb] *= (float)(1 << B);   // the biased sums' factor 2^B
    if (rb_valid) wave_finish<NCB>(acc, T, N, rb, split, splits, partial, counters, bf16_out, y);
}

// Packed layout: thread per (chunk, row block, lane); the lane's 8 B bytes are
// its 4 groups' 2 B bytes back to back, stored as 16-byte pieces (+ an 8-byte
// tail) piece-major within the (chunk, row block) block.
template <int B>
__global__ __launch_bounds__(256) void pack_qbits_kernel(const uint8_t* __restrict__ src, int64_t N, int64_t K,
                                                         uint8_t* __restrict__ dst, int64_t n_items) {
    using L = QbLayout<B>;
    const int64_t nrb = (N + 15) / 16;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n_items; i += (int64_t)gridDim.x * 256) {
        const int lane = (int)(i & 63);
        const int64_t cr = i >> 6;
        const int64_t rb = cr % nrb, c = cr / nrb;
        const int64_t row = rb * 16 + (lane & 15);
        const int g = lane >> 4;
        uint8_t bytes[L::LANE_BYTES];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int j = 0; j < 2 * B; ++j)
                bytes[q * 2 * B + j] =
                    row < N ? src[row * (K * B / 8) + B * (32 * c + 8 * q + 2 * g) + j] : (uint8_t)0;
        uint8_t* blk = dst + (c * nrb + rb) * L::BLOCK_CHUNK;
#pragma unroll
        for (int p = 0; p < L::NP16; ++p)
#pragma unroll
            for (int j = 0; j < 16; ++j) blk[(int64_t)p * 1024 + lane * 16 + j] = bytes[16 * p + j];
        if constexpr (L::TAIL8)
#pragma unroll
            for (int j = 0; j < 8; ++j) blk[(int64_t)L::NP16 * 1024 + lane * 8 + j] = bytes[16 * L::NP16 + j];
    }
}

// Widening to int8: one thread per group of 64 codes (8 B bytes in, 64 out).
template <int B>
__global__ __launch_bounds__(256) void unpack_qbits_to_int8_kernel(const uint8_t* __restrict__ src, int64_t n_groups,
                                                                   int8_t* __restrict__ out) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n_groups; i += (int64_t)gridDim.x * 256) {
        uint32_t wd[2 * B + 1];
        const uint32_t* p = reinterpret_cast<const uint32_t*>(src + i * 8 * B);   // 8 B bytes: 8-byte aligned
#pragma unroll
        for (int j = 0; j < 2 * B; ++j) wd[j] = p[j];
        wd[2 * B] = 0u;
        uint32_t o[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            uint32_t v = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) v |= ((uint32_t)extract_code<B>(wd, B * (4 * k + e)) & 0xFFu) << (8 * e);
            o[k] = v;
        }
        uint4* dst = reinterpret_cast<uint4*>(out + i * 64);
#pragma unroll
        for (int k = 0; k < 4; ++k) dst[k] = make_uint4(o[4 * k], o[4 * k + 1], o[4 * k + 2], o[4 * k + 3]);
    }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
int qbits_of(int fmt) { return fmt == W_Q3G64 ? 3 : fmt == W_Q5G64 ? 5 : fmt == W_Q6G64 ? 6 : 0; }

int64_t gemv_qbits_workspace_bytes(int64_t T, int64_t N, int64_t K) {
    if (T <= 0 || N <= 0 || K <= 0 || K % WG_KC != 0) return 0;
    int64_t need = 0;
    for (int64_t tc = 1; tc <= (T < 64 ? T : 64); tc += 15) {     // the largest over the passes' plans
        const int64_t w = wave_workspace(plan_wave(N, K, tc, 3), tc);   // Q3's plan: the most splits
        if (w > need) need = w;
    }
    const int64_t tl = T < 64 ? T : 64;
    const int64_t wl = wave_workspace(plan_wave(N, K, tl, 3), tl);
    if (wl > need) need = wl;
    if (T > 64 && T % 64) {                                       // the remainder pass
        const int64_t wr = wave_workspace(plan_wave(N, K, T % 64, 3), T % 64);
        if (wr > need) need = wr;
    }
    return need;
}

template <int B, int NCB, bool PK, int XS = 0>
static void launch_qb_ncb(const WavePlan& p, const void* w, const uint16_t* wsc, const uint16_t* x, int Tc, int64_t N,
                          int64_t K, bool bf16_out, void* y, float* partial, unsigned* counters, hipStream_t stream) {
    constexpr bool SH = NCB >= 2;
    constexpr int NW = SH ? WG_WAVES : 1;
    gemv_qbits_kernel<B, NCB, PK, SH, XS><<<dim3((unsigned)((p.rbs + NW - 1) / NW), (unsigned)p.splits), 64 * NW, 0,
                                            stream>>>(
        reinterpret_cast<const uint8_t*>(w), wsc, x, Tc, (int)N, K, p.chunks_per_split, p.splits, partial, counters,
        bf16_out ? 1 : 0, y);
}

template <int B, bool PK>
static void launch_qb(const WavePlan& p, const void* w, const uint16_t* wsc, const uint16_t* x, int Tc, int64_t N,
                      int64_t K, bool bf16_out, void* y, float* partial, unsigned* counters, hipStream_t stream) {
    // one token block: the wave stages its first 2, 4 or 8 token rows itself (T <= 8)
    switch (Tc <= 2 ? 1 : Tc <= 4 ? 2 : Tc <= 8 ? 4 : (Tc + 15) / 16 + 8) {
        case 1: launch_qb_ncb<B, 1, PK, 1>(p, w, wsc, x, Tc, N, K, bf16_out, y, partial, counters, stream); break;
        case 2: launch_qb_ncb<B, 1, PK, 2>(p, w, wsc, x, Tc, N, K, bf16_out, y, partial, counters, stream); break;
        case 4: launch_qb_ncb<B, 1, PK, 4>(p, w, wsc, x, Tc, N, K, bf16_out, y, partial, counters, stream); break;
        case 9: launch_qb_ncb<B, 1, PK>(p, w, wsc, x, Tc, N, K, bf16_out, y, partial, counters, stream); break;
        // two or more token blocks: the last 8-row staging round is skipped when it holds no token
        case 10:
            if (Tc <= 24) launch_qb_ncb<B, 2, PK, 3>(p, w, wsc, x, Tc, N, K, bf16_out, y, partial, counters, stream);
            else launch_qb_ncb<B, 2, PK>(p, w, wsc, x, Tc, N, K, bf16_out, y, partial, counters, stream);
            break;
        case 11:
            if (Tc <= 40) launch_qb_ncb<B, 3, PK, 5>(p, w, wsc, x, Tc, N, K, bf16_out, y, partial, counters, stream);
            else launch_qb_ncb<B, 3, PK>(p, w, wsc, x, Tc, N, K, bf16_out, y, partial, counters, stream);
            break;
        default:
            if (Tc <= 56) launch_qb_ncb<B, 4, PK, 7>(p, w, wsc, x, Tc, N, K, bf16_out, y, partial, counters, stream);
            else launch_qb_ncb<B, 4, PK>(p, w, wsc, x, Tc, N, K, bf16_out, y, partial, counters, stream);
            break;
    }
}

hipError_t launch_gemv_qbits(int fmt, const void* w, const uint16_t* w_scale, const uint16_t* x, int64_t T, int64_t N,
                             int64_t K, bool bf16_out, void* y, void* workspace, int64_t workspace_bytes,
                             hipStream_t stream, bool packed) {
    const int b = qbits_of(fmt);
    if (b == 0 || K % WG_KC != 0) return hipErrorInvalidValue;
    if (T == 0 || N == 0) return hipSuccess;
    const size_t ybytes = bf16_out ? 2 : 4;
    for (int64_t t0 = 0; t0 < T; t0 += 64) {
        const int Tc = (int)((T - t0) < 64 ? (T - t0) : 64);
        float* partial;
        unsigned* counters;
        const WavePlan p = plan_wave_with(N, K, Tc, b, workspace, workspace_bytes, &partial, &counters);
        const uint16_t* xc = x + t0 * K;
        void* yc = reinterpret_cast<char*>(y) + t0 * N * ybytes;
#define NQ_QB_CASE(BITS)                                                                                         \
    if (b == BITS) {                                                                                             \
        if (packed) launch_qb<BITS, true>(p, w, w_scale, xc, Tc, N, K, bf16_out, yc, partial, counters, stream);  \
        else launch_qb<BITS, false>(p, w, w_scale, xc, Tc, N, K, bf16_out, yc, partial, counters, stream);       \
    }
        NQ_QB_CASE(3)
        NQ_QB_CASE(5)
        NQ_QB_CASE(6)
#undef NQ_QB_CASE
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_pack_qbits(int fmt, const void* src, int64_t N, int64_t K, void* dst, hipStream_t stream) {
    const int b = qbits_of(fmt);
    if (b == 0 || K % WG_KC != 0) return hipErrorInvalidValue;
    if (N == 0 || K == 0) return hipSuccess;
    const int64_t n_items = (N + 15) / 16 * (K / WG_KC) * 64;
    int64_t blocks = (n_items + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    const uint8_t* s = reinterpret_cast<const uint8_t*>(src);
    uint8_t* d = reinterpret_cast<uint8_t*>(dst);
    if (b == 3) pack_qbits_kernel<3><<<(unsigned)blocks, 256, 0, stream>>>(s, N, K, d, n_items);
    if (b == 5) pack_qbits_kernel<5><<<(unsigned)blocks, 256, 0, stream>>>(s, N, K, d, n_items);
    if (b == 6) pack_qbits_kernel<6><<<(unsigned)blocks, 256, 0, stream>>>(s, N, K, d, n_items);
    return hipGetLastError();
}

hipError_t launch_unpack_qbits_to_int8(int fmt, const uint8_t* codes, int64_t N, int64_t K, int8_t* out,
                                       hipStream_t stream) {
    const int b = qbits_of(fmt);
    if (b == 0 || K % 64 != 0) return hipErrorInvalidValue;
    const int64_t n_groups = N * (K / 64);
    if (n_groups == 0) return hipSuccess;
    int64_t blocks = (n_groups + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (b == 3) unpack_qbits_to_int8_kernel<3><<<(unsigned)blocks, 256, 0, stream>>>(codes, n_groups, out);
    if (b == 5) unpack_qbits_to_int8_kernel<5><<<(unsigned)blocks, 256, 0, stream>>>(codes, n_groups, out);
    if (b == 6) unpack_qbits_to_int8_kernel<6><<<(unsigned)blocks, 256, 0, stream>>>(codes, n_groups, out);
    return hipGetLastError();
}

}  // namespace nq
