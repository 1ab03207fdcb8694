// Decode GEMV / skinny GEMM: y[t][n] = sum_k x[t][k] * W[n][k] for a few
// tokens (T <= 64 per pass), weights decoded on the fly in registers.
//
// Main path (K % 256 == 0): BF16 MFMA 16x16x32 on exactly decoded weights.
//   - A workgroup of 4 waves owns 64 weight rows (4 row blocks of 16) and a K
//     range walked in chunks of 256 columns.  Wave w takes columns
//     [64 w, 64 w + 64) of every chunk for all 4 row blocks, so each wave
//     reads only the activation fragments of its own two k-steps (a quarter of
//     what a wave owning 16 rows over the whole chunk would read from LDS) and
//     runs 4 x (token blocks) independent MFMA chains.  At the end the four
//     waves' partial sums are added in LDS, in wave order.
//   - Weights go from HBM straight into registers, depth<FMT>() chunks ahead
//     of use, in a static register ring (the loop is unrolled by the depth).
//     Each lane reads 8- or 16-byte pieces; one load instruction covers 64
//     contiguous bytes of 16 rows (row-major) or 512 B / 1 KiB (packed).
//   - The hot loop has no branches: every chunk is full, prefetch indices are
//     clamped to the last chunk (the repeated loads at the end hit in cache),
//     and activations / scales come through buffer loads whose out-of-range
//     offsets read as zero.  Branches inside the loop would make the compiler
//     drain every outstanding load at each join.
//   - Activations: either staged once in LDS for the whole K range of the
//     workgroup (resident variant) or double-buffered chunk by chunk with one
//     barrier per chunk (streaming variant).  Rows past T read as zero.
//   - Decode in registers: E4M3 -> BF16 by the hardware scaled convert
//     (exact; MXFP8 passes its power-of-two group scale to the convert),
//     int8 / int4 -> FP32 -> BF16 (exact for |q| <= 128), BF16 as stored;
//     Q4 with one token block in a biased form (1.5 + q / 16, exact, see
//     chunk_mfma) corrected by the group's activation sum.
//   - Grouped formats run one MFMA chain per scale group and fold the FP16
//     group scale in FP32 (acc += sc * D); row-scaled FP8 applies its BF16
//     row scale once at the end.
//   - With a workspace the K range is split across workgroups; each split
//     writes an FP32 partial and the last workgroup of a row tile (atomic
//     counter) sums the partials in split order: deterministic results.
//   - With a few more row tiles than CUs (formats without group scales),
//     the leftover tiles' chunks are spread over extra workgroups that run
//     beside the whole tiles (direct_spread), with the same deterministic
//     exchange; the whole tiles' waves take the higher issue priority.
// Fallback (any K): one wave per (row, 8 tokens), scalar decode, FP32 sums.
#pragma once

#include "nq_device.h"
#include "nq_launch.h"

namespace nq {

constexpr int GV_ROWS = 64;   // rows per workgroup (4 row blocks of 16)
constexpr int GV_KC = 256;    // columns per chunk
constexpr unsigned BUF_FLAGS = 0x00020000u;

template <int FMT>
constexpr int group_size() {
    return FMT == W_Q8G32 ? 32 : ((FMT == W_Q4G64 || FMT == W_Q8G64) ? 64 : 0);
}

// Ring depth (chunks in flight per wave) of the streaming variant; shallower
// with three or more token blocks so that two waves fit per SIMD (a second
// round of workgroups costs more than the shorter prefetch), and with two
// token blocks for the formats with group scales, whose deeper ring there
// needs more than 256 VGPRs (the excess lives in AGPRs, copied back and forth).
template <int FMT, int NCB>
constexpr int depth() {
    constexpr bool grouped = FMT == W_Q4G64 || FMT == W_Q8G32 || FMT == W_Q8G64;
    return (FMT == W_BF16 || NCB >= 3 || (grouped && NCB == 2)) ? 2 : (FMT == W_Q4G64 ? 4 : 3);
}

template <int FMT>
__device__ __forceinline__ int64_t row_bytes(int64_t K) {
    if (FMT == W_Q4G64) return K >> 1;
    if (FMT == W_BF16) return K << 1;
    return K;
}

// Pieces.  Within a chunk of 256 columns, lane 16 g + i of a row block (row i,
// lane group g) owns, per piece q, these bytes of its row:
//   FP8ROW / MXFP8 / Q8G64: 4 pieces of 16 B at byte 64q + 16g   (k = 64q + 16g + [0,16))
//   Q4G64:                  4 pieces of  8 B at byte 32q + 8g    (k = 64q + 16g + [0,16))
//   Q8G32:                  8 pieces of  8 B at byte 32q + 8g    (k = 32q + 8g + [0,8))
//   BF16:                   8 pieces of 16 B at byte 64q + 16g   (k = 32q + 8g + [0,8))
// Wave w takes the PW pieces covering chunk columns [64w, 64w + 64) of each of
// the 4 row blocks.  Packed Q4G64 pieces hold their codes biased and reordered
// within each 32-bit word (q4_pack_word); every other format's bytes are copied.
template <int FMT>
struct PieceFmt {
    static constexpr bool WIDE = (FMT == W_FP8ROW || FMT == W_MXFP8 || FMT == W_Q8G64 || FMT == W_BF16);
    static constexpr int NP = (FMT == W_Q8G32 || FMT == W_BF16) ? 8 : 4;   // pieces per row block and chunk
    static constexpr int PW = NP / 4;                                     // ... per row block and wave
    static constexpr int PB = WIDE ? 16 : 8;                               // bytes per lane and piece
    static constexpr int64_t BLOCK_CHUNK = (int64_t)NP * 64 * PB;         // packed bytes per (chunk, row block)
    using Piece = typename std::conditional<WIDE, uint4, uint2>::type;
};

// One wave's share of a chunk: slot j = PW * (row block) + (piece of the wave).
template <int FMT>
struct WChunk {
    typename PieceFmt<FMT>::Piece p[4 * PieceFmt<FMT>::PW];
    uint32_t e8[FMT == W_MXFP8 ? 4 : 1];
};

// Byte offset, within a row-major row, of piece q of chunk c for lane group g.
template <int FMT>
__host__ __device__ __forceinline__ int64_t piece_offset(int64_t c, int q, int g) {
    const int64_t kc0 = c * GV_KC;
    if (FMT == W_Q4G64) return (kc0 >> 1) + 32 * q + 8 * g;
    if (FMT == W_Q8G32) return kc0 + 32 * q + 8 * g;
    if (FMT == W_BF16) return 2 * kc0 + 64 * q + 16 * g;
    return kc0 + 64 * q + 16 * g;
}

// Where a wave's weights come from: per row block, the lane's row (row-major)
// or the lane's piece base in the packed layout (see pack_weights_kernel).
// Rows past N are clamped (their outputs are never written).
struct WSrc {
    const uint8_t* base[4];
    const uint8_t* e8[4];    // MXFP8: the lane's row of scale bytes [K/32]
    int64_t cstride;         // packed: bytes from chunk c to chunk c + 1
    int q0;                  // first piece of this wave
    int g;                   // lane group of the load (row-major: lane % 4, see rowmajor_to_frag)
    int ge;                  // lane group of the fragment (MXFP8 scale bytes)
};

template <int FMT, bool PK>
__device__ __forceinline__ WSrc make_wsrc(const uint8_t* w, const void* scales, int64_t row0, int N, int64_t K,
                                          int lane, int wv) {
    using P = PieceFmt<FMT>;
    WSrc s;
    const int64_t nrb = ((int64_t)N + 15) / 16;
    s.cstride = PK ? nrb * P::BLOCK_CHUNK : 0;
    s.q0 = P::PW * wv;
    s.g = PK ? lane >> 4 : lane & 3;
    s.ge = lane >> 4;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        int64_t row = row0 + 16 * r + (lane & 15);
        if (row > N - 1) row = N - 1;
        int64_t rowc = row0 + 16 * r + (lane >> 2);     // row-major loads: four lanes per row
        if (rowc > N - 1) rowc = N - 1;
        if (PK) {
            int64_t rb = (row0 >> 4) + r;
            if (rb > nrb - 1) rb = nrb - 1;
            s.base[r] = w + rb * P::BLOCK_CHUNK + (int64_t)lane * P::PB;
        } else {
            s.base[r] = w + rowc * row_bytes<FMT>(K);
        }
        s.e8[r] = reinterpret_cast<const uint8_t*>(scales) + row * (K >> 5);
    }
    return s;
}

// NT (packed only): non-temporal loads, for the kernels and weight sizes where
// they measured faster (see launch_mfma).
template <int FMT, bool PK, bool NT = false>
__device__ __forceinline__ void load_chunk(WChunk<FMT>& r, const WSrc& src, int64_t c) {
    using P = PieceFmt<FMT>;
#pragma unroll
    for (int j = 0; j < 4 * P::PW; ++j) {
        const int rb = j / P::PW;
        const int q = src.q0 + j % P::PW;
        const uint8_t* p = PK ? src.base[rb] + c * src.cstride + q * (64 * P::PB)
                              : src.base[rb] + piece_offset<FMT>(c, q, src.g);
        if constexpr (PK && NT) ld_nt(r.p[j], p);
        else r.p[j] = *reinterpret_cast<const typename P::Piece*>(p);
        if constexpr (FMT == W_MXFP8) r.e8[j] = src.e8[rb][(c * GV_KC + 64 * q + 16 * src.ge) >> 5];
    }
}

// Row-major weights are loaded with four neighbouring lanes on one row (lane
// l: row l / 4 of the row block, the piece's bytes of lane group l % 4), so
// that each quad of lanes reads one contiguous run of its row; loaded in the
// fragment's own order (lane 16 g + i on row i) every lane of a quad would
// address another row, four times the memory requests per load.  The MFMA
// fragment wants lane 16 g + i on row i: each word is fetched from lane 4 i + g
// (ds_bpermute: a cross-lane move, no LDS memory).  Packed weights are stored
// in fragment order already.
template <int FMT, bool PK>
__device__ __forceinline__ void rowmajor_to_frag(WChunk<FMT>& r) {
    if constexpr (!PK) {
        using P = PieceFmt<FMT>;
        constexpr int WORDS = P::PB / 4;
        const int lane = threadIdx.x & 63;
        const int addr = 4 * (4 * (lane & 15) + (lane >> 4));
#pragma unroll
        for (int j = 0; j < 4 * P::PW; ++j) {
            uint32_t v[WORDS];
            __builtin_memcpy(v, &r.p[j], P::PB);
#pragma unroll
            for (int d = 0; d < WORDS; ++d) v[d] = (uint32_t)__builtin_amdgcn_ds_bpermute(addr, (int)v[d]);
            __builtin_memcpy(&r.p[j], v, P::PB);
        }
    }
}

// Chunk column of k-step s (0..7) for lane group g: the B fragment of lane
// (i, g) holds activations [t = i][col, col + 8).
template <int FMT>
__device__ __forceinline__ int kstep_col(int s, int g) {
    if constexpr (FMT == W_Q8G32 || FMT == W_BF16) return 32 * s + 8 * g;
    else return 64 * (s >> 1) + 16 * g + 8 * (s & 1);
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

// Q4 codes are multiplied in a biased form: the nibble u = q + 8 (0..15)
// written into mantissa bits 3..6 of the BF16 1.0 is exactly 1 + u / 16 =
// 1.5 + q / 16, so a group's MFMA sum over the biased weights, started from
// C = -1.5 sum x (chunk_mfma), is exactly sum x q / 16 up to FP32 rounding.
// The packed layout stores u with the two codes of a BF16 pair 16 bits apart
// (code 2i at bits 4i, code 2i + 1 at bits 16 + 4i of each 32-bit word), so a
// pair costs one shift and one and-or; the row-major layout (natural order,
// two's complement) builds the same values with a few more operations, so
// packed and row-major results stay identical.
constexpr uint32_t Q4_ONE = 0x3F803F80u;        // two BF16 1.0
constexpr uint32_t Q4_NEG15 = 0xBFC0BFC0u;      // two BF16 -1.5
constexpr uint32_t Q4_MANT = 0x00780078u;       // mantissa bits 3..6 of both halves
// (t & mask) | one: with literal constants the compiler emits a separate and
// + or (the VOP3 and-or takes no literal on this target); with the constants
// in registers (readfirstlane makes them opaque, once per kernel) it emits
// one v_and_or_b32.
__device__ __forceinline__ uint32_t q4_packed_pair(uint32_t d, int i, uint32_t mask, uint32_t one) {
    const uint32_t t = i == 0 ? (d << 3) : (d >> (4 * i - 3));
    return (t & mask) | one;      // one v_and_or_b32 (mask uniform, one in a VGPR: see decode_afrag)
}
__device__ __forceinline__ uint32_t q4_natural_pair(uint32_t d, int i) {  // codes 2i, 2i + 1 of a row-major word
    const uint32_t b = ((d >> (8 * i)) ^ 0x88u) & 0xFFu;                  // u of both codes
    return ((b & 0xFu) << 3) | ((b & 0xF0u) << 15) | Q4_ONE;
}
__device__ __forceinline__ uint32_t q4_packed_exact_pair(uint32_t x, int i) {   // x = packed word ^ 0x88888888
    const float a = (float)((int32_t)(x << (28 - 4 * i)) >> 28);
    const float b = (float)((int32_t)(x << (12 - 4 * i)) >> 28);
    return f32x2_to_bf16x2(a, b);
}

// The A fragment (8 BF16 weights) of row block rb at the wave's local k-step ls.
template <int FMT, bool PK = false, bool BIAS = false>
__device__ __forceinline__ v8bf decode_afrag(const WChunk<FMT>& r, int rb, int ls) {
    uint32_t o[4];
    if constexpr (FMT == W_FP8ROW || FMT == W_MXFP8) {
        const uint4 q = r.p[rb];
        const uint32_t d0 = ls ? q.z : q.x, d1 = ls ? q.w : q.y;
        float sc = 1.0f;
        if constexpr (FMT == W_MXFP8) sc = ue8m0_to_f32(r.e8[rb]);
        o[0] = e4m3x2_to_bf16x2<false>(d0, sc);
        o[1] = e4m3x2_to_bf16x2<true>(d0, sc);
        o[2] = e4m3x2_to_bf16x2<false>(d1, sc);
        o[3] = e4m3x2_to_bf16x2<true>(d1, sc);
    } else if constexpr (FMT == W_Q8G64) {
        const uint4 q = r.p[rb];
        const uint32_t d0 = ls ? q.z : q.x, d1 = ls ? q.w : q.y;
        o[0] = i8x2_to_bf16x2(d0, 0);
        o[1] = i8x2_to_bf16x2(d0, 16);
        o[2] = i8x2_to_bf16x2(d1, 0);
        o[3] = i8x2_to_bf16x2(d1, 16);
    } else if constexpr (FMT == W_Q4G64) {
        const uint2 q = r.p[rb];
        const uint32_t d0 = ls ? q.y : q.x;
        const uint32_t xq = d0 ^ 0x88888888u;
        // The and-or takes at most one scalar operand on this target: the mask
        // stays uniform, the constant 1.0 pair is moved to a vector register
        // (a plain VALU move, consumed by VALU instructions only), so the
        // compiler emits one v_and_or_b32 per pair instead of an and and an or.
        const uint32_t mask = __builtin_amdgcn_readfirstlane(Q4_MANT);
        uint32_t one;
        asm("v_mov_b32 %0, %1" : "=v"(one) : "s"(__builtin_amdgcn_readfirstlane(Q4_ONE)));
#pragma unroll
        for (int i = 0; i < 4; ++i)
            o[i] = BIAS ? (PK ? q4_packed_pair(d0, i, mask, one) : q4_natural_pair(d0, i))
                        : (PK ? q4_packed_exact_pair(xq, i) : i4x2_to_bf16x2(d0, 8 * i));
    } else if constexpr (FMT == W_Q8G32) {
        const uint2 q = r.p[2 * rb + ls];
        o[0] = i8x2_to_bf16x2(q.x, 0);
        o[1] = i8x2_to_bf16x2(q.x, 16);
        o[2] = i8x2_to_bf16x2(q.y, 0);
        o[3] = i8x2_to_bf16x2(q.y, 16);
    } else {  // W_BF16
        const uint4 q = r.p[2 * rb + ls];
        o[0] = q.x; o[1] = q.y; o[2] = q.z; o[3] = q.w;
    }
    return __builtin_bit_cast(v8bf, make_uint4(o[0], o[1], o[2], o[3]));
}

// One chunk of one wave: xrow(cb) gives the LDS element index of the B
// fragment row for token block cb (lane's token), kl the chunk's first column
// in the LDS activation rows, scs / sbase the group scales of the chunk.  The
// weights are in fragment order (rowmajor_to_frag already applied).
template <int FMT, int NCB, bool PK>
__device__ __forceinline__ void chunk_mfma(const WChunk<FMT>& wc, const uint16_t* xs, const int (&xrow)[NCB], int kl,
                                           const uint16_t* scs, int sgroup0, int wv, int lg,
                                           v4f (&acc)[4][NCB]) {
    constexpr int GS = group_size<FMT>();
    if constexpr (GS == 0) {
#pragma unroll
        for (int ls = 0; ls < 2; ++ls) {
            const int col = kl + kstep_col<FMT>(2 * wv + ls, lg);
            v8bf b[NCB];
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) b[cb] = *reinterpret_cast<const v8bf*>(&xs[xrow[cb] + col]);
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const v8bf a = decode_afrag<FMT>(wc, rb, ls);
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
                    acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[cb], acc[rb][cb], 0, 0, 0);
            }
        }
    } else {
        // GS == 64: the wave's two k-steps are one group; GS == 32: each k-step is one.
        constexpr int NGW = 64 / GS;                     // groups per wave and chunk
        if constexpr (FMT == W_Q4G64) {
            // Biased Q4 weights (1.5 + q / 16, see decode_afrag), every token
            // block: the bias is removed inside the matrix unit.  C = -1.5 sum x
            // over the group comes from two MFMAs of a fragment of -1.5s
            // against the activations (once per token block, shared by the
            // row blocks), and each row block's chain starts from C, so it ends
            // at sum x (1.5 + q / 16) - 1.5 sum x = sum x q / 16 (the factor 16
            // is applied once per wave, q4_bias_finish).  The group scale is
            // then one FMA per element.
            v8bf b[2][NCB];
#pragma unroll
            for (int ls = 0; ls < 2; ++ls) {
                const int col = kl + kstep_col<FMT>(2 * wv + ls, lg);
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) b[ls][cb] = *reinterpret_cast<const v8bf*>(&xs[xrow[cb] + col]);
            }
            const v8bf neg = __builtin_bit_cast(v8bf, make_uint4(Q4_NEG15, Q4_NEG15, Q4_NEG15, Q4_NEG15));
            v4f c0[NCB];
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                c0[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(neg, b[0][cb], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                c0[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(neg, b[1][cb], c0[cb], 0, 0, 0);
            }
            const int gi = sgroup0 + wv;
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const v8bf a0 = decode_afrag<FMT, PK, true>(wc, rb, 0);
                const v8bf a1 = decode_afrag<FMT, PK, true>(wc, rb, 1);
                const uint2 s4 = *reinterpret_cast<const uint2*>(&scs[gi * GV_ROWS + 16 * rb + 4 * lg]);
                const float sc[4] = {f16_bits_to_f32(s4.x & 0xFFFFu), f16_bits_to_f32(s4.x >> 16),
                                     f16_bits_to_f32(s4.y & 0xFFFFu), f16_bits_to_f32(s4.y >> 16)};
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    v4f d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b[0][cb], c0[cb], 0, 0, 0);
                    d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b[1][cb], d, 0, 0, 0);
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[rb][cb][e] = fmaf(d[e], sc[e], acc[rb][cb][e]);
                }
            }
        } else if constexpr (NGW == 1) {
            // GS == 64: row blocks in two pairs, the pair's chains interleaved;
            // 2 NCB group sums are live at a time (not 4 NCB), which keeps the
            // four-token-block build within 256 registers (two waves per SIMD).
            v8bf b[2][NCB];
#pragma unroll
            for (int ls = 0; ls < 2; ++ls) {
                const int col = kl + kstep_col<FMT>(2 * wv + ls, lg);
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) b[ls][cb] = *reinterpret_cast<const v8bf*>(&xs[xrow[cb] + col]);
            }
            const int gi = sgroup0 + wv;
#pragma unroll
            for (int rp = 0; rp < 2; ++rp) {
                v4f d[2][NCB];
#pragma unroll
                for (int ls = 0; ls < 2; ++ls)
#pragma unroll
                    for (int r = 0; r < 2; ++r) {
                        const v8bf a = decode_afrag<FMT, PK, false>(wc, 2 * rp + r, ls);
#pragma unroll
                        for (int cb = 0; cb < NCB; ++cb)
                            d[r][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                a, b[ls][cb], ls == 0 ? v4f{0.f, 0.f, 0.f, 0.f} : d[r][cb], 0, 0, 0);
                    }
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    const int rb = 2 * rp + r;
                    const uint2 s4 = *reinterpret_cast<const uint2*>(&scs[gi * GV_ROWS + 16 * rb + 4 * lg]);
                    const float sc[4] = {f16_bits_to_f32(s4.x & 0xFFFFu), f16_bits_to_f32(s4.x >> 16),
                                         f16_bits_to_f32(s4.y & 0xFFFFu), f16_bits_to_f32(s4.y >> 16)};
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[rb][cb][e] = fmaf(d[r][cb][e], sc[e], acc[rb][cb][e]);
                }
            }
        } else {
            v4f d[4][NCB];
#pragma unroll
            for (int ls = 0; ls < 2; ++ls) {
                const int col = kl + kstep_col<FMT>(2 * wv + ls, lg);
                v8bf b[NCB];
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) b[cb] = *reinterpret_cast<const v8bf*>(&xs[xrow[cb] + col]);
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    const v8bf a = decode_afrag<FMT, PK, false>(wc, rb, ls);
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) {
                        const v4f c0 = (NGW == 2 || ls == 0) ? v4f{0.f, 0.f, 0.f, 0.f} : d[rb][cb];
                        d[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[cb], c0, 0, 0, 0);
                    }
                }
                if (NGW == 2 || ls == 1) {
                    const int gi = sgroup0 + (NGW == 2 ? 2 * wv + ls : wv);
#pragma unroll
                    for (int rb = 0; rb < 4; ++rb) {
                        const uint2 s4 = *reinterpret_cast<const uint2*>(&scs[gi * GV_ROWS + 16 * rb + 4 * lg]);
                        const float sc[4] = {f16_bits_to_f32(s4.x & 0xFFFFu), f16_bits_to_f32(s4.x >> 16),
                                             f16_bits_to_f32(s4.y & 0xFFFFu), f16_bits_to_f32(s4.y >> 16)};
#pragma unroll
                        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                            for (int e = 0; e < 4; ++e) acc[rb][cb][e] = fmaf(d[rb][cb][e], sc[e], acc[rb][cb][e]);
                    }
                }
            }
        }
    }
}

// The factor 16 of the biased Q4 sums (see chunk_mfma), once per wave.
template <int FMT, int NCB>
__device__ __forceinline__ void q4_bias_finish(v4f (&acc)[4][NCB]) {
    if constexpr (FMT == W_Q4G64)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) acc[rb][cb] *= 16.0f;
}

// Sum the four waves' partials of row block wv in wave order through LDS
// (red: 16 KiB per token block, 16-byte aligned; the caller's LDS reads of the
// main loop must be finished, which the leading barrier guarantees).
template <int NCB>
__device__ __forceinline__ void reduce_waves(v4f (&acc)[4][NCB], v4f (&fin)[NCB], v4f* red, int wv, int lane) {
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) red[((wv * 4 + rb) * NCB + cb) * 64 + lane] = acc[rb][cb];
    __syncthreads();
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        v4f s = red[((0 * 4 + wv) * NCB + cb) * 64 + lane];
#pragma unroll
        for (int w2 = 1; w2 < 4; ++w2) s += red[((w2 * 4 + wv) * NCB + cb) * 64 + lane];
        fin[cb] = s;
    }
}

// reduce_waves for the waves with `mine` set: the barriers are the whole
// workgroup's, the writes and sums only theirs.
template <int NCB>
__device__ __forceinline__ void reduce_waves_half(v4f (&acc)[4][NCB], v4f (&fin)[NCB], v4f* red, int wv, int lane,
                                                  bool mine) {
    __syncthreads();
    if (mine) {
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) red[((wv * 4 + rb) * NCB + cb) * 64 + lane] = acc[rb][cb];
    }
    __syncthreads();
    if (mine) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            v4f s = red[((0 * 4 + wv) * NCB + cb) * 64 + lane];
#pragma unroll
            for (int w2 = 1; w2 < 4; ++w2) s += red[((w2 * 4 + wv) * NCB + cb) * 64 + lane];
            fin[cb] = s;
        }
    }
}

// reduce_waves for sums held transposed, as MFMAs with the activations in the
// A operand leave them (lane 16 g + i: tokens 4 g + e of row i): each value is
// first written to its place in the usual layout (lane 16 g' + i': rows
// 4 g' + e' of token i'), then the waves' sums are added alike.
template <int NCB>
__device__ __forceinline__ void reduce_waves_t(v4f (&acc)[4][NCB], v4f (&fin)[NCB], v4f* red, int wv, int lane) {
    const int li = lane & 15, lg = lane >> 4;
    float* rf = reinterpret_cast<float*>(red);
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                rf[(((wv * 4 + rb) * NCB + cb) * 64 + (li >> 2) * 16 + 4 * lg + e) * 4 + (li & 3)] = acc[rb][cb][e];
    __syncthreads();
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        v4f s = red[((0 * 4 + wv) * NCB + cb) * 64 + lane];
#pragma unroll
        for (int w2 = 1; w2 < 4; ++w2) s += red[((w2 * 4 + wv) * NCB + cb) * 64 + lane];
        fin[cb] = s;
    }
}

// FP32 partials between workgroups: 16-byte buffer stores and loads with the
// cache policy the compiler gives an agent-scope atomic access (sc1), so they
// bypass the per-XCD L2, which is not coherent across XCDs.  Ordering comes
// from the exchange protocol: stores complete (s_waitcnt) before the counter
// moves, loads are issued after the counter is seen.
constexpr int CPOL_DEVICE = 16;    // sc1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t partial_rsrc(float* p) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, 0x7FFFFFF0, BUF_FLAGS);
}
__device__ __forceinline__ void store_partial(__amdgpu_buffer_rsrc_t r, int64_t idx, v4f v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v), r, (int)(idx * 4), 0, CPOL_DEVICE);
}
// An element index whose byte offset lies past the partial buffer's range:
// a load of it reads zeros.
constexpr int64_t PARTIAL_OOB = 0x7FFFFFF0 / 4;
__device__ __forceinline__ v4f load_partial(__amdgpu_buffer_rsrc_t r, int64_t idx) {
    return __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(r, (int)(idx * 4), 0, CPOL_DEVICE));
}

// BF16 row scales of rows n0 .. n0 + 3 as FP32 (row-FP8; the other formats
// need none).  Four 2-byte buffer loads with no branch between them, so they
// are in flight together; rows past N read as zero (never written).  Loaded
// once per lane before the token blocks' writes: guarded loads per write
// would each wait for memory, NCB x 4 round trips at the end of every tile.
template <int FMT>
__device__ __forceinline__ v4f row_scales(const void* __restrict__ scales, int64_t n0, int N) {
    v4f s = v4f{1.f, 1.f, 1.f, 1.f};
    if constexpr (FMT == W_FP8ROW) {
        const __amdgpu_buffer_rsrc_t r =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(scales), (short)0, N * 2, BUF_FLAGS);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            s[i] = bf16_bits_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, (int)((n0 + i) * 2), 0, 0));
    }
    return s;
}

// Output rows n0 .. n0 + 3 of token t from FP32 values v; rsc from
// row_scales (row-FP8: the row scale is applied here).
template <int FMT>
__device__ __forceinline__ void write_rows(v4f v, int t, int64_t n0, v4f rsc, int T, int N, int bf16_out,
                                           void* __restrict__ y) {
    if (t >= T) return;
    if constexpr (FMT == W_FP8ROW) {
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = v[r] * rsc[r];
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
}

// Output of row block wv: the FP32 values fin (row-FP8 scale applied here),
// either written to y or, with splits > 1, published as a partial and summed
// by the last workgroup of the tile.
template <int FMT, int NCB>
__device__ __forceinline__ void finish_tile(v4f (&fin)[NCB], const void* __restrict__ scales, int T, int N,
                                            int64_t row0, int wv, int lane, int tile, int split, int splits,
                                            float* __restrict__ partial, unsigned* __restrict__ counters,
                                            int bf16_out, void* __restrict__ y, int* s_last) {
    const int li = lane & 15, lg = lane >> 4;
    const int tid = threadIdx.x;
    const int64_t npad = (int64_t)gridDim.x * GV_ROWS;
    const int64_t n0 = row0 + wv * 16 + 4 * lg;           // this lane's 4 output rows
    const v4f rsc = row_scales<FMT>(scales, n0, N);
    auto write_out = [&](int cb, v4f v) { write_rows<FMT>(v, cb * 16 + li, n0, rsc, T, N, bf16_out, y); };

    if (splits == 1) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) write_out(cb, fin[cb]);
        return;
    }

    // Split-K: publish this split's partial; the last workgroup of the tile sums.
    // Partials move only through device-coherent stores and loads (see
    // store_partial); each wave waits for its stores to complete before the
    // counter is bumped.  No device-scope fence: on this part it would write
    // back and invalidate the whole L2.
    const __amdgpu_buffer_rsrc_t pr = partial_rsrc(partial);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        const int t = cb * 16 + li;
        if (t < T) store_partial(pr, ((int64_t)split * T + t) * npad + n0, fin[cb]);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) {
        const unsigned prev = __hip_atomic_fetch_add(&counters[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_last = (prev == (unsigned)(splits - 1));
    }
    __syncthreads();
    if (!*s_last) return;
    // The loads of a batch of splits, for all token blocks, are in flight
    // together (one memory round trip per batch; tokens past T and splits past
    // the last read as zero through out-of-range offsets, so no branch sits
    // between them); each token block's sum runs in split order.
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
            for (int j = 0; j < SB; ++j)
                part[cb][j] = load_partial(pr, (t < T && sb + j < splits) ? ((int64_t)(sb + j) * T + t) * npad + n0
                                                                         : PARTIAL_OOB);
        }
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int j = 0; j < SB; ++j)
                if (sb + j < splits) sum[cb] += part[cb][j];
    }
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) write_out(cb, sum[cb]);
    if (tid == 0) __hip_atomic_store(&counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Spread workgroups (see gemv_direct_kernel, gemv_mfma_kernel): workgroup e
// of E owns the units [e U / E, (e + 1) U / E) of the leftover tiles
// [tile0, tile0 + R) (U = R x chunks, one unit = one chunk of one tile,
// tile-major; E <= U so no range is empty).  Activation fragments come
// straight from memory as in the direct kernel.  When the range leaves a tile
// (and at its end) the tile's sums are added across the waves and published
// as an FP32 partial in slot (e - first workgroup of the tile), or written
// directly when the range covers the tile; the last workgroup of a tile to
// arrive (atomic counter) adds the slots in slot order, so the result does
// not depend on timing.  A spread workgroup runs a few units, so the
// boundary work (which waits for its loads) costs little.
constexpr int SPREAD_MAXSEG = 3;

// The spread workgroup whose range holds leftover unit v.
__device__ __forceinline__ int spread_owner(int64_t v, int64_t U, int E) { return (int)(((v + 1) * E - 1) / U); }

template <int FMT, int NCB, bool PK, bool NT = false>
__device__ __forceinline__ void direct_spread(const uint8_t* __restrict__ w, const void* __restrict__ scales,
                                              const uint16_t* __restrict__ x, int T, int N, int64_t K, int tile0,
                                              int R, int e, int E, int maxslots, float* __restrict__ partial,
                                              unsigned* __restrict__ counters, int bf16_out, void* __restrict__ y,
                                              v4f* red, int* s_last) {
    using P = PieceFmt<FMT>;
    constexpr int D = 2;
    constexpr int GS = group_size<FMT>();
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int li = lane & 15;
    const int lg = lane >> 4;
    const int C = (int)(K / GV_KC);
    const int64_t U = (int64_t)R * C;
    const int64_t u0 = (int64_t)e * U / E, u1 = (int64_t)(e + 1) * U / E;
    const int nu = (int)(u1 - u0);
    const int lt0 = (int)(u0 / C);                           // first leftover tile touched (local index)
    const int nseg = (int)((u1 - 1) / C) - lt0 + 1;

    const int64_t nrb = ((int64_t)N + 15) / 16;
    const int64_t cstride = PK ? nrb * P::BLOCK_CHUNK : 0;
    const int q0 = P::PW * wv;
    const uint8_t* wlane = w + (int64_t)lane * P::PB;     // packed: the lane's piece within a block chunk
    const __amdgpu_buffer_rsrc_t xrsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, (int)((int64_t)T * K * 2), BUF_FLAGS);
    const __amdgpu_buffer_rsrc_t pr = partial_rsrc(partial);
    int xoff[2][NCB];
#pragma unroll
    for (int ls = 0; ls < 2; ++ls)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
            xoff[ls][cb] = (int)(((int64_t)(cb * 16 + li) * K + kstep_col<FMT>(2 * wv + ls, lg)) * 2);

    struct XFrag {
        uint4 v[2][NCB];
    };
    WChunk<FMT> wr[D];
    XFrag xr[D];
    // formats with group scales: per row block, the scales of the lane's row
    // for the wave's groups of the unit's chunk (GS = 64: one; GS = 32: two)
    uint32_t sr[D][4];
    // (tile, chunk) of the next unit to load (stops at the last unit) and the
    // chunk of the next unit to compute
    int ld_t = tile0 + lt0, ld_c = (int)(u0 - (int64_t)lt0 * C), ld_i = 0;
    int cp_c = ld_c, cp_i = 0;
    auto load = [&](int slot) {
        const int tl = ld_t, c = ld_c;
        if (ld_i < nu - 1) {
            ++ld_i;
            if (++ld_c == C) {
                ld_c = 0;
                ++ld_t;
            }
        }
#pragma unroll
        for (int ls = 0; ls < 2; ++ls)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
                xr[slot].v[ls][cb] = __builtin_bit_cast(
                    uint4, __builtin_amdgcn_raw_buffer_load_b128(xrsrc, xoff[ls][cb] + c * (GV_KC * 2), 0, 0));
#pragma unroll
        for (int j = 0; j < 4 * P::PW; ++j) {
            const int rb = j / P::PW;
            const int q = q0 + j % P::PW;
            const int64_t rowb = (int64_t)tl * GV_ROWS + 16 * rb;             // first row of the row block
            const uint8_t* pw;
            int64_t row = 0;
            if constexpr (PK) {
                const int64_t rbg = rowb / 16 < nrb - 1 ? rowb / 16 : nrb - 1;   // blocks past N are clamped
                pw = wlane + (rbg * P::BLOCK_CHUNK + (int64_t)c * cstride + q * (64 * P::PB));
            }
            if constexpr (FMT == W_MXFP8 || GS != 0) {     // the lane's fragment row (scales)
                const int64_t lim = (int64_t)N - 1 - rowb;                   // rows past N are clamped
                const int lr = (int64_t)li < lim ? li : (int)lim;
                row = rowb + lr;
            }
            if constexpr (!PK) {
                // four lanes per row (see rowmajor_to_frag)
                const int64_t lim = (int64_t)N - 1 - rowb;
                const int lc = (int64_t)(lane >> 2) < lim ? (lane >> 2) : (int)lim;
                pw = w + (rowb + lc) * row_bytes<FMT>(K) + piece_offset<FMT>(c, q, lane & 3);
            }
            if constexpr (PK && NT) ld_nt(wr[slot].p[j], pw);
            else wr[slot].p[j] = *reinterpret_cast<const typename P::Piece*>(pw);
            if constexpr (GS != 0) {
                if (j % P::PW == 0) {
                    // the wave's columns [64 wv, 64 wv + 64) of chunk c are group 4 c + wv
                    // (GS = 64) or groups 8 c + 2 wv + {0, 1} (GS = 32)
                    const uint16_t* s16 = reinterpret_cast<const uint16_t*>(scales) + row * (K / GS);
                    if constexpr (GS == 64) sr[slot][rb] = s16[4 * c + wv];
                    else sr[slot][rb] = *reinterpret_cast<const uint32_t*>(s16 + 8 * c + 2 * wv);
                }
            }
            if constexpr (FMT == W_MXFP8)
                wr[slot].e8[j] = reinterpret_cast<const uint8_t*>(scales)[row * (K >> 5) +
                                                                          ((c * GV_KC + 64 * q + 16 * lg) >> 5)];
        }
    };

    auto seg_full = [&](int k) {        // segment k (leftover tile lt0 + k) covered whole by this range
        const int64_t tb = (int64_t)(lt0 + k) * C;
        const int64_t b = tb > u0 ? tb : u0, en = tb + C < u1 ? tb + C : u1;
        return en - b == C;
    };
    auto seg_slots = [&](int k) {       // this workgroup's slot and the tile's slot count
        const int64_t tb = (int64_t)(lt0 + k) * C;
        const int first = spread_owner(tb, U, E);
        return make_int2(e - first, spread_owner(tb + C - 1, U, E) - first + 1);
    };
    v4f acc[4][NCB];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) acc[rb][cb] = v4f{0.f, 0.f, 0.f, 0.f};
    // segment k's sums: written directly or published as a partial; acc restarts
    auto close_segment = [&](int k) {
        v4f fin[NCB];
        if constexpr (GS != 0) reduce_waves_t<NCB>(acc, fin, red, wv, lane);
        else reduce_waves<NCB>(acc, fin, red, wv, lane);
        const int tl = tile0 + lt0 + k;
        const int64_t n0 = (int64_t)tl * GV_ROWS + wv * 16 + 4 * lg;
        if (seg_full(k)) {
            const v4f rsc = row_scales<FMT>(scales, n0, N);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) write_rows<FMT>(fin[cb], cb * 16 + li, n0, rsc, T, N, bf16_out, y);
        } else {
            const int slot = seg_slots(k).x;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                const int t = cb * 16 + li;
                if (t < T)
                    store_partial(pr, (((int64_t)(lt0 + k) * maxslots + slot) * T + t) * GV_ROWS + wv * 16 + 4 * lg,
                                  fin[cb]);
            }
        }
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) acc[rb][cb] = v4f{0.f, 0.f, 0.f, 0.f};
    };
    int kseg = 0;
    auto step = [&](int slot) {
        if (cp_c == 0 && cp_i > 0) close_segment(kseg++);   // this unit opens the next tile (uniform)
        ++cp_i;
        if (++cp_c == C) cp_c = 0;
        rowmajor_to_frag<FMT, PK>(wr[slot]);
        if constexpr (GS != 0) {
            // Group scales: the MFMAs take the activations as A and the
            // weights as B (both fragments hold the same k of their lane, so
            // the group sums are the same), which leaves lane 16 g + i the
            // sums of tokens 4 g + e of row i: one scale per row block and
            // group.  Q4 codes are decoded exactly here (no bias).
            constexpr int NGW = 64 / GS;
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const float sc[2] = {f16_bits_to_f32(sr[slot][rb] & 0xFFFFu), f16_bits_to_f32(sr[slot][rb] >> 16)};
                v4f d[NCB];
#pragma unroll
                for (int ls = 0; ls < 2; ++ls) {
                    const v8bf wf = decode_afrag<FMT, PK, false>(wr[slot], rb, ls);
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) {
                        const v4f c0 = (NGW == 2 || ls == 0) ? v4f{0.f, 0.f, 0.f, 0.f} : d[cb];
                        d[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, xr[slot].v[ls][cb]),
                                                                        wf, c0, 0, 0, 0);
                    }
                    if (NGW == 2 || ls == 1) {
                        const float g = sc[NGW == 2 ? ls : 0];
#pragma unroll
                        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                            for (int e = 0; e < 4; ++e) acc[rb][cb][e] = fmaf(d[cb][e], g, acc[rb][cb][e]);
                    }
                }
            }
        } else {
#pragma unroll
            for (int ls = 0; ls < 2; ++ls) {
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    const v8bf a = decode_afrag<FMT>(wr[slot], rb, ls);
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb)
                        acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            a, __builtin_bit_cast(v8bf, xr[slot].v[ls][cb]), acc[rb][cb], 0, 0, 0);
                }
            }
        }
    };

#pragma unroll
    for (int d = 0; d < D; ++d) load(d);
    int i = 0;
    for (; i + D <= nu; i += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
            step(u);
            load(u);
        }
    }
#pragma unroll
    for (int u = 0; u < D - 1; ++u)
        if (i + u < nu) step(u);
    close_segment(kseg);

    // Each wave waits for its partial stores before the counters move.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) {
        // all counters move before any result is looked at: one round trip
        unsigned prev[SPREAD_MAXSEG];
#pragma unroll
        for (int k = 0; k < SPREAD_MAXSEG; ++k)
            prev[k] = (k < nseg && !seg_full(k))
                          ? __hip_atomic_fetch_add(&counters[tile0 + lt0 + k], 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT)
                          : 0u;
#pragma unroll
        for (int k = 0; k < SPREAD_MAXSEG; ++k)
            s_last[k] = (k < nseg && !seg_full(k)) && prev[k] == (unsigned)(seg_slots(k).y - 1);
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < SPREAD_MAXSEG; ++k) {
        if (k >= nseg || !s_last[k]) continue;
        const int tl = tile0 + lt0 + k;
        const int nslots = seg_slots(k).y;
        const int64_t n0 = (int64_t)tl * GV_ROWS + wv * 16 + 4 * lg;
        const v4f rsc = row_scales<FMT>(scales, n0, N);
        // The loads of a batch of slots, for all token blocks, are in flight
        // together (one memory round trip per batch; tokens past T and slots
        // past the last read as zero through out-of-range offsets, so no
        // branch sits between them); each token block's sum runs in slot order.
        constexpr int SB = NCB == 1 ? 16 : 12;
        v4f sum[NCB];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) sum[cb] = v4f{0.f, 0.f, 0.f, 0.f};
        for (int sb = 0; sb < nslots; sb += SB) {
            v4f part[NCB][SB];
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                const int t = cb * 16 + li;
#pragma unroll
                for (int j = 0; j < SB; ++j) {
                    const int64_t idx = (((int64_t)(lt0 + k) * maxslots + sb + j) * T + t) * GV_ROWS + wv * 16 + 4 * lg;
                    part[cb][j] = load_partial(pr, (t < T && sb + j < nslots) ? idx : PARTIAL_OOB);
                }
            }
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                for (int j = 0; j < SB; ++j)
                    if (sb + j < nslots) sum[cb] += part[cb][j];
        }
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) write_rows<FMT>(sum[cb], cb * 16 + li, n0, rsc, T, N, bf16_out, y);
        if (tid == 0) __hip_atomic_store(&counters[tl], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ---------------------------------------------------------------------------
// Streaming variant: the activation chunk [16 NCB][256] is double-buffered in
// LDS (rows past T read as zero); the next chunk's activations are requested
// before the next weights so that waiting for them never waits for weights.
// One barrier per chunk.
// ---------------------------------------------------------------------------
// Waves per SIMD the streaming kernel is compiled for: two, so that a spread
// workgroup fits beside a whole-tile one on every CU (see direct_spread) and
// two K splits of a tile share a CU, except at four token blocks for BF16
// weights, which would spill at that budget, and for the grouped formats,
// which run no spread workgroups there and fit in 256 registers without the
// bound.  At two token blocks the two-wave budget measured faster for the
// grouped formats too (5120 x 17408, T = 17: Q4 23.4 -> 22.7 us packed,
// Q8 group-32 row-major 35.2 -> 33.0 us).
template <int FMT, int NCB>
constexpr int stream_min_waves() {
    return (NCB < 4 || (FMT != W_BF16 && group_size<FMT>() == 0)) ? 2 : 1;
}

// The builds with two row tiles per workgroup (the one-byte formats without
// group scales; eight waves on a CU's four SIMDs fit the two-wave register
// budget there).
template <int FMT, int NCB>
constexpr bool two_tile_format() {
    return (FMT == W_FP8ROW || FMT == W_MXFP8) && stream_min_waves<FMT, NCB>() == 2;
}

// With spread_wgs > 0 (one split; the grouped formats at one token block only): workgroups
// [0, spread_wgs) share the tiles [main_tiles, tiles) unit by unit
// (direct_spread) and the main_tiles after them take one whole tile each as
// below.  The spread workgroups come first so that they are dispatched first:
// their partial exchange then ends well inside the whole tiles' time.
//
// TH = 2 (formats without group scales, one K split, no spread workgroups,
// many tiles per CU): eight waves take two neighbouring row tiles, waves
// 4 h + q tile h and column quarter q, and share one activation stage, which
// halves the activation bytes staged per weight byte.
//
// WNT: non-temporal weight loads (packed weights; see launch_mfma).
//
// XSKIP (TH = 1, one token block, T <= 8): the second 8-row round of the
// activation staging holds no token, so it is not loaded; the B fragment
// rows of the lanes past the staged rows read one zero row instead (row 8 of
// each buffer, cleared once).  Loads of absent token rows read zero through
// the buffer bounds but cost the address unit as much as real ones
// (17408x5120 Q8G32 T = 1 / 8: 23.2 / 24.4 -> 21.6 / 22.5 us, 5120x17408
// 25.0 / 25.5 -> 22.2 / 22.5; row-FP8 T = 1 / 4 17.8 / 17.6 -> 17.4 / 17.3).
// Skipping the last round at three token blocks (T = 33..40) did not help
// row-FP8 and cost the grouped formats 1-4 %, so it is used at one block only.
template <int FMT, int NCB, bool PK, int TH = 1, bool XSKIP = false, bool WNT = false>
__global__ __launch_bounds__(256 * TH, (TH == 1 ? stream_min_waves<FMT, NCB>() : 2)) void gemv_mfma_kernel(
    const uint8_t* __restrict__ w, const void* __restrict__ scales, const uint16_t* __restrict__ x, int T, int N,
    int64_t K, int chunks_per_split, int splits, float* __restrict__ partial, unsigned* __restrict__ counters,
    int bf16_out, void* __restrict__ y, int main_tiles, int spread_wgs, int maxslots) {
    constexpr int TP = 16 * NCB;
    constexpr int XPITCH = GV_KC + 8;                 // bf16 per LDS row: rows shift by 4 banks
    constexpr int XPR = GV_KC / 8;                    // 16-byte activation pieces per row and chunk
    constexpr int NT = 256 * TH;                      // threads
    constexpr int XP = TP * XPR / NT;                 // ... per thread
    static_assert(!XSKIP || (TH == 1 && NCB == 1), "skipped staging round: one tile, one token block");
    constexpr int XPS = XSKIP ? XP - 1 : XP;          // staging rounds loaded
    constexpr int ZROW = XPS * NT / XPR;              // XSKIP: the zero row (first row not staged)
    constexpr int GS = group_size<FMT>();
    static_assert(TH == 1 || GS == 0, "two tiles per workgroup: formats without group scales");
    constexpr int NG = GS ? GV_KC / (GS ? GS : 1) : 1;   // scale groups per chunk
    constexpr int SP = GS ? (NG * GV_ROWS + 255) / 256 : 1;
    constexpr int D = depth<FMT, NCB>();
    // xs doubles as the buffer of the final cross-wave sum (16 KiB per token block)
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][TP * XPITCH];
    __shared__ __attribute__((aligned(16))) uint16_t scs[2][GS ? NG * GV_ROWS : 1];
    __shared__ int s_last;
    static_assert(sizeof(xs) >= 16384 * NCB, "reduction buffer");
    if constexpr ((GS == 0 || NCB == 1) && TH == 1) {
        __shared__ int s_last_sp[SPREAD_MAXSEG];
        if ((int)blockIdx.x < spread_wgs) {
            const int tiles_all = (int)((N + GV_ROWS - 1) / GV_ROWS);
            direct_spread<FMT, NCB, PK, WNT>(w, scales, x, T, N, K, main_tiles, tiles_all - main_tiles,
                                        (int)blockIdx.x, spread_wgs, maxslots, partial, counters,
                                        bf16_out, y, reinterpret_cast<v4f*>(&xs[0][0]), s_last_sp);
            return;
        }
    }

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = TH == 1 ? tid >> 6 : (tid >> 6) & 3;   // the wave's column quarter of a chunk
    const int half = TH == 1 ? 0 : tid >> 8;              // the wave's row tile of the TH
    const int li = lane & 15;
    const int lg = lane >> 4;
    const int tile = ((int)blockIdx.x - spread_wgs) * TH + half;   // spread workgroups come first
    // A whole tile's waves issue ahead of a spread workgroup's on the same CU
    // (these are younger, and equal priority favours the oldest wave): the
    // spread work then fills the cycles the tile leaves idle.
    if (spread_wgs > 0) __builtin_amdgcn_s_setprio(2);
    const int split = blockIdx.y;
    const int64_t row0 = (int64_t)tile * GV_ROWS;
    const int64_t total_chunks = K / GV_KC;
    const int64_t c_begin = (int64_t)split * chunks_per_split;
    int nch = (int)(total_chunks - c_begin);
    if (nch > chunks_per_split) nch = chunks_per_split;
    const int64_t k_begin = c_begin * GV_KC;

    const WSrc src = make_wsrc<FMT, PK>(w, scales, row0, N, K, lane, wv);

    // activations: rows >= T fall outside the buffer and read as zero
    const __amdgpu_buffer_rsrc_t xrsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, (int)((int64_t)T * K * 2), BUF_FLAGS);
    __amdgpu_buffer_rsrc_t srsrc = xrsrc;
    if constexpr (GS != 0)
        srsrc = __builtin_amdgcn_make_buffer_rsrc((void*)scales, (short)0, (int)((int64_t)N * (K / GS) * 2),
                                                  BUF_FLAGS);

    // Activations (and group scales) of a chunk are loaded into registers D
    // chunks ahead, in the same order as the chunk's weights, and stored to
    // LDS one chunk ahead of use: waiting for them then never waits for more
    // than the weights the current chunk needs anyway.
    // WSC (group-64 formats in the XSKIP build): the chunk's group scales come
    // from one 8-byte load per row by wave 0 instead of one 2-byte load per
    // scale by every thread (four load instructions per chunk down to one;
    // two comparisons in separate runs, T = 1 / 8: Q4G64 17408x5120 14.8 /
    // 15.6 -> 14.0 / 15.5 us and 14.5 / 15.4 -> 14.3 / 15.6, 5120x17408 16.3 /
    // 16.8 -> 15.3 / 15.7 and 16.1 / 16.7 -> 15.7 / 16.2, Q8G64 -2..3 %; in the
    // other builds the branch made the compiler spill, 2-5x slower with the
    // 16-byte form for group-32 scales).
    constexpr bool WSC = GS == 64 && XSKIP;
    uint4 xreg[D][XP];
    uint32_t sreg[D][WSC ? 2 : SP];
    const int wv_s = __builtin_amdgcn_readfirstlane(tid >> 6);
    auto load_x = [&](int slot, int c) {
        const int64_t kc0 = k_begin + (int64_t)c * GV_KC;
#pragma unroll
        for (int j = 0; j < XPS; ++j) {
            const int idx = tid + NT * j;
            const int t = idx / XPR, pc = idx % XPR;
            const int off = (int)(((int64_t)t * K + kc0 + 8 * pc) * 2);
            xreg[slot][j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xrsrc, off, 0, 0));
        }
        if constexpr (WSC) {
            // wave 0 only: lane r loads row row0 + r's four scales of the
            // chunk (contiguous 8 bytes) in one load; rows >= N read as zero
            if (wv_s == 0) {
                const int64_t row = row0 + lane;
                const int off = (int)((row * (K / GS) + kc0 / GS) * 2);
                const v2u v = __builtin_bit_cast(v2u, __builtin_amdgcn_raw_buffer_load_b64(srsrc, off, 0, 0));
                sreg[slot][0] = v[0];
                sreg[slot][1] = v[1];
            }
        } else if constexpr (GS != 0) {
#pragma unroll
            for (int j = 0; j < SP; ++j) {
                const int idx = tid + 256 * j;          // idx = row * NG + group
                const int r = idx / NG, gi = idx % NG;
                const int64_t row = row0 + r;           // rows >= N read as zero
                const int off = (int)((row * (K / GS) + kc0 / GS + gi) * 2);
                sreg[slot][j] = __builtin_amdgcn_raw_buffer_load_b16(srsrc, off, 0, 0);
            }
        }
    };
    auto store_x = [&](int buf, int slot) {
#pragma unroll
        for (int j = 0; j < XPS; ++j) {
            const int idx = tid + NT * j;
            const int t = idx / XPR, pc = idx % XPR;
            *reinterpret_cast<uint4*>(&xs[buf][t * XPITCH + 8 * pc]) = xreg[slot][j];
        }
        if constexpr (WSC) {
            if (wv_s == 0) {
#pragma unroll
                for (int g = 0; g < NG; ++g)
                    scs[buf][g * GV_ROWS + lane] = (uint16_t)(sreg[slot][g >> 1] >> (16 * (g & 1)));
            }
        } else if constexpr (GS != 0) {
#pragma unroll
            for (int j = 0; j < SP; ++j) {
                const int idx = tid + 256 * j;
                if (SP * 256 == NG * GV_ROWS || idx < NG * GV_ROWS)
                    scs[buf][(idx % NG) * GV_ROWS + idx / NG] = (uint16_t)sreg[slot][j];
            }
        }
    };

    v4f acc[4][NCB];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) acc[rb][cb] = v4f{0.f, 0.f, 0.f, 0.f};
    int xrow[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) xrow[cb] = (XSKIP && cb * 16 + li > ZROW ? ZROW : cb * 16 + li) * XPITCH;
    if constexpr (XSKIP) {     // the zero row of both buffers (threads 0..63), before the first barrier
        if (tid < 64)
            *reinterpret_cast<uint4*>(&xs[tid >> 5][ZROW * XPITCH + 8 * (tid & 31)]) = make_uint4(0u, 0u, 0u, 0u);
    }

    // One chunk c (c = u mod D): compute from ring slot u and LDS buffer c & 1,
    // stage the activations of chunk c + 1 (register slot (u + 1) mod D),
    // request activations and weights of chunk c + D into slot u (indices
    // clamped to the last chunk, so the body has no branch), barrier.
    WChunk<FMT> ring[D];
    auto body = [&](int c, int u) {
        const int buf = c & 1;
        rowmajor_to_frag<FMT, PK>(ring[u]);
        chunk_mfma<FMT, NCB, PK>(ring[u], xs[buf], xrow, 0, scs[buf], 0, wv, lg, acc);
        store_x((c + 1) & 1, (u + 1) % D);
        load_x(u, min(c + D, nch - 1));
        load_chunk<FMT, PK, WNT>(ring[u], src, c_begin + min(c + D, nch - 1));
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
    };

    if (nch > 0) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            load_x(d, min(d, nch - 1));
            load_chunk<FMT, PK, WNT>(ring[d], src, c_begin + min(d, nch - 1));
        }
        store_x(0, 0);
        __syncthreads();
        int c = 0;
        for (; c + D <= nch; c += D) {
#pragma unroll
            for (int u = 0; u < D; ++u) body(c + u, u);
        }
#pragma unroll
        for (int u = 0; u < D - 1; ++u)
            if (c + u < nch) body(c + u, u);
    }

    v4f fin[NCB];
    q4_bias_finish<FMT, NCB>(acc);
    if constexpr (TH == 1) {
        reduce_waves<NCB>(acc, fin, reinterpret_cast<v4f*>(&xs[0][0]), wv, lane);
    } else {
        // the two tiles' sums in turn through the one buffer
#pragma unroll
        for (int h = 0; h < TH; ++h) {
            v4f fh[NCB];
            reduce_waves_half<NCB>(acc, fh, reinterpret_cast<v4f*>(&xs[0][0]), wv, lane, half == h);
            if (half == h)
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) fin[cb] = fh[cb];
        }
    }
    finish_tile<FMT, NCB>(fin, scales, T, N, row0, wv, lane, tile, split, splits, partial, counters, bf16_out, y,
                          &s_last);
}

// ---------------------------------------------------------------------------
// Resident-activation variant: when the workgroup's activation slice
// [T][k range] (and its rows' group scales) fits in LDS, it is staged once and
// the waves then stream weights with no barrier at all, each with its own
// register ring of 3 chunks (4 for MXFP8, whose scale loads are small).  Deeper
// rings were measured slower: more bytes in flight per wave only lengthens the
// memory queues and spreads the waves' finishing times.  B fragments of tokens
// t >= T read a zero row.
// ---------------------------------------------------------------------------
template <int FMT>
constexpr int depth_resident() {
    return FMT == W_MXFP8 ? 4 : 3;
}

template <int FMT, int NCB, bool PK>
__global__ __launch_bounds__(256) void gemv_resident_kernel(const uint8_t* __restrict__ w,
                                                            const void* __restrict__ scales,
                                                            const uint16_t* __restrict__ x, int T, int N,
                                                            int64_t K, int chunks_per_split, int splits,
                                                            float* __restrict__ partial,
                                                            unsigned* __restrict__ counters, int bf16_out,
                                                            void* __restrict__ y) {
    constexpr int GS = group_size<FMT>();
    constexpr int D = depth_resident<FMT>();
    // The dynamic LDS also holds the final cross-wave sum (16 KiB per token block).
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    __shared__ int s_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int li = lane & 15;
    const int lg = lane >> 4;
    const int tile = blockIdx.x;
    const int split = blockIdx.y;
    const int64_t row0 = (int64_t)tile * GV_ROWS;
    const int64_t total_chunks = K / GV_KC;
    const int64_t c_begin = (int64_t)split * chunks_per_split;
    int nch = (int)(total_chunks - c_begin);
    if (nch > chunks_per_split) nch = chunks_per_split;
    const int64_t k_begin = c_begin * GV_KC;
    const int krange = nch * GV_KC;
    const int xpitch = chunks_per_split * GV_KC + 8;      // bf16 per LDS row (rows shift by 4 banks)
    uint16_t* xs = lds;                                    // [T + 1][xpitch], row T is zero
    uint16_t* scs = lds + (T + 1) * xpitch;                // [groups of the slice][64 rows]

    const WSrc src = make_wsrc<FMT, PK>(w, scales, row0, N, K, lane, wv);

    // the first weight chunks are requested before the activations are staged
    WChunk<FMT> ring[D];
    if (nch > 0) {
#pragma unroll
        for (int d = 0; d < D; ++d) load_chunk<FMT, PK>(ring[d], src, c_begin + min(d, nch - 1));
    }

    // stage activations (16-byte pieces), the zero row and the group scales
    {
        const int pieces = krange / 8;
        for (int i = tid; i < (T + 1) * pieces; i += 256) {
            const int t = i / pieces, pc = i - t * pieces;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (t < T) v = *reinterpret_cast<const uint4*>(x + (int64_t)t * K + k_begin + 8 * pc);
            *reinterpret_cast<uint4*>(&xs[t * xpitch + 8 * pc]) = v;
        }
        if constexpr (GS != 0) {
            const uint16_t* sc16 = reinterpret_cast<const uint16_t*>(scales);
            const int ng = krange / GS;
            for (int i = tid; i < ng * GV_ROWS; i += 256) {
                const int r = i / ng, gi = i - r * ng;
                int64_t row = row0 + r;
                if (row >= N) row = N - 1;
                scs[gi * GV_ROWS + r] = sc16[row * (K / GS) + k_begin / GS + gi];
            }
        }
        __syncthreads();
    }

    v4f acc[4][NCB];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) acc[rb][cb] = v4f{0.f, 0.f, 0.f, 0.f};
    int xrow[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) xrow[cb] = min(cb * 16 + li, T) * xpitch;

    auto compute = [&](WChunk<FMT>& wc, int c) {
        rowmajor_to_frag<FMT, PK>(wc);
        chunk_mfma<FMT, NCB, PK>(wc, xs, xrow, c * GV_KC, scs, GS ? c * GV_KC / (GS ? GS : 1) : 0, wv, lg, acc);
    };

    if (nch > 0) {
        int c = 0;
        for (; c + D <= nch; c += D) {
#pragma unroll
            for (int u = 0; u < D; ++u) {
                compute(ring[u], c + u);
                load_chunk<FMT, PK>(ring[u], src, c_begin + min(c + u + D, nch - 1));
                // keep each refill right after the compute that frees its slot
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int u = 0; u < D - 1; ++u)
            if (c + u < nch) compute(ring[u], c + u);
    }

    v4f fin[NCB];
    q4_bias_finish<FMT, NCB>(acc);
    reduce_waves<NCB>(acc, fin, reinterpret_cast<v4f*>(lds), wv, lane);
    finish_tile<FMT, NCB>(fin, scales, T, N, row0, wv, lane, tile, split, splits, partial, counters, bf16_out, y,
                          &s_last);
}

// ---------------------------------------------------------------------------
// Direct variant (formats without group scales): each wave loads the
// activation fragments of its own k-steps straight from memory (L2: the
// activations are small and read by every workgroup) into the same register
// ring as its weights, so nothing is staged in LDS, no barrier runs in the
// loop, and waiting for a chunk never waits for anything but that chunk.
// Tokens t >= T lie outside the activation buffer and read as zero.
// ---------------------------------------------------------------------------
template <int NCB>
constexpr int depth_direct() {
    return NCB >= 3 ? 2 : 3;
}

// With spread_wgs > 0 (and one split): workgroups [0, spread_wgs) share the
// tiles [main_tiles, tiles) unit by unit (direct_spread), dispatched first so
// that their partial exchange ends well inside the whole tiles' time, and the
// main_tiles workgroups after them each take one whole tile as below.  With more tiles
// than CUs but not a multiple of them, whole tiles alone leave a few CUs with
// one tile more and the launch takes nearly twice as long; the spread
// workgroups (a few units each, resident beside the whole-tile ones) even the
// CUs out, and their partial exchange ends long before the whole tiles do.
template <int FMT, int NCB, bool PK, bool NT = false>
__global__ __launch_bounds__(256) void gemv_direct_kernel(const uint8_t* __restrict__ w,
                                                          const void* __restrict__ scales,
                                                          const uint16_t* __restrict__ x, int T, int N, int64_t K,
                                                          int chunks_per_split, int splits,
                                                          float* __restrict__ partial,
                                                          unsigned* __restrict__ counters, int bf16_out,
                                                          void* __restrict__ y, int main_tiles, int spread_wgs,
                                                          int maxslots) {
    static_assert(group_size<FMT>() == 0, "grouped formats stage their scales in LDS");
    constexpr int D = depth_direct<NCB>();
    __shared__ __attribute__((aligned(16))) v4f red[4 * 4 * NCB * 64];   // final cross-wave sum
    __shared__ int s_last;
    __shared__ int s_last_sp[SPREAD_MAXSEG];
    if ((int)blockIdx.x < spread_wgs) {
        const int tiles_all = (int)((N + GV_ROWS - 1) / GV_ROWS);
        direct_spread<FMT, NCB, PK, NT>(w, scales, x, T, N, K, main_tiles, tiles_all - main_tiles,
                                    (int)blockIdx.x, spread_wgs, maxslots, partial, counters, bf16_out,
                                    y, red, s_last_sp);
        return;
    }

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int li = lane & 15;
    const int lg = lane >> 4;
    const int tile = (int)blockIdx.x - spread_wgs;   // spread workgroups come first
    const int split = blockIdx.y;
    const int64_t row0 = (int64_t)tile * GV_ROWS;
    const int64_t total_chunks = K / GV_KC;
    const int64_t c_begin = (int64_t)split * chunks_per_split;
    int nch = (int)(total_chunks - c_begin);
    if (nch > chunks_per_split) nch = chunks_per_split;

    const WSrc src = make_wsrc<FMT, PK>(w, scales, row0, N, K, lane, wv);
    const __amdgpu_buffer_rsrc_t xrsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, (int)((int64_t)T * K * 2), BUF_FLAGS);
    // byte offset of the lane's B fragment (token cb * 16 + li, k-step 2 wv + ls) in chunk 0
    int xoff[2][NCB];
#pragma unroll
    for (int ls = 0; ls < 2; ++ls)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
            xoff[ls][cb] = (int)(((int64_t)(cb * 16 + li) * K + kstep_col<FMT>(2 * wv + ls, lg)) * 2);

    struct XFrag {
        uint4 v[2][NCB];
    };
    WChunk<FMT> wr[D];
    XFrag xr[D];
    auto load = [&](int u, int64_t c) {
#pragma unroll
        for (int ls = 0; ls < 2; ++ls)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
                xr[u].v[ls][cb] = __builtin_bit_cast(
                    uint4, __builtin_amdgcn_raw_buffer_load_b128(xrsrc, xoff[ls][cb] + (int)(c * GV_KC * 2), 0, 0));
        load_chunk<FMT, PK, NT>(wr[u], src, c);
    };

    v4f acc[4][NCB];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) acc[rb][cb] = v4f{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int u) {
        rowmajor_to_frag<FMT, PK>(wr[u]);
#pragma unroll
        for (int ls = 0; ls < 2; ++ls) {
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const v8bf a = decode_afrag<FMT>(wr[u], rb, ls);
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
                    acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        a, __builtin_bit_cast(v8bf, xr[u].v[ls][cb]), acc[rb][cb], 0, 0, 0);
            }
        }
    };

    if (nch > 0) {
#pragma unroll
        for (int d = 0; d < D; ++d) load(d, c_begin + min(d, nch - 1));
        int c = 0;
        for (; c + D <= nch; c += D) {
#pragma unroll
            for (int u = 0; u < D; ++u) {
                compute(u);
                load(u, c_begin + min(c + u + D, nch - 1));
                // keep each refill right after the compute that frees its slot
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int u = 0; u < D - 1; ++u)
            if (c + u < nch) compute(u);
    }

    v4f fin[NCB];
    reduce_waves<NCB>(acc, fin, red, wv, lane);
    finish_tile<FMT, NCB>(fin, scales, T, N, row0, wv, lane, tile, split, splits, partial, counters, bf16_out, y,
                          &s_last);
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
    bool direct;             // activation fragments loaded per wave (formats without group scales)
    bool resident;           // activation slice staged once in LDS (no barriers in the loop)
    int64_t main_tiles;      // direct variant with spread workgroups: tiles taken whole
    int spread_wgs;          // ... workgroups sharing the other tiles (0: none)
    int maxslots;            // ... partial slots per shared tile
    int kc;                  // chunk width (always GV_KC)
    int64_t tiles;
    int splits;
    int chunks_per_split;
    int64_t lds_bytes;       // dynamic LDS of the resident kernel
    bool two_tiles;          // streaming kernel with two row tiles per workgroup (TH = 2)
};

constexpr int64_t RESIDENT_LDS_MAX = 64 << 10;

template <int FMT, int NCB, bool PK>
static void launch_mfma(const GemvPlan& p, const void* w, const void* scales, const uint16_t* x, int Tc, int64_t N,
                        int64_t K, bool bf16_out, void* y, float* partial, unsigned* counters,
                        hipStream_t stream) {
    dim3 grid((unsigned)p.tiles, (unsigned)p.splits);
    // Non-temporal weight loads (packed weights of 32 MiB or more; the direct
    // kernel, the two-tile kernel up to two token blocks, and the one-tile
    // streaming kernel on many tiles at one token block).  Measured against
    // plain loads: row-FP8 152064x5120 T = 1 / 4 / 8 / 16 / 32 129.2 / 128.7 /
    // 130.6 / 132.0 / 141.2 -> 114.2 / 112.5 / 118.3 / 120.3 / 132.3 us,
    // 5120x17408 T = 1 18.1 -> 17.2; slower: the two-tile kernel at T = 48 / 64
    // (+2 / +4 %), the one-tile streaming kernel with one tile per CU and
    // spread workgroups (17408x5120 row-FP8 T = 16 +5 %, Q8G32 T = 1 +6 %),
    // small matrices that the last-level cache keeps
    // between launches (96x5120 BF16 +15 %), and row-major weights, whose rows
    // four waves read in quarters of a line (+7..24 %).
    const bool nt = PK && (int64_t)N * (FMT == W_BF16 ? 2 * K : K) >= ((int64_t)32 << 20);
    if constexpr (group_size<FMT>() == 0) {
        if (p.direct) {
            const dim3 g = p.spread_wgs > 0 ? dim3((unsigned)(p.main_tiles + p.spread_wgs)) : grid;
            if (nt)
                gemv_direct_kernel<FMT, NCB, PK, true><<<g, 256, 0, stream>>>(
                    reinterpret_cast<const uint8_t*>(w), scales, x, Tc, (int)N, K, p.chunks_per_split, p.splits,
                    partial, counters, bf16_out ? 1 : 0, y, (int)p.main_tiles, p.spread_wgs, p.maxslots);
            else
                gemv_direct_kernel<FMT, NCB, PK><<<g, 256, 0, stream>>>(
                    reinterpret_cast<const uint8_t*>(w), scales, x, Tc, (int)N, K, p.chunks_per_split, p.splits,
                    partial, counters, bf16_out ? 1 : 0, y, (int)p.main_tiles, p.spread_wgs, p.maxslots);
            return;
        }
    }
    if (p.resident) {
        gemv_resident_kernel<FMT, NCB, PK><<<grid, 256, (size_t)p.lds_bytes, stream>>>(
            reinterpret_cast<const uint8_t*>(w), scales, x, Tc, (int)N, K, p.chunks_per_split, p.splits, partial,
            counters, bf16_out ? 1 : 0, y);
        return;
    }
    if constexpr (two_tile_format<FMT, NCB>()) {
        if (p.two_tiles) {
            if (nt && NCB <= 2)
                gemv_mfma_kernel<FMT, NCB, PK, 2, false, true><<<dim3((unsigned)((p.tiles + 1) / 2)), 512, 0, stream>>>(
                    reinterpret_cast<const uint8_t*>(w), scales, x, Tc, (int)N, K, p.chunks_per_split, 1, partial,
                    counters, bf16_out ? 1 : 0, y, 0, 0, 0);
            else
                gemv_mfma_kernel<FMT, NCB, PK, 2><<<dim3((unsigned)((p.tiles + 1) / 2)), 512, 0, stream>>>(
                    reinterpret_cast<const uint8_t*>(w), scales, x, Tc, (int)N, K, p.chunks_per_split, 1, partial,
                    counters, bf16_out ? 1 : 0, y, 0, 0, 0);
            return;
        }
    }
    const dim3 g = p.spread_wgs > 0 ? dim3((unsigned)(p.main_tiles + p.spread_wgs)) : grid;
    // the one-tile streaming kernel takes non-temporal loads on many tiles per
    // CU at one token block only (152064x5120 Q8G32 T = 1 / 8 / 16 140.8 /
    // 155.0 / 168.1 -> 132.6 / 146.9 / 162.7 us; level to +2 % from 17 tokens on)
    const bool snt = nt && NCB == 1 && p.tiles >= 4 * (int64_t)device_cu_count();
    if (NCB == 1 && Tc <= 8 && snt)
        gemv_mfma_kernel<FMT, 1, PK, 1, true, true><<<g, 256, 0, stream>>>(
            reinterpret_cast<const uint8_t*>(w), scales, x, Tc, (int)N, K, p.chunks_per_split, p.splits, partial,
            counters, bf16_out ? 1 : 0, y, (int)p.main_tiles, p.spread_wgs, p.maxslots);
    else if (NCB == 1 && Tc <= 8)      // no token in the second 8-row staging round
        gemv_mfma_kernel<FMT, 1, PK, 1, true><<<g, 256, 0, stream>>>(
            reinterpret_cast<const uint8_t*>(w), scales, x, Tc, (int)N, K, p.chunks_per_split, p.splits, partial,
            counters, bf16_out ? 1 : 0, y, (int)p.main_tiles, p.spread_wgs, p.maxslots);
    else if (snt)
        gemv_mfma_kernel<FMT, 1, PK, 1, false, true><<<g, 256, 0, stream>>>(
            reinterpret_cast<const uint8_t*>(w), scales, x, Tc, (int)N, K, p.chunks_per_split, p.splits, partial,
            counters, bf16_out ? 1 : 0, y, (int)p.main_tiles, p.spread_wgs, p.maxslots);
    else
        gemv_mfma_kernel<FMT, NCB, PK><<<g, 256, 0, stream>>>(
            reinterpret_cast<const uint8_t*>(w), scales, x, Tc, (int)N, K, p.chunks_per_split, p.splits, partial,
            counters, bf16_out ? 1 : 0, y, (int)p.main_tiles, p.spread_wgs, p.maxslots);
}

template <int FMT, bool PK>
static void launch_ncb(const GemvPlan& p, const void* w, const void* scales, const uint16_t* x, int Tc, int64_t N,
                       int64_t K, bool bf16_out, void* y, float* partial, unsigned* counters, hipStream_t stream) {
    switch ((Tc + 15) / 16) {
        case 1: launch_mfma<FMT, 1, PK>(p, w, scales, x, Tc, N, K, bf16_out, y, partial, counters, stream); break;
        case 2: launch_mfma<FMT, 2, PK>(p, w, scales, x, Tc, N, K, bf16_out, y, partial, counters, stream); break;
        case 3: launch_mfma<FMT, 3, PK>(p, w, scales, x, Tc, N, K, bf16_out, y, partial, counters, stream); break;
        default: launch_mfma<FMT, 4, PK>(p, w, scales, x, Tc, N, K, bf16_out, y, partial, counters, stream); break;
    }
}

template <int FMT>
static void launch_fmt(const GemvPlan& p, bool packed, const void* w, const void* scales, const uint16_t* x, int Tc,
                       int64_t N, int64_t K, bool bf16_out, void* y, float* partial, unsigned* counters,
                       hipStream_t stream) {
    if (p.mfma) {
        if (packed) launch_ncb<FMT, true>(p, w, scales, x, Tc, N, K, bf16_out, y, partial, counters, stream);
        else launch_ncb<FMT, false>(p, w, scales, x, Tc, N, K, bf16_out, y, partial, counters, stream);
    } else {
        dim3 grid((unsigned)N, (unsigned)((Tc + 7) / 8));
        gemv_generic_kernel<FMT><<<grid, 64, 0, stream>>>(reinterpret_cast<const uint8_t*>(w), scales, x, Tc,
                                                          (int)N, K, bf16_out ? 1 : 0, y);
    }
}

// Launch the MFMA or generic kernels of one format for one pass of at most 64
// tokens (each format's kernels are instantiated in a translation unit of
// their own, nq_gemv_<format>.hip, so that they compile in parallel).
#define NQ_GEMV_FMT_ENTRY(name)                                                                                   \
    void name(const GemvPlan& p, bool packed, const void* w, const void* scales, const uint16_t* x, int Tc,       \
              int64_t N, int64_t K, bool bf16_out, void* y, float* partial, unsigned* counters, hipStream_t stream)
NQ_GEMV_FMT_ENTRY(gemv_launch_fp8row);
NQ_GEMV_FMT_ENTRY(gemv_launch_mxfp8);
NQ_GEMV_FMT_ENTRY(gemv_launch_bf16);
NQ_GEMV_FMT_ENTRY(gemv_launch_q8g64);
NQ_GEMV_FMT_ENTRY(gemv_launch_q4g64);
NQ_GEMV_FMT_ENTRY(gemv_launch_q8g32);

}  // namespace nq
