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
    int g;                   // lane group
};

template <int FMT, bool PK>
__device__ __forceinline__ WSrc make_wsrc(const uint8_t* w, const void* scales, int64_t row0, int N, int64_t K,
                                          int lane, int wv) {
    using P = PieceFmt<FMT>;
    WSrc s;
    const int64_t nrb = ((int64_t)N + 15) / 16;
    s.cstride = PK ? nrb * P::BLOCK_CHUNK : 0;
    s.q0 = P::PW * wv;
    s.g = lane >> 4;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        int64_t row = row0 + 16 * r + (lane & 15);
        if (row > N - 1) row = N - 1;
        if (PK) {
            int64_t rb = (row0 >> 4) + r;
            if (rb > nrb - 1) rb = nrb - 1;
            s.base[r] = w + rb * P::BLOCK_CHUNK + (int64_t)lane * P::PB;
        } else {
            s.base[r] = w + row * row_bytes<FMT>(K);
        }
        s.e8[r] = reinterpret_cast<const uint8_t*>(scales) + row * (K >> 5);
    }
    return s;
}

template <int FMT, bool PK>
__device__ __forceinline__ void load_chunk(WChunk<FMT>& r, const WSrc& src, int64_t c) {
    using P = PieceFmt<FMT>;
#pragma unroll
    for (int j = 0; j < 4 * P::PW; ++j) {
        const int rb = j / P::PW;
        const int q = src.q0 + j % P::PW;
        const uint8_t* p = PK ? src.base[rb] + c * src.cstride + q * (64 * P::PB)
                              : src.base[rb] + piece_offset<FMT>(c, q, src.g);
        r.p[j] = *reinterpret_cast<const typename P::Piece*>(p);
        if constexpr (FMT == W_MXFP8) r.e8[j] = src.e8[rb][(c * GV_KC + 64 * q + 16 * src.g) >> 5];
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

// With one token block, Q4 codes are multiplied in a biased form: the nibble
// u = q + 8 (0..15) written into mantissa bits 3..6 of the BF16 1.0 is
// exactly 1 + u / 16 = 1.5 + q / 16, so a group's MFMA sum D over the biased
// weights gives the exact group sum as sum x q = 16 (D - 1.5 sum x) (sum x
// from one more MFMA against a fragment of ones).  The packed layout stores u
// with the two codes of a BF16 pair 16 bits apart (code 2i at bits 4i, code
// 2i + 1 at bits 16 + 4i of each 32-bit word), so a pair costs one shift and
// one and-or; the row-major layout (natural order, two's complement) builds
// the same values with a few more operations.  With more token blocks the
// decode is shared by their MFMAs while the sum of x and the correction are
// per block, so there both layouts decode q itself (the same values, so
// packed and row-major results stay identical).
constexpr uint32_t Q4_ONE = 0x3F803F80u;        // two BF16 1.0
constexpr uint32_t Q4_MANT = 0x00780078u;       // mantissa bits 3..6 of both halves
// (t & mask) | one: with literal constants the compiler emits a separate and
// + or (the VOP3 and-or takes no literal on this target); with the constants
// in registers (readfirstlane makes them opaque, once per kernel) it emits
// one v_and_or_b32.
__device__ __forceinline__ uint32_t q4_packed_pair(uint32_t d, int i, uint32_t mask, uint32_t one) {
    const uint32_t t = i == 0 ? (d << 3) : (d >> (4 * i - 3));
    return (t & mask) | (one & ~mask);
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
        const uint32_t mask = __builtin_amdgcn_readfirstlane(Q4_MANT), one = __builtin_amdgcn_readfirstlane(Q4_ONE);
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
// in the LDS activation rows, scs / sbase the group scales of the chunk.
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
        constexpr bool BIAS = FMT == W_Q4G64 && NCB == 1;   // biased Q4 weights: also sum x per group
        v4f d[4][NCB];
        v4f xsum[NCB];
#pragma unroll
        for (int ls = 0; ls < 2; ++ls) {
            const int col = kl + kstep_col<FMT>(2 * wv + ls, lg);
            v8bf b[NCB];
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) b[cb] = *reinterpret_cast<const v8bf*>(&xs[xrow[cb] + col]);
            if constexpr (BIAS) {
                const v8bf ones = __builtin_bit_cast(v8bf, make_uint4(Q4_ONE, Q4_ONE, Q4_ONE, Q4_ONE));
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
                    xsum[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        ones, b[cb], ls == 0 ? v4f{0.f, 0.f, 0.f, 0.f} : xsum[cb], 0, 0, 0);
            }
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const v8bf a = decode_afrag<FMT, PK, BIAS>(wc, rb, ls);
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
                    // biased Q4: sum x q = 16 (D - 1.5 sum x); the factor 16 is applied once
                    // to the finished sums (q4_bias_finish: exact, a power of two)
                    const float sc[4] = {f16_bits_to_f32(s4.x & 0xFFFFu), f16_bits_to_f32(s4.x >> 16),
                                         f16_bits_to_f32(s4.y & 0xFFFFu), f16_bits_to_f32(s4.y >> 16)};
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float v = BIAS ? fmaf(xsum[cb][e], -1.5f, d[rb][cb][e]) : d[rb][cb][e];
                            acc[rb][cb][e] = fmaf(v, sc[e], acc[rb][cb][e]);
                        }
                }
            }
        }
    }
}

// The factor 16 of the biased Q4 sums (see chunk_mfma), once per wave.
template <int FMT, int NCB>
__device__ __forceinline__ void q4_bias_finish(v4f (&acc)[4][NCB]) {
    if constexpr (FMT == W_Q4G64 && NCB == 1)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) acc[rb][0] *= 16.0f;
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

template <int FMT, int NCB, bool PK>
__device__ __forceinline__ void direct_spread(const uint8_t* __restrict__ w, const void* __restrict__ scales,
                                              const uint16_t* __restrict__ x, int T, int N, int64_t K, int tile0,
                                              int R, int e, int E, int maxslots, float* __restrict__ partial,
                                              unsigned* __restrict__ counters, int bf16_out, void* __restrict__ y,
                                              v4f* red, int* s_last) {
    using P = PieceFmt<FMT>;
    constexpr int D = 2;
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
            if constexpr (!PK || FMT == W_MXFP8) {
                const int64_t lim = (int64_t)N - 1 - rowb;                   // rows past N are clamped
                const int lr = (int64_t)li < lim ? li : (int)lim;
                row = rowb + lr;
            }
            if constexpr (!PK) pw = w + row * row_bytes<FMT>(K) + piece_offset<FMT>(c, q, lg);
            wr[slot].p[j] = *reinterpret_cast<const typename P::Piece*>(pw);
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
        reduce_waves<NCB>(acc, fin, red, wv, lane);
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
// Waves per SIMD the streaming kernel is compiled for: two for the formats
// without group scales, so that a spread workgroup fits beside a whole-tile
// one on every CU (see direct_spread), and for the grouped formats at three
// token blocks (two K splits per tile then share a CU); one for the other
// grouped cases, and for BF16 weights at four token blocks, which would spill
// at that budget (a spread launch then runs its spread workgroups after the
// whole tiles).
template <int FMT, int NCB>
constexpr int stream_min_waves() {
    return (!(FMT == W_BF16 && NCB == 4) && (group_size<FMT>() == 0 || NCB == 3)) ? 2 : 1;
}

// With spread_wgs > 0 (formats without group scales, one split): workgroups
// [0, spread_wgs) share the tiles [main_tiles, tiles) unit by unit
// (direct_spread) and the main_tiles after them take one whole tile each as
// below.  The spread workgroups come first so that they are dispatched first:
// their partial exchange then ends well inside the whole tiles' time.
template <int FMT, int NCB, bool PK>
__global__ __launch_bounds__(256, (stream_min_waves<FMT, NCB>())) void gemv_mfma_kernel(
    const uint8_t* __restrict__ w, const void* __restrict__ scales, const uint16_t* __restrict__ x, int T, int N,
    int64_t K, int chunks_per_split, int splits, float* __restrict__ partial, unsigned* __restrict__ counters,
    int bf16_out, void* __restrict__ y, int main_tiles, int spread_wgs, int maxslots) {
    constexpr int TP = 16 * NCB;
    constexpr int XPITCH = GV_KC + 8;                 // bf16 per LDS row: rows shift by 4 banks
    constexpr int XPR = GV_KC / 8;                    // 16-byte activation pieces per row and chunk
    constexpr int XP = TP * XPR / 256;                // ... per thread
    constexpr int GS = group_size<FMT>();
    constexpr int NG = GS ? GV_KC / (GS ? GS : 1) : 1;   // scale groups per chunk
    constexpr int SP = GS ? (NG * GV_ROWS + 255) / 256 : 1;
    constexpr int D = depth<FMT, NCB>();
    // xs doubles as the buffer of the final cross-wave sum (16 KiB per token block)
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][TP * XPITCH];
    __shared__ __attribute__((aligned(16))) uint16_t scs[2][GS ? NG * GV_ROWS : 1];
    __shared__ int s_last;
    static_assert(sizeof(xs) >= 16384 * NCB, "reduction buffer");
    if constexpr (GS == 0) {
        __shared__ int s_last_sp[SPREAD_MAXSEG];
        if ((int)blockIdx.x < spread_wgs) {
            const int tiles_all = (int)((N + GV_ROWS - 1) / GV_ROWS);
            direct_spread<FMT, NCB, PK>(w, scales, x, T, N, K, main_tiles, tiles_all - main_tiles,
                                        (int)blockIdx.x, spread_wgs, maxslots, partial, counters,
                                        bf16_out, y, reinterpret_cast<v4f*>(&xs[0][0]), s_last_sp);
            return;
        }
    }

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int li = lane & 15;
    const int lg = lane >> 4;
    const int tile = (int)blockIdx.x - spread_wgs;   // spread workgroups come first
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
    uint4 xreg[D][XP];
    uint32_t sreg[D][SP];
    auto load_x = [&](int slot, int c) {
        const int64_t kc0 = k_begin + (int64_t)c * GV_KC;
#pragma unroll
        for (int j = 0; j < XP; ++j) {
            const int idx = tid + 256 * j;
            const int t = idx / XPR, pc = idx % XPR;
            const int off = (int)(((int64_t)t * K + kc0 + 8 * pc) * 2);
            xreg[slot][j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xrsrc, off, 0, 0));
        }
        if constexpr (GS != 0) {
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
        for (int j = 0; j < XP; ++j) {
            const int idx = tid + 256 * j;
            const int t = idx / XPR, pc = idx % XPR;
            *reinterpret_cast<uint4*>(&xs[buf][t * XPITCH + 8 * pc]) = xreg[slot][j];
        }
        if constexpr (GS != 0) {
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
    for (int cb = 0; cb < NCB; ++cb) xrow[cb] = (cb * 16 + li) * XPITCH;

    // One chunk c (c = u mod D): compute from ring slot u and LDS buffer c & 1,
    // stage the activations of chunk c + 1 (register slot (u + 1) mod D),
    // request activations and weights of chunk c + D into slot u (indices
    // clamped to the last chunk, so the body has no branch), barrier.
    WChunk<FMT> ring[D];
    auto body = [&](int c, int u) {
        const int buf = c & 1;
        chunk_mfma<FMT, NCB, PK>(ring[u], xs[buf], xrow, 0, scs[buf], 0, wv, lg, acc);
        store_x((c + 1) & 1, (u + 1) % D);
        load_x(u, min(c + D, nch - 1));
        load_chunk<FMT, PK>(ring[u], src, c_begin + min(c + D, nch - 1));
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
    };

    if (nch > 0) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            load_x(d, min(d, nch - 1));
            load_chunk<FMT, PK>(ring[d], src, c_begin + min(d, nch - 1));
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
    reduce_waves<NCB>(acc, fin, reinterpret_cast<v4f*>(&xs[0][0]), wv, lane);
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

    auto compute = [&](const WChunk<FMT>& wc, int c) {
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
template <int FMT, int NCB, bool PK>
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
        direct_spread<FMT, NCB, PK>(w, scales, x, T, N, K, main_tiles, tiles_all - main_tiles,
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
        load_chunk<FMT, PK>(wr[u], src, c);
    };

    v4f acc[4][NCB];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) acc[rb][cb] = v4f{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int u) {
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
};

constexpr int64_t RESIDENT_LDS_MAX = 64 << 10;

static int fmt_group(int fmt) {
    return fmt == W_Q8G32 ? 32 : ((fmt == W_Q4G64 || fmt == W_Q8G64) ? 64 : 0);
}

static double fmt_bytes_per_weight(int fmt) {
    return fmt == W_Q4G64 ? 0.5 : (fmt == W_BF16 ? 2.0 : 1.0);
}

// Staged activations [Tc + 1][span + 8] and group scales [span / G][64]; at
// least the 16 KiB per token block that the final cross-wave sum reuses.
static int64_t resident_lds(int fmt, int64_t Tc, int64_t cps, int kc) {
    const int gs = fmt_group(fmt);
    const int64_t span = cps * kc;
    const int64_t stage = ((Tc + 1) * (span + 8) + (gs ? span / gs * GV_ROWS : 0)) * 2;
    const int64_t red = 16384 * ((Tc + 15) / 16);
    return stage > red ? stage : red;
}

// More tiles than CUs, not a multiple of them, one split: whole tiles for the
// first m x CUs, the R others spread over at most one more workgroup per CU
// (at most SPREAD_MAXSEG tiles each).  The busiest CU then holds lmax =
// ceil(U / min(U, CUs)) units beside its tile; the fewest workgroups that keep
// that bound, ceil(U / lmax), give a leftover tile the fewest partial slots,
// and so the shortest final sum for its last workgroup, which slows the
// whole tile sharing its CU (17408 x 5120: 160 workgroups of 2 chunks, 10
// slots a tile, instead of 256 of 1 or 2 chunks, 16 or 17 slots).
static void plan_spread(GemvPlan& p, int64_t chunks) {
    const int64_t cus = (int64_t)device_cu_count();
    const int64_t R = p.tiles % cus, U = R * chunks;
    if (p.splits != 1 || p.tiles <= cus || R == 0 || U >= ((int64_t)1 << 31)) return;
    const int64_t E0 = U < cus ? U : cus;
    const int64_t lmax = (U + E0 - 1) / E0;
    const int64_t E = (U + lmax - 1) / lmax;
    const int64_t lmin = U / E;
    if ((lmax - 1 + chunks - 1) / chunks + 1 > SPREAD_MAXSEG) return;
    p.main_tiles = p.tiles - R;
    p.spread_wgs = (int)E;
    p.maxslots = (int)((chunks + lmin - 1) / lmin + 1);
}

// K split count for fewer row tiles than CUs: the one (up to smax) that
// minimizes the chunks of the busiest CU, ceil(tiles s / CUs) x ceil(chunks / s)
// with one workgroup per (tile, split); ties go to fewer splits.
static int64_t balanced_splits(int64_t tiles, int64_t chunks, int64_t smax) {
    const int64_t cus = (int64_t)device_cu_count();
    int64_t best = 1, best_cost = -1;
    for (int64_t s = 1; s <= smax; ++s) {
        const int64_t cps = (chunks + s - 1) / s;
        const int64_t se = (chunks + cps - 1) / cps;
        const int64_t cost = ((tiles * se + cus - 1) / cus) * cps;
        if (best_cost < 0 || cost < best_cost) {
            best_cost = cost;
            best = se;
        }
    }
    return best;
}

static GemvPlan plan_gemv(int fmt, int64_t Tc, int64_t N, int64_t K, bool allow_spread = true) {
    GemvPlan p{};
    // buffer offsets are 32-bit: the activation block must stay below 2 GiB
    p.mfma = (K > 0) && (K % GV_KC == 0) && (Tc * K * 2 < ((int64_t)1 << 31)) &&
             (N * (K / 32) * 2 < ((int64_t)1 << 31));
    p.kc = GV_KC;
    p.tiles = (N + GV_ROWS - 1) / GV_ROWS;
    p.splits = 1;
    p.chunks_per_split = p.mfma ? (int)(K / p.kc) : 0;
    if (!p.mfma) return p;
    const int64_t chunks = K / p.kc;
    constexpr int64_t min_chunks = 4;          // chunks per K split at least
    int64_t smax = chunks / min_chunks;        // keep whole chunks, at least min_chunks per split
    if (smax > 32) smax = 32;
    if (smax < 1) smax = 1;
    // One whole tile per CU plus a few leftover tiles (at most CUs / 8)
    // spread beside them, over a long K (at least 16 chunks): the streaming
    // kernel, whose whole tiles issue ahead of the spread work (see
    // gemv_mfma_kernel), is faster than the direct kernel at every T there
    // (17408 x 5120: T = 1 17.8 against 18.2 us, T = 4 17.3 / 18.0, T = 16
    // 18.8 / 20.6; 16448 x 5120: T = 16 18.1 / 19.2); the resident kernel's K
    // split is slower than both.  With more leftover tiles or a shorter K the
    // direct kernel is as fast or faster (24576 x 5120: 24.5 against 26.7 us;
    // 17408 x 2048: 10.9 against 11.6 us at T = 1).
    const int64_t cus_n = (int64_t)device_cu_count();
    const bool spread_one_round = fmt_group(fmt) == 0 && allow_spread && p.tiles > cus_n &&
                                  8 * (p.tiles - cus_n) <= cus_n && chunks >= 16;
    if (fmt_group(fmt) == 0 && Tc <= 16 && !spread_one_round) {
        // direct variant (no group scales, one token block): about one
        // workgroup per CU (measured: more per CU only slow it down); with
        // fewer tiles than CUs, K split so that the busiest CU has the fewest chunks
        const int64_t sd = p.tiles < (int64_t)device_cu_count() ? balanced_splits(p.tiles, chunks, smax) : 1;
        const int64_t cps = (chunks + sd - 1) / sd;
        p.direct = true;
        p.chunks_per_split = (int)cps;
        p.splits = (int)((chunks + cps - 1) / cps);
        if (allow_spread) plan_spread(p, chunks);
        return p;
    }
    // resident variant: from the split count that leaves the busiest CU the
    // fewest chunks, the smallest whose slice fits in LDS and whose FP32
    // partials stay within 12% of the weight bytes; only for one token block
    // with the row tiles covering the CUs (17408 x 5120 T = 1, 5 splits: Q4
    // 19.4 against 21.3 us for the streaming kernel without a split, Q8G32
    // 26.8 / 30.7).  With fewer tiles than CUs the streaming kernel with the
    // balanced split is as fast or faster: the slice that fits in LDS forces
    // more splits than the balance needs (5120 x 17408: row-FP8 T = 17 32.9
    // -> 19.3 us, Q8G32 T = 8 36.8 -> 24.8, Q4 T = 1 21.7 -> 19.1; Q8G32
    // 4096 x 4096 T = 8 11.6 -> 10.0).
    const double wbytes = (double)N * (double)K * fmt_bytes_per_weight(fmt);
    // With at least 4 row tiles per CU whole tiles already balance within a
    // quarter: the streaming kernel without a K split is faster there
    // (measured on 2376 tiles, Q8G32: 148-170 us at T = 1..16, against 152-222
    // us for the resident kernel, whose split adds the partial exchange).
    const bool many_tiles = p.tiles >= 4 * (int64_t)device_cu_count();
    // Grouped formats between one and two tiles per CU, not a multiple of the
    // CUs: from 5 tokens on the streaming kernel with K split in three (see
    // below) beats the resident kernel (17408 x 5120 Q8G32 T = 8 / 16: 30.2 /
    // 32.6 -> 28.6 / 30.3 us; Q4 level); below that the resident one wins (T = 1:
    // Q4 19.5 against 21.2 us, Q8G32 26.9 / 28.1).
    const bool grouped_leftover = fmt_group(fmt) != 0 && p.tiles > (int64_t)device_cu_count() &&
                                  p.tiles < 2 * (int64_t)device_cu_count() &&
                                  p.tiles % (int64_t)device_cu_count() != 0 && chunks >= 3 * (int64_t)min_chunks;
    // Grouped formats with the tiles a multiple of the CUs (1-3 per CU): from
    // 4 tokens on the streaming kernel with K split in two beats the resident
    // kernel too (16384 x 5120 T = 4 / 8 / 12 / 16: Q8G32 25.3 / 26.1 / 31.5 /
    // 31.9 -> 22.5 / 21.9 / 22.6 / 23.2 us, Q4 21.0 / 18.9 / 19.1 / 16.4 ->
    // 16.5 / 16.2 / 16.7 / 17.2; 32768 x 5120 Q8G32 T = 8 / 16: 47.1 / 52.0 ->
    // 39.8 / 41.7).
    const bool grouped_even = fmt_group(fmt) != 0 && p.tiles >= (int64_t)device_cu_count() &&
                              p.tiles % (int64_t)device_cu_count() == 0 && !many_tiles;
    const bool try_resident = Tc <= 16 && p.tiles >= (int64_t)device_cu_count() && !many_tiles && !spread_one_round &&
                              !(grouped_leftover && Tc > 4) && !(grouped_even && Tc >= 4);
    const int64_t sr = balanced_splits(p.tiles, chunks, smax);
    for (int64_t s = sr; try_resident && s <= 32 && s <= chunks; ++s) {
        const int64_t cps = (chunks + s - 1) / s;
        const int64_t se = (chunks + cps - 1) / cps;
        const double partial_bytes = se > 1 ? 8.0 * (double)se * (double)Tc * (double)N : 0.0;
        const int64_t lds = resident_lds(fmt, Tc, cps, p.kc);
        if (lds <= RESIDENT_LDS_MAX && partial_bytes <= 0.12 * wbytes) {
            p.resident = true;
            p.chunks_per_split = (int)cps;
            p.splits = (int)se;
            p.lds_bytes = lds;
            return p;
        }
    }
    // streaming variant: once the row tiles alone cover every CU, splitting K
    // only adds workgroups that compete for LDS bandwidth plus the partial
    // exchange; below that, the split that leaves the busiest CU the fewest chunks
    // Grouped formats with more than one token block (their per-weight work
    // is heavier) gain from two workgroups per CU: with up to 4 tiles per CU,
    // K is split in two (17408x5120 T = 33: Q4 36.4 -> 35.4 us, Q8G32 42.6 ->
    // 40.4 us); the formats without group scales do not (FP8 28 -> 31 us).
    const bool two_per_cu = fmt_group(fmt) != 0 && (Tc > 16 || (grouped_even && Tc >= 4)) &&
                            p.tiles < 4 * (int64_t)device_cu_count();
    int64_t s0 = p.tiles >= (int64_t)device_cu_count() ? (two_per_cu ? 2 : 1) : balanced_splits(p.tiles, chunks, smax);
    // Between one and two tiles per CU, not a multiple of the CUs: two or
    // three splits, whichever leaves the busiest CU the smaller share of a
    // tile (ceil(tiles s / CUs) / s).  272 tiles: 4/3 against 3/2, three
    // splits (17408 x 5120 T = 17 / 33 / 48, Q4 28.0 / 35.9 / 37.5 -> 26.6 /
    // 33.8 / 35.7 us, Q8G32 34.7 / 40.5 / 42.3 -> 32.2 / 37.9 / 40.8 us; 20480
    // x 5120 Q8G32 T = 33 40.9 -> 39.1); 384 tiles: 5/3 against 3/2, two
    // (24576 x 5120 T = 8 / 33: Q8G32 35.9 / 46.8 against 33.0 / 42.1 us, Q4
    // 26.6 / 40.9 against 24.1 / 37.0).  Four or five splits are slower
    // again (the exchange).
    if (grouped_leftover && Tc > 4) {
        const int64_t cus = (int64_t)device_cu_count();
        const int64_t w2 = (2 * p.tiles + cus - 1) / cus, w3 = (3 * p.tiles + cus - 1) / cus;
        s0 = 2 * w3 < 3 * w2 ? 3 : 2;
    }
    const int64_t cps = (chunks + s0 - 1) / s0;
    p.chunks_per_split = (int)cps;
    p.splits = (int)((chunks + cps - 1) / cps);
    if (fmt_group(fmt) == 0 && allow_spread) plan_spread(p, chunks);
    return p;
}

static int64_t align256(int64_t v) { return (v + 255) & ~(int64_t)255; }

static int64_t plan_workspace(const GemvPlan& p, int64_t Tc) {
    if (p.spread_wgs > 0) return align256(p.tiles * 4) + (p.tiles - p.main_tiles) * p.maxslots * Tc * GV_ROWS * 4;
    if (!p.mfma || p.splits == 1) return 0;
    return align256(p.tiles * 4) + (int64_t)p.splits * Tc * p.tiles * GV_ROWS * 4;
}

int64_t gemv_workspace_bytes(int fmt, int64_t T, int64_t N, int64_t K) {
    if (fmt < 0) fmt = W_FP8ROW;
    const int64_t Tc = T < 64 ? T : 64;
    int64_t need = plan_workspace(plan_gemv(fmt, Tc, N, K), Tc);
    if (T > 64) {                                   // the remainder pass may plan differently
        const int64_t Tr = T % 64;
        if (Tr) {
            const int64_t r = plan_workspace(plan_gemv(fmt, Tr, N, K), Tr);
            if (r > need) need = r;
        }
    }
    return need;
}

template <int FMT, int NCB, bool PK>
static void launch_mfma(const GemvPlan& p, const void* w, const void* scales, const uint16_t* x, int Tc, int64_t N,
                        int64_t K, bool bf16_out, void* y, float* partial, unsigned* counters,
                        hipStream_t stream) {
    dim3 grid((unsigned)p.tiles, (unsigned)p.splits);
    if constexpr (group_size<FMT>() == 0) {
        if (p.direct) {
            const dim3 g = p.spread_wgs > 0 ? dim3((unsigned)(p.main_tiles + p.spread_wgs)) : grid;
            gemv_direct_kernel<FMT, NCB, PK><<<g, 256, 0, stream>>>(
                reinterpret_cast<const uint8_t*>(w), scales, x, Tc, (int)N, K, p.chunks_per_split, p.splits, partial,
                counters, bf16_out ? 1 : 0, y, (int)p.main_tiles, p.spread_wgs, p.maxslots);
            return;
        }
    }
    if (p.resident)
        gemv_resident_kernel<FMT, NCB, PK><<<grid, 256, (size_t)p.lds_bytes, stream>>>(
            reinterpret_cast<const uint8_t*>(w), scales, x, Tc, (int)N, K, p.chunks_per_split, p.splits, partial,
            counters, bf16_out ? 1 : 0, y);
    else {
        const dim3 g = p.spread_wgs > 0 ? dim3((unsigned)(p.main_tiles + p.spread_wgs)) : grid;
        gemv_mfma_kernel<FMT, NCB, PK><<<g, 256, 0, stream>>>(reinterpret_cast<const uint8_t*>(w), scales, x, Tc,
                                                                  (int)N, K, p.chunks_per_split, p.splits, partial,
                                                                  counters, bf16_out ? 1 : 0, y, (int)p.main_tiles,
                                                                  p.spread_wgs, p.maxslots);
    }
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

// ---------------------------------------------------------------------------
// Packed weight layout.  Rows are grouped in blocks of 16 (the last block
// zero-padded).  Chunk-major: for every chunk c of 256 columns, for every row
// block, for every piece q of the chunk (see PieceFmt), the 64 lanes' pieces
// are stored one after another in lane order (lane = 16 g + i holds row i,
// lane group g).  Every load instruction of a wave reads 64 x piece contiguous
// bytes, and the waves of the whole grid, walking chunk by chunk, sweep one
// contiguous window of memory at a time.  A pure permutation of the row-major
// bytes (K % 256 == 0).
// ---------------------------------------------------------------------------
// Packed Q4 word: the row-major word's codes c0..c7 (c_j at bits 4j, two's
// complement) as biased nibbles u = c ^ 8 = c + 8, c_2i at bits 4i and
// c_2i+1 at bits 16 + 4i (see q4_packed_pair).
__device__ __forceinline__ uint32_t q4_pack_word(uint32_t w) {
    w ^= 0x88888888u;
    uint32_t o = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o |= ((w >> (8 * i)) & 0xFu) << (4 * i);
        o |= ((w >> (8 * i + 4)) & 0xFu) << (16 + 4 * i);
    }
    return o;
}

template <int FMT>
__global__ __launch_bounds__(256) void pack_weights_kernel(const uint8_t* __restrict__ src, int64_t N, int64_t K,
                                                           uint8_t* __restrict__ dst, int64_t n_pieces) {
    constexpr int NP = PieceFmt<FMT>::NP;
    constexpr int PB = PieceFmt<FMT>::PB;
    const int64_t nrb = (N + 15) / 16;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n_pieces; i += (int64_t)gridDim.x * 256) {
        // i = ((c * nrb + rb) * NP + q) * 64 + lane
        const int lane = (int)(i & 63);
        const int64_t j = i >> 6;
        const int q = (int)(j % NP);
        const int64_t cr = j / NP;
        const int64_t rb = cr % nrb, c = cr / nrb;
        const int64_t row = rb * 16 + (lane & 15);
        uint8_t* d = dst + i * PB;
        if (row < N) {
            const uint8_t* s = src + row * row_bytes<FMT>(K) + piece_offset<FMT>(c, q, lane >> 4);
            if constexpr (PB == 16) {
                *reinterpret_cast<uint4*>(d) = *reinterpret_cast<const uint4*>(s);
            } else if constexpr (FMT == W_Q4G64) {
                const uint2 v = *reinterpret_cast<const uint2*>(s);
                *reinterpret_cast<uint2*>(d) = make_uint2(q4_pack_word(v.x), q4_pack_word(v.y));
            } else {
                *reinterpret_cast<uint2*>(d) = *reinterpret_cast<const uint2*>(s);
            }
        } else {
            if constexpr (PB == 16) *reinterpret_cast<uint4*>(d) = make_uint4(0, 0, 0, 0);
            else *reinterpret_cast<uint2*>(d) = make_uint2(0, 0);
        }
    }
}

static int64_t row_bytes_host(int fmt, int64_t K) {
    return fmt == W_Q4G64 ? K / 2 : (fmt == W_BF16 ? 2 * K : K);
}

int64_t packed_weight_bytes(int fmt, int64_t N, int64_t K) {
    return (N + 15) / 16 * 16 * row_bytes_host(fmt, K);
}

template <int FMT>
static void launch_pack_fmt(const void* src, int64_t N, int64_t K, void* dst, hipStream_t stream) {
    const int64_t n_pieces = (N + 15) / 16 * (K / GV_KC) * PieceFmt<FMT>::NP * 64;
    int64_t blocks = (n_pieces + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    pack_weights_kernel<FMT><<<(unsigned)blocks, 256, 0, stream>>>(reinterpret_cast<const uint8_t*>(src), N, K,
                                                                   reinterpret_cast<uint8_t*>(dst), n_pieces);
}

hipError_t launch_pack_weights(int fmt, const void* src, int64_t N, int64_t K, void* dst, hipStream_t stream) {
    if (N == 0 || K == 0) return hipSuccess;
    switch (fmt) {
        case W_FP8ROW: launch_pack_fmt<W_FP8ROW>(src, N, K, dst, stream); break;
        case W_MXFP8: launch_pack_fmt<W_MXFP8>(src, N, K, dst, stream); break;
        case W_BF16: launch_pack_fmt<W_BF16>(src, N, K, dst, stream); break;
        case W_Q8G64: launch_pack_fmt<W_Q8G64>(src, N, K, dst, stream); break;
        case W_Q4G64: launch_pack_fmt<W_Q4G64>(src, N, K, dst, stream); break;
        case W_Q8G32: launch_pack_fmt<W_Q8G32>(src, N, K, dst, stream); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_gemv(int fmt, const void* w, const void* scales, const uint16_t* x, int64_t T, int64_t N,
                       int64_t K, bool bf16_out, void* y, void* workspace, int64_t workspace_bytes,
                       hipStream_t stream, bool packed) {
    if (T == 0 || N == 0) return hipSuccess;
    const size_t ybytes = bf16_out ? 2 : 4;
    for (int64_t t0 = 0; t0 < T; t0 += 64) {
        const int Tc = (int)((T - t0) < 64 ? (T - t0) : 64);
        GemvPlan p = plan_gemv(fmt, Tc, N, K);
        if (packed && !p.mfma) return hipErrorInvalidValue;    // only the MFMA kernels read packed weights
        float* partial = nullptr;
        unsigned* counters = nullptr;
        if (p.spread_wgs > 0) {
            if (workspace != nullptr && workspace_bytes >= plan_workspace(p, Tc)) {
                counters = reinterpret_cast<unsigned*>(workspace);
                partial = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + align256(p.tiles * 4));
            } else {
                p = plan_gemv(fmt, Tc, N, K, false);           // no room for partials: whole tiles only
            }
        }
        if (p.splits > 1) {
            const int64_t need = plan_workspace(p, Tc);
            if (workspace != nullptr && workspace_bytes >= need) {
                counters = reinterpret_cast<unsigned*>(workspace);
                partial = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + align256(p.tiles * 4));
            } else {
                p.splits = 1;
                p.chunks_per_split = (int)(K / p.kc);
                if (p.resident) {
                    p.lds_bytes = resident_lds(fmt, Tc, p.chunks_per_split, p.kc);
                    p.resident = p.lds_bytes <= RESIDENT_LDS_MAX;
                }
            }
        }
        const uint16_t* xc = x + t0 * K;
        void* yc = reinterpret_cast<char*>(y) + t0 * N * ybytes;
        switch (fmt) {
            case W_FP8ROW: launch_fmt<W_FP8ROW>(p, packed, w, scales, xc, Tc, N, K, bf16_out, yc, partial, counters, stream); break;
            case W_MXFP8: launch_fmt<W_MXFP8>(p, packed, w, scales, xc, Tc, N, K, bf16_out, yc, partial, counters, stream); break;
            case W_BF16: launch_fmt<W_BF16>(p, packed, w, scales, xc, Tc, N, K, bf16_out, yc, partial, counters, stream); break;
            case W_Q8G64: launch_fmt<W_Q8G64>(p, packed, w, scales, xc, Tc, N, K, bf16_out, yc, partial, counters, stream); break;
            case W_Q4G64: launch_fmt<W_Q4G64>(p, packed, w, scales, xc, Tc, N, K, bf16_out, yc, partial, counters, stream); break;
            case W_Q8G32: launch_fmt<W_Q8G32>(p, packed, w, scales, xc, Tc, N, K, bf16_out, yc, partial, counters, stream); break;
            default: return hipErrorInvalidValue;
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace nq
