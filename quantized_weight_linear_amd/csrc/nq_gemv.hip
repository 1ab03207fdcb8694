// Decode GEMV host side: the launch plan (kernel variant, K splits, spread
// workgroups), the workspace size, the packed weight layout, and the entry
// that runs a call in passes of at most 64 tokens.  The kernels are in
// nq_gemv_kernels.h, instantiated per format in nq_gemv_<format>.hip.
#include <mutex>

#include "nq_gemv_kernels.h"

namespace nq {

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
    // buffer offsets are 32-bit: the activation rows a pass addresses (padded
    // to whole token blocks; the padding reads zero) must stay below 2 GiB
    p.mfma = (K > 0) && (K % GV_KC == 0) && ((Tc + 15) / 16 * 16 * K * 2 < ((int64_t)1 << 31)) &&
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
    // 17408 x 2048: 10.9 against 11.6 us at T = 1).  The grouped formats take
    // the same path at one token block (their spread units load their own
    // scales, see direct_spread): 17408 x 5120 Q4 T = 1 / 4 / 8 19.2 / 19.7 /
    // 21.0 -> 15.4 / 15.6 / 16.0 us and Q8G32 27.3 / 29.5 / 29.9 -> 22.7 /
    // 23.3 / 24.2 against the resident kernel or the streaming kernel's K split.
    const int64_t cus_n = (int64_t)device_cu_count();
    const bool spread_one_round = (fmt_group(fmt) == 0 || Tc <= 16) && allow_spread && p.tiles > cus_n &&
                                  8 * (p.tiles - cus_n) <= cus_n && chunks >= 16;
    // One-byte formats without group scales on at least 4 tiles per CU: two
    // row tiles per workgroup share one activation stage (gemv_mfma_kernel
    // with TH = 2), in place of the spread workgroups, from 5 tokens on for
    // row-FP8 and 8 for MXFP8 (below that the direct kernel is as fast, and
    // MXFP8 packed at T = 5 faster: 171.0 against 178.6 us on the head).
    // Measured, 152064 x 5120 row-FP8 packed, T = 8 / 12 / 16 / 17 / 24 / 32 /
    // 33 / 48 / 64: 129.6 / 134.6 / 141.7 / 138.7 / 149.3 / 161.1 / 168.7 /
    // 185.7 / 206.7 -> 130.1 / 132.4 / 133.6 / 134.8 / 139.0 / 143.4 / 142.7 /
    // 155.0 / 177.1 us; row-major T = 5 / 16 / 32 / 64 158.7 / 185.2 / 185.9 /
    // 233.9 -> 147.3 / 153.9 / 170.2 / 201.4; 65536 x 5120 packed T = 16 / 32
    // / 64 61.4 / 67.5 / 80.6 -> 57.0 / 60.9 / 74.9; MXFP8 packed T = 16 / 32 /
    // 64 198.7 / 217.1 / 269 -> 186.3 / 197.6 / 238.  The plan is the same for
    // both weight layouts, so that their results agree bit for bit; row-major
    // MXFP8 loses at T = 17 / 24 (215.2 / 222.4 -> 225.9 / 229.9 us).  Not for
    // BF16 weights, whose activation bytes weigh half as much against the
    // weights' (packed 65536 x 5120 T = 33 110.5 -> 116.0 us).
    const bool two_tiles = ((fmt == W_FP8ROW && Tc > 4) || (fmt == W_MXFP8 && Tc >= 8)) && p.tiles >= 4 * cus_n;
    if (fmt_group(fmt) == 0 && Tc <= 16 && !spread_one_round && !two_tiles) {
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
    // with the row tiles covering the CUs and more leftover tiles than the
    // spread path takes (measured on 17408 x 5120 T = 1 before that shape went
    // to the spread path, 5 splits: Q4 19.4 against 21.3 us for the streaming
    // kernel without a split, Q8G32 26.8 / 30.7).  With fewer tiles than CUs the streaming kernel with the
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
    // CUs (and not taken by the spread path): from 5 tokens on the streaming
    // kernel with K split in three (see below) beats the resident kernel
    // (measured on 17408 x 5120 before the spread path: Q8G32 T = 8 / 16:
    // 30.2 / 32.6 -> 28.6 / 30.3 us; Q4 level); below that the resident one
    // wins (T = 1: Q4 19.5 against 21.2 us, Q8G32 26.9 / 28.1).
    const bool grouped_leftover = fmt_group(fmt) != 0 && p.tiles > (int64_t)device_cu_count() &&
                                  p.tiles < 2 * (int64_t)device_cu_count() &&
                                  p.tiles % (int64_t)device_cu_count() != 0 && chunks >= 3 * (int64_t)min_chunks;
    // Grouped formats with the tiles a multiple of the CUs (1-3 per CU): the
    // streaming kernel beats the resident kernel at every T, without a K split
    // below 4 tokens (16384 x 5120 T = 1: Q4 18.8 -> 14.3 us, Q8G32 25.4 ->
    // 21.5) and with K split in two from 4 tokens on (T = 4 / 8 / 12 / 16:
    // Q8G32 25.3 / 26.1 / 31.5 / 31.9 -> 22.5 / 21.9 / 22.6 / 23.2 us, Q4 21.0 /
    // 18.9 / 19.1 / 16.4 -> 16.5 / 16.2 / 16.7 / 17.2; 32768 x 5120 Q8G32 T = 8
    // / 16: 47.1 / 52.0 -> 39.8 / 41.7).
    const bool grouped_even = fmt_group(fmt) != 0 && p.tiles >= (int64_t)device_cu_count() &&
                              p.tiles % (int64_t)device_cu_count() == 0 && !many_tiles;
    const bool try_resident = Tc <= 16 && p.tiles >= (int64_t)device_cu_count() && !many_tiles && !spread_one_round &&
                              !(grouped_leftover && Tc > 4) && !grouped_even;
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
    if (grouped_leftover && Tc > 4 && !spread_one_round) {
        const int64_t cus = (int64_t)device_cu_count();
        const int64_t w2 = (2 * p.tiles + cus - 1) / cus, w3 = (3 * p.tiles + cus - 1) / cus;
        s0 = 2 * w3 < 3 * w2 ? 3 : 2;
    }
    const int64_t cps = (chunks + s0 - 1) / s0;
    p.chunks_per_split = (int)cps;
    p.splits = (int)((chunks + cps - 1) / cps);
    p.two_tiles = two_tiles && p.splits == 1;
    if ((fmt_group(fmt) == 0 || spread_one_round) && allow_spread && !p.two_tiles) plan_spread(p, chunks);
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
            case W_FP8ROW: gemv_launch_fp8row(p, packed, w, scales, xc, Tc, N, K, bf16_out, yc, partial, counters, stream); break;
            case W_MXFP8: gemv_launch_mxfp8(p, packed, w, scales, xc, Tc, N, K, bf16_out, yc, partial, counters, stream); break;
            case W_BF16: gemv_launch_bf16(p, packed, w, scales, xc, Tc, N, K, bf16_out, yc, partial, counters, stream); break;
            case W_Q8G64: gemv_launch_q8g64(p, packed, w, scales, xc, Tc, N, K, bf16_out, yc, partial, counters, stream); break;
            case W_Q4G64: gemv_launch_q4g64(p, packed, w, scales, xc, Tc, N, K, bf16_out, yc, partial, counters, stream); break;
            case W_Q8G32: gemv_launch_q8g32(p, packed, w, scales, xc, Tc, N, K, bf16_out, yc, partial, counters, stream); break;
            default: return hipErrorInvalidValue;
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}


// ---------------------------------------------------------------------------
// GEMV without a caller workspace, for callers that cannot allocate (graph
// capture, tight serving loops): the K-split / spread partials and counters
// live in a fixed device array of GEMV_STATIC_SCRATCH_BYTES, one per GPU,
// held until the process ends.  Host code never passes the array's name to a
// kernel (on the host it is only a stand-in for the symbol): its device
// address is looked up once per device with hipGetSymbolAddress and kept.
// Every call clears the counters it will use with a fill kernel first (no
// memset node, so the call can be captured in a graph); the partials need no
// clearing.  Calls that overlap on one GPU share the array and race.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[GEMV_STATIC_SCRATCH_BYTES];

__global__ __launch_bounds__(256) void zero_words_kernel(unsigned* __restrict__ p, int n) {
    for (int i = (int)(blockIdx.x * 256 + threadIdx.x); i < n; i += (int)(gridDim.x * 256)) p[i] = 0u;
}

static hipError_t scratch_address(void** out) {
    static std::mutex mu;
    static void* ptrs[64] = {nullptr};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> g(mu);
    if (ptrs[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        ptrs[dev] = p;
    }
    *out = ptrs[dev];
    return hipSuccess;
}

hipError_t launch_gemv_noalloc(int fmt, const void* w, const void* scales, const uint16_t* x, int64_t T, int64_t N,
                               int64_t K, bool bf16_out, void* y, hipStream_t stream, bool packed) {
    if (T == 0 || N == 0) return hipSuccess;
    const int64_t need = gemv_workspace_bytes(fmt, T, N, K);
    if (need > GEMV_STATIC_SCRATCH_BYTES) return hipErrorInvalidValue;   // validated by the caller
    void* ws = nullptr;
    if (need > 0) {
        hipError_t e = scratch_address(&ws);
        if (e != hipSuccess) return e;
        // the counters (one per row tile) lead the workspace and must start at zero
        const int n = (int)((N + GV_ROWS - 1) / GV_ROWS);
        zero_words_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(reinterpret_cast<unsigned*>(ws), n);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return launch_gemv(fmt, w, scales, x, T, N, K, bf16_out, y, ws, need > 0 ? GEMV_STATIC_SCRATCH_BYTES : 0, stream,
                       packed);
}

}  // namespace nq
