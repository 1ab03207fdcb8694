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
// writes 1 KB of LDS in lane order, eight lanes per row reading the row's 128
// contiguous bytes of the stage.  Whole 128-byte lines per row matter: loads
// of 64 bytes per row reach about half the L2-to-CU rate.  The 16-byte pieces
// of a row are XOR-swizzled so that the MFMA fragment reads (16 bytes per
// lane) are conflict-free.  One stage holds 128 K-columns of both panels
// (plus, for W8A8 with K % 512 != 0, the activation and weight scales of its
// two groups; with K % 512 == 0 the scales come in windows of several stages,
// see ScaleWin); a ring of S stages (W8A8 3, FP8 2: as many as LDS holds) with
// one barrier per stage.  Rows past M / N and columns past K are out of the buffer range or
// masked, and read as zero.
//
// W8A8 (64-channel groups, two per stage): two v_mfma_i32_32x32x32_i8 per
// tile sum a group exactly in int32.  The first MFMA's C operand is the
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
#include <type_traits>
#include <utility>

#include "nq_device.h"
#include "nq_launch.h"

// m0 is written by the LDS-mode loads below; nothing else in this file uses it.
#pragma clang diagnostic ignored "-Winline-asm"

namespace nq {

constexpr int GB_K = 128;    // K columns (bytes) per stage: whole 128-byte lines of every row
constexpr unsigned GB_FLAGS = 0x00020000u;
constexpr int GB_OOB = 0x40000000;   // a buffer offset past every range used here

template <bool W8A8>
struct GemmCfg {
    static constexpr int WM = W8A8 ? 4 : 4, WN = W8A8 ? 2 : 2;   // wave grid
    static constexpr int TM = W8A8 ? 2 : 2, TN = W8A8 ? 2 : 4;   // 32 x 32 tiles per wave
    static constexpr int S = W8A8 ? 3 : 2;                       // stages in the LDS ring
    static constexpr int NW = WM * WN;
    static constexpr int BM = 32 * TM * WM, BN = 32 * TN * WN;
    static constexpr int LOADS = (BM + BN) / 8 / NW;    // panel loads per wave and stage (8 rows each)
    static_assert((BM + BN) % (8 * NW) == 0, "panel loads must divide evenly over the waves");
    // W8A8 scale loads per stage: two groups of activation scales (BM / 64
    // loads each) and of weight scales (BN / 64 each), two per wave.
    static constexpr int SCALE_LOADS = W8A8 ? 2 : 0;
    static_assert(!W8A8 || BM / 64 + BN / 64 <= NW, "scale load plan");
};

// 16-byte aligned size: every stage of the ring starts on a 16-byte boundary,
// so fragment reads stay single 16-byte LDS reads.
template <bool W8A8, bool SW>
struct alignas(16) GemmStage {
    static constexpr int BM = GemmCfg<W8A8>::BM, BN = GemmCfg<W8A8>::BN;
    static constexpr bool PER_STAGE = W8A8 && !SW;   // scales staged with the panels
    uint8_t a[BM * GB_K];
    uint8_t b[BN * GB_K];
    float as[PER_STAGE ? 2 * BM : 1];       // activation scales of the stage's two groups
    uint32_t ws[PER_STAGE ? 2 * BN : 1];    // weight scales of the two groups (FP16 bits, zero-extended:
                                            // a 2-byte load in LDS mode still writes 4 bytes per lane)
    uint32_t sink[PER_STAGE ? 128 : 1];     // target of the empty scale loads (they write zeros)
};

// W8A8 scale windows (K % 512 == 0, so that scale rows start on 16-byte
// boundaries).  Staging two groups of scales per stage takes one gather per
// row and group: a 64-lane load that touches 64 cache lines, as many address
// lookups as 8 panel loads, which made the address unit the bottleneck.  A
// window instead takes one 16-byte load per row for the activation scales of
// four groups (two stages) or the FP16 weight scales of eight groups (four
// stages), five times fewer lookups; two slots each, the one in use and the
// one being filled.  Layout [slot][row][group within the window].
template <bool SW>
struct alignas(16) ScaleWin {
    static constexpr int BM = GemmCfg<true>::BM, BN = GemmCfg<true>::BN;
    float as[SW ? 2 : 1][SW ? 4 * BM : 1];
    uint16_t ws[SW ? 2 : 1][SW ? 8 * BN : 1];
};

// 32x32 MFMA output layout: lane l holds column (l % 32) and rows
// 8 j + 4 (l / 32) + r for j, r in 0..3 (element 4 j + r).
__device__ __forceinline__ int d_row(int lane, int e) { return 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3); }

// Row scales for the W8A8 rescale.  Accumulator element e of a 32 x 32 tile
// sits on row d_row(lane, e): 8 (e / 4) + e % 4 in lanes [0, 32) and 4 more in
// lanes [32, 64), the same row across each half wave.  A register whose lane
// n + 16 r (r = 0..3) holds the scale of row d_row(32 (r / 2), n) carries the
// 32 row scales a tile needs; DPP row_newbcast:e hands lane e of each 16-lane
// row to the whole row, which is then the scale of element e's row in every
// lane.  One 4-byte LDS read per tile replaces eight 16-byte ones.
__device__ __forceinline__ int row_scale_lane_row(int lane) {
    return 8 * ((lane & 15) >> 2) + 4 * (lane >> 5) + (lane & 3);
}
// acc + bcast_e(s) * x, one v_fmac_f32 with the DPP broadcast on its first
// source (the compiler does not fold a separate DPP move into the FMA).  s is
// never written by the vector ALU (it comes from an LDS read), so the DPP
// source needs no wait states.
template <int E>
__device__ __forceinline__ float fmac_row_bcast(float acc, float s, float x) {
    asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
        : "+v"(acc) : "v"(s), "v"(x), "n"(E));
    return acc;
}
template <int... E>
__device__ __forceinline__ void rescale_tile(v16f& acc, const v16i& d, float ws, float wsc, float s,
                                             std::integer_sequence<int, E...>) {
    ((acc[E] = fmac_row_bcast<E>(acc[E], s, fmaf(__int_as_float(d[E]), ws, wsc))), ...);
}

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

template <bool W8A8, bool SUMS, bool KTAIL, bool SW>
__global__ __launch_bounds__(64 * GemmCfg<W8A8>::NW) void gemm_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ a_scale, const uint8_t* __restrict__ W,
    const uint16_t* __restrict__ w_scale, int M, int N, int K, int bf16_out, void* __restrict__ y,
    int32_t* __restrict__ group_sums) {
    using C = GemmCfg<W8A8>;
    constexpr int BM = C::BM, BN = C::BN, TM = C::TM, TN = C::TN, S = C::S;
    constexpr int DMA_PER_STAGE = C::LOADS + C::SCALE_LOADS;   // load instructions per wave and stage
    static_assert(!SW || (W8A8 && !KTAIL), "scale windows: W8A8 with K % 512 == 0");
    using Stage = GemmStage<W8A8, SW>;
    __shared__ __attribute__((aligned(16))) Stage st[S];
    __shared__ __attribute__((aligned(16))) ScaleWin<SW> win;
    __shared__ float s_rs[W8A8 ? 1 : BM + BN];                 // FP8: token scales, then weight-row scales

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar branches, SGPR resources
    const int wm = wv % C::WM, wn = wv / C::WM;
    // Tile order.  Workgroups are handed to the 8 XCDs round-robin by linear
    // id, and each XCD has its own L2.  Workgroup b runs on XCD b % 8, and
    // XCD j's workgroups take a contiguous range of tiles in M-fastest order:
    // the ones that share an L2 at the same time cover all M tiles of a few
    // N tiles, so each panel slice enters that L2 about once.
    const int tiles_m = (M + BM - 1) / BM;
    const int b = blockIdx.x;
    const int xq = (int)gridDim.x / 8, xr = (int)gridDim.x % 8;   // XCD j gets xq + (j < xr) tiles
    const int t = (b % 8) * xq + min(b % 8, xr) + b / 8;
    const int m0 = (t % tiles_m) * BM;
    const int n0 = (t / tiles_m) * BN;
    const int G = K >> 6;                       // W8A8: 64-channel groups, two per stage
    const int nsteps = (K + GB_K - 1) / GB_K;
    const int rows_a = min(M - m0, BM);
    const int rows_b = min(N - n0, BN);

    // Buffer ranges start at the tile: rows past M / N fall outside them.
    const v4u ra = buffer_desc(A + (int64_t)m0 * K, (uint32_t)(rows_a * K));
    const v4u rb = buffer_desc(W + (int64_t)n0 * K, (uint32_t)(rows_b * K));

    // Panel layout in LDS: row r of a panel at byte 128 r, its 16-byte piece
    // c (columns k0 + 16 c + [0, 16)) in slot c ^ ((r >> 1) & 7).  Panel
    // loads cover 8 rows each: A rows first, then B rows; wave wv issues loads
    // wv * LOADS + [0, LOADS).  Lane L writes slot L % 8 of row L / 8 of its
    // load, so eight lanes read one row's 128 contiguous bytes (one whole
    // cache line).  The XOR keeps fragment reads conflict-free (see frag_off).
    const int lslot = lane & 7;
    int voff_ld[C::LOADS];
    uint32_t lds_ld_a[C::LOADS];   // LDS byte offset within the stage
    int lk_ld[C::LOADS];           // column of the lane's piece within the stage
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
        const int q = wv * C::LOADS + i;                  // wave-uniform
        const int rq = q < BM / 8 ? q : q - BM / 8;       // load index within its panel
        const int r = 8 * rq + (lane >> 3);               // row within the panel
        lk_ld[i] = 16 * (lslot ^ ((r >> 1) & 7));
        voff_ld[i] = r * K + lk_ld[i];
        lds_ld_a[i] = (q < BM / 8) ? (uint32_t)(1024 * q) : (uint32_t)(BM * GB_K + 1024 * rq);
    }
    // W8A8 scale loads, two per wave: slot z = 2 wv + u.  Slots [0, 2 BM/64)
    // load activation scales (group h = z / (BM/64) of the stage, rows
    // 64 (z % (BM/64)) + lane), the next 2 BN/64 slots weight scales alike,
    // and the rest issue empty loads into sink, so that every wave issues the
    // same number of loads per stage.
    constexpr int NAS = W8A8 ? 2 * (BM / 64) : 0, NWS = W8A8 ? 2 * (BN / 64) : 0;
    v4u rs = ra;
    int voff_s[2] = {GB_OOB, GB_OOB}, grp_s[2] = {0, 0}, sz_s = 0;
    uint32_t lds_s[2] = {0, 0};
    if constexpr (W8A8 && SW) {
        // Windows: waves [0, BM/64) load the activation rows 64 wv + lane,
        // the next BN/64 waves the weight rows; lane L writes LDS bytes
        // 16 L + [0, 16) of its 64-row block.
        if (wv < BM / 64) {
            rs = buffer_desc(a_scale + (int64_t)m0 * G, (uint32_t)(rows_a * G * 4));
            voff_s[0] = (64 * wv + lane) * G * 4;
            lds_s[0] = (uint32_t)(1024 * wv);
            sz_s = 4;
        } else if (wv < BM / 64 + BN / 64) {
            rs = buffer_desc(w_scale + (int64_t)n0 * G, (uint32_t)(rows_b * G * 2));
            voff_s[0] = (64 * (wv - BM / 64) + lane) * G * 2;
            lds_s[0] = (uint32_t)(1024 * (wv - BM / 64));
            sz_s = 2;
        }
    } else if constexpr (W8A8) {
        if (2 * wv < NAS) {
            rs = buffer_desc(a_scale + (int64_t)m0 * G, (uint32_t)(rows_a * G * 4));
            sz_s = 4;
        } else if (2 * wv < NAS + NWS) {
            rs = buffer_desc(w_scale + (int64_t)n0 * G, (uint32_t)(rows_b * G * 2));
            sz_s = 2;
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int z = 2 * wv + u;
            if (z < NAS) {
                const int h = z / (BM / 64), jj = z % (BM / 64);
                voff_s[u] = (64 * jj + lane) * G * 4;
                grp_s[u] = h;
                lds_s[u] = (uint32_t)(offsetof(Stage, as) + 4 * (h * BM + 64 * jj));
            } else if (z < NAS + NWS) {
                const int h = (z - NAS) / (BN / 64), jj = (z - NAS) % (BN / 64);
                voff_s[u] = (64 * jj + lane) * G * 2;
                grp_s[u] = h;
                lds_s[u] = (uint32_t)(offsetof(Stage, ws) + 4 * (h * BN + 64 * jj));
            } else {
                lds_s[u] = (uint32_t)(offsetof(Stage, sink) + 256 * u);
            }
        }
    }

    // Loads [lo, hi) of stage s (and, with lo == 0, its scale loads).  The
    // loops issue a stage's loads in two parts after MFMAs have been queued:
    // a wave blocks while the address unit takes its loads (64 per CU and
    // stage), so issuing them all right after the barrier would leave the
    // matrix unit idle.
    auto issue = [&](Stage& Sg, int s, int lo, int hi) {
        const uint32_t base = lds_addr(&Sg);
        const int k0 = s < nsteps ? s * GB_K : GB_OOB;   // stages past the end load nothing
#pragma unroll
        for (int i = 0; i < C::LOADS; ++i) {
            if (i < lo || i >= hi) continue;
            const int q = wv * C::LOADS + i;
            int vo = voff_ld[i] + k0;
            if constexpr (KTAIL) {
                if (k0 + lk_ld[i] >= K) vo = GB_OOB;          // K % 16 == 0: pieces are whole
            }
            lds_dma<16>(q < BM / 8 ? ra : rb, base + lds_ld_a[i], vo);
        }
        if constexpr (W8A8 && SW) {
            // Stage s = 2w issues activation window w (stages 2w, 2w + 1),
            // stage s = 4v weight window v (stages 4v .. 4v + 3).  A window
            // goes out with its first stage's panels, two stages ahead of its
            // use, into the slot whose last reader every wave has passed.
            if (lo != 0) return;
            const bool live = s < nsteps;
            if (sz_s == 4 && (s & 1) == 0) {
                const int w = s >> 1;
                lds_dma<16>(rs, lds_addr(&win.as[w & 1][0]) + lds_s[0], live ? voff_s[0] + 16 * w : GB_OOB);
            } else if (sz_s == 2 && (s & 3) == 0) {
                const int v = s >> 2;
                lds_dma<16>(rs, lds_addr(&win.ws[v & 1][0]) + lds_s[0], live ? voff_s[0] + 16 * v : GB_OOB);
            }
        } else if constexpr (W8A8) {
            if (lo != 0) return;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int g = 2 * s + grp_s[u];                 // past the last group: an empty load
                const bool live = voff_s[u] < GB_OOB && g < G;
                if (sz_s == 4) lds_dma<4>(rs, base + lds_s[u], live ? voff_s[u] + 4 * g : GB_OOB);
                else lds_dma<2>(rs, base + lds_s[u], live ? voff_s[u] + 2 * g : GB_OOB);
            }
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
    // wave (16 lanes, 16 rows, one piece) r & 1 and the XOR spread the rows
    // over all 16 four-bank groups.
    auto frag_off = [&](int rt, int c0) {
        const int r = rt + (lane & 31);
        return 128 * r + 16 * ((c0 + (lane >> 5)) ^ ((r >> 1) & 7));
    };
    const int wr0 = 32 * TM * wm;       // first panel row of the wave, A
    const int wc0 = 32 * TN * wn;       // ... and B

    // W8A8.  d holds 12582912 + P (as float bits) for the wave's tiles of one
    // group.  mfma_group fills it for group gh of stage Mst.
    v16i bias = {0x4B400000, 0x4B400000, 0x4B400000, 0x4B400000, 0x4B400000, 0x4B400000,
                 0x4B400000, 0x4B400000, 0x4B400000, 0x4B400000, 0x4B400000, 0x4B400000,
                 0x4B400000, 0x4B400000, 0x4B400000, 0x4B400000};
    v16i d[W8A8 ? TM : 1][W8A8 ? TN : 1];
    auto load_frags = [&](const Stage& Mst, int mgh, v4i (&af)[2][TM], v4i (&bf)[2][TN]) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
                af[h][i] = *reinterpret_cast<const v4i*>(&Mst.a[frag_off(wr0 + 32 * i, 4 * mgh + 2 * h)]);
#pragma unroll
            for (int j = 0; j < TN; ++j)
                bf[h][j] = *reinterpret_cast<const v4i*>(&Mst.b[frag_off(wc0 + 32 * j, 4 * mgh + 2 * h)]);
        }
    };
    auto mfma_group = [&](const Stage& Mst, int mgh) {
        v4i af[2][TM], bf[2][TN];
        load_frags(Mst, mgh, af, bf);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                d[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[0][i], bf[0][j], bias, 0, 0, 0);
                d[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[1][i], bf[1][j], d[i][j], 0, 0, 0);
            }
    };
    // One group step: rescale group g (group rgh of stage R) from d,
    //     acc += (P * ws) * as,
    // and, with MF, refill d tile by tile with the next group (group mgh of
    // stage Mst): the matrix unit works on tile t while the vector ALU
    // rescales tile t + 1, and only one set of group sums is live.  The MFMAs
    // have no memory effects, so the compiler would otherwise hoist them all
    // ahead of the rescale (keeping old and new sums live together): the
    // empty asm takes the tile's rescaled acc as input and passes the bias
    // operand through, which pins the tile's MFMAs after its rescale.
    auto group_step = [&](auto mf, const Stage& R, int rgh, int g, const Stage& Mst, int mgh,
                          auto after_row) {
        constexpr bool MF = decltype(mf)::value;
        v4i af[2][TM], bf[2][TN];
        if constexpr (MF) load_frags(Mst, mgh, af, bf);
        float wsf[TN], wsc[TN], asr[TM];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int col = wc0 + 32 * j + (lane & 31);
            if constexpr (SW) wsf[j] = f16_bits_to_f32(win.ws[(g >> 3) & 1][8 * col + (g & 7)]);
            else wsf[j] = f16_bits_to_f32(R.ws[rgh * BN + col] & 0xFFFFu);
            wsc[j] = -12582912.0f * wsf[j];
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int row = wr0 + 32 * i + row_scale_lane_row(lane);
            if constexpr (SW) asr[i] = win.as[(g >> 2) & 1][4 * row + (g & 3)];
            else asr[i] = R.as[rgh * BM + row];
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                rescale_tile(acc[i][j], d[i][j], wsf[j], wsc[j], asr[i], std::make_integer_sequence<int, 16>{});
                if constexpr (SUMS) {
                    const int n = n0 + wc0 + 32 * j + (lane & 31);
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int m = m0 + wr0 + 32 * i + d_row(lane, e);
                        if (m < M && n < N) group_sums[((int64_t)m * N + n) * G + g] = d[i][j][e] - 0x4B400000;
                    }
                }
                if constexpr (MF) {
                    asm volatile("" : "+v"(bias) : "v"(acc[i][j]));
                    d[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[0][i], bf[0][j], bias, 0, 0, 0);
                    d[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[1][i], bf[1][j], d[i][j], 0, 0, 0);
                }
            }
            after_row(i);
        }
    };

    // FP8, one stage.  For column pair p each lane reads 16 consecutive codes
    // of its row (k = 32 p + 16 (lane / 32) + [0, 16)) in one conflict-free
    // read and feeds bytes [0, 8) to one 32x32x16 MFMA and bytes [8, 16) to a
    // second.  The first MFMA thus sums k in {32p + [0,8), 32p + 16 + [0,8)},
    // the second the other 16: the A and B fragments use the same lane -> k
    // assignment, so the two MFMAs together form the exact dot product over
    // the 32 columns.
    auto compute_fp8 = [&](const Stage& Sg, auto after_pair) {
        constexpr int NP = GB_K / 32;
        v4u ca[TM], cb[TN];
        auto read_pair = [&](int p, v4u (&xa)[TM], v4u (&xb)[TN]) {
#pragma unroll
            for (int i = 0; i < TM; ++i) xa[i] = *reinterpret_cast<const v4u*>(&Sg.a[frag_off(wr0 + 32 * i, 2 * p)]);
#pragma unroll
            for (int j = 0; j < TN; ++j) xb[j] = *reinterpret_cast<const v4u*>(&Sg.b[frag_off(wc0 + 32 * j, 2 * p)]);
        };
        // the BF16 fragments of half hh (bytes [8 hh, 8 hh + 8) of each lane's 16 codes)
        auto convert = [&](const v4u (&xa)[TM], const v4u (&xb)[TN], int hh, v8bf (&af)[TM], v8bf (&bf)[TN]) {
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const uint32_t w0 = hh ? xa[i].z : xa[i].x, w1 = hh ? xa[i].w : xa[i].y;
                af[i] = __builtin_bit_cast(v8bf, make_uint4(e4m3x2_to_bf16x2<false>(w0, 1.0f),
                                                            e4m3x2_to_bf16x2<true>(w0, 1.0f),
                                                            e4m3x2_to_bf16x2<false>(w1, 1.0f),
                                                            e4m3x2_to_bf16x2<true>(w1, 1.0f)));
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const uint32_t w0 = hh ? xb[j].z : xb[j].x, w1 = hh ? xb[j].w : xb[j].y;
                bf[j] = __builtin_bit_cast(v8bf, make_uint4(e4m3x2_to_bf16x2<false>(w0, 1.0f),
                                                            e4m3x2_to_bf16x2<true>(w0, 1.0f),
                                                            e4m3x2_to_bf16x2<false>(w1, 1.0f),
                                                            e4m3x2_to_bf16x2<true>(w1, 1.0f)));
            }
        };
        auto mfmas = [&](const v8bf (&af)[TM], const v8bf (&bf)[TN]) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
        };
        read_pair(0, ca, cb);
        if constexpr (!KTAIL && TM == 2 && TN == 4) {
            // Software-pipelined by half column pairs: the converts of the next
            // half (of this pair, or the first half of the next pair, whose
            // codes were read one pair ahead) are issued among the 8 MFMAs of
            // the current half, 3 converts after each MFMA (sched_group_barrier),
            // so the matrix unit is fed while the vector ALU converts.
            v8bf af[2][TM], bf[2][TN];
            convert(ca, cb, 0, af[0], bf[0]);
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                v4u na[TM], nb[TN];
                if (p + 1 < NP) read_pair(p + 1, na, nb);
                asm volatile("" : "+v"(ca[0]), "+v"(ca[1]), "+v"(cb[0]), "+v"(cb[1]), "+v"(cb[2]), "+v"(cb[3]) :: "memory");
                // half 0 of pair p multiplied, half 1 converted
                convert(ca, cb, 1, af[1], bf[1]);
                mfmas(af[0], bf[0]);
#pragma unroll
                for (int g = 0; g < TM * TN; ++g) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);    // three VALU
                }
                __builtin_amdgcn_sched_barrier(0);
                // half 1 of pair p multiplied, half 0 of pair p + 1 converted
                if (p + 1 < NP) convert(na, nb, 0, af[0], bf[0]);
                mfmas(af[1], bf[1]);
                if (p + 1 < NP) {
#pragma unroll
                    for (int g = 0; g < TM * TN; ++g) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);   // pair p's MFMAs stay ahead of pair p + 1's wait
                after_pair(p);
                if (p + 1 < NP) {
#pragma unroll
                    for (int i = 0; i < TM; ++i) ca[i] = na[i];
#pragma unroll
                    for (int j = 0; j < TN; ++j) cb[j] = nb[j];
                }
            }
        } else {
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                // The reads of pair p + 1 go out before pair p is converted and
                // multiplied, so their latency hides behind this pair's MFMAs.
                // The empty asm (a memory clobber, with pair p's codes passed
                // through it) keeps the compiler from sinking those reads below
                // the MFMAs.
                v4u na[TM], nb[TN];
                if (p + 1 < NP) read_pair(p + 1, na, nb);
                if constexpr (TM == 2 && TN == 4)
                    asm volatile("" : "+v"(ca[0]), "+v"(ca[1]), "+v"(cb[0]), "+v"(cb[1]), "+v"(cb[2]), "+v"(cb[3]) :: "memory");
                else if constexpr (TM == 2 && TN == 2)
                    asm volatile("" : "+v"(ca[0]), "+v"(ca[1]), "+v"(cb[0]), "+v"(cb[1]) :: "memory");
                else
                    static_assert(TM == 2 && (TN == 2 || TN == 4), "operand list of the ordering asm");
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    v8bf af[TM], bf[TN];
                    convert(ca, cb, hh, af, bf);
                    mfmas(af, bf);
                }
                __builtin_amdgcn_sched_barrier(0);   // pair p's MFMAs stay ahead of pair p + 1's wait
                after_pair(p);
                if (p + 1 < NP) {
#pragma unroll
                    for (int i = 0; i < TM; ++i) ca[i] = na[i];
#pragma unroll
                    for (int j = 0; j < TN; ++j) cb[j] = nb[j];
                }
            }
        }
    };

    auto sync_stage = [&]() {
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

#pragma unroll
    for (int s = 0; s < S - 1; ++s) issue(st[s], s, 0, C::LOADS);
    if constexpr (!W8A8) {
        for (int i = tid; i < BM + BN; i += 64 * C::NW) {
            s_rs[i] = i < BM ? (i < rows_a ? a_scale[m0 + i] : 0.f)
                             : (i - BM < rows_b ? bf16_bits_to_f32(w_scale[n0 + i - BM]) : 0.f);
        }
        __syncthreads();
    }

    if constexpr (W8A8) {
        // Stage s holds groups 2s and 2s + 1.  Iteration s: rescale(2s) with
        // the MFMAs of 2s + 1 (both stage s); wait for stage s + 1 and pass the
        // barrier; refill the buffer of stage s - 1 (whose last reader, the
        // step of group 2s - 1, every wave has finished) with stage s + S - 1;
        // rescale(2s + 1) from stage s with the MFMAs of 2s + 2 from stage
        // s + 1.  Those MFMAs run unconditionally: past the last group the
        // stage holds zeros and d is not used.  An odd last group (K % 128 ==
        // 64) is rescaled after the loop.  With S = 3 one stage is in flight
        // while two are read.
        static_assert(S == 3, "ring of three stages");
        // Stage 1 (odd) carries no scale window: its loads are the last LOADS.
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(SW ? C::LOADS : DMA_PER_STAGE) : "memory");
        sync_stage();
        mfma_group(st[0], 0);
        const int full = G >> 1;                       // stages with two groups
        auto no_hook = [](int) {};
        for (int s = 0; s < full; ++s) {
            group_step(std::true_type{}, st[s % S], 0, 2 * s, st[s % S], 1, no_hook);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // also drains group-sum stores
            sync_stage();
            Stage& nxt = st[(s + S - 1) % S];
            group_step(std::true_type{}, st[s % S], 1, 2 * s + 1, st[(s + 1) % S], 0, [&](int i) {
                if (i == 0) issue(nxt, s + S - 1, 0, C::LOADS / 2);
                if (i == TM - 1) issue(nxt, s + S - 1, C::LOADS / 2, C::LOADS);
            });
        }
        if (G & 1) group_step(std::false_type{}, st[full % S], 0, 2 * full, st[full % S], 0, no_hook);
    } else {
        // Ring: before consuming stage s this wave waits for its own loads of
        // stage s (the S - 2 later stages may stay in flight); the barrier
        // makes every wave's loads visible and shows that buffer (s - 1) % S,
        // refilled next, is no longer read.
        for (int s = 0; s < nsteps; ++s) {
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(DMA_PER_STAGE * (S - 2)) : "memory");
            sync_stage();
            Stage& nxt = st[(s + S - 1) % S];
            compute_fp8(st[s % S], [&](int p) {
                if (p == 0) issue(nxt, s + S - 1, 0, C::LOADS / 2);
                if (p == 1) issue(nxt, s + S - 1, C::LOADS / 2, C::LOADS);
            });
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // drain the empty tail loads

    // Output.  A tile inside the matrix (every tile of the prefill shapes)
    // writes without per-element bounds checks, each output type in a loop of
    // its own: checked per element, every store had become a branch of its own
    // (64 per wave and tile).
    auto value = [&](int i, int j, int e, int ml, int nl) {
        float v = acc[i][j][e];
        if constexpr (!W8A8) v = (v * s_rs[ml]) * s_rs[BM + nl];
        return v;
    };
    if (m0 + BM <= M && n0 + BN <= N) {
        if (bf16_out) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int nl = wc0 + 32 * j + (lane & 31);
                    uint16_t* yc = reinterpret_cast<uint16_t*>(y) + (int64_t)m0 * N + n0 + nl;
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int ml = wr0 + 32 * i + d_row(lane, e);
                        yc[(int64_t)ml * N] = (uint16_t)f32_to_bf16_rne(value(i, j, e, ml, nl));
                    }
                }
        } else {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int nl = wc0 + 32 * j + (lane & 31);
                    float* yc = reinterpret_cast<float*>(y) + (int64_t)m0 * N + n0 + nl;
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int ml = wr0 + 32 * i + d_row(lane, e);
                        yc[(int64_t)ml * N] = value(i, j, e, ml, nl);
                    }
                }
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int nl = wc0 + 32 * j + (lane & 31);
            const int n = n0 + nl;
            if (n >= N) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int ml = wr0 + 32 * i + d_row(lane, e);
                const int m = m0 + ml;
                if (m >= M) continue;
                const float v = value(i, j, e, ml, nl);
                if (bf16_out) reinterpret_cast<uint16_t*>(y)[(int64_t)m * N + n] = (uint16_t)f32_to_bf16_rne(v);
                else reinterpret_cast<float*>(y)[(int64_t)m * N + n] = v;
            }
        }
}

template <bool W8A8, bool SUMS, bool KTAIL, bool SW = false>
static hipError_t launch_gemm_t(const uint8_t* A, const float* a_scale, const uint8_t* W, const uint16_t* w_scale,
                                int64_t M, int64_t N, int64_t K, bool bf16_out, void* y, int32_t* sums,
                                hipStream_t stream) {
    using C = GemmCfg<W8A8>;
    const int64_t tiles = ((N + C::BN - 1) / C::BN) * ((M + C::BM - 1) / C::BM);
    if (tiles >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    gemm_kernel<W8A8, SUMS, KTAIL, SW><<<dim3((unsigned)tiles), 64 * C::NW, 0, stream>>>(A, a_scale, W, w_scale, (int)M, (int)N, (int)K,
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
    const bool tail = K % GB_K != 0;   // an odd number of groups: the last stage holds one
    const bool win = K % 512 == 0;     // scale windows (16-byte aligned scale rows)
    if (group_sums != nullptr)
        return win ? launch_gemm_t<true, true, false, true>(A, a_scale, W, w_scale, M, N, K, bf16_out, y, group_sums, stream)
             : tail ? launch_gemm_t<true, true, true>(A, a_scale, W, w_scale, M, N, K, bf16_out, y, group_sums, stream)
                    : launch_gemm_t<true, true, false>(A, a_scale, W, w_scale, M, N, K, bf16_out, y, group_sums, stream);
    return win ? launch_gemm_t<true, false, false, true>(A, a_scale, W, w_scale, M, N, K, bf16_out, y, nullptr, stream)
         : tail ? launch_gemm_t<true, false, true>(A, a_scale, W, w_scale, M, N, K, bf16_out, y, nullptr, stream)
                : launch_gemm_t<true, false, false>(A, a_scale, W, w_scale, M, N, K, bf16_out, y, nullptr, stream);
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
