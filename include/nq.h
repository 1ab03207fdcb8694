/*
 * nq.h — quantized-weight linear projection for AMD MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels.  Packed low-bit weights are decoded
 * on the fly against their stored scales and multiplied by BF16 activations:
 * a bandwidth-bound GEMV / skinny GEMM for decode and verify steps (a few
 * tokens) and MFMA GEMMs for prefill chunks.
 *
 * Sources (the web pages the method is described on), cited by title and
 * section below:
 *   [MXFP8 card]   "Qwen3.8-27B "MXFP8-CRACK" — NInfer artifact"
 *   [FP8 card]     "Qwen3.8-27B EfficientThink-Uncensored FP8 for NInfer"
 *   [NVFP4 card]   "Qwen3.8-27B-NVIDIA-NVFP4-NInferV3"
 *   [RTX5080 card] "Qwen3.8-27B for NInfer — RTX 5080 16 GB, true 128K + Vision"
 *   [int8 card]    "Qwen3.8-27B, NInfer int8-prefill artifact for the RTX 4090"
 *
 * Conventions for every entry point
 *   - Matrices are dense and row-major.  A weight matrix is [N][K]: N output
 *     rows, K input channels; activations are [T][K] (T tokens); outputs are
 *     [T][N]; y[t][n] = sum_k x[t][k] * W[n][k].  Group and block axes run
 *     along K.
 *   - BF16 / FP16 values are passed as their 16-bit patterns (uint16_t), FP32
 *     as float, E4M3 codes as uint8_t (OCP E4M3, "e4m3fn": bias 7, largest
 *     finite 448, S.1111.111 is NaN).
 *   - All data pointers are DEVICE pointers and must be 16-byte aligned.  The
 *     caller owns every buffer; the library allocates nothing and keeps no
 *     state between calls.  `stream` is a hipStream_t (NULL = the default
 *     stream); every call only enqueues work on it and returns without
 *     synchronizing.  Output buffers must not overlap inputs.
 *   - A buffer whose size is zero may be NULL.  Calls with nothing to compute
 *     (N == 0 or T == 0) return NQ_OK without launching.
 *   - Every call validates all arguments before enqueuing anything and returns
 *     the first failing check; on any error nothing is written.  No C++
 *     exception crosses this interface.
 */
#ifndef NQ_H
#define NQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NQ_ABI_VERSION 1

typedef enum {
    NQ_OK = 0,
    NQ_ERR_NULL = 1,    /* a required pointer is NULL */
    NQ_ERR_SHAPE = 2,   /* a size is negative, a divisibility rule fails, or a grid does not match */
    NQ_ERR_ALIGN = 3,   /* a pointer is not 16-byte aligned */
    NQ_ERR_FORMAT = 4,  /* an enum value is unknown */
    NQ_ERR_RANGE = 5,   /* a row range is empty or outside [0, N] */
    NQ_ERR_HIP = 6,     /* the HIP runtime reported an error when enqueuing */
    NQ_ERR_SCRATCH = 7  /* the call needs more scratch than the library's static array holds */
} nq_status;

typedef enum { NQ_OUT_F32 = 0, NQ_OUT_BF16 = 1 } nq_out;

typedef enum {
    NQ_W_Q4G64_F16S = 0,  /* 4-bit two's-complement codes, element 2j in the low nibble of byte j
                             ([N][K/2] bytes), one FP16 scale per 64 elements ([N][K/64]) */
    NQ_W_Q8G32_F16S = 1,  /* int8 codes [N][K], one FP16 scale per 32 elements [N][K/32] */
    NQ_W_Q8G64_F16S = 2,  /* int8 codes [N][K], one FP16 scale per 64 elements [N][K/64] */
    NQ_W_MXFP8_G32 = 3,   /* four E4M3 codes per little-endian u32 word ([N][K/4]), one UE8M0
                             byte per 32 elements ([N][K/32]) worth 2^(b-127); b = 255 is NaN */
    NQ_W_BF16 = 4,        /* BF16 weights [N][K], no scales */
    NQ_W_Q3G64_F16S = 5,  /* 3-, 5- and 6-bit two's-complement codes as a dense little-endian bit stream */
    NQ_W_Q5G64_F16S = 6,  /* along each row: element j at bits [b j, b j + b) of the row's K b / 8 bytes */
    NQ_W_Q6G64_F16S = 7   /* (b = 4 would be the Q4 layout); one FP16 scale per 64 elements [N][K/64] */
} nq_wfmt;

typedef enum { NQ_ROUTE_BF16 = 0, NQ_ROUTE_A8 = 1, NQ_ROUTE_A8_DECODE = 2 } nq_route_kind;

/* Flags of the routed calls (nq_route, nq_linear_*): which steps may run with
 * int8 activations.  NQ_A8_PREFILL: steps of 129 tokens or more (the W8A8
 * GEMM); NQ_A8_DECODE: steps of at most 128 tokens (the A8 decode GEMV, for
 * the MLP projections of an engine that enables it).  1 keeps the meaning of
 * the former boolean argument. */
#define NQ_A8_PREFILL 1
#define NQ_A8_DECODE 2

/* Version of this interface (NQ_ABI_VERSION). */
int nq_abi_version(void);

/* Static text for a status code (never NULL). */
const char* nq_status_string(int status);

/*
 * MXFP8 decode.  [MXFP8 card, "How it was built", item 1]: four E4M3 codes
 * per 32-bit word, one UE8M0 scale byte 2^(b-127) per 32-element group, decoded
 * to BF16.
 *   words  [N][K/4] u32, element 4j+i in bits 8i..8i+7 of word j
 *   e8m0   [N][K/32] u8
 *   w_out  [N][K] FP32 (out_dt = NQ_OUT_F32) or BF16 bits (NQ_OUT_BF16): the
 *          exact value e4m3(code) * 2^(b-127) rounded once to nearest-even
 *          (overflow to infinity; NaN codes or b = 255 give the quiet NaN
 *          0x7FC00000 / 0x7FC0).
 * Errors: K % 32 != 0 -> NQ_ERR_SHAPE.
 */
nq_status nq_decode_mxfp8(const uint32_t* words, const uint8_t* e8m0, int64_t N, int64_t K,
                          int out_dt, void* w_out, void* stream);

/*
 * MLX affine int8 decode.  [MXFP8 card, "How it was built", item 2]: uint8
 * codes with one FP16 scale and one FP16 bias per 128-element group decode as
 * w = q * scale + bias, written as BF16.
 *   codes          [N][K] u8 (16-byte aligned)
 *   scales, biases [N][K/128] FP16 bits, groups along K
 *   w_out          [N][K] FP32 (out_dt = NQ_OUT_F32) or BF16 bits (NQ_OUT_BF16,
 *                  16-byte aligned): the exact value of q * scale + bias
 *                  rounded once to nearest-even (NaN -> 0x7FC00000 / 0x7FC0).
 * Errors: K % 128 != 0 -> NQ_ERR_SHAPE.
 */
nq_status nq_decode_mlx_affine_int8(const uint8_t* codes, const uint16_t* scales, const uint16_t* biases,
                                    int64_t N, int64_t K, int out_dt, void* w_out, void* stream);

/*
 * Block-128x128 E4M3 -> one BF16 scale per output row ("fp8_row_maxabs").
 * [FP8 card, "Conversion and verification", "Block-wise to per-row,
 * exactly"]: each code is decoded in FP32 as e4m3(code) times the scale of its
 * 128x128 block (weight_scale_inv), the grid is checked against the code shape,
 * the values are re-encoded with one BF16 scale per row, and a row range reads
 * only the block rows it touches.
 *   codes      [N][K] E4M3 codes
 *   wsi        [gr][gc] FP32, gr = ceil(N/128), gc = ceil(K/128)
 *   rows       [row_begin, row_end) of the N rows are re-encoded
 *   out_codes  [row_end-row_begin][K]: e4m3_rne_sat(fp32(v / s)) where v is the
 *              FP32 decoded value and s the row scale
 *   out_scale  [row_end-row_begin] BF16 bits: s = bf16_rne(fp32(max|v| / 448))
 * A row of zeros gets s = +0 and keeps its signed zero codes; a row holding a
 * NaN code gets s = NaN (0x7FC0) and NaN codes (0x7F).  A row so small that s
 * is a BF16 subnormal (max|v| below ~5.3e-36) or rounds to zero follows the
 * same rule: quotients beyond 448 saturate to +-448 (code 0x7E / 0xFE).
 * Errors: gr/gc mismatch -> NQ_ERR_SHAPE; bad row range -> NQ_ERR_RANGE.
 */
nq_status nq_reencode_block128_to_row(const uint8_t* codes, const float* wsi, int64_t N, int64_t K,
                                      int64_t gr, int64_t gc, int64_t row_begin, int64_t row_end,
                                      uint8_t* out_codes, uint16_t* out_scale, void* stream);

/*
 * BF16 -> row-scaled FP8, the same per-row encoding as above applied to BF16
 * values.  [NVFP4 card, "How it was created"]: the token embedding goes from
 * its BF16 source to row-scale FP8.
 *   w          [N][K] BF16 bits;  out_codes [N][K];  out_scale [N] BF16 bits
 */
nq_status nq_encode_fp8row_bf16(const uint16_t* w, int64_t N, int64_t K, uint8_t* out_codes,
                                uint16_t* out_scale, void* stream);

/*
 * Int8 activation quantization for the W8A8 prefill route.  [int8 card, "What
 * changes"]: per token and per 64 channels, scale = amax / 127.
 *   x      [T][K] BF16 bits, K % 64 == 0
 *   q      [T][K] int8: clamp(rne(fp32(x / s)), -127, 127); an all-zero group
 *          (s = 0) gives 0, a NaN quotient gives 0
 *   scale  [T][K/64] FP32: s = fp32(amax / 127) (IEEE division)
 */
nq_status nq_quantize_act_int8_g64(const uint16_t* x, int64_t T, int64_t K, int8_t* q, float* scale,
                                   void* stream);

/*
 * Per-token E4M3 activation quantization for the FP8-activation GEMM.  The
 * pages name FP8-activation routes ([FP8 card, "Conversion and verification",
 * "Hardware fit"]) without describing their quantizer; this is the reading
 * used here: s = fp32(amax_t / 448), codes e4m3_rne_sat(fp32(x / s)), an
 * all-zero token gets s = 0 and keeps its signed zeros.
 *   x [M][K] BF16 bits;  codes [M][K];  scale [M] FP32
 */
nq_status nq_quantize_act_fp8_row(const uint16_t* x, int64_t M, int64_t K, uint8_t* codes, float* scale,
                                  void* stream);

/*
 * Decode GEMV on row-scaled FP8 weights, BF16 activations, FP32 accumulation.
 * [FP8 card, introduction]: one BF16 scale per output row; [int8 card, "What
 * changes"]: decode and verify steps use BF16 activations; [NVFP4 card, "How
 * it was created"]: weights are dequantized on the fly against their scales.
 *   w        [N][K] E4M3 codes;  w_scale [N] BF16 bits;  x [T][K] BF16 bits
 *   y        [T][N] FP32 or BF16 bits: y = s[n] * sum_k x[t][k] * e4m3(w[n][k]);
 *            a BF16 output is the RNE rounding of the FP32 result
 *   workspace, workspace_bytes   optional device scratch (see
 *            nq_gemv_workspace_bytes); NULL / 0 is always valid
 * Any K >= 0 and any T >= 0 are accepted.
 */
nq_status nq_gemv_fp8row(const uint8_t* w, const uint16_t* w_scale, const uint16_t* x, int64_t T,
                         int64_t N, int64_t K, int out_dt, void* y, void* workspace,
                         int64_t workspace_bytes, void* stream);

/*
 * Bytes of optional workspace that let the decode GEMVs split K across
 * workgroups for a (format, T, N, K) call (0 when the call does not use one).
 * With a workspace of at least this size the K range of each 64-row tile is
 * divided among several workgroups; each writes an FP32 partial and the last
 * one to finish (an atomic counter per tile) sums the partials in a fixed
 * order, so results stay deterministic.  Without it (NULL, or smaller) one
 * workgroup covers the whole K range of its tile; both are correct, the
 * split is faster when N is small.  The workspace must be zero-filled once
 * before its first use; every call leaves it zero-filled again.  Calls that
 * share a workspace must be ordered (the same stream); the workspace holds
 * no data between calls.  `fmt` is an nq_wfmt, or -1 for row-scaled FP8.
 */
int64_t nq_gemv_workspace_bytes(int fmt, int64_t T, int64_t N, int64_t K);

/*
 * Packed weight layout for the decode GEMVs.  A one-time permutation of a
 * row-major weight matrix (codes only; scales stay as they are) into the
 * order in which the GEMV kernels stream it: rows in blocks of 16 (the last
 * block zero-padded); chunk-major: for every chunk of 256 columns, for every
 * row block, for every 8- or 16-byte piece of the chunk, the pieces of all 64
 * lanes of a wavefront stored contiguously (lane 16 g + i holds row i of the
 * block, lane group g).  Pieces per row and chunk: FP8 / MXFP8 / Q8G64 four
 * of 16 B (64 columns each, lane group g at byte 16 g), Q4G64 four of 8 B,
 * Q8G32 eight of 8 B (32 columns, byte 8 g), BF16 eight of 16 B.  Q3 / Q5 /
 * Q6: per chunk and row block, each lane's 8 b bytes (the codes 64 q + 16 g +
 * [0, 16) of its row for q = 0..3, the bit stream's bytes back to back) stored
 * as 16-byte pieces (and an 8-byte tail for b = 3, 5), piece-major.  Every
 * load instruction of the GEMV reads a contiguous 512 B or 1 KiB, and the
 * grid, walking chunk by chunk, sweeps one contiguous window at a time.  The pages store weights in engine-specific tiled
 * layouts too ([NVFP4 card, "How it was created"]: the NVFP4 storage layout
 * works in 128-row tiles).
 *   fmt       an nq_wfmt, or -1 for row-scaled FP8 codes
 *   w         row-major codes as nq_gemv_fp8row / nq_gemv_qgroup take them
 *   w_packed  nq_packed_weight_bytes(fmt, N, K) bytes, caller-owned
 * Errors: K % 256 != 0 (or K == 0 with N > 0) -> NQ_ERR_SHAPE; unknown fmt ->
 * NQ_ERR_FORMAT.
 */
int64_t nq_packed_weight_bytes(int fmt, int64_t N, int64_t K);
nq_status nq_pack_weights(int fmt, const void* w, int64_t N, int64_t K, void* w_packed, void* stream);

/*
 * nq_gemv_fp8row / nq_gemv_qgroup on packed codes (from nq_pack_weights with
 * the same fmt, N and K); every other argument as in the row-major calls, and
 * the results are bit-identical to them.
 */
nq_status nq_gemv_fp8row_packed(const uint8_t* w_packed, const uint16_t* w_scale, const uint16_t* x,
                                int64_t T, int64_t N, int64_t K, int out_dt, void* y, void* workspace,
                                int64_t workspace_bytes, void* stream);
nq_status nq_gemv_qgroup_packed(int fmt, const void* w_packed, const void* w_scales, const uint16_t* x,
                                int64_t T, int64_t N, int64_t K, int out_dt, void* y, void* workspace,
                                int64_t workspace_bytes, void* stream);

/*
 * nq_gemv_fp8row_packed without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The K-split / spread partials and
 * counters go to a static device array of NQ_GEMV_STATIC_SCRATCH_BYTES that
 * the library holds on every GPU it runs on until the process ends; this call
 * allocates nothing and calls no allocating routine.  Each call first clears
 * the counters it uses with a small fill kernel on `stream` (no memset node),
 * then runs the same kernels and plan as nq_gemv_fp8row_packed with a
 * workspace: the results are bit-identical to that call's.  All calls on one
 * GPU share its array, which keeps the last call's partials: calls that
 * overlap on one GPU (different streams, or threads) race and must not be
 * issued.
 * Errors: as nq_gemv_fp8row_packed; NQ_ERR_SCRATCH when the call's plan needs
 * more than NQ_GEMV_STATIC_SCRATCH_BYTES (nq_gemv_workspace_bytes(-1, T, N, K)
 * tells in advance), checked before anything is enqueued.
 */
#define NQ_GEMV_STATIC_SCRATCH_BYTES (8 << 20)
nq_status nq_gemv_fp8row_packed_noalloc(const uint8_t* w_packed, const uint16_t* w_scale, const uint16_t* x,
                                        int64_t T, int64_t N, int64_t K, int out_dt, void* y, void* stream);

/*
 * Decode GEMV on grouped weights (see nq_wfmt for layouts), BF16 activations,
 * FP32 accumulation: y[t][n] = sum_g sc[n][g] * sum_{k in g} x[t][k] * q[n][k].
 * [NVFP4 card, "What is in the file"] (grouped Q4/Q5/Q6/Q8 with FP16 scales,
 * BF16 projections); [RTX5080 card, "Quantization profile"] (Q3/Q4/Q5
 * group-64 with FP16 scales); [MXFP8 card, "How it was built"] (MXFP8).
 *   w_codes, w_scales  per nq_wfmt (w_scales is ignored and may be NULL for BF16)
 * Errors: K not a multiple of the group size -> NQ_ERR_SHAPE; for Q3/Q5/Q6
 * also K % 256 != 0, or code bytes (rows padded to 16) of 2 GiB or more.
 */
nq_status nq_gemv_qgroup(int fmt, const void* w_codes, const void* w_scales, const uint16_t* x,
                         int64_t T, int64_t N, int64_t K, int out_dt, void* y, void* workspace,
                         int64_t workspace_bytes, void* stream);

/*
 * W8A8 prefill GEMM.  [int8 card, "What changes"]: int8 activation codes times
 * int8 weight codes, summed exactly in int32 per 64-channel group; each group
 * sum is scaled by weight_scale x activation_scale in FP32 and the scaled
 * groups are summed.
 *   a_q [M][K] int8, a_scale [M][K/64] FP32 (from nq_quantize_act_int8_g64)
 *   w_q [N][K] int8, w_scale [N][K/64] FP16 bits (Q8 group-64 weights)
 *   y   [M][N] FP32 or BF16 bits
 *   group_sums  NULL, or [M][N][K/64] int32 receiving every exact group sum
 *               (a check hook for small shapes)
 * Errors: K % 64 != 0 -> NQ_ERR_SHAPE.
 */
nq_status nq_gemm_w8a8_g64(const int8_t* a_q, const float* a_scale, const int8_t* w_q,
                           const uint16_t* w_scale, int64_t M, int64_t N, int64_t K, int out_dt,
                           void* y, int32_t* group_sums, void* stream);

/*
 * FP8-activation prefill GEMM on row-scaled FP8 weights.  [FP8 card,
 * "Conversion and verification", "Hardware fit"]: row-scaled FP8 weights feed
 * FP8-activation matrix routes (E4M3 activations times E4M3 weights) rather
 * than a BF16 copy of the weights.  Activations are quantized as
 * nq_quantize_act_fp8_row, into the caller-owned workspaces a_codes [M][K] and
 * a_scale [M] (readable afterwards);
 * y[m][n] = a_scale[m] * w_scale[n] * sum_k e4m3(a_codes[m][k]) * e4m3(w[n][k]).
 * How it is computed here: both E4M3 operands are decoded exactly to BF16 in
 * registers and multiplied on the BF16 matrix units with FP32 accumulation
 * (every product of two E4M3 values is exact in FP32).  The FP8 matrix
 * instructions are not used because their dot products were measured with
 * relative errors of 1.3e-5 .. 5e-5, outside the 1e-5 bound this library keeps.
 * Errors: K % 16 != 0 -> NQ_ERR_SHAPE.
 */
nq_status nq_gemm_fp8row(const uint16_t* x, const uint8_t* w, const uint16_t* w_scale, int64_t M,
                         int64_t N, int64_t K, uint8_t* a_codes, float* a_scale, int out_dt, void* y,
                         void* stream);

/*
 * Route rule.  [int8 card, "What changes"]: a projection permitted to use
 * int8 activations in prefill takes that route only in steps of 129 tokens
 * or more (NQ_ROUTE_A8); decode and verify steps keep the BF16-activation
 * route.  [FP8 card, "Start the server"]: a server variant also runs the MLP
 * with int8 activations in decode; with NQ_A8_DECODE in the flags, steps of
 * at most 128 tokens take the A8 decode GEMV (NQ_ROUTE_A8_DECODE).  The pages
 * give no details of that variant; the arithmetic here is the W8A8 one
 * (per-token-per-64 int8 activations, exact int32 group sums, FP32 rescale).
 * Host-only; returns an nq_route_kind.
 */
int nq_route(int64_t T, int a8_flags);

/*
 * A8 decode GEMV: the W8A8 arithmetic of nq_gemm_w8a8_g64 at decode sizes
 * (any T; tuned for T <= 64), streaming the weights once.
 *   fmt      NQ_W_Q8G64_F16S (int8 codes [N][K]) or NQ_W_Q4G64_F16S (nibbles
 *            [N][K/2], see nq_wfmt); row-major here, or packed by
 *            nq_pack_weights(fmt, ...) for nq_gemv_a8_g64_packed
 *   w_scale  [N][K/64] FP16 bits
 *   a_q, a_scale   [T][K] int8 and [T][K/64] FP32 from nq_quantize_act_int8_g64
 *   y        [T][N] FP32 or BF16 bits:
 *            y[t][n] = sum_g P[t][n][g] * w_scale[n][g] * a_scale[t][g], each
 *            P the exact int32 sum of a 64-channel group; the group terms are
 *            summed in FP32 (a BF16 output is the RNE rounding of it)
 *   workspace, workspace_bytes   optional, as for the BF16 GEMVs
 *            (nq_gemv_a8_workspace_bytes; zero-filled once, left zero-filled)
 * Errors: K % 256 != 0 -> NQ_ERR_SHAPE; another fmt -> NQ_ERR_FORMAT.
 */
int64_t nq_gemv_a8_workspace_bytes(int64_t T, int64_t N, int64_t K);
nq_status nq_gemv_a8_g64(int fmt, const void* w_codes, const uint16_t* w_scale, const int8_t* a_q,
                         const float* a_scale, int64_t T, int64_t N, int64_t K, int out_dt, void* y,
                         void* workspace, int64_t workspace_bytes, void* stream);
nq_status nq_gemv_a8_g64_packed(int fmt, const void* w_packed, const uint16_t* w_scale, const int8_t* a_q,
                                const float* a_scale, int64_t T, int64_t N, int64_t K, int out_dt, void* y,
                                void* workspace, int64_t workspace_bytes, void* stream);

/*
 * The Q8 group-64 projection as an engine step runs it: routed by
 * nq_route(T, a8_flags).  BF16 route: nq_gemv_qgroup(NQ_W_Q8G64_F16S, ...).
 * A8 routes: nq_quantize_act_int8_g64 into the caller-owned workspaces a_q_ws
 * [T][K] and a_scale_ws [T][K/64] (needed only when an A8 route is taken),
 * then nq_gemm_w8a8_g64 (prefill) or nq_gemv_a8_g64 (decode; K % 256 == 0).
 * `workspace` is the optional GEMV workspace (size the larger of
 * nq_gemv_workspace_bytes and nq_gemv_a8_workspace_bytes).
 */
nq_status nq_linear_q8g64(const uint16_t* x, int64_t T, const int8_t* w_q, const uint16_t* w_scale,
                          int64_t N, int64_t K, int a8_flags, int8_t* a_q_ws, float* a_scale_ws,
                          int out_dt, void* y, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * Q4 group-64 codes as int8 (the A8 route's weights).  [int8 card, "What
 * changes"]: in prefill the Q4 codes feed the int8 matrix units exactly.
 *   codes [N][K/2] bytes, two's complement nibbles, low nibble first
 *         (16-byte aligned)
 *   out   [N][K] int8 in [-8, 7] (16-byte aligned)
 * Errors: K % 64 != 0 -> NQ_ERR_SHAPE.
 */
nq_status nq_unpack_q4_to_int8(const uint8_t* codes, int64_t N, int64_t K, int8_t* out, void* stream);

/*
 * The Q4 group-64 projection as an engine step runs it: routed by
 * nq_route(T, a8_flags).  [int8 card, "What changes"]: BF16 route
 * nq_gemv_qgroup(NQ_W_Q4G64_F16S, ...); A8 prefill route:
 * nq_quantize_act_int8_g64 into a_q_ws [T][K] and a_scale_ws [T][K/64], the
 * codes widened by nq_unpack_q4_to_int8 into w_i8_ws [N][K] (caller-owned; a
 * caller that keeps a widened copy can call nq_gemm_w8a8_g64 directly), then
 * nq_gemm_w8a8_g64 with the same FP16 scales; A8 decode route: the same
 * quantization, then nq_gemv_a8_g64 on the Q4 codes as stored (no widened
 * copy; K % 256 == 0).  The A8 workspaces are needed only when their route is
 * taken (w_i8_ws only for the prefill one); `workspace` is the optional GEMV
 * workspace.
 */
nq_status nq_linear_q4g64(const uint16_t* x, int64_t T, const uint8_t* w_codes, const uint16_t* w_scale,
                          int64_t N, int64_t K, int a8_flags, int8_t* a_q_ws, float* a_scale_ws,
                          int8_t* w_i8_ws, int out_dt, void* y, void* workspace, int64_t workspace_bytes,
                          void* stream);

/*
 * Measurement helper: a plain streaming read of `bytes` of device memory (a
 * multiple of 16), nothing computed but a fold of the bytes into one word per
 * workgroup written to sink [nq_stream_read_sink_words()].  It gives the HBM
 * read rate that the weight-streaming GEMVs are compared against: [int8 card,
 * "Files"] notes that decode is bandwidth bound.
 * Errors: bytes % 16 != 0, or bytes of 2 GiB - 16 or more -> NQ_ERR_SHAPE.
 */
int64_t nq_stream_read_sink_words(void);
nq_status nq_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream);

/*
 * Q3 / Q5 / Q6 group-64 codes as int8 (the A8 routes' weights).  [int8 card,
 * "What changes"]: in prefill the low-bit codes feed the int8 matrix units
 * exactly.
 *   fmt   NQ_W_Q3G64_F16S, NQ_W_Q5G64_F16S or NQ_W_Q6G64_F16S
 *   codes [N][K b / 8] bytes (see nq_wfmt), 16-byte aligned
 *   out   [N][K] int8, each code sign-extended
 * Errors: K % 64 != 0 -> NQ_ERR_SHAPE; another fmt -> NQ_ERR_FORMAT.
 */
nq_status nq_unpack_qbits_to_int8(int fmt, const uint8_t* codes, int64_t N, int64_t K, int8_t* out,
                                  void* stream);

/*
 * The Q3 / Q5 / Q6 group-64 projection as an engine step runs it, routed by
 * nq_route(T, a8_flags) ([RTX5080 card, "Quantization profile"]; [int8 card,
 * "What changes"]).  BF16 route: nq_gemv_qgroup(fmt, ...).  A8 routes:
 * nq_quantize_act_int8_g64 into a_q_ws [T][K] and a_scale_ws [T][K/64], the
 * codes widened by nq_unpack_qbits_to_int8 into w_i8_ws [N][K], then
 * nq_gemm_w8a8_g64 (prefill) or the A8 decode GEMV on the widened codes
 * (decode), both with the same FP16 scales.  The A8 workspaces are needed only
 * when an A8 route is taken; `workspace` is the optional GEMV workspace.
 * Errors: K % 256 != 0 -> NQ_ERR_SHAPE; another fmt -> NQ_ERR_FORMAT.
 */
nq_status nq_linear_qbits_g64(int fmt, const uint16_t* x, int64_t T, const uint8_t* w_codes,
                              const uint16_t* w_scale, int64_t N, int64_t K, int a8_flags, int8_t* a_q_ws,
                              float* a_scale_ws, int8_t* w_i8_ws, int out_dt, void* y, void* workspace,
                              int64_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NQ_H */
