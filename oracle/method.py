"""The steps of the quantized-weight linear projection, written from the pages.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Layout conventions (readings; the pages do not fix them):
  * a weight matrix is [N][K] row-major, N output rows by K input channels, and
    the projection is y[t, n] = sum_k x[t, k] * W[n, k];
  * activations are [T][K], outputs [T][N];
  * group and block axes run along K.
All arrays are numpy arrays; BF16 / FP16 / FP32 tensors are passed as their
bit patterns (uint16 / uint16 / uint32) so that nothing is rounded on the way
in.
"""

import numpy as np

from .formats import (
    bf16_decode, e4m3_decode, encode_bf16, encode_e4m3, f16_decode, f32_bits,
    f32_decode, f32_div, round_bf16, round_f32, ue8m0_decode,
)

# ---------------------------------------------------------------------------
# a1. MXFP8 decode.
# [MXFP8 card, "How it was built", item 1]: four E4M3 codes are packed in one
# 32-bit word and every 32 consecutive elements share one UE8M0 scale byte
# worth 2^(b-127); the converter turns them into BF16.
# Readings: element 4j+i sits in bits 8i..8i+7 of word j (little-endian); the
# scale array is [N][K/32]; the output is BF16 (as the page) or FP32, rounded
# to nearest-even from the exact product.
# ---------------------------------------------------------------------------


def unpack_mxfp8_codes(words):
    """u32 words [N][K/4] -> uint8 codes [N][K] (element 4j+i = byte i of word j)."""
    w = np.asarray(words, dtype=np.uint32)
    n, kw = w.shape
    out = np.empty((n, kw * 4), dtype=np.uint8)
    for i in range(4):
        out[:, i::4] = ((w >> np.uint32(8 * i)) & np.uint32(0xFF)).astype(np.uint8)
    return out


def mxfp8_values(words, e8m0):
    """Exact decoded values (float64) of an MXFP8 matrix."""
    codes = unpack_mxfp8_codes(words)
    n, k = codes.shape
    scale = ue8m0_decode(np.asarray(e8m0, dtype=np.uint8))          # [N][K/32]
    per_elem = np.repeat(scale, 32, axis=1)[:, :k]
    with np.errstate(invalid="ignore", over="ignore"):
        return e4m3_decode(codes) * per_elem          # 4 significant bits x 2^e: exact


def decode_mxfp8(words, e8m0, out="bf16"):
    """MXFP8 -> BF16 (uint16 bits) or FP32 (uint32 bits), single rounding."""
    v = mxfp8_values(words, e8m0)
    if out == "bf16":
        return encode_bf16(v)
    r = round_f32(v)
    bits = f32_bits(np.where(np.isnan(r), 0.0, r))
    return np.where(np.isnan(r), np.uint32(0x7FC00000), bits).astype(np.uint32)


# ---------------------------------------------------------------------------
# MLX affine int8 decode (the draft layer's storage, the step before the path
# in the conversion pipeline).
# [MXFP8 card, "How it was built", item 2]: uint8 codes with one FP16 scale and
# one FP16 bias per 128-element group decode as w = q * scale + bias, written
# as BF16.
# Readings: codes [N][K] uint8, groups of 128 along K, scales and biases
# [N][K/128] FP16 bits; w is the exact value of q * scale + bias (float64 holds
# it: q * scale has at most 19 significant bits and every FP16 value is a
# multiple of 2^-24 below 2^16, so the sum spans under 50 bits) rounded once
# to BF16 (nearest-even, overflow to infinity; NaN -> 0x7FC0), or to FP32.
# ---------------------------------------------------------------------------


def mlx_affine_int8_values(codes, scales, biases):
    """Exact values (float64) of an MLX affine int8 matrix."""
    q = np.asarray(codes, dtype=np.uint8).astype(np.float64)
    n, k = q.shape
    s = np.repeat(f16_decode(np.asarray(scales, dtype=np.uint16)), 128, axis=1)[:, :k]
    b = np.repeat(f16_decode(np.asarray(biases, dtype=np.uint16)), 128, axis=1)[:, :k]
    with np.errstate(invalid="ignore", over="ignore"):
        return q * s + b


def decode_mlx_affine_int8(codes, scales, biases, out="bf16"):
    """MLX affine int8 -> BF16 (uint16 bits) or FP32 (uint32 bits), single rounding."""
    v = mlx_affine_int8_values(codes, scales, biases)
    if out == "bf16":
        return encode_bf16(v)
    r = round_f32(v)
    bits = f32_bits(np.where(np.isnan(r), 0.0, r))
    return np.where(np.isnan(r), np.uint32(0x7FC00000), bits).astype(np.uint32)


# ---------------------------------------------------------------------------
# a2. Block-128x128 E4M3 -> one BF16 scale per output row (fp8_row_maxabs).
# [FP8 card, "Conversion and verification", "Block-wise to per-row,
# exactly"]: codes carry a weight_scale_inv value per 128x128 block; each code
# is decoded in FP32 (the E4M3 significand times the block scale), the grid is
# checked against the code shape, the decoded values are re-encoded with one
# BF16 scale per output row, and a row range reads only the block rows it
# touches.  [FP8 card, introduction] names the per-row encoding
# fp8_row_maxabs.
# Readings: the block scale multiplies; the row scale is the row's largest
# magnitude over 448 (the largest E4M3 value) rounded to BF16, the division
# done in IEEE FP32; each code is the E4M3 round-to-nearest-even (saturating)
# of the FP32 quotient value / scale; a row of zeros gets scale +0 and keeps the
# signed zeros; NaN propagates (a row holding NaN gets a NaN scale and NaN
# codes).
# ---------------------------------------------------------------------------


class GridShapeError(ValueError):
    pass


def block_decode_f32(codes, wsi):
    """Decode block-scaled E4M3 codes to FP32 values (returned as float64)."""
    codes = np.asarray(codes, dtype=np.uint8)
    n, k = codes.shape
    wsi = np.asarray(wsi, dtype=np.float32)
    gr, gc = wsi.shape
    if gr != -(-n // 128) or gc != -(-k // 128):
        raise GridShapeError(f"scale grid {gr}x{gc} does not match codes {n}x{k} in 128x128 blocks")
    s = f32_decode(wsi.view(np.uint32))
    per_elem = np.repeat(np.repeat(s, 128, axis=0)[:n], 128, axis=1)[:, :k]
    with np.errstate(invalid="ignore", over="ignore"):
        return round_f32(e4m3_decode(codes) * per_elem)


def encode_rows_fp8(values):
    """fp8_row_maxabs of FP32-representable values [R][K] -> (codes u8, scale bf16 bits)."""
    v = np.asarray(values, dtype=np.float64)
    m = np.max(np.abs(v), axis=1) if v.shape[1] else np.zeros(v.shape[0])   # NaN propagates
    s_bits = encode_bf16(f32_div(m, 448.0))
    s = bf16_decode(s_bits)
    with np.errstate(invalid="ignore", divide="ignore"):
        q = f32_div(v, s[:, None])
    zero_over_zero = (v == 0) & (s[:, None] == 0)
    q = np.where(zero_over_zero, np.copysign(0.0, v), q)
    return encode_e4m3(q), s_bits


def reencode_block128_to_row(codes, wsi, row_begin=None, row_end=None):
    codes = np.asarray(codes, dtype=np.uint8)
    n = codes.shape[0]
    r0 = 0 if row_begin is None else row_begin
    r1 = n if row_end is None else row_end
    if not (0 <= r0 < r1 <= n):
        raise ValueError("row range out of bounds")
    v = block_decode_f32(codes, wsi)           # grid check on the full shape
    return encode_rows_fp8(v[r0:r1])


def encode_fp8row_bf16(w_bf16):
    """BF16 [N][K] -> fp8_row_maxabs.  [NVFP4 card, "How it was created": the
    token embedding goes from its BF16 source to the same row-scale FP8]."""
    return encode_rows_fp8(bf16_decode(np.asarray(w_bf16, dtype=np.uint16)))


# ---------------------------------------------------------------------------
# a3 / a4. Decode GEMVs on the BF16-activation route.
# [int8 card, "What changes"]: decode and verify steps keep BF16 activations;
# [NVFP4 card, "How it was created"]: weights are dequantized on the fly
# against their stored scales.  Row FP8: one BF16 scale per output row [FP8
# card]; grouped formats: symmetric codes with one FP16 scale per group of 32
# or 64 along K [NVFP4 card, "What is in the file"; RTX5080 card,
# "Quantization profile"]; BF16: weights used as stored [NVFP4 card, the GDN
# a/b gating projections].
# Readings: Q4 codes are two's-complement nibbles, element 2j in the low nibble
# of byte j; Q8 codes are int8; scales are [N][K/G].
# ---------------------------------------------------------------------------


def gemv_fp8row(w_codes, w_scale_bf16, x_bf16):
    """y[t,n] = s[n] * sum_k x[t,k] * e4m3(q[n,k]), float64."""
    wv = e4m3_decode(w_codes)
    s = bf16_decode(w_scale_bf16)
    xv = bf16_decode(x_bf16)
    return (xv @ wv.T) * s[None, :]


def unpack_q4(packed, k):
    """bytes [N][K/2] -> int codes [N][K] in [-8, 7]."""
    p = np.asarray(packed, dtype=np.uint8).astype(np.int64)
    lo = p & 0xF
    hi = p >> 4
    q = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.int64)
    q[:, 0::2] = np.where(lo >= 8, lo - 16, lo)
    q[:, 1::2] = np.where(hi >= 8, hi - 16, hi)
    return q[:, :k]


# Q3 / Q5 / Q6 group-64 codes.  [RTX5080 card, "Quantization profile"]: the
# main text weights are Q3, Q4 and Q5 group-64 codes with FP16 scales;
# [NVFP4 card, "What is in the file"]: grouped Q4 / Q5 / Q6 / Q8 formats.  The
# pages give no bit layout.  Reading: symmetric b-bit two's-complement codes
# (q in [-2^(b-1), 2^(b-1) - 1], w = q * scale), stored as a dense
# little-endian bit stream along each row: element j of a row occupies bits
# [b j, b j + b) of the row's bytes, bit i of the stream being bit i % 8 of
# byte i // 8.  For b = 4 this is the nibble layout above (element 2j in the
# low nibble of byte j).  A group of 64 codes spans 8 b bytes, so groups and
# rows start on byte boundaries; one FP16 scale per 64 codes, [N][K/64].


def unpack_qbits(packed, k, bits):
    """Dense little-endian b-bit two's-complement codes [N][K*b/8] bytes -> int codes [N][K]."""
    p = np.asarray(packed, dtype=np.uint8)
    n = p.shape[0]
    stream = np.unpackbits(p, axis=1, bitorder="little")[:, :k * bits].astype(np.int64)   # bit i = stream[i]
    fields = stream.reshape(n, k, bits)
    u = np.zeros((n, k), dtype=np.int64)
    for i in range(bits):
        u += fields[:, :, i] << i
    return np.where(u >= (1 << (bits - 1)), u - (1 << bits), u)


QBITS = {"q3g64": 3, "q5g64": 5, "q6g64": 6}

GROUP = {"q4g64": 64, "q8g32": 32, "q8g64": 64, "mxfp8": 32, "bf16": None, "q3g64": 64, "q5g64": 64, "q6g64": 64}


def grouped_codes_and_scales(fmt, codes, scales, k):
    """Decoded integer/E4M3 codes [N][K] (float64) and per-group scales [N][G]."""
    if fmt == "q4g64":
        return unpack_q4(codes, k).astype(np.float64), f16_decode(scales)
    if fmt in ("q8g32", "q8g64"):
        return np.asarray(codes, dtype=np.int8).astype(np.float64), f16_decode(scales)
    if fmt == "mxfp8":
        return e4m3_decode(unpack_mxfp8_codes(codes)), ue8m0_decode(np.asarray(scales, np.uint8))
    if fmt in QBITS:
        return unpack_qbits(codes, k, QBITS[fmt]).astype(np.float64), f16_decode(scales)
    raise ValueError(fmt)


def gemv_qgroup(fmt, codes, scales, x_bf16):
    """y[t,n] = sum_g sc[n,g] * sum_{k in g} x[t,k] * q[n,k], float64."""
    xv = bf16_decode(x_bf16)
    t, k = xv.shape
    if fmt == "bf16":
        return xv @ bf16_decode(codes).T
    gs = GROUP[fmt]
    q, sc = grouped_codes_and_scales(fmt, codes, scales, k)
    y = np.zeros((t, q.shape[0]))
    for g in range(k // gs):
        sl = slice(g * gs, (g + 1) * gs)
        with np.errstate(invalid="ignore"):
            y += (xv[:, sl] @ q[:, sl].T) * sc[None, :, g]
    return y


# ---------------------------------------------------------------------------
# a5 / a6. W8A8 prefill.
# [int8 card, "What changes"]: for prefill steps of 129 tokens or more, the
# activations are quantized per token and per 64 channels with scale =
# amax / 127 (the same groups as the weight scales), integer codes are
# multiplied on int8 matrix units exactly, and each group's int32 sum is scaled
# by weight_scale x activation_scale in FP32; the scaled groups are summed.
# Readings: amax is exact on BF16 inputs; the scale is the IEEE FP32 quotient
# amax / 127; a code is the FP32 quotient x / scale rounded to nearest-even and
# clamped to [-127, 127]; an all-zero group has scale 0 and codes 0; a NaN
# quotient gives code 0.
# ---------------------------------------------------------------------------


def quantize_act_int8_g64(x_bf16):
    """BF16 [T][K] -> (int8 codes [T][K], FP32 scales as uint32 bits [T][K/64])."""
    xv = bf16_decode(x_bf16)
    t, k = xv.shape
    if k % 64:
        raise ValueError("K must be a multiple of 64")
    xg = xv.reshape(t, k // 64, 64)
    amax = np.max(np.abs(xg), axis=2)
    s = f32_div(amax, 127.0)
    with np.errstate(invalid="ignore", divide="ignore"):
        r = np.rint(f32_div(xg, s[:, :, None]))
    r = np.where(np.isnan(r), 0.0, np.clip(r, -127, 127))
    s_bits = f32_bits(np.where(np.isnan(s), 0.0, s))
    s_bits = np.where(np.isnan(s), np.uint32(0x7FC00000), s_bits).astype(np.uint32)
    return r.reshape(t, k).astype(np.int8), s_bits


def w8a8_group_sums(a_q, w_q):
    """P[m,n,g] = sum_{k in g} a_q[m,k] * w_q[n,k], exact (int64)."""
    a = np.asarray(a_q, dtype=np.int64)
    w = np.asarray(w_q, dtype=np.int64)
    m, k = a.shape
    g = k // 64
    p = np.empty((m, w.shape[0], g), dtype=np.int64)
    for j in range(g):
        sl = slice(j * 64, (j + 1) * 64)
        # float64 products and sums of at most 64 terms of |127*127| are exact
        p[:, :, j] = np.rint(a[:, sl].astype(np.float64) @ w[:, sl].astype(np.float64).T).astype(np.int64)
    return p


def gemm_w8a8_g64(a_q, a_scale_bits, w_q, w_scale_f16, return_sums=False):
    """y[m,n] = sum_g P[m,n,g] * (w_scale[n,g] * a_scale[m,g]), float64."""
    a_s = f32_decode(np.asarray(a_scale_bits, dtype=np.uint32))
    w_s = f16_decode(np.asarray(w_scale_f16, dtype=np.uint16))
    a = np.asarray(a_q, dtype=np.int64)
    w = np.asarray(w_q, dtype=np.int64)
    m, k = a.shape
    y = np.zeros((m, w.shape[0]))
    sums = [] if return_sums else None
    for j in range(k // 64):
        sl = slice(j * 64, (j + 1) * 64)
        p = a[:, sl].astype(np.float64) @ w[:, sl].astype(np.float64).T     # exact integers
        y += p * (a_s[:, j][:, None] * w_s[:, j][None, :])
        if return_sums:
            sums.append(p.astype(np.int64))
    if return_sums:
        return y, (np.stack(sums, axis=2) if sums else np.zeros((m, w.shape[0], 0), np.int64))
    return y


# ---------------------------------------------------------------------------
# a7. FP8-activation prefill GEMM on row-scaled FP8 weights.
# [FP8 card, "Conversion and verification", "Hardware fit"]: the row-scaled
# FP8 weights feed FP8-activation matrix-unit routes directly, without a BF16
# dequantization first.  The pages do not describe how activations are
# quantized for that route (parity unpinned with respect to the pages).
# Reading: one scale per token, amax / 448 in IEEE FP32, codes the saturating
# E4M3 round-to-nearest-even of the FP32 quotient x / scale, an all-zero token
# keeps its signed zeros with scale 0.
# ---------------------------------------------------------------------------


def quantize_act_fp8_row(x_bf16):
    """BF16 [M][K] -> (E4M3 codes [M][K], FP32 scale bits [M])."""
    xv = bf16_decode(x_bf16)
    amax = np.max(np.abs(xv), axis=1) if xv.shape[1] else np.zeros(xv.shape[0])
    s = f32_div(amax, 448.0)
    with np.errstate(invalid="ignore", divide="ignore"):
        q = f32_div(xv, s[:, None])
    q = np.where((xv == 0) & (s[:, None] == 0), np.copysign(0.0, xv), q)
    s_bits = np.where(np.isnan(s), np.uint32(0x7FC00000), f32_bits(np.where(np.isnan(s), 0.0, s)))
    return encode_e4m3(q), s_bits.astype(np.uint32)


def gemm_fp8row(x_bf16, w_codes, w_scale_bf16):
    """Returns (y float64 [M][N], activation codes, activation scale bits)."""
    qa, sa_bits = quantize_act_fp8_row(x_bf16)
    sa = f32_decode(sa_bits)
    sw = bf16_decode(w_scale_bf16)
    acc = e4m3_decode(qa) @ e4m3_decode(w_codes).T
    return acc * sa[:, None] * sw[None, :], qa, sa_bits


# ---------------------------------------------------------------------------
# a8. Route rule.
# [int8 card, "What changes"]: a projection allowed to run with int8
# activations takes that route only in prefill steps of 129 tokens or more;
# decode and verification steps keep the BF16 route, so output is unchanged
# when no step reaches 129 tokens.
# ---------------------------------------------------------------------------

A8_MIN_TOKENS = 129

# [FP8 card, "Start the server"]: one server variant also runs the MLP with
# int8 activations in decode steps.  The pages give no details of it.
# Reading: an A8 decode step is the W8A8 computation above (per-token-per-64
# int8 activations, exact int32 group sums, FP32 rescale) at decode sizes,
# enabled by its own flag for steps of at most 128 tokens.


def route(t, allow_a8, a8_decode=False):
    if allow_a8 and t >= A8_MIN_TOKENS:
        return "a8"
    if a8_decode and t < A8_MIN_TOKENS:
        return "a8_decode"
    return "bf16"


def linear_w8g64(x_bf16, w_q, w_scale_f16, allow_a8, a8_decode=False):
    """The projection as an engine step runs it: routed by token count."""
    t = np.asarray(x_bf16).shape[0]
    if route(t, allow_a8, a8_decode) != "bf16":
        qa, sa = quantize_act_int8_g64(x_bf16)
        return gemm_w8a8_g64(qa, sa, w_q, w_scale_f16)
    return gemv_qgroup("q8g64", w_q, w_scale_f16, x_bf16)


# Q4 group-64 weights on both routes.  [int8 card, "What changes"]: in
# prefill the Q4 (and Q5) codes feed the int8 matrix units exactly, with the
# per-64 weight scales applied to each group's int32 sum as for Q8.
# Reading: the A8 route is the W8A8 GEMM on the Q4 codes taken as int8 values
# in [-8, 7]; the BF16 route is the grouped GEMV.


def linear_q4g64(x_bf16, w_packed, w_scale_f16, allow_a8, a8_decode=False):
    """The Q4 group-64 projection routed by token count."""
    t, k = np.asarray(x_bf16).shape
    if route(t, allow_a8, a8_decode) != "bf16":
        qa, sa = quantize_act_int8_g64(x_bf16)
        return gemm_w8a8_g64(qa, sa, unpack_q4(w_packed, k), w_scale_f16)
    return gemv_qgroup("q4g64", w_packed, w_scale_f16, x_bf16)


def linear_qbits_g64(fmt, x_bf16, w_packed, w_scale_f16, allow_a8, a8_decode=False):
    """The Q3 / Q5 / Q6 group-64 projection routed by token count: on the A8
    routes the codes feed the int8 arithmetic exactly, as Q4's do [int8 card,
    "What changes": Q4 / Q5 codes go to the int8 units exactly]."""
    t, k = np.asarray(x_bf16).shape
    if route(t, allow_a8, a8_decode) != "bf16":
        qa, sa = quantize_act_int8_g64(x_bf16)
        return gemm_w8a8_g64(qa, sa, unpack_qbits(w_packed, k, QBITS[fmt]), w_scale_f16)
    return gemv_qgroup(fmt, w_packed, w_scale_f16, x_bf16)


# ---------------------------------------------------------------------------
# Output roundings (what an FP32- or BF16-output kernel should produce from
# the float64 result, up to the kernel's own summation order).
# ---------------------------------------------------------------------------


def to_f32(y):
    return round_f32(y)


def to_bf16(y):
    return round_bf16(y)
