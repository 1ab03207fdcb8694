"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin fails.

Each mutation replaces one oracle function or table for the duration of the
test; the listed pins must then raise.  This shows that the pins are sensitive
to a dropped term, a wrong sign or index, a transposed operand, a wrong
constant or a wrong rounding rule anywhere in the oracle.
"""

import numpy as np
import pytest

import oracle_pins as P
from oracle import formats as F
from oracle import method as M


def _table_with(bias=7, sub_exp=-6):
    t = F.E4M3_TABLE.copy()
    for c in range(256):
        e, m = (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            continue
        s = -1.0 if c >> 7 else 1.0
        v = (m / 8) * 2.0 ** sub_exp if e == 0 else (1 + m / 8) * 2.0 ** (e - bias)
        t[c] = s * v
    return t


def _rne_ties_away(x, p, emin, max_finite, saturate):
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    with np.errstate(invalid="ignore", over="ignore"):
        _, e = np.frexp(ax)
        qexp = np.maximum(e - 1, emin) - (p - 1)
        r = np.ldexp(np.floor(np.ldexp(ax, -qexp) + 0.5), qexp)
        r = np.where(r > max_finite, max_finite if saturate else np.inf, r)
        r = np.where(np.isnan(ax), np.nan, r)
    return np.copysign(r, x)


def _unpack_mxfp8_big_endian(words):
    w = np.asarray(words, dtype=np.uint32)
    out = np.empty((w.shape[0], w.shape[1] * 4), dtype=np.uint8)
    for i in range(4):
        out[:, i::4] = ((w >> np.uint32(8 * (3 - i))) & np.uint32(0xFF)).astype(np.uint8)
    return out


def _unpack_q4_swapped(packed, k):
    q = M.__dict__["_orig_unpack_q4"](packed, k)
    q2 = q.copy()
    q2[:, 0::2], q2[:, 1::2] = q[:, 1::2], q[:, 0::2]
    return q2


def _unpack_q4_unsigned(packed, k):
    p = np.asarray(packed, dtype=np.uint8).astype(np.int64)
    q = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.int64)
    q[:, 0::2] = p & 0xF
    q[:, 1::2] = p >> 4
    return q[:, :k]


def _encode_rows_scale127(values):
    v = np.asarray(values, dtype=np.float64)
    m = np.max(np.abs(v), axis=1)
    s_bits = F.encode_bf16(F.f32_div(m, 127.0))
    s = F.bf16_decode(s_bits)
    with np.errstate(invalid="ignore", divide="ignore"):
        q = F.f32_div(v, s[:, None])
    return F.encode_e4m3(q), s_bits


def _encode_rows_no_bf16(values):
    v = np.asarray(values, dtype=np.float64)
    m = np.max(np.abs(v), axis=1)
    s = F.f32_div(m, 448.0)
    s_bits = F.encode_bf16(s)          # stored rounded, but codes divide by the unrounded scale
    with np.errstate(invalid="ignore", divide="ignore"):
        q = F.f32_div(v, s[:, None])
    q = np.where(v == 0, np.copysign(0.0, v), q)
    return F.encode_e4m3(q), s_bits


def _quant_reciprocal(x_bf16):
    xv = F.bf16_decode(x_bf16)
    t, k = xv.shape
    xg = xv.reshape(t, k // 64, 64)
    amax = np.max(np.abs(xg), axis=2)
    s = F.f32_div(amax, 127.0)
    with np.errstate(invalid="ignore", divide="ignore"):
        inv = F.f32_div(1.0, s)
        r = np.rint(F.round_f32(xg * inv[:, :, None]))
    r = np.where(np.isnan(r), 0.0, np.clip(r, -127, 127))
    return r.reshape(t, k).astype(np.int8), F.f32_bits(np.nan_to_num(s))


def _gemv_fp8row_no_scale(w_codes, w_scale_bf16, x_bf16):
    return F.bf16_decode(x_bf16) @ F.e4m3_decode(w_codes).T


def _w8a8_shifted_scale(a_q, a_scale_bits, w_q, w_scale_f16, return_sums=False):
    a_s = F.f32_decode(np.asarray(a_scale_bits, np.uint32))
    w_s = F.f16_decode(np.asarray(w_scale_f16, np.uint16))
    a = np.asarray(a_q, np.int64).astype(np.float64)
    w = np.asarray(w_q, np.int64).astype(np.float64)
    g = a.shape[1] // 64
    y = np.zeros((a.shape[0], w.shape[0]))
    sums = []
    for j in range(g):
        sl = slice(j * 64, (j + 1) * 64)
        p = a[:, sl] @ w[:, sl].T
        jj = (j + 1) % g                        # wrong group's scales
        y += p * (a_s[:, jj][:, None] * w_s[:, jj][None, :])
        sums.append(p.astype(np.int64))
    return (y, np.stack(sums, axis=2)) if return_sums else y


def _w8a8_no_act_scale(a_q, a_scale_bits, w_q, w_scale_f16, return_sums=False):
    ones = np.ones_like(np.asarray(a_scale_bits, np.uint32)).astype(np.float32).view(np.uint32)
    return M.__dict__["_orig_gemm_w8a8_g64"](a_q, ones, w_q, w_scale_f16, return_sums)


def _block_decode_transposed(codes, wsi):
    """Index the scale grid as [column block][row block] (wrapped to fit)."""
    codes = np.asarray(codes, dtype=np.uint8)
    n, k = codes.shape
    s = F.f32_decode(np.asarray(wsi, dtype=np.float32).view(np.uint32))
    gr, gc = s.shape
    rb = (np.arange(n) // 128)[:, None]
    cb = (np.arange(k) // 128)[None, :]
    return F.round_f32(F.e4m3_decode(codes) * s[cb % gr, rb % gc])


def _f32_div_unrounded(a, b):
    with np.errstate(divide="ignore", invalid="ignore"):
        return np.asarray(a, np.float64) / np.asarray(b, np.float64)


def _route_128(t, allow_a8):
    return "a8" if (allow_a8 and t >= 128) else "bf16"


def _ue8m0_off_by_one(b):
    b = np.asarray(b, dtype=np.int64)
    return np.where(b == 255, np.nan, np.ldexp(1.0, b - 128))


def _quant_fp8_amax127(x_bf16):
    xv = F.bf16_decode(x_bf16)
    amax = np.max(np.abs(xv), axis=1)
    s = F.f32_div(amax, 127.0)
    with np.errstate(invalid="ignore", divide="ignore"):
        q = F.f32_div(xv, s[:, None])
    q = np.where(xv == 0, np.copysign(0.0, xv), q)
    return F.encode_e4m3(q), F.f32_bits(s)


def _mlx_group64(codes, scales, biases):
    q = np.asarray(codes, dtype=np.uint8).astype(np.float64)
    n, k = q.shape
    s = np.repeat(F.f16_decode(scales), 64, axis=1)[:, :k]
    b = np.repeat(F.f16_decode(biases), 64, axis=1)[:, :k]
    s = np.pad(s, ((0, 0), (0, k - s.shape[1])), mode="edge")
    b = np.pad(b, ((0, 0), (0, k - b.shape[1])), mode="edge")
    return q * s + b


def _mlx_minus_bias(codes, scales, biases):
    q = np.asarray(codes, dtype=np.uint8).astype(np.float64)
    n, k = q.shape
    return q * np.repeat(F.f16_decode(scales), 128, axis=1)[:, :k] - np.repeat(F.f16_decode(biases), 128, axis=1)[:, :k]


def _mlx_through_f32(codes, scales, biases):
    q = np.asarray(codes, dtype=np.uint8).astype(np.float32)
    n, k = q.shape
    s = np.repeat(F.f16_decode(scales), 128, axis=1)[:, :k].astype(np.float32)
    b = np.repeat(F.f16_decode(biases), 128, axis=1)[:, :k].astype(np.float32)
    return (q * s + b).astype(np.float64)           # an FP32 value first, then BF16: two roundings


def _unpack_qbits_msb_first(packed, k, bits):
    p = np.asarray(packed, dtype=np.uint8)
    n = p.shape[0]
    stream = np.unpackbits(p, axis=1, bitorder="big")[:, :k * bits].astype(np.int64)
    fields = stream.reshape(n, k, bits)
    u = np.zeros((n, k), dtype=np.int64)
    for i in range(bits):
        u += fields[:, :, i] << i
    return np.where(u >= (1 << (bits - 1)), u - (1 << bits), u)


def _unpack_qbits_unsigned(packed, k, bits):
    p = np.asarray(packed, dtype=np.uint8)
    stream = np.unpackbits(p, axis=1, bitorder="little")[:, :k * bits].astype(np.int64)
    return (stream.reshape(p.shape[0], k, bits) << np.arange(bits)).sum(axis=2)


def _route_no_decode(t, allow_a8, a8_decode=False):
    return "a8" if (allow_a8 and t >= 129) else "bf16"


MUTATIONS = [
    ("qbits bit order within bytes reversed", lambda mp: mp.setattr(M, "unpack_qbits", _unpack_qbits_msb_first),
     [P.pin_qbits]),
    ("qbits unsigned codes", lambda mp: mp.setattr(M, "unpack_qbits", _unpack_qbits_unsigned), [P.pin_qbits]),
    ("route ignores the A8 decode flag", lambda mp: mp.setattr(M, "route", _route_no_decode), [P.pin_route]),
    ("mlx groups of 64", lambda mp: mp.setattr(M, "mlx_affine_int8_values", _mlx_group64),
     [P.pin_mlx_affine_int8]),
    ("mlx bias subtracted", lambda mp: mp.setattr(M, "mlx_affine_int8_values", _mlx_minus_bias),
     [P.pin_mlx_affine_int8]),
    ("mlx value rounded to FP32 first", lambda mp: mp.setattr(M, "mlx_affine_int8_values", _mlx_through_f32),
     [P.pin_mlx_affine_int8]),

    ("e4m3 bias 8", lambda mp: mp.setattr(F, "E4M3_TABLE", _table_with(bias=8)),
     [P.pin_e4m3_golden, P.pin_e4m3_vs_torch]),
    ("e4m3 subnormal exponent", lambda mp: mp.setattr(F, "E4M3_TABLE", _table_with(sub_exp=-7)),
     [P.pin_e4m3_structure]),
    ("ties away from zero", lambda mp: mp.setattr(F, "round_rne", _rne_ties_away),
     [P.pin_e4m3_encode, P.pin_round_bf16_f16_f32]),
    ("ue8m0 2^(b-128)", lambda mp: mp.setattr(M, "ue8m0_decode", _ue8m0_off_by_one),
     [P.pin_mxfp8_decode]),
    ("mxfp8 big-endian", lambda mp: mp.setattr(M, "unpack_mxfp8_codes", _unpack_mxfp8_big_endian),
     [P.pin_mxfp8_decode]),
    ("q4 nibbles swapped", lambda mp: (mp.setattr(M, "_orig_unpack_q4", M.unpack_q4, raising=False),
                                       mp.setattr(M, "unpack_q4", _unpack_q4_swapped)),
     [P.pin_gemv_qgroup]),
    ("q4 unsigned nibbles", lambda mp: mp.setattr(M, "unpack_q4", _unpack_q4_unsigned),
     [P.pin_gemv_qgroup]),
    ("row scale amax/127", lambda mp: mp.setattr(M, "encode_rows_fp8", _encode_rows_scale127),
     [P.pin_reencode_invariants]),
    ("row scale not rounded to bf16 before dividing",
     lambda mp: mp.setattr(M, "encode_rows_fp8", _encode_rows_no_bf16),
     [P.pin_reencode_bruteforce]),
    ("int8 quant by reciprocal", lambda mp: mp.setattr(M, "quantize_act_int8_g64", _quant_reciprocal),
     [P.pin_quantize_int8]),
    ("gemv drops row scale", lambda mp: mp.setattr(M, "gemv_fp8row", _gemv_fp8row_no_scale),
     [P.pin_gemv_fp8row]),
    ("w8a8 scales of the wrong group",
     lambda mp: mp.setattr(M, "gemm_w8a8_g64", _w8a8_shifted_scale), [P.pin_w8a8]),
    ("w8a8 drops activation scale",
     lambda mp: (mp.setattr(M, "_orig_gemm_w8a8_g64", M.gemm_w8a8_g64, raising=False),
                 mp.setattr(M, "gemm_w8a8_g64", _w8a8_no_act_scale)), [P.pin_w8a8]),
    ("block grid transposed", lambda mp: mp.setattr(M, "block_decode_f32", _block_decode_transposed),
     [P.pin_reencode_bruteforce, P.pin_reencode_invariants]),
    ("FP32 division not rounded", lambda mp: (mp.setattr(F, "f32_div", _f32_div_unrounded),
                                              mp.setattr(M, "f32_div", _f32_div_unrounded)),
     [P.pin_f32_div, P.pin_quantize_int8]),
    ("route threshold 128", lambda mp: mp.setattr(M, "route", _route_128), [P.pin_route]),
    ("fp8 activation scale amax/127", lambda mp: mp.setattr(M, "quantize_act_fp8_row", _quant_fp8_amax127),
     [P.pin_fp8_act_and_gemm]),
]


@pytest.mark.parametrize("name,apply,pins", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(monkeypatch, name, apply, pins):
    apply(monkeypatch)
    caught = False
    for pin in pins:
        try:
            pin()
        except AssertionError:
            caught = True
            break
    assert caught, f"no pin caught the planted mistake: {name}"
