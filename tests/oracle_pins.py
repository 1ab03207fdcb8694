"""Pins that tie the CPU oracle to something other than itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
the format definitions, exact rational arithmetic, an invariant the pages
state, or a library routine that implements the same textbook operation.
They are plain functions (not collected by pytest) so that the mutation tests
can plant a mistake in the oracle and check that some pin fails.

Sources are cited by page title and section (see ``oracle/__init__.py``).
"""

import os
from fractions import Fraction

import numpy as np
import torch

from oracle import formats as F
from oracle import method as M

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _frac(s):
    if s in ("nan",):
        return None
    if s == "-0":
        return "-0"
    return Fraction(s)


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append(line.split())
    return rows


# ----------------------------------------------------------------------------
# Independent brute-force rounding: enumerate the target format's values and
# take the nearest (ties to the even code).  This is a different algorithm from
# the oracle's scale-and-rint rounding.
# ----------------------------------------------------------------------------

_E4M3_NONNEG = []
for _c in range(0x7F):
    _e, _m = _c >> 3, _c & 7
    _v = Fraction(_m, 8) / 64 if _e == 0 else (1 + Fraction(_m, 8)) * Fraction(2) ** (_e - 7)
    _E4M3_NONNEG.append((_v, _c))


def brute_e4m3(x):
    """Exact Fraction (or float) -> E4M3 code, RNE, saturating, sign of zero kept."""
    if isinstance(x, float) and x != x:
        return 0x7F
    neg = (x < 0) or (isinstance(x, float) and x == 0 and np.signbit(x))
    a = abs(Fraction(x)) if not isinstance(x, Fraction) else abs(x)
    if a >= 448:
        best = 0x7E
    else:
        best, bestd = None, None
        for v, c in _E4M3_NONNEG:
            d = abs(v - a)
            if bestd is None or d < bestd or (d == bestd and (c & 1) == 0):
                best, bestd = c, d
    return best | (0x80 if neg else 0)


def frac_to_f32(x):
    """Exact rational -> nearest float32 (Fraction->float is correctly rounded to
    double; double->float32 is numpy's cast; both round to nearest even, and the
    double rounding is exact for quotients/products of float32 values)."""
    return np.float32(float(x))


def brute_f32_div(a, b):
    return Fraction(float(frac_to_f32(Fraction(a) / Fraction(b))))


# ----------------------------------------------------------------------------
# Formats
# ----------------------------------------------------------------------------


def pin_e4m3_golden():
    for code_s, val_s in _read_golden("e4m3_values.txt"):
        code = int(code_s, 16)
        got = F.e4m3_decode(np.array([code], np.uint8))[0]
        if val_s == "nan":
            assert np.isnan(got), (code_s, got)
        elif val_s == "-0":
            assert got == 0 and np.signbit(got), (code_s, got)
        else:
            assert Fraction(got) == Fraction(val_s), (code_s, got, val_s)


def pin_e4m3_structure():
    t = F.E4M3_TABLE
    assert np.isnan(t).sum() == 2 and np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0), "positive codes must increase"
    for c in range(0x80):
        if c == 0x7F:
            continue
        assert t[c | 0x80] == -t[c] and np.signbit(t[c | 0x80])
    # number of finite, non-NaN, nonzero codes
    assert int(np.sum(np.isfinite(t) & (t != 0))) == 252
    # spacing: 8 values per binade, subnormal quantum 2^-9
    assert t[1] == 2.0 ** -9 and t[8] == 2.0 ** -6 and t[0x7E] == 448.0


def pin_e4m3_vs_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F.e4m3_decode(np.arange(256, dtype=np.uint8))
    same = (ref == got) | (np.isnan(ref) & np.isnan(got))
    assert same.all()
    assert np.array_equal(np.signbit(ref[~np.isnan(ref)]), np.signbit(got[~np.isnan(got)]))


def pin_ue8m0():
    for b in range(255):
        assert Fraction(float(F.ue8m0_decode(b))) == Fraction(2) ** (b - 127), b
    assert np.isnan(F.ue8m0_decode(255))


def pin_binary_decoders():
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref_bf = torch.from_numpy(allbits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    got_bf = F.bf16_decode(allbits)
    ok = (ref_bf == got_bf) | (np.isnan(ref_bf) & np.isnan(got_bf))
    assert ok.all(), "bf16 decode"
    ref_h = allbits.view(np.float16).astype(np.float64)
    got_h = F.f16_decode(allbits)
    ok = (ref_h == got_h) | (np.isnan(ref_h) & np.isnan(got_h))
    assert ok.all(), "f16 decode"
    rng = np.random.default_rng(5)
    b32 = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    ref_f = b32.view(np.float32).astype(np.float64)
    got_f = F.f32_decode(b32)
    ok = (ref_f == got_f) | (np.isnan(ref_f) & np.isnan(got_f))
    assert ok.all(), "f32 decode"


def _bf16_of_f32_torch(x32):
    return torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()


def pin_round_bf16_f16_f32():
    rng = np.random.default_rng(6)
    # random float32 over a wide range plus exact ties between BF16 neighbours
    b32 = rng.integers(0, 2 ** 32, 300000, dtype=np.uint64).astype(np.uint32)
    x32 = b32.view(np.float32)
    x32 = x32[np.isfinite(x32)]
    ties = ((rng.integers(0, 2 ** 16, 50000).astype(np.uint32) << 16) | 0x8000).view(np.float32)
    ties = ties[np.isfinite(ties)]
    for x in (x32, ties):
        ref = _bf16_of_f32_torch(x)
        got = F.round_bf16(x.astype(np.float64))
        ok = (ref == got) | (np.isnan(ref) & np.isnan(got))
        assert ok.all(), "bf16 RNE"
    # known tie: 1 + 2^-8 -> 1.0 ; 1 + 3*2^-8 -> 1 + 2^-6
    assert F.round_bf16(1 + 2.0 ** -8) == 1.0
    assert F.round_bf16(1 + 3 * 2.0 ** -8) == 1 + 2.0 ** -6
    x64 = rng.standard_normal(300000) * np.exp2(rng.integers(-30, 30, 300000))
    with np.errstate(over="ignore"):
        ref_h = x64.astype(np.float16).astype(np.float64)
    got_h = F.round_f16(x64)
    assert np.array_equal(ref_h, got_h), "f16 RNE"
    tiny = rng.standard_normal(100000) * 2.0 ** -20         # f16 subnormals
    assert np.array_equal(tiny.astype(np.float16).astype(np.float64), F.round_f16(tiny))
    x64 = rng.standard_normal(300000) * np.exp2(rng.integers(-140, 120, 300000))
    assert np.array_equal(x64.astype(np.float32).astype(np.float64), F.round_f32(x64)), "f32 RNE"


def pin_f32_div():
    rng = np.random.default_rng(7)
    a = (rng.standard_normal(200000) * 100).astype(np.float32)
    b = (rng.standard_normal(200000) * 3).astype(np.float32)
    ref = (a / b).astype(np.float64)
    assert np.array_equal(ref, F.f32_div(a.astype(np.float64), b.astype(np.float64)))


def pin_e4m3_encode():
    for kind, xin, want in _read_golden("rounding_cases.txt"):
        if kind != "e4m3":
            continue
        x = float(Fraction(xin)) if xin != "-0" else -0.0
        code = int(F.encode_e4m3(np.array([x]))[0])
        if want == "-0":
            assert code == 0x80, (xin, hex(code))
        else:
            assert Fraction(float(F.E4M3_TABLE[code])) == Fraction(want), (xin, hex(code), want)
    rng = np.random.default_rng(8)
    xs = np.concatenate([rng.standard_normal(3000) * np.exp2(rng.integers(-12, 10, 3000)),
                         [0.0, -0.0, np.nan, np.inf, -np.inf, 447.99, 448.0, 463.99, 1e30]])
    # midpoints between neighbouring E4M3 values, nudged either way
    vals = F.E4M3_TABLE[:0x7F]
    mids = (vals[:-1] + vals[1:]) / 2
    xs = np.concatenate([xs, mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9)])
    got = F.encode_e4m3(xs)
    for x, c in zip(xs, got):
        if np.isinf(x):
            want = 0x7E | (0x80 if x < 0 else 0)
        else:
            want = brute_e4m3(Fraction(x) if np.isfinite(x) and x != 0 else x)
        assert int(c) == want, (x, hex(int(c)), hex(want))
    # library cross-check where torch's (non-saturating) cast is defined the same way
    fin = xs[np.isfinite(xs) & (np.abs(xs) < 464)]
    fin = fin[fin.astype(np.float32).astype(np.float64) == fin]     # no float32 pre-rounding in torch
    ref = torch.from_numpy(fin).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ref, F.encode_e4m3(fin))


ORACLE_FORMAT_PINS = [pin_e4m3_golden, pin_e4m3_structure, pin_e4m3_vs_torch, pin_ue8m0,
                      pin_binary_decoders, pin_round_bf16_f16_f32, pin_f32_div, pin_e4m3_encode]


# ----------------------------------------------------------------------------
# Method steps
# ----------------------------------------------------------------------------


def _bf16_bits_from_f32(x32):
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def pin_mxfp8_decode():
    # byte order: word 0x04030201 holds elements 1,2,3,4 in that order
    w = np.array([[0x44434241, 0x38383838, 0, 0, 0, 0, 0, 0]], dtype=np.uint32)
    codes = M.unpack_mxfp8_codes(w)
    assert list(codes[0, :8]) == [0x41, 0x42, 0x43, 0x44, 0x38, 0x38, 0x38, 0x38]
    # every code x every b in [120, 130]: exact closed form
    allc = np.arange(256, dtype=np.uint32)
    words = (allc[0::4] | (allc[1::4] << 8) | (allc[2::4] << 16) | (allc[3::4] << 24)).reshape(1, 64)
    words = np.repeat(words, 11, axis=0)
    e8 = np.repeat(np.arange(120, 131, dtype=np.uint8)[:, None], 8, axis=1)
    v = M.mxfp8_values(words, e8)
    for i, b in enumerate(range(120, 131)):
        for c in range(256):
            fv = F.e4m3_fraction(c)
            if fv is None:
                assert np.isnan(v[i, c])
            else:
                assert Fraction(v[i, c]) == fv * Fraction(2) ** (b - 127), (b, c)
    # group boundaries: element k uses scale k // 32
    w2 = np.full((1, 16), 0x38383838, dtype=np.uint32)     # all ones, K = 64
    e2 = np.array([[127, 130]], dtype=np.uint8)
    v2 = M.mxfp8_values(w2, e2)
    assert np.all(v2[0, :32] == 1.0) and np.all(v2[0, 32:] == 8.0)
    # outputs are single roundings of the exact value (library casts)
    out32 = M.decode_mxfp8(words, e8, out="f32")
    fin = ~np.isnan(v)
    assert np.array_equal(out32.view(np.float32)[fin].astype(np.float64), v[fin])
    outbf = M.decode_mxfp8(words, e8, out="bf16")
    ref = _bf16_bits_from_f32(v.astype(np.float32))
    assert np.array_equal(outbf[fin], ref[fin])
    assert np.all(outbf[~fin] == 0x7FC0)
    # far scales: overflow to inf in FP32; BF16 subnormal rounding for tiny values
    e_far = np.array([[254, 1, 0, 250, 245, 2, 3, 255]], dtype=np.uint8)
    wf = words[:1]
    vf = M.mxfp8_values(wf, e_far)
    with np.errstate(over="ignore"):
        ref32 = vf.astype(np.float32)
    got32 = M.decode_mxfp8(wf, e_far, out="f32").view(np.float32)
    fin = ~np.isnan(vf)
    assert np.array_equal(got32[fin], ref32[fin])
    gotbf = M.decode_mxfp8(wf, e_far, out="bf16")
    # bf16 by exact enumeration of the rounding: compare to torch's cast of the
    # float32 value, which is exact whenever the float32 value is exact
    exact32 = fin & (ref32.astype(np.float64) == vf)
    assert np.array_equal(gotbf[exact32], _bf16_bits_from_f32(ref32)[exact32])


def _brute_bf16_bits(v):
    """Exact rational -> BF16 bits by round-to-nearest-even on the rational
    value (normal range only), independent of the oracle's rounding."""
    if v == 0:
        return 0
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1                                   # 2^e <= a < 2^(e+1)
    assert -126 <= e <= 127
    ulp = Fraction(2) ** (e - 7)
    m = a / ulp
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = float(fl * ulp) * (-1.0 if v < 0 else 1.0)
    return int(np.array([r], np.float32).view(np.uint32)[0] >> 16)


def pin_mlx_affine_int8():
    """[MXFP8 card, "How it was built", item 2]: w = q * scale + bias per
    128-element group, written as BF16."""
    one_group = lambda q: np.array([q + [0] * (128 - len(q))], np.uint8)
    # hand values: 3 * 0.5 - 1 = 0.5; 0 * 0.5 - 1 = -1
    out = M.decode_mlx_affine_int8(one_group([3]), np.array([[0x3800]], np.uint16), np.array([[0xBC00]], np.uint16))
    assert out[0, 0] == 0x3F00 and out[0, 1] == 0xBF80
    # ties to even: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 (-> 1);
    # 1 + 3 * 2^-8 halfway between 1 + 2^-7 and 1 + 2^-6 (-> the even 1 + 2^-6)
    out = M.decode_mlx_affine_int8(one_group([1, 3]), np.array([[0x1C00]], np.uint16), np.array([[0x3C00]], np.uint16))
    assert out[0, 0] == 0x3F80 and out[0, 1] == 0x3F82
    # one rounding of the exact value: 1 + 2^-8 + 2^-24 is above the tie (-> 1 + 2^-7);
    # rounding it to FP32 first would land on the tie and then on 1
    out = M.decode_mlx_affine_int8(one_group([1]), np.array([[0x0001]], np.uint16), np.array([[0x3C04]], np.uint16))
    assert out[0, 0] == 0x3F81
    # groups of 128 along K: element 127 takes group 0, element 128 group 1
    q2 = np.full((1, 256), 2, np.uint8)
    out = M.decode_mlx_affine_int8(q2, np.array([[0x3C00, 0x4000]], np.uint16), np.array([[0, 0]], np.uint16))
    assert out[0, 127] == 0x4000 and out[0, 128] == 0x4080          # 2 * 1, 2 * 2
    # brute force with exact rationals on random groups
    rng = np.random.default_rng(11)
    n, k = 3, 384
    q = rng.integers(0, 256, (n, k)).astype(np.uint8)
    sc = np.exp2(rng.uniform(-14, -4, (n, k // 128))).astype(np.float16).view(np.uint16)
    bi = (-rng.uniform(96, 160, (n, k // 128)) * F.f16_decode(sc)).astype(np.float16).view(np.uint16)
    got = M.decode_mlx_affine_int8(q, sc, bi)
    got32 = M.decode_mlx_affine_int8(q, sc, bi, out="f32")
    for i in range(n):
        for j in range(k):
            g = j // 128
            v = int(q[i, j]) * Fraction(F.f16_decode(sc[i, g])) + Fraction(F.f16_decode(bi[i, g]))
            assert got[i, j] == _brute_bf16_bits(v), (i, j)
            assert Fraction(float(got32[i:i + 1, j:j + 1].view(np.float32)[0, 0])) == Fraction(float(np.float32(float(v))))
    # NaN scale -> canonical NaN, infinite bias -> infinity
    out = M.decode_mlx_affine_int8(one_group([5]), np.array([[0x7E00]], np.uint16), np.array([[0x7C00]], np.uint16))
    assert out[0, 0] == 0x7FC0
    out = M.decode_mlx_affine_int8(one_group([5]), np.array([[0x3C00]], np.uint16), np.array([[0xFC00]], np.uint16))
    assert out[0, 0] == 0xFF80


def _brute_reencode_row(codes_row, wsi_row_blocks):
    """One row by exact rationals: returns (codes list, scale Fraction)."""
    k = len(codes_row)
    v = []
    for j in range(k):
        fv = F.e4m3_fraction(int(codes_row[j]))
        sc = Fraction(float(wsi_row_blocks[j // 128]))
        v.append(Fraction(float(frac_to_f32(fv * sc))))
    m = max(abs(a) for a in v) if v else Fraction(0)
    s32 = brute_f32_div(m, 448)
    s = Fraction(float(torch.tensor(float(s32), dtype=torch.float32).to(torch.bfloat16).item()))
    q = []
    for a, c in zip(v, codes_row):
        if s == 0:
            q.append(0x80 if (a == 0 and (int(c) & 0x80)) else 0x00)
            continue
        z = brute_f32_div(a, s)
        neg_zero = (z == 0) and bool(int(c) & 0x80)
        q.append(brute_e4m3(-0.0) if neg_zero else brute_e4m3(z))
    return q, s


def pin_reencode_bruteforce():
    rng = np.random.default_rng(9)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    for (n, k) in [(4, 8), (3, 200), (130, 5)]:
        codes = rng.choice(finite, size=(n, k))
        gr, gc = -(-n // 128), -(-k // 128)
        wsi = _bf16_bits_from_f32(np.exp2(rng.uniform(-10, -4, (gr, gc))).astype(np.float32))
        wsi = (wsi.astype(np.uint32) << 16).view(np.float32)
        qo, so = M.reencode_block128_to_row(codes, wsi)
        for r in range(n):
            q, s = _brute_reencode_row(codes[r], wsi[r // 128])
            assert list(qo[r]) == q, (n, k, r)
            assert Fraction(float(F.bf16_decode(so[r]))) == s, (n, k, r)


def pin_reencode_invariants():
    rng = np.random.default_rng(10)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    n, k = 256, 384
    codes = rng.choice(finite, size=(n, k))
    # (i) shared-scale invariant: every block of a 128-row band shares one
    # BF16-representable scale and every row holds a +-448 code.
    codes_s = codes.copy()
    codes_s[:, 5] = 0x7E
    codes_s[1::2, 5] = 0xFE
    band_scale = np.array([2.0 ** -7 * 1.5, 2.0 ** -9 * 1.25], dtype=np.float32)
    wsi = np.repeat(band_scale[:, None], 3, axis=1)
    qo, so = M.reencode_block128_to_row(codes_s, wsi)
    assert np.array_equal(qo, codes_s)
    assert np.array_equal(F.bf16_decode(so), np.repeat(band_scale.astype(np.float64), 128))
    # (ii) every nonzero row reaches +-448; (iii) the FP8 card's per-element
    # bound: within half an E4M3 ulp at the element's magnitude, in units of
    # the row scale (the source is exact here, so no BF16 term).
    wsi2 = np.exp2(rng.uniform(-10, -4, (2, 3))).astype(np.float32)
    wsi2 = (_bf16_bits_from_f32(wsi2).astype(np.uint32) << 16).view(np.float32)
    qo, so = M.reencode_block128_to_row(codes, wsi2)
    assert np.all(np.any((qo & 0x7F) == 0x7E, axis=1))
    v = M.block_decode_f32(codes, wsi2)
    s = F.bf16_decode(so)[:, None]
    deq = F.e4m3_decode(qo) * s
    mag = np.abs(v) / s
    _, e = np.frexp(mag)
    ulp = np.exp2(np.maximum(e - 1, -6) - 3)          # E4M3 ulp at |v|/s
    assert np.all(np.abs(deq - v) <= 0.5 * ulp * s * (1 + 2.0 ** -20))
    # (iv) a row range gives the same slice as the full re-encode
    q2, s2 = M.reencode_block128_to_row(codes, wsi2, 100, 200)
    assert np.array_equal(q2, qo[100:200]) and np.array_equal(s2, so[100:200])
    # (v) zero rows: scale +0, signed zeros kept
    z = np.zeros((2, 8), np.uint8)
    z[1, ::2] = 0x80
    qz, sz = M.reencode_block128_to_row(z, np.ones((1, 1), np.float32))
    assert np.all(sz == 0) and np.array_equal(qz, z)
    # grid must match the code shape
    try:
        M.reencode_block128_to_row(codes, np.ones((2, 2), np.float32))
    except M.GridShapeError:
        pass
    else:
        raise AssertionError("grid shape not validated")


def pin_encode_fp8row_bf16():
    rng = np.random.default_rng(11)
    w = _bf16_bits_from_f32((rng.standard_normal((5, 300)) * 0.02).astype(np.float32))
    q, s = M.encode_fp8row_bf16(w)
    wv = F.bf16_decode(w)
    for r in range(5):
        m = max(abs(Fraction(x)) for x in wv[r])
        s32 = brute_f32_div(m, 448)
        sb = Fraction(float(torch.tensor(float(s32), dtype=torch.float32).to(torch.bfloat16).item()))
        assert Fraction(float(F.bf16_decode(s[r]))) == sb
        for j in range(300):
            assert int(q[r, j]) == brute_e4m3(brute_f32_div(Fraction(wv[r, j]), sb)) or \
                (wv[r, j] == 0 and int(q[r, j]) in (0, 0x80))


def _brute_encode_row(vals, neg_zero):
    """fp8_row_maxabs of one row by exact rationals, for any row maximum:
    vals are the exact FP32 source values (Fractions), neg_zero[j] marks a -0
    element.  s = bf16(f32(m / 448)); a zero element keeps its signed zero (0 / s
    is a zero, and 0 / 0 is not evaluated); with s = 0 a nonzero element's
    quotient is infinite and saturates to +-448; otherwise the E4M3 RNE
    (saturating) of the FP32 quotient.  Returns (codes, s, largest quotient)."""
    m = max(abs(a) for a in vals)
    s = Fraction(float(torch.tensor(float(brute_f32_div(m, 448)), dtype=torch.float32).to(torch.bfloat16).item()))
    q, zmax = [], Fraction(0)
    for a, nz in zip(vals, neg_zero):
        if a == 0:
            q.append(0x80 if nz else 0x00)
        elif s == 0:
            q.append(0xFE if a < 0 else 0x7E)
        else:
            z = brute_f32_div(a, s)
            zmax = max(zmax, abs(z))
            q.append(brute_e4m3(z))
    return q, s, zmax


def tiny_row_bf16(seed):
    """BF16 rows whose maxima put m / 448 in or below BF16's subnormal range
    (m from ~1e-38 to ~5.3e-36, where the row scale keeps 1..7 significant
    bits), plus the normal boundary s = 2^-126; the other elements uniform in
    [-m, m] (many of them BF16 subnormals), one -0 and one +0 per row."""
    rng = np.random.default_rng(seed)
    maxima = [1e-37, -3.3e-37, 2.0e-36, 5.25e-36, 448 * 2.0 ** -126, 4.0e-38, 2.9e-38, 1.0e-38, 6.1e-38, 7.7e-37]
    rows = []
    for m in maxima:
        r = rng.uniform(-1, 1, 40) * abs(m)
        r[rng.integers(0, 40)] = m
        r[3], r[7] = -0.0, 0.0
        rows.append(r)
    return _bf16_bits_from_f32(np.array(rows, np.float64).astype(np.float32))


def pin_encode_tiny_rows():
    """[FP8 card, "Conversion and verification"]: the per-row encoding for
    rows whose scale m / 448 is a BF16 subnormal (or rounds to zero).  The
    scale then carries few significant bits and quotients reach ~670 (beyond
    E4M3's 448), which saturate to +-448 (the saturating encode)."""
    w = tiny_row_bf16(31)
    q, s = M.encode_fp8row_bf16(w)
    wv = F.bf16_decode(w)
    zmax = Fraction(0)
    for r in range(w.shape[0]):
        vals = [Fraction(float(v)) for v in wv[r]]
        qb, sb, zm = _brute_encode_row(vals, [bool(np.signbit(v)) and v == 0 for v in wv[r]])
        assert Fraction(float(F.bf16_decode(s[r]))) == sb, r
        assert list(q[r]) == qb, r
        zmax = max(zmax, zm)
    assert zmax > 464                      # the saturating case is exercised
    assert np.any(s == 0) and np.any((s > 0) & (s < 0x80))  # zero and subnormal scales
    # block-scaled source with a weight_scale_inv near 2^-131 (FP32 subnormal,
    # not BF16-rounded): decoded values and the row scale are subnormal
    rng = np.random.default_rng(32)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    codes = rng.choice(finite, size=(3, 200))
    codes[:, 17] = 0x7E
    wsi = np.array([[1.37 * 2.0 ** -131, 0.9 * 2.0 ** -131]], np.float32)
    qo, so = M.reencode_block128_to_row(codes, wsi)
    zmax = Fraction(0)
    for r in range(3):
        vals, nz = [], []
        for j in range(200):
            fv = F.e4m3_fraction(int(codes[r, j]))
            vals.append(Fraction(float(frac_to_f32(fv * Fraction(float(wsi[0, j // 128]))))))
            nz.append(vals[-1] == 0 and bool(int(codes[r, j]) & 0x80))
        qb, sb, zm = _brute_encode_row(vals, nz)
        assert Fraction(float(F.bf16_decode(so[r]))) == sb, r
        assert list(qo[r]) == qb, r
        zmax = max(zmax, zm)
    assert zmax > 464 and np.all(so < 0x80)          # subnormal scales, saturating quotients


def pin_quantize_int8():
    # closed-form ties: a group whose amax is 127 has scale exactly 1
    cases = [(Fraction(a), int(b)) for kind, a, b in _read_golden("rounding_cases.txt") if kind == "int8_s1"]
    xs = np.zeros((1, 64), np.float32)
    xs[0, 0] = 127.0
    for i, (a, _) in enumerate(cases):
        xs[0, 1 + i] = float(a)
    q, s = M.quantize_act_int8_g64(_bf16_bits_from_f32(xs))
    assert s.view(np.float32)[0, 0] == 1.0
    for i, (_, want) in enumerate(cases):
        assert int(q[0, 1 + i]) == want, (cases[i], int(q[0, 1 + i]))
    # zero group -> scale 0, codes 0; amax element -> +-127; |q| <= 127
    rng = np.random.default_rng(12)
    x = rng.standard_normal((7, 256)).astype(np.float32)
    x[3, 64:128] = 0.0
    x[2, 5] = -40.0
    xb = _bf16_bits_from_f32(x)
    q, s = M.quantize_act_int8_g64(xb)
    assert np.all(s.view(np.float32)[3, 1] == 0) and np.all(q[3, 64:128] == 0)
    assert q[2, 5] == -127
    assert np.all(np.abs(q.astype(np.int32)) <= 127)
    # library IEEE float32 arithmetic (numpy) on a large sample: catches a
    # reciprocal-multiply or a double rounding, which touch ~0.1% of elements
    xl = rng.standard_normal((512, 1024)).astype(np.float32)
    xl = xl * np.where(rng.random(xl.shape) < 0.01, 20.0, 1.0).astype(np.float32)
    xlb = _bf16_bits_from_f32(xl)
    xl32 = (xlb.astype(np.uint32) << 16).view(np.float32).reshape(512, 16, 64)
    amax32 = np.max(np.abs(xl32), axis=2)
    s32 = amax32 / np.float32(127.0)
    ref = np.clip(np.rint(xl32 / s32[:, :, None]), -127, 127).astype(np.int8).reshape(512, 1024)
    ql, sl = M.quantize_act_int8_g64(xlb)
    assert np.array_equal(sl.view(np.float32), s32)
    assert np.array_equal(ql, ref)
    xv = F.bf16_decode(xb)
    for t in range(7):
        for g in range(4):
            grp = xv[t, g * 64:(g + 1) * 64]
            amax = max(abs(Fraction(v)) for v in grp)
            if amax == 0:
                continue
            s_ref = brute_f32_div(amax, 127)
            assert Fraction(float(s.view(np.float32)[t, g])) == s_ref
            for j in range(64):
                z = brute_f32_div(Fraction(grp[j]), s_ref)
                r = round(z)                       # Python rounds half to even
                r = max(-127, min(127, r))
                assert int(q[t, g * 64 + j]) == r


def pin_gemv_fp8row():
    rng = np.random.default_rng(13)
    n, k, t = 8, 40, 4
    w = rng.integers(0, 256, (n, k)).astype(np.uint8)
    w[w == 0x7F] = 0x7E
    w[w == 0xFF] = 0xFE
    sb = _bf16_bits_from_f32(np.exp2(rng.uniform(-12, -4, n)).astype(np.float32))
    # one-hot activations reproduce the decoded weight columns exactly
    eye = _bf16_bits_from_f32(np.eye(k, dtype=np.float32))
    y = M.gemv_fp8row(w, sb, eye)
    assert np.array_equal(y, (F.e4m3_decode(w) * F.bf16_decode(sb)[:, None]).T)
    # exact rational brute force
    x = _bf16_bits_from_f32(rng.standard_normal((t, k)).astype(np.float32))
    y = M.gemv_fp8row(w, sb, x)
    xv, sv = F.bf16_decode(x), F.bf16_decode(sb)
    for ti in range(t):
        for ni in range(n):
            terms = [Fraction(xv[ti, j]) * F.e4m3_fraction(w[ni, j]) for j in range(k)]
            ex = Fraction(sv[ni]) * sum(terms)
            bound = Fraction(sv[ni]) * sum(abs(v) for v in terms) * Fraction(1, 2 ** 45)
            assert abs(Fraction(y[ti, ni]) - ex) <= bound


def _brute_group_gemv(fmt, q_int, sc, xv, gs):
    t, k = xv.shape
    n = len(q_int)
    out = np.zeros((t, n))
    mag = np.zeros((t, n))
    for ti in range(t):
        for ni in range(n):
            acc = Fraction(0)
            a = Fraction(0)
            for g in range(k // gs):
                terms = [Fraction(xv[ti, j]) * q_int[ni][j] for j in range(g * gs, (g + 1) * gs)]
                acc += Fraction(sc[ni][g]) * sum(terms)
                a += Fraction(sc[ni][g]) * sum(abs(v) for v in terms)
            out[ti, ni] = float(acc)
            mag[ti, ni] = float(a)
    return out, mag


def pin_gemv_qgroup():
    rng = np.random.default_rng(14)
    t, n = 4, 8
    # nibble order: byte 0x8F holds element 0 = -1 (low nibble) and element 1 = -8
    q = M.unpack_q4(np.array([[0x8F, 0x70]], np.uint8), 4)
    assert list(q[0]) == [-1, -8, 0, 7]
    for fmt, gs in (("q4g64", 64), ("q8g32", 32), ("q8g64", 64), ("mxfp8", 32)):
        k = 2 * gs
        if fmt == "q4g64":
            codes = rng.integers(0, 256, (n, k // 2)).astype(np.uint8)
            qi = [[int(v) for v in row] for row in M.unpack_q4(codes, k)]
        elif fmt.startswith("q8"):
            codes = rng.integers(-127, 128, (n, k)).astype(np.int8)
            qi = [[int(v) for v in row] for row in codes]
        else:
            finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint32)
            b = rng.choice(finite, (n, k))
            codes = (b[:, 0::4] | (b[:, 1::4] << 8) | (b[:, 2::4] << 16) | (b[:, 3::4] << 24)).astype(np.uint32)
            qi = [[F.e4m3_fraction(int(v)) for v in row] for row in b]
        if fmt == "mxfp8":
            scales = rng.integers(120, 131, (n, k // gs)).astype(np.uint8)
            scv = [[Fraction(2) ** (int(v) - 127) for v in row] for row in scales]
        else:
            scales = np.exp2(rng.uniform(-9, -5, (n, k // gs))).astype(np.float16).view(np.uint16)
            scv = [[Fraction(float(v)) for v in row] for row in scales.view(np.float16)]
        x = _bf16_bits_from_f32(rng.standard_normal((t, k)).astype(np.float32))
        y = M.gemv_qgroup(fmt, codes, scales, x)
        ref, mag = _brute_group_gemv(fmt, qi, scv, F.bf16_decode(x), gs)
        assert np.all(np.abs(y - ref) <= mag * 2.0 ** -45), fmt
        # one-hot: column k of the decoded matrix
        kk = 3
        e = np.zeros((1, k), np.float32)
        e[0, kk] = 1
        y1 = M.gemv_qgroup(fmt, codes, scales, _bf16_bits_from_f32(e))
        for ni in range(n):
            assert Fraction(y1[0, ni]) == Fraction(qi[ni][kk]) * scv[ni][kk // gs], (fmt, ni)
    # bf16 weights: plain products
    wb = _bf16_bits_from_f32(rng.standard_normal((n, 16)).astype(np.float32))
    x = _bf16_bits_from_f32(rng.standard_normal((t, 16)).astype(np.float32))
    y = M.gemv_qgroup("bf16", wb, None, x)
    ref = torch.from_numpy(F.bf16_decode(x)) @ torch.from_numpy(F.bf16_decode(wb)).T
    assert np.allclose(y, ref.numpy(), rtol=1e-14, atol=1e-14)


def _pack_stream(codes, bits):
    """Independent packer: each row's codes as one Python integer, code j at
    bit b j (two's complement), written out little-endian."""
    out = []
    for row in codes:
        acc = 0
        for j, c in enumerate(row):
            acc |= (int(c) & ((1 << bits) - 1)) << (bits * j)
        out.append(list(acc.to_bytes(len(row) * bits // 8, "little")))
    return np.array(out, np.uint8)


def pin_qbits():
    """[RTX5080 card, "Quantization profile"]: Q3 / Q5 group-64 codes; the
    dense little-endian bit-stream reading (element j at bits [b j, b j + b))."""
    # hand-packed: Q5 codes -16, 15, 0, -1, 7, -8, 1, 2 are the 5-bit fields
    # 10000 01111 00000 11111 00111 11000 00001 00010 (written MSB first) at bits
    # 0, 5, 10, ..., 35: byte 0 = bits 7..0 = 1111 0000, byte 1 = 1000 0001,
    # byte 2 = 0111 1111, byte 3 = 0111 0000, byte 4 = 0001 0000
    q5 = M.unpack_qbits(np.array([[0xF0, 0x81, 0x7F, 0x70, 0x10]], np.uint8), 8, 5)
    assert list(q5[0]) == [-16, 15, 0, -1, 7, -8, 1, 2]
    # Q3 codes -4, 3, 0, -1, 1, 2, -2, -3: fields 100 011 000 111 001 010 110 101
    # at bits 0, 3, ..., 21: bytes 0001 1100, 0001 1110, 1011 1001
    q3 = M.unpack_qbits(np.array([[0x1C, 0x1E, 0xB9]], np.uint8), 8, 3)
    assert list(q3[0]) == [-4, 3, 0, -1, 1, 2, -2, -3]
    rng = np.random.default_rng(24)
    for bits in (3, 5, 6):
        lo = -(1 << (bits - 1))
        codes = rng.integers(lo, -lo, (5, 128))
        packed = _pack_stream(codes, bits)
        assert packed.shape == (5, 16 * bits)
        assert np.array_equal(M.unpack_qbits(packed, 128, bits), codes)
        # and bit by bit from the bytes, with Python integers
        for r in range(5):
            v = int.from_bytes(bytes(packed[r]), "little")
            for j in range(128):
                u = (v >> (bits * j)) & ((1 << bits) - 1)
                assert M.unpack_qbits(packed[r:r + 1], 128, bits)[0, j] == (u - (1 << bits) if u >> (bits - 1) else u)
    # b = 4 is the Q4 nibble layout
    b4 = rng.integers(0, 256, (3, 64)).astype(np.uint8)
    assert np.array_equal(M.unpack_qbits(b4, 128, 4), M.unpack_q4(b4, 128))
    # grouped GEMV on Q5 / Q3 codes by exact rationals
    t, n, k = 3, 5, 128
    for fmt, bits in (("q5g64", 5), ("q3g64", 3), ("q6g64", 6)):
        lo = -(1 << (bits - 1))
        codes = rng.integers(lo, -lo, (n, k))
        packed = _pack_stream(codes, bits)
        scales = np.exp2(rng.uniform(-9, -5, (n, 2))).astype(np.float16).view(np.uint16)
        scv = [[Fraction(float(v)) for v in row] for row in scales.view(np.float16)]
        x = _bf16_bits_from_f32(rng.standard_normal((t, k)).astype(np.float32))
        y = M.gemv_qgroup(fmt, packed, scales, x)
        ref, mag = _brute_group_gemv(fmt, [[int(v) for v in row] for row in codes], scv, F.bf16_decode(x), 64)
        assert np.all(np.abs(y - ref) <= mag * 2.0 ** -45), fmt
        # A8 routes: the codes enter the int8 arithmetic exactly
        xa = _bf16_bits_from_f32(rng.standard_normal((130, k)).astype(np.float32))
        qa, sa = M.quantize_act_int8_g64(xa)
        ya, sums = M.gemm_w8a8_g64(qa, sa, codes.astype(np.int8), scales, return_sums=True)
        assert np.array_equal(M.linear_qbits_g64(fmt, xa, packed, scales, True), ya)
        assert np.array_equal(M.linear_qbits_g64(fmt, xa[:9], packed, scales, False, True), ya[:9])
        assert np.array_equal(M.linear_qbits_g64(fmt, xa[:9], packed, scales, True), M.gemv_qgroup(fmt, packed, scales, xa[:9]))
        for i in (0, 129):
            for j in range(n):
                assert sums[i, j, 1] == sum(int(qa[i, kk]) * int(codes[j, kk]) for kk in range(64, 128))


def pin_w8a8():
    rng = np.random.default_rng(15)
    m, n, k = 3, 5, 128
    a = rng.integers(-127, 128, (m, k)).astype(np.int8)
    w = rng.integers(-127, 128, (n, k)).astype(np.int8)
    p = M.w8a8_group_sums(a, w)
    for i in range(m):
        for j in range(n):
            for g in range(2):
                s = sum(int(a[i, kk]) * int(w[j, kk]) for kk in range(g * 64, (g + 1) * 64))
                assert p[i, j, g] == s
    # power-of-two scales, one group: the scaled sum is exact
    a_s = np.exp2(rng.integers(-8, -2, (m, 2))).astype(np.float32)
    w_s = np.exp2(rng.integers(-9, -5, (n, 2))).astype(np.float16)
    y, sums = M.gemm_w8a8_g64(a, a_s.view(np.uint32), w, w_s.view(np.uint16), return_sums=True)
    assert np.array_equal(sums, p)
    for i in range(m):
        for j in range(n):
            ex = sum(Fraction(int(p[i, j, g])) * Fraction(float(a_s[i, g])) * Fraction(float(w_s[j, g]))
                     for g in range(2))
            assert Fraction(y[i, j]) == ex
    # general FP16 / FP32 scales: rational brute force
    a_s = (np.abs(rng.standard_normal((m, 2))) * 0.05 + 1e-3).astype(np.float32)
    w_s = np.exp2(rng.uniform(-9, -5, (n, 2))).astype(np.float16)
    y = M.gemm_w8a8_g64(a, a_s.view(np.uint32), w, w_s.view(np.uint16))
    for i in range(m):
        for j in range(n):
            ex = sum(Fraction(int(p[i, j, g])) * Fraction(float(a_s[i, g])) * Fraction(float(w_s[j, g]))
                     for g in range(2))
            assert abs(Fraction(y[i, j]) - ex) <= abs(ex) * Fraction(1, 2 ** 50)


def pin_fp8_act_and_gemm():
    rng = np.random.default_rng(16)
    m, n, k = 3, 4, 50
    x = rng.standard_normal((m, k)).astype(np.float32)
    x[1] = 0
    x[1, 3] = -0.0
    xb = _bf16_bits_from_f32(x)
    qa, sa = M.quantize_act_fp8_row(xb)
    xv = F.bf16_decode(xb)
    for i in range(m):
        amax = max(abs(Fraction(v)) for v in xv[i])
        s_ref = brute_f32_div(amax, 448) if amax else Fraction(0)
        assert Fraction(float(sa.view(np.float32)[i])) == s_ref
        for j in range(k):
            if s_ref == 0:
                want = 0x80 if np.signbit(xv[i, j]) else 0
            else:
                z = brute_f32_div(Fraction(xv[i, j]), s_ref)
                want = brute_e4m3(-0.0 if (z == 0 and np.signbit(xv[i, j])) else z)
            assert int(qa[i, j]) == want
        if amax:
            assert np.any((qa[i] & 0x7F) == 0x7E)
    w = rng.integers(0, 256, (n, k)).astype(np.uint8)
    w[(w & 0x7F) == 0x7F] = 0x3C
    sw = _bf16_bits_from_f32(np.exp2(rng.uniform(-12, -4, n)).astype(np.float32))
    y, qa2, sa2 = M.gemm_fp8row(xb, w, sw)
    assert np.array_equal(qa2, qa)
    for i in range(m):
        for j in range(n):
            ex = Fraction(float(sa.view(np.float32)[i])) * Fraction(F.bf16_decode(sw[j])) * sum(
                F.e4m3_fraction(int(qa[i, kk])) * F.e4m3_fraction(int(w[j, kk])) for kk in range(k))
            assert abs(Fraction(y[i, j]) - ex) <= abs(ex) * Fraction(1, 2 ** 48) + Fraction(1, 2 ** 300)


def pin_route():
    assert M.route(128, True) == "bf16" and M.route(129, True) == "a8"
    assert M.route(1792, False) == "bf16" and M.route(1, True) == "bf16"
    rng = np.random.default_rng(17)
    n, k = 6, 128
    w = rng.integers(-127, 128, (n, k)).astype(np.int8)
    ws = np.exp2(rng.uniform(-9, -5, (n, 2))).astype(np.float16).view(np.uint16)
    x = _bf16_bits_from_f32(rng.standard_normal((129, k)).astype(np.float32))
    below = M.linear_w8g64(x[:128], w, ws, True)
    assert np.array_equal(below, M.gemv_qgroup("q8g64", w, ws, x[:128]))
    at = M.linear_w8g64(x, w, ws, True)
    qa, sa = M.quantize_act_int8_g64(x)
    assert np.array_equal(at, M.gemm_w8a8_g64(qa, sa, w, ws))
    assert not np.array_equal(at[:128], below)        # a different rounding of the activations
    # the A8 decode flag: steps of at most 128 tokens take the W8A8 arithmetic
    assert M.route(1, False, True) == "a8_decode" and M.route(128, True, True) == "a8_decode"
    assert M.route(129, False, True) == "bf16" and M.route(129, True, True) == "a8"
    dec = M.linear_w8g64(x[:33], w, ws, False, True)
    assert np.array_equal(dec, M.gemm_w8a8_g64(qa[:33], sa[:33], w, ws))      # per-token quantization
    # the group sums by integer brute force (each 64-channel group exact)
    _, sums = M.gemm_w8a8_g64(qa[:3], sa[:3], w, ws, return_sums=True)
    for i in range(3):
        for j in range(n):
            for g in range(2):
                assert sums[i, j, g] == sum(int(qa[i, kk]) * int(w[j, kk]) for kk in range(64 * g, 64 * g + 64))


def pin_linear_q4g64():
    """Q4 on both routes: below 129 tokens the grouped GEMV, from 129 on the
    W8A8 GEMM whose int32 group sums are the exact integer dot products of
    the int8 activation codes and the Q4 codes."""
    rng = np.random.default_rng(23)
    n, k = 5, 128
    w = rng.integers(0, 256, (n, k // 2)).astype(np.uint8)
    ws = np.exp2(rng.uniform(-9, -5, (n, 2))).astype(np.float16).view(np.uint16)
    x = _bf16_bits_from_f32(rng.standard_normal((129, k)).astype(np.float32))
    assert np.array_equal(M.linear_q4g64(x[:128], w, ws, True), M.gemv_qgroup("q4g64", w, ws, x[:128]))
    assert np.array_equal(M.linear_q4g64(x[:130], w, ws, False), M.gemv_qgroup("q4g64", w, ws, x[:130]))
    qa, sa = M.quantize_act_int8_g64(x)
    y, sums = M.gemm_w8a8_g64(qa, sa, M.unpack_q4(w, k), ws, return_sums=True)
    assert np.array_equal(M.linear_q4g64(x, w, ws, True), y)
    # A8 decode: below 129 tokens with the decode flag, the same W8A8 arithmetic
    assert np.array_equal(M.linear_q4g64(x[:16], w, ws, False, True), y[:16])
    # the group sums by brute force over the nibbles (low nibble first, two's complement)
    for i in (0, 64, 128):
        for j in range(n):
            for g in range(2):
                acc = 0
                for kk in range(64 * g, 64 * g + 64):
                    b = int(w[j, kk // 2])
                    nib = (b >> 4) if kk % 2 else (b & 15)
                    acc += int(qa[i, kk]) * (nib - 16 if nib >= 8 else nib)
                assert sums[i, j, g] == acc


ORACLE_METHOD_PINS = [pin_mxfp8_decode, pin_mlx_affine_int8, pin_reencode_bruteforce, pin_reencode_invariants,
                      pin_encode_fp8row_bf16, pin_encode_tiny_rows, pin_quantize_int8, pin_gemv_fp8row, pin_gemv_qgroup,
                      pin_w8a8, pin_fp8_act_and_gemm, pin_route, pin_linear_q4g64, pin_qbits]

ALL_PINS = ORACLE_FORMAT_PINS + ORACLE_METHOD_PINS
