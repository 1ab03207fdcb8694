"""HIP library vs the CPU oracle, through the C ABI (needs an MI355X).

Integer and encoded results (decoded weights, re-encoded codes and scales,
int8 codes and scales, int32 group sums, FP8 activation codes) must match the
oracle bit for bit.  FP32 outputs must be within a relative Frobenius error of
1e-5 of the float64 oracle; a BF16 output must be the round-to-nearest-even of
the same kernel's FP32 output, bit for bit, and within 2^-8 of the oracle.
Inputs come from the seeded generators; the oracle never sees a GPU result.
"""

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import method as M
from quantized_weight_linear_amd import nq
from quantized_weight_linear_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"
FP32_TOL = 1e-5
BF16_TOL = 2.0 ** -8

_NP2T = {np.uint8: torch.uint8, np.int8: torch.int8, np.uint16: torch.int16, np.int16: torch.int16,
         np.uint32: torch.int32, np.int32: torch.int32, np.float32: torch.float32}


def dev(a):
    a = np.ascontiguousarray(a)
    view = {np.dtype(np.uint16): np.int16, np.dtype(np.uint32): np.int32}.get(a.dtype)
    if view is not None:
        a = a.view(view)
    return torch.from_numpy(a).to(DEV)


def host(t, dtype):
    torch.cuda.synchronize()
    return t.cpu().numpy().view(dtype)


def empty(shape, np_dtype):
    return torch.empty(shape, dtype=_NP2T[np_dtype], device=DEV)


def rel_fro(got, ref):
    ref = np.asarray(ref, np.float64)
    d = np.linalg.norm(np.asarray(got, np.float64) - ref)
    n = np.linalg.norm(ref)
    return d / n if n > 0 else d


def bf16_of_f32_bits(f32):
    return F.encode_bf16(np.asarray(f32, np.float32).astype(np.float64))


def say(msg):
    print(msg, flush=True)


@pytest.fixture(autouse=True)
def _announce(request):
    say(f"[gpu] {request.node.name}")
    yield
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# a1: MXFP8 decode
# ---------------------------------------------------------------------------

def _all_code_words(rows):
    c = np.arange(256, dtype=np.uint32)
    words = (c[0::4] | (c[1::4] << 8) | (c[2::4] << 16) | (c[3::4] << 24)).reshape(1, 64)
    return np.repeat(words, rows, axis=0)


@pytest.mark.parametrize("bvals", [list(range(120, 131)), [0, 1, 2, 3, 127, 245, 246, 247, 250, 254, 255]])
def test_decode_mxfp8_every_code(bvals):
    words = _all_code_words(len(bvals))
    e8 = np.repeat(np.array(bvals, np.uint8)[:, None], 8, axis=1)
    n, k = words.shape[0], 256
    for out in ("f32", "bf16"):
        y = empty((n, k), np.float32 if out == "f32" else np.uint16)
        nq.nq_decode_mxfp8(dev(words), dev(e8), n, k, y)
        got = host(y, np.uint32 if out == "f32" else np.uint16)
        ref = M.decode_mxfp8(words, e8, out=out)
        assert np.array_equal(got, ref), out


def test_decode_mxfp8_config1():
    d = W.mxfp8_gemv()
    n, k = d["words"].shape[0], d["words"].shape[1] * 4
    for out in ("f32", "bf16"):
        y = empty((n, k), np.float32 if out == "f32" else np.uint16)
        nq.nq_decode_mxfp8(dev(d["words"]), dev(d["e8m0"]), n, k, y)
        assert np.array_equal(host(y, np.uint32 if out == "f32" else np.uint16),
                              M.decode_mxfp8(d["words"], d["e8m0"], out=out))


# ---------------------------------------------------------------------------
# a2: block-128 -> per-row re-encode, and BF16 -> per-row encode
# ---------------------------------------------------------------------------

def _block_inputs(n, k, seed, bf16_scales=True):
    g = W.rng(90, seed)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    codes = finite[g.integers(0, finite.size, (n, k))]
    shape = (-(-n // 128), -(-k // 128))
    if bf16_scales:
        wsi = W.bf16_log_uniform_as_f32(g, shape, -10, -4)
    else:
        wsi = np.exp2(g.uniform(-10, -4, shape)).astype(np.float32)    # full 24-bit significands
    return codes, wsi


def _gpu_reencode(codes, wsi, r0, r1):
    n, k = codes.shape
    oc = empty((r1 - r0, k), np.uint8)
    osc = empty((r1 - r0,), np.uint16)
    nq.nq_reencode_block128_to_row(dev(codes), dev(wsi), n, k, r0, r1, oc, osc)
    return host(oc, np.uint8), host(osc, np.uint16)


@pytest.mark.parametrize("n,k,bf16_scales", [(300, 520, True), (130, 200, False), (4, 8, True),
                                             (256, 384, False), (129, 1000, True)])
def test_reencode_small(n, k, bf16_scales):
    codes, wsi = _block_inputs(n, k, n * 7 + k, bf16_scales)
    codes[1] = 0x00                        # zero row: scale +0, codes unchanged
    codes[2, ::3] = 0x80
    codes[2, 1::3] = 0x00
    codes[2, 2::3] = 0x80
    if n > 5:
        codes[5, 3] = 0x7F                 # NaN row
    for r0, r1 in [(0, n), (1, min(n, 3)), (n // 2, n)]:
        q, s = _gpu_reencode(codes, wsi, r0, r1)
        qo, so = M.reencode_block128_to_row(codes, wsi, r0, r1)
        assert np.array_equal(s, so), (r0, r1)
        assert np.array_equal(q, qo), (r0, r1)


def test_reencode_config3_full():
    """Every row of the 5120x17408 re-encode, bit for bit (the oracle runs in
    bands of 512 rows, four block rows each)."""
    d = W.block128_codes()
    n, k = d["codes"].shape
    q, s = _gpu_reencode(d["codes"], d["wsi"], 0, n)
    for r0 in range(0, n, 512):
        r1 = min(n, r0 + 512)
        qo, so = M.reencode_block128_to_row(d["codes"][r0:r1], d["wsi"][r0 // 128:(r1 + 127) // 128], 0, r1 - r0)
        assert np.array_equal(so, s[r0:r1]), r0
        assert np.array_equal(qo, q[r0:r1]), r0
    # a row range reads only its block rows and gives the same slice
    q2, s2 = _gpu_reencode(d["codes"], d["wsi"], 1000, 1300)
    assert np.array_equal(q2, q[1000:1300]) and np.array_equal(s2, s[1000:1300])


@pytest.mark.parametrize("n,k", [(64, 5120), (33, 200), (4, 8), (17, 16)])
def test_encode_fp8row_bf16_small(n, k):
    w = W.bf16_normal(W.rng(92, n + k), (n, k), std=0.02)
    w[0, :] = 0
    oc, osc = empty((n, k), np.uint8), empty((n,), np.uint16)
    nq.nq_encode_fp8row_bf16(dev(w), n, k, oc, osc)
    qo, so = M.encode_fp8row_bf16(w)
    assert np.array_equal(host(osc, np.uint16), so) and np.array_equal(host(oc, np.uint8), qo)


def _tiny_rows_bf16(k, seed):
    """BF16 rows whose maxima put m / 448 in or below BF16's subnormal range
    (the row scale keeps 0..7 significant bits, quotients reach ~670 and
    saturate), the normal boundary 448 * 2^-126, and a normal row; elements
    uniform in [-m, m], with signed zeros."""
    g = W.rng(120, seed)
    maxima = [1e-37, -3.3e-37, 2.0e-36, 5.25e-36, 448 * 2.0 ** -126, 4.0e-38, 2.9e-38, 1.0e-38, 6.1e-38,
              7.7e-37, 1.3e-36, 0.25]
    rows = []
    for m in maxima:
        r = g.uniform(-1, 1, k) * abs(m)
        r[g.integers(0, k)] = m
        r[3], r[7] = -0.0, 0.0
        rows.append(r)
    return W.to_bf16_bits(np.array(rows, np.float64).astype(np.float32))


@pytest.mark.parametrize("k", [256, 5120, 40])
def test_encode_fp8row_bf16_tiny_rows(k):
    w = _tiny_rows_bf16(k, k)
    n = w.shape[0]
    oc, osc = empty((n, k), np.uint8), empty((n,), np.uint16)
    nq.nq_encode_fp8row_bf16(dev(w), n, k, oc, osc)
    qo, so = M.encode_fp8row_bf16(w)
    assert np.any(so == 0) and np.any((so > 0) & (so < 0x80))     # zero and subnormal scales occur
    assert np.array_equal(host(osc, np.uint16), so)
    assert np.array_equal(host(oc, np.uint8), qo)


@pytest.mark.parametrize("n,k", [(300, 520), (130, 256)])
def test_reencode_tiny_block_scales(n, k):
    """weight_scale_inv near 2^-131 (FP32 subnormal, not BF16-rounded) in some
    blocks: decoded values and row scales subnormal, quotients saturating."""
    codes, wsi = _block_inputs(n, k, 77 + n, bf16_scales=False)
    codes[:, 17] = 0x7E
    wsi[0, :] = np.array([1.37, 0.9, 1.11, 1.6, 1.2][:wsi.shape[1]], np.float64) * 2.0 ** -131
    if wsi.shape[0] > 1:
        wsi[1, 0] = 3.1 * 2.0 ** -140
    q, s = _gpu_reencode(codes, wsi, 0, n)
    qo, so = M.reencode_block128_to_row(codes, wsi)
    assert np.all(so[:128] < 0x80)
    assert np.array_equal(s, so)
    assert np.array_equal(q, qo)


# ---------------------------------------------------------------------------
# a5: int8 activation quantization; a7 input: E4M3 per-token quantization
# ---------------------------------------------------------------------------

def _special_activations(t, k):
    x = W.bf16_normal(W.rng(93, t * k), (t, k), outlier_p=0.01)
    xf = (x.astype(np.uint32) << 16).view(np.float32).copy()
    xf[0, :64] = 0.0                                       # zero group
    xf[1, :64] = np.array([127.0, 2.5, 3.5, -2.5, 126.5, -126.5, 0.5, 1.5] * 8, np.float32)  # ties
    xf[2, 64:128] = -3.0                                    # constant group
    xf[3, 5] = np.nan                                       # NaN group
    xf[3, 70] = np.inf                                      # inf group
    xf[4, :] = -0.0
    return W.to_bf16_bits(xf)


@pytest.mark.parametrize("t,k", [(7, 256), (33, 5120), (1, 64)])
def test_quantize_int8_small(t, k):
    x = _special_activations(max(t, 5), k)[:t] if t >= 5 else W.bf16_normal(W.rng(94, k), (t, k))
    q, s = empty((t, k), np.int8), empty((t, k // 64), np.float32)
    nq.nq_quantize_act_int8_g64(dev(x), t, k, q, s)
    qo, so = M.quantize_act_int8_g64(x)
    assert np.array_equal(host(s, np.uint32), so)
    assert np.array_equal(host(q, np.int8), qo)


def test_quantize_int8_config5_full():
    d = W.w8a8_prefill()
    m, k = d["x"].shape
    q, s = empty((m, k), np.int8), empty((m, k // 64), np.float32)
    nq.nq_quantize_act_int8_g64(dev(d["x"]), m, k, q, s)
    qo, so = M.quantize_act_int8_g64(d["x"])
    assert np.array_equal(host(s, np.uint32), so)
    assert np.array_equal(host(q, np.int8), qo)


def _near_half_groups(n_groups, seed):
    """Groups of 64 BF16 values whose quotients x / s (s = f32(amax / 127)) lie
    within 2^-12 of a half-integer: each group holds its amax and 63 values
    picked among all BF16 values in [0, amax] by that criterion, random signs."""
    g = np.random.default_rng(seed)
    out = np.zeros((n_groups, 64), np.uint16)
    all_bf = np.arange(0, 0x7F80, dtype=np.uint32)                        # positive finite BF16
    all_v = (all_bf << 16).view(np.float32).astype(np.float64)
    for r in range(n_groups):
        mb = np.uint32(g.integers(0x3C00, 0x4400))                         # amax in [2^-7, 2^9)
        m = float((np.array([mb << 16], np.uint32)).view(np.float32)[0])
        sc = float(np.float32(m) / np.float32(127.0))                     # IEEE FP32 division
        cand = all_bf[(all_v <= m)]
        t = all_v[(all_v <= m)] / sc
        d = np.abs((t - np.floor(t)) - 0.5)
        pick = cand[d < 2.0 ** -12]
        if len(pick) > 63:
            pick = g.choice(pick, 63, replace=False)
        fill = g.choice(cand, 63 - len(pick)) if len(pick) < 63 else np.zeros(0, np.uint32)
        vals = np.concatenate([pick, fill]).astype(np.uint16)
        vals = vals | (g.integers(0, 2, 63).astype(np.uint16) << 15)
        out[r, 0] = mb
        out[r, 1:] = vals
    return out


def test_quantize_int8_near_half_quotients():
    x = _near_half_groups(96, 5)
    # and groups of exact ties: amax = 127 * 2^e makes s = 2^e, and (j + 0.5) 2^e are ties
    ties = np.zeros((8, 64), np.float32)
    for r, e in enumerate(range(-4, 4)):
        ties[r, 0] = 127.0 * 2.0 ** e
        ties[r, 1:] = (np.arange(63) % 64 + 0.5) * 2.0 ** e * (1 - 2 * (np.arange(63) % 2))
    tb = (ties.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((tb.astype(np.uint32) << 16).view(np.float32), ties)   # all BF16-exact
    x = np.concatenate([x, tb]).reshape(13, 512)
    t, k = x.shape
    q, s = empty((t, k), np.int8), empty((t, k // 64), np.float32)
    nq.nq_quantize_act_int8_g64(dev(x), t, k, q, s)
    qo, so = M.quantize_act_int8_g64(x)
    assert np.array_equal(host(s, np.uint32), so)
    assert np.array_equal(host(q, np.int8), qo)


@pytest.mark.parametrize("m,k", [(7, 256), (70, 400), (3, 8), (12, 512)])
def test_quantize_fp8_row(m, k):
    if m == 12:
        x = _tiny_rows_bf16(k, 5)           # FP32-subnormal token scales (quotients stay below 450)
    else:
        x = _special_activations(max(m, 5), k)[:m] if m >= 5 else W.bf16_normal(W.rng(95, k), (m, k))
    c, s = empty((m, k), np.uint8), empty((m,), np.float32)
    nq.nq_quantize_act_fp8_row(dev(x), m, k, c, s)
    co, so = M.quantize_act_fp8_row(x)
    assert np.array_equal(host(s, np.uint32), so)
    assert np.array_equal(host(c, np.uint8), co)


# ---------------------------------------------------------------------------
# a3 / a4: decode GEMVs
# ---------------------------------------------------------------------------

def _run_gemv_fp8row(wq, ws, x, workspace_mode, out):
    t, k = x.shape
    n = wq.shape[0]
    y = empty((t, n), np.float32 if out == "f32" else np.uint16)
    wsp = nq.alloc_gemv_workspace(-1, t, n, k, DEV) if workspace_mode else None
    nq.nq_gemv_fp8row(dev(wq), dev(ws), dev(x), t, n, k, y, wsp)
    return host(y, np.float32 if out == "f32" else np.uint16), wsp


def _check_float_out(got_f32, got_bf16, ref):
    assert rel_fro(got_f32, ref) <= FP32_TOL, rel_fro(got_f32, ref)
    assert np.array_equal(got_bf16, bf16_of_f32_bits(got_f32))
    assert rel_fro(F.bf16_decode(got_bf16), ref) <= BF16_TOL


GEMV_SHAPES = [(1000, 1536), (200, 1408), (64, 256), (37, 200), (8, 8), (130, 100), (16, 0)]


@pytest.mark.parametrize("n,k", GEMV_SHAPES)
@pytest.mark.parametrize("t", [1, 4, 16, 17, 33, 64, 65])
def test_gemv_fp8row(n, k, t):
    w = W.bf16_normal(W.rng(96, n * 3 + k), (n, k), std=0.02)
    wq, ws = M.encode_fp8row_bf16(w)
    x = W.bf16_normal(W.rng(97, t + k), (t, k))
    ref = M.gemv_fp8row(wq, ws, x)
    for wmode in (False, True):
        y32, wsp = _run_gemv_fp8row(wq, ws, x, wmode, "f32")
        y16, _ = _run_gemv_fp8row(wq, ws, x, wmode, "bf16")
        if k == 0:
            assert np.all(y32 == 0)
            continue
        _check_float_out(y32, y16, ref)
        if wsp is not None:
            assert int(wsp.view(torch.int32)[:64].abs().sum().item()) == 0     # counters reset


# Tile counts just above / well below the CU count, and a K split over many
# workgroups (partials exchanged through the workspace).  16448 x 4096: one
# leftover tile over a long K, where the row-FP8 plan takes the streaming
# kernel with spread workgroups also for one token block.
@pytest.mark.parametrize("n,k,t", [(4160, 8192, 1), (16448, 1024, 16), (17408, 1280, 4), (1000, 1536, 16),
                                   (16448, 4096, 1), (16448, 4096, 16)])
def test_gemv_fp8row_irregular_tile_counts(n, k, t):
    w = W.bf16_normal(W.rng(96, n * 7 + k), (n, k), std=0.02)
    wq, ws = M.encode_fp8row_bf16(w)
    x = W.bf16_normal(W.rng(97, t * 3 + k), (t, k))
    ref = M.gemv_fp8row(wq, ws, x)
    y32, wsp = _run_gemv_fp8row(wq, ws, x, True, "f32")
    y16, _ = _run_gemv_fp8row(wq, ws, x, True, "bf16")
    _check_float_out(y32, y16, ref)
    if wsp is not None:
        assert int(wsp.view(torch.int32)[:(n + 63) // 64].abs().sum().item()) == 0     # counters reset


def test_gemv_fp8row_one_hot_is_exact():
    n, k = 300, 512
    w = W.bf16_normal(W.rng(98, 0), (n, k), std=0.02)
    wq, ws = M.encode_fp8row_bf16(w)
    cols = [0, 1, 100, 511]
    x = np.zeros((len(cols), k), np.float32)
    for i, c in enumerate(cols):
        x[i, c] = 1.0
    xb = W.to_bf16_bits(x)
    y, _ = _run_gemv_fp8row(wq, ws, xb, True, "f32")
    ref = M.gemv_fp8row(wq, ws, xb)
    assert np.array_equal(y.astype(np.float64), F.round_f32(ref))


GROUP_FMTS = [("q4g64", nq.NQ_W_Q4G64_F16S), ("q8g32", nq.NQ_W_Q8G32_F16S), ("q8g64", nq.NQ_W_Q8G64_F16S),
              ("mxfp8", nq.NQ_W_MXFP8_G32), ("bf16", nq.NQ_W_BF16)]


def _grouped_inputs(name, n, k, seed):
    if name in ("q4g64", "q8g32", "q8g64"):
        d = W.grouped(name, n, k, seed)
        return d["codes"], d["scales"]
    if name == "mxfp8":
        g = W.rng(99, seed)
        words = W.pack_bytes_to_words(W.e4m3_codes(g, (n, k)))
        return words, g.integers(120, 131, (n, k // 32)).astype(np.uint8)
    return W.bf16_normal(W.rng(99, seed), (n, k), std=0.02), None


def _run_gemv_q(fmt, codes, scales, x, n, workspace_mode, out):
    t, k = x.shape
    y = empty((t, n), np.float32 if out == "f32" else np.uint16)
    wsp = nq.alloc_gemv_workspace(fmt, t, n, k, DEV) if workspace_mode else None
    nq.nq_gemv_qgroup(fmt, dev(codes), dev(scales) if scales is not None else None, dev(x), t, n, k, y, wsp)
    return host(y, np.float32 if out == "f32" else np.uint16)


@pytest.mark.parametrize("name,fmt", GROUP_FMTS)
@pytest.mark.parametrize("n,k", [(1000, 1536), (200, 1408), (70, 192), (9, 64)])
@pytest.mark.parametrize("t", [1, 8, 33, 64])
def test_gemv_qgroup(name, fmt, n, k, t):
    codes, scales = _grouped_inputs(name, n, k, n + k + t)
    x = W.bf16_normal(W.rng(100, t + k), (t, k))
    ref = M.gemv_qgroup(name, codes, scales, x)
    for wmode in (False, True):
        y32 = _run_gemv_q(fmt, codes, scales, x, n, wmode, "f32")
        y16 = _run_gemv_q(fmt, codes, scales, x, n, wmode, "bf16")
        _check_float_out(y32, y16, ref)


@pytest.mark.parametrize("t", [1, 8, 40])
def test_gemv_q4_every_code_large_offset(t):
    """Q4: every code value at every position, activations 30 + N(0, 1): the
    biased decode's worst case (group sums of x far above those of x q)."""
    n, k = 64, 1024
    q = (np.arange(n)[:, None] * 7 + np.arange(k)[None, :]) % 16 - 8
    u = (q & 15).astype(np.uint8)
    codes = (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)
    assert np.array_equal(M.unpack_q4(codes, k), q)
    scales = W.grouped("q4g64", n, k, seed=12)["scales"]
    x = W.to_bf16_bits((30.0 + W.rng(152, t).standard_normal((t, k))).astype(np.float32))
    ref = M.gemv_qgroup("q4g64", codes, scales, x)
    fmt = nq.NQ_W_Q4G64_F16S
    cd, sd = dev(codes), dev(scales)
    pk = _pack_dev(fmt, cd, n, k)
    g32, g16, _ = _gemv_both_layouts(fmt, cd, pk, sd, x, n, k)
    _check_float_out(g32, g16, ref)


# Four token blocks on 272 row tiles (17408 rows), the shape where the group
# formats' four-token-block streaming build has to fit two waves per SIMD
# (Q8 group-64: its row blocks in pairs), packed and row-major, every row.
@pytest.mark.parametrize("name,fmt", GROUP_FMTS[:3])
@pytest.mark.parametrize("t", [49, 64])
def test_gemv_qgroup_four_token_blocks_many_tiles(name, fmt, t):
    n, k = W.FFN, 1280
    codes, scales = _grouped_inputs(name, n, k, 31 * t + 7)
    x = W.bf16_normal(W.rng(100, 3 * t + k), (t, k))
    ref = M.gemv_qgroup(name, codes, scales, x)
    cd, sd = dev(codes), dev(scales)
    pk = _pack_dev(fmt, cd, n, k)
    g32, g16, _ = _gemv_both_layouts(fmt, cd, pk, sd, x, n, k)
    _check_float_out(g32, g16, ref)


# One-byte formats without group scales on at least four row tiles per CU,
# from 5 (row-FP8) or 8 (MXFP8) tokens on: the streaming kernel's two-tile
# workgroups (eight waves, one activation stage for both tiles); below that
# the direct kernel.  1025 tiles: the last workgroup's
# second tile lies wholly past the matrix (its reads clamp to the last row,
# its writes are dropped).  Packed and row-major, every row.
@pytest.mark.parametrize("name,fmt", [("fp8row", -1)] + GROUP_FMTS[3:])
@pytest.mark.parametrize("t", [4, 5, 8, 16, 17, 32, 40, 64])
def test_gemv_two_tile_workgroups(name, fmt, t):
    n, k = 1025 * 64 - 5, 512
    if fmt == -1:
        w = W.bf16_normal(W.rng(96, 31 * t), (n, k), std=0.02)
        codes, scales = M.encode_fp8row_bf16(w)
    else:
        codes, scales = _grouped_inputs(name, n, k, 41 * t + 3)
    x = W.bf16_normal(W.rng(100, 5 * t + k), (t, k))
    ref = (M.gemv_fp8row(codes, scales, x) if fmt == -1 else M.gemv_qgroup(name, codes, scales, x))
    cd = dev(codes)
    sd = dev(scales) if scales is not None else None
    pk = _pack_dev(fmt, cd, n, k)
    g32, g16, _ = _gemv_both_layouts(fmt, cd, pk, sd, x, n, k)
    _check_float_out(g32, g16, ref)
    assert rel_fro(g32[:, -64:], ref[:, -64:]) <= FP32_TOL


def test_gemv_mxfp8_config1():
    d = W.mxfp8_gemv()
    n, k = d["words"].shape[0], d["words"].shape[1] * 4
    y32 = _run_gemv_q(nq.NQ_W_MXFP8_G32, d["words"], d["e8m0"], d["x"], n, True, "f32")
    y16 = _run_gemv_q(nq.NQ_W_MXFP8_G32, d["words"], d["e8m0"], d["x"], n, True, "bf16")
    _check_float_out(y32, y16, M.gemv_qgroup("mxfp8", d["words"], d["e8m0"], d["x"]))


def _sampled_rows(n, seed, count=96):
    return np.unique(np.concatenate([[0, 63, 64, n - 1], W.rng(101, seed).integers(0, n, count)]))


def _leftover_rows(n, seed, count=96):
    """Every row of the row tiles beyond the last whole multiple of 256 tiles
    (those the GEMV spreads over extra workgroups or splits), plus a sample."""
    tiles = -(-n // 64)
    first = (tiles - tiles % 256) * 64 if tiles > 256 and tiles % 256 else n
    return np.unique(np.concatenate([np.arange(first, n), _sampled_rows(n, seed, count)]))


def _banded(fn, n, band=512):
    """Run a row-wise oracle step over row bands in threads (numpy releases
    the GIL in its elementwise kernels); the bands are independent rows."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(8) as ex:
        return list(ex.map(lambda r0: fn(r0, min(n, r0 + band)), range(0, n, band)))


def _oracle_fp8row_encode(w):
    parts = _banded(lambda a, b: M.encode_fp8row_bf16(w[a:b]), w.shape[0])
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def _gpu_fp8row_weights(w):
    n, k = w.shape
    wd = dev(w)
    q_d, s_d = empty((n, k), np.uint8), empty((n,), np.uint16)
    nq.nq_encode_fp8row_bf16(wd, n, k, q_d, s_d)
    del wd
    return q_d, s_d


def _pack_dev(fmt, codes_d, n, k):
    pk = empty((nq.nq_packed_weight_bytes(fmt, n, k),), np.uint8)
    nq.nq_pack_weights(fmt, codes_d, n, k, pk)
    return pk


def _counters_zero(wsp, n, rows_per_counter=64):
    """The workspace's counters (one per row tile, or per 16-row block for the
    wave-per-row-block kernels) are back at zero."""
    c = (n + rows_per_counter - 1) // rows_per_counter
    return wsp is None or int(wsp.view(torch.int32)[:c].abs().sum().item()) == 0


def _gemv_both_layouts(fmt, codes_d, pk, scales_d, x, n, k):
    """The call as bench.py times it (packed, shared workspace, BF16 out) plus
    FP32 out, and the row-major call; returns (fp32 packed, bf16 packed, fp32
    row-major) after checking the workspace counters are reset."""
    t = x.shape[0]
    xd = dev(x)
    wsp = nq.alloc_gemv_workspace(fmt, t, n, k, DEV)
    y32, y16, yr = empty((t, n), np.float32), empty((t, n), np.uint16), empty((t, n), np.float32)
    if fmt == -1:
        nq.nq_gemv_fp8row_packed(pk, scales_d, xd, t, n, k, y16, wsp)
        nq.nq_gemv_fp8row_packed(pk, scales_d, xd, t, n, k, y32, wsp)
        nq.nq_gemv_fp8row(codes_d, scales_d, xd, t, n, k, yr, wsp)
    else:
        nq.nq_gemv_qgroup_packed(fmt, pk, scales_d, xd, t, n, k, y16, wsp)
        nq.nq_gemv_qgroup_packed(fmt, pk, scales_d, xd, t, n, k, y32, wsp)
        nq.nq_gemv_qgroup(fmt, codes_d, scales_d, xd, t, n, k, yr, wsp)
    g32, g16, gr = host(y32, np.float32), host(y16, np.uint16), host(yr, np.float32)
    wave_kernel = fmt in (nq.NQ_W_Q3G64_F16S, nq.NQ_W_Q5G64_F16S, nq.NQ_W_Q6G64_F16S)
    assert _counters_zero(wsp, n, 16 if wave_kernel else 64)
    assert np.array_equal(g16, bf16_of_f32_bits(g32))          # BF16 = RNE of the same FP32 result
    assert np.array_equal(g32.view(np.uint32), gr.view(np.uint32))   # packed = row-major, bit for bit
    return g32, g16, gr


# The headline launches: packed row-FP8 17408 x 5120 (272 row tiles: whole
# tiles on every CU plus 16 spread over extra workgroups), T = 1, 4, 16, 33 as
# bench.py runs them (shared workspace, BF16 out), every row against the
# oracle (the oracle encodes the whole matrix in row bands).
@pytest.mark.slow
def test_gemv_fp8row_headline_all_rows():
    n, k = W.FFN, W.HIDDEN
    w = W.fp8row_weights_bf16(n, k)
    q_d, s_d = _gpu_fp8row_weights(w)
    qo, so = _oracle_fp8row_encode(w)
    assert np.array_equal(host(s_d, np.uint16), so) and np.array_equal(host(q_d, np.uint8), qo)
    pk = _pack_dev(-1, q_d, n, k)
    x33 = W.activations(33, k)
    ref33 = M.gemv_fp8row(qo, so, x33)
    for t in (1, 4, 16, 33):
        g32, g16, _ = _gemv_both_layouts(-1, q_d, pk, s_d, x33[:t].copy(), n, k)
        assert rel_fro(g32, ref33[:t]) <= FP32_TOL, t
        assert rel_fro(F.bf16_decode(g16), ref33[:t]) <= BF16_TOL, t
        # the leftover tiles' rows on their own (the exchanged partial sums)
        assert rel_fro(g32[:, 16384:], ref33[:t, 16384:]) <= FP32_TOL, t


@pytest.mark.slow
@pytest.mark.parametrize("n,k,ts", [(W.HIDDEN, W.FFN, [1, 17, 33])])
def test_gemv_fp8row_full_size(n, k, ts):
    w = W.fp8row_weights_bf16(n, k)
    q_d, s_d = _gpu_fp8row_weights(w)
    rows = _sampled_rows(n, n)
    wq_o, ws_o = M.encode_fp8row_bf16(w[rows])
    assert np.array_equal(host(q_d, np.uint8)[rows], wq_o) and np.array_equal(host(s_d, np.uint16)[rows], ws_o)
    for t in ts:
        x = W.activations(t, k)
        y = empty((t, n), np.float32)
        wsp = nq.alloc_gemv_workspace(-1, t, n, k, DEV)
        nq.nq_gemv_fp8row(q_d, s_d, dev(x), t, n, k, y, wsp)
        got = host(y, np.float32)[:, rows]
        assert rel_fro(got, M.gemv_fp8row(wq_o, ws_o, x)) <= FP32_TOL, t


# Config 3 as bench.py times it: the re-encoded 5120 x 17408 down projection,
# packed, T = 1 and 33, every row; the 96 x 5120 BF16 gate, packed.
@pytest.mark.slow
def test_gemv_config3_reencode_then_gemv_and_gate():
    d = W.block128_codes()
    n, k = d["codes"].shape
    q_d, s_d = empty((n, k), np.uint8), empty((n,), np.uint16)
    nq.nq_reencode_block128_to_row(dev(d["codes"]), dev(d["wsi"]), n, k, 0, n, q_d, s_d)
    parts = _banded(lambda a, b: M.reencode_block128_to_row(d["codes"][a:b], d["wsi"][a // 128:(b + 127) // 128],
                                                            0, b - a), n)
    qo, so = np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])
    assert np.array_equal(host(s_d, np.uint16), so) and np.array_equal(host(q_d, np.uint8), qo)
    pk = _pack_dev(-1, q_d, n, k)
    for t in (1, 33):
        x = W.activations(t, k, workload=3, tensor=3)
        g32, g16, _ = _gemv_both_layouts(-1, q_d, pk, s_d, x, n, k)
        ref = M.gemv_fp8row(qo, so, x)
        assert rel_fro(g32, ref) <= FP32_TOL, t
        assert rel_fro(F.bf16_decode(g16), ref) <= BF16_TOL, t
    gate = W.gate_bf16()
    gn, gk = gate.shape
    gd = dev(gate)
    gpk = _pack_dev(nq.NQ_W_BF16, gd, gn, gk)
    for t in (1, 33):
        x = W.activations(t, gk, workload=3, tensor=4)
        g32, g16, _ = _gemv_both_layouts(nq.NQ_W_BF16, gd, gpk, None, x, gn, gk)
        _check_float_out(g32, g16, M.gemv_qgroup("bf16", gate, None, x))


# Config 4 as bench.py times it: Q4 group-64 and Q8 group-32, packed, both
# shapes, T = 1, 8, 33 (and 17, two token blocks), every row.
@pytest.mark.slow
@pytest.mark.parametrize("name,fmt", GROUP_FMTS[:2])
@pytest.mark.parametrize("n,k", [(W.FFN, W.HIDDEN), (W.HIDDEN, W.FFN)])
def test_gemv_qgroup_config4_full_size(name, fmt, n, k):
    d = W.grouped(name, n, k)
    cd, sd = dev(d["codes"]), dev(d["scales"])
    pk = _pack_dev(fmt, cd, n, k)
    x33 = W.activations(33, k, workload=4, tensor=50)
    ref33 = M.gemv_qgroup(name, d["codes"], d["scales"], x33)
    for t in (1, 8, 17, 33):
        g32, g16, _ = _gemv_both_layouts(fmt, cd, pk, sd, x33[:t].copy(), n, k)
        assert rel_fro(g32, ref33[:t]) <= FP32_TOL, (name, t)
        assert rel_fro(F.bf16_decode(g16), ref33[:t]) <= BF16_TOL, (name, t)


# 384 row tiles (1.5 per CU) with 12 chunks: from 5 tokens on the grouped
# formats split K in two (the busiest CU then holds 3 halves against 5 thirds).
@pytest.mark.slow
@pytest.mark.parametrize("name,fmt", GROUP_FMTS[:2])
def test_gemv_qgroup_two_split_leftover(name, fmt):
    n, k = 24576, 3072
    assert nq.nq_gemv_workspace_bytes(fmt, 8, n, k) == 1536 + 2 * 8 * 384 * 64 * 4
    d = W.grouped(name, n, k, seed=3)
    cd, sd = dev(d["codes"]), dev(d["scales"])
    pk = _pack_dev(fmt, cd, n, k)
    x33 = W.activations(33, k, workload=4, tensor=51)
    ref33 = M.gemv_qgroup(name, d["codes"], d["scales"], x33)
    for t in (8, 33):
        g32, _, _ = _gemv_both_layouts(fmt, cd, pk, sd, x33[:t].copy(), n, k)
        assert rel_fro(g32, ref33[:t]) <= FP32_TOL, (name, t)


# Grouped formats with a few row tiles past the CU count (257 tiles, and 258
# with the last one ragged: 12 rows): whole tiles plus spread workgroups whose
# units apply the group scales themselves; one token block (T <= 16).  The
# workspace size shows the plan took that path.
@pytest.mark.slow
@pytest.mark.parametrize("name,fmt", GROUP_FMTS[:3])
@pytest.mark.parametrize("n", [16448, 16460])
def test_gemv_qgroup_spread(name, fmt, n):
    k = 4096
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tiles, chunks = (n + 63) // 64, k // 256
    r = tiles % cus
    assert 0 < r and 8 * r <= cus
    units = r * chunks
    lmax = -(-units // min(units, cus))
    e = -(-units // lmax)
    maxslots = -(-chunks // (units // e)) + 1
    d = W.grouped(name, n, k, seed=5)
    cd, sd = dev(d["codes"]), dev(d["scales"])
    pk = _pack_dev(fmt, cd, n, k)
    x16 = W.activations(16, k, workload=4, tensor=52)
    ref16 = M.gemv_qgroup(name, d["codes"], d["scales"], x16)
    for t in (1, 5, 16):
        assert nq.nq_gemv_workspace_bytes(fmt, t, n, k) == -(-tiles * 4 // 256) * 256 + r * maxslots * t * 64 * 4
        g32, g16, _ = _gemv_both_layouts(fmt, cd, pk, sd, x16[:t].copy(), n, k)
        assert rel_fro(g32, ref16[:t]) <= FP32_TOL, (name, t)
        assert rel_fro(g32[:, (tiles - r) * 64:], ref16[:t, (tiles - r) * 64:]) <= FP32_TOL, (name, t)
        assert rel_fro(F.bf16_decode(g16), ref16[:t]) <= BF16_TOL, (name, t)


# The output head as bench.py times it (packed row-FP8, 2376 row tiles: 2304
# whole, 72 spread), T = 1, 16, 33, 64; every row of the 72 spread tiles and a
# sample; plus the row-major sweep.
@pytest.mark.slow
def test_gemv_head_full_size_sweep():
    n, k = W.HEAD_ROWS, W.HIDDEN
    w = W.head_weights_bf16()
    q_d, s_d = _gpu_fp8row_weights(w)
    rows = _leftover_rows(n, 5)
    qo, so = _oracle_fp8row_encode(w[rows])
    assert np.array_equal(host(q_d, np.uint8)[rows], qo) and np.array_equal(host(s_d, np.uint16)[rows], so)
    pk = _pack_dev(-1, q_d, n, k)
    x64 = W.activations(64, k, workload=5, tensor=4)
    ref64 = M.gemv_fp8row(qo, so, x64)
    for t in (1, 16, 33, 64):
        g32, g16, _ = _gemv_both_layouts(-1, q_d, pk, s_d, x64[:t].copy(), n, k)
        assert rel_fro(g32[:, rows], ref64[:t]) <= FP32_TOL, t
        assert rel_fro(F.bf16_decode(g16[:, rows]), ref64[:t]) <= BF16_TOL, t
    for t in (2, 7, 34, 48):
        x = x64[:t].copy()
        y = empty((t, n), np.float32)
        nq.nq_gemv_fp8row(q_d, s_d, dev(x), t, n, k, y, nq.alloc_gemv_workspace(-1, t, n, k, DEV))
        assert rel_fro(host(y, np.float32)[:, rows], ref64[:t]) <= FP32_TOL, t


@pytest.mark.slow
def test_gemv_head_q8g32_full_size_packed():
    """The output head as Q8 group-32 (the FP8-versus-Q8 comparison's other
    side), packed as the benchmark runs it: every row of the spread tiles and
    a sample, against the oracle."""
    n, k = W.HEAD_ROWS, W.HIDDEN
    fmt = nq.NQ_W_Q8G32_F16S
    d = W.grouped("q8g32", n, k, seed=7)
    cd, sd = dev(d["codes"]), dev(d["scales"])
    pk = _pack_dev(fmt, cd, n, k)
    rows = _leftover_rows(n, 5)
    x64 = W.activations(64, k, workload=5, tensor=4)
    ref64 = M.gemv_qgroup("q8g32", d["codes"][rows], d["scales"][rows], x64)
    for t in (1, 16, 33, 34, 64):
        g32, _, _ = _gemv_both_layouts(fmt, cd, pk, sd, x64[:t].copy(), n, k)
        assert rel_fro(g32[:, rows], ref64[:t]) <= FP32_TOL, t


# bench.py's pattern: back-to-back launches over rotating weight copies (here
# four different matrices) and distinct activations, all sharing one
# workspace, nothing synchronized in between; every launch against the oracle
# on every row of the leftover tiles (the partial exchange) and a sample.
@pytest.mark.slow
@pytest.mark.parametrize("t", [33, 16, 1])
def test_gemv_back_to_back_shared_workspace(t):
    n, k = W.FFN, W.HIDDEN
    rows = _leftover_rows(n, 11, 160)
    mats, refs = [], []
    for i in range(4):
        w = W.fp8row_weights_bf16(n, k, seed=20 + i)
        q_d, s_d = _gpu_fp8row_weights(w)
        mats.append((_pack_dev(-1, q_d, n, k), s_d))
        del q_d
        refs.append(_oracle_fp8row_encode(w[rows]))
    xs = [W.activations(t, k, seed=30 + j) for j in range(8)]
    xds = [dev(x) for x in xs]
    wsp = nq.alloc_gemv_workspace(-1, t, n, k, DEV)
    ys = [empty((t, n), np.float32) for _ in range(8)]
    torch.cuda.synchronize()
    for j in range(8):
        pk, s_d = mats[j % 4]
        nq.nq_gemv_fp8row_packed(pk, s_d, xds[j], t, n, k, ys[j], wsp)
    for j in range(8):
        qo, so = refs[j % 4]
        got = host(ys[j], np.float32)[:, rows]
        assert rel_fro(got, M.gemv_fp8row(qo, so, xs[j])) <= FP32_TOL, j
    assert _counters_zero(wsp, n)


# ---------------------------------------------------------------------------
# MLX affine int8 decode (the draft layer's storage): bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,k", [(1, 128), (3, 384), (257, 1024), (130, 5120)])
def test_decode_mlx_affine_int8(n, k):
    d = W.mlx_affine_int8(n, k, seed=n + k)
    c, s, b = dev(d["codes"]), dev(d["scales"]), dev(d["biases"])
    ybf, y32 = empty((n, k), np.uint16), empty((n, k), np.float32)
    nq.nq_decode_mlx_affine_int8(c, s, b, n, k, ybf)
    nq.nq_decode_mlx_affine_int8(c, s, b, n, k, y32)
    assert np.array_equal(host(ybf, np.uint16), M.decode_mlx_affine_int8(d["codes"], d["scales"], d["biases"]))
    assert np.array_equal(host(y32, np.uint32), M.decode_mlx_affine_int8(d["codes"], d["scales"], d["biases"], out="f32"))


def test_decode_mlx_affine_int8_edges():
    # per group (row r, two groups): ties, the single-rounding case, subnormal,
    # zero, NaN and infinite scales and biases, the largest magnitudes
    pairs = [(0x1C00, 0x3C00), (0x0001, 0x3C04), (0x0001, 0x8000), (0x0000, 0x0000), (0x7E00, 0x3C00),
             (0x3C00, 0xFC00), (0x7C00, 0x0000), (0x7BFF, 0x7BFF), (0x7BFF, 0xFBFF), (0x03FF, 0x8400)]
    n, k = len(pairs), 256
    codes = np.tile(np.arange(256, dtype=np.uint8), (n, 1))
    scales = np.array([[p[0], p[0] ^ 0x8000] for p in pairs], np.uint16)
    biases = np.array([[p[1], p[1]] for p in pairs], np.uint16)
    ybf, y32 = empty((n, k), np.uint16), empty((n, k), np.float32)
    nq.nq_decode_mlx_affine_int8(dev(codes), dev(scales), dev(biases), n, k, ybf)
    nq.nq_decode_mlx_affine_int8(dev(codes), dev(scales), dev(biases), n, k, y32)
    assert np.array_equal(host(ybf, np.uint16), M.decode_mlx_affine_int8(codes, scales, biases))
    assert np.array_equal(host(y32, np.uint32), M.decode_mlx_affine_int8(codes, scales, biases, out="f32"))


@pytest.mark.slow
def test_decode_mlx_affine_int8_full_size_sampled():
    n, k = W.FFN, W.HIDDEN
    d = W.mlx_affine_int8(n, k)
    y = empty((n, k), np.uint16)
    nq.nq_decode_mlx_affine_int8(dev(d["codes"]), dev(d["scales"]), dev(d["biases"]), n, k, y)
    rows = _sampled_rows(n, 9)
    got = host(y, np.uint16)[rows]
    assert np.array_equal(got, M.decode_mlx_affine_int8(d["codes"][rows], d["scales"][rows], d["biases"][rows]))


# ---------------------------------------------------------------------------
# a6: W8A8 GEMM; a7: FP8 GEMM; a8: route
# ---------------------------------------------------------------------------

def _w8a8_inputs(m, n, k, seed):
    g = W.rng(102, seed)
    x = W.bf16_normal(g, (m, k), outlier_p=0.01)
    qa, sa = M.quantize_act_int8_g64(x)
    w = W.int8_uniform(g, (n, k))
    ws = W.f16_log_uniform(g, (n, k // 64), -9, -5)
    return qa, sa, w, ws


# (300, 300, 192) and (257, 129, 320): odd group counts (the last 128-column
# stage holds one group) over several tiles in both directions.  K % 512 == 0
# takes the scale-window path: (257, 129, 1536) and (300, 300, 2048) reuse both
# window slots of both scale kinds on ragged tiles.
@pytest.mark.parametrize("m,n,k", [(64, 128, 5120), (70, 100, 640), (130, 257, 128), (1, 1, 64), (300, 300, 192),
                                   (257, 129, 320), (257, 129, 1536), (300, 300, 2048), (513, 385, 512)])
def test_w8a8_group_sums_and_output(m, n, k):
    qa, sa, w, ws = _w8a8_inputs(m, n, k, m + n + k)
    y32, y16 = empty((m, n), np.float32), empty((m, n), np.uint16)
    gsum = empty((m, n, k // 64), np.int32)
    nq.nq_gemm_w8a8_g64(dev(qa), dev(sa), dev(w), dev(ws), m, n, k, y32, gsum)
    nq.nq_gemm_w8a8_g64(dev(qa), dev(sa), dev(w), dev(ws), m, n, k, y16)
    ref, sums = M.gemm_w8a8_g64(qa, sa, w, ws, return_sums=True)
    assert np.array_equal(host(gsum, np.int32).astype(np.int64), sums)
    _check_float_out(host(y32, np.float32), host(y16, np.uint16), ref)


def test_w8a8_power_of_two_scales_exact():
    m, n, k = 40, 72, 64
    g = W.rng(103, 0)
    qa = W.int8_uniform(g, (m, k))
    w = W.int8_uniform(g, (n, k))
    sa = np.exp2(g.integers(-8, -2, (m, 1))).astype(np.float32)
    ws = np.exp2(g.integers(-9, -5, (n, 1))).astype(np.float16).view(np.uint16)
    y = empty((m, n), np.float32)
    nq.nq_gemm_w8a8_g64(dev(qa), dev(sa.view(np.uint32)), dev(w), dev(ws), m, n, k, y)
    ref = M.gemm_w8a8_g64(qa, sa.view(np.uint32), w, ws)
    assert np.array_equal(host(y, np.float32).astype(np.float64), ref)


@pytest.mark.slow
def test_w8a8_config5_full_sampled():
    d = W.w8a8_prefill()
    m, k = d["x"].shape
    n = d["w"].shape[0]
    qa, sa = empty((m, k), np.int8), empty((m, k // 64), np.float32)
    nq.nq_quantize_act_int8_g64(dev(d["x"]), m, k, qa, sa)
    y = empty((m, n), np.float32)
    nq.nq_gemm_w8a8_g64(qa, sa, dev(d["w"]), dev(d["w_scale"]), m, n, k, y)
    qo, so = M.quantize_act_int8_g64(d["x"])
    rows = W.rng(104, 0).choice(m, 48, replace=False)
    cols = _sampled_rows(n, 6, 160)
    got = host(y, np.float32)[np.ix_(rows, cols)]
    ref = M.gemm_w8a8_g64(qo[rows], so[rows], d["w"][cols], d["w_scale"][cols])
    assert rel_fro(got, ref) <= FP32_TOL


# (300, 520, 1040): K % 128 == 16 over 2 x 3 tiles
@pytest.mark.parametrize("m,n,k", [(70, 100, 400), (128, 256, 5120), (1, 3, 16), (129, 130, 256), (300, 520, 1040)])
def test_fp8_gemm(m, n, k):
    x = W.bf16_normal(W.rng(105, m + n + k), (m, k), outlier_p=0.01)
    w = W.bf16_normal(W.rng(106, m + n + k), (n, k), std=0.02)
    wq, ws = M.encode_fp8row_bf16(w)
    ac, asc = empty((m, k), np.uint8), empty((m,), np.float32)
    y32, y16 = empty((m, n), np.float32), empty((m, n), np.uint16)
    nq.nq_gemm_fp8row(dev(x), dev(wq), dev(ws), m, n, k, ac, asc, y32)
    ref, qa, sa = M.gemm_fp8row(x, wq, ws)
    assert np.array_equal(host(ac, np.uint8), qa) and np.array_equal(host(asc, np.uint32), sa)
    nq.nq_gemm_fp8row(dev(x), dev(wq), dev(ws), m, n, k, ac, asc, y16)
    _check_float_out(host(y32, np.float32), host(y16, np.uint16), ref)


@pytest.mark.slow
def test_fp8_gemm_full_sampled():
    m, n, k = W.PREFILL_CHUNK, W.FFN, W.HIDDEN
    w = W.fp8row_weights_bf16(n, k)
    wq_d, ws_d = empty((n, k), np.uint8), empty((n,), np.uint16)
    nq.nq_encode_fp8row_bf16(dev(w), n, k, wq_d, ws_d)
    x = W.activations(m, k, workload=5, tensor=6)
    ac, asc, y = empty((m, k), np.uint8), empty((m,), np.float32), empty((m, n), np.float32)
    nq.nq_gemm_fp8row(dev(x), wq_d, ws_d, m, n, k, ac, asc, y)
    rows = W.rng(107, 0).choice(m, 48, replace=False)
    cols = _sampled_rows(n, 7, 160)
    wq_o, ws_o = M.encode_fp8row_bf16(w[cols])
    ref, qa, sa = M.gemm_fp8row(x[rows], wq_o, ws_o)
    assert np.array_equal(host(ac, np.uint8)[rows], qa)
    assert rel_fro(host(y, np.float32)[np.ix_(rows, cols)], ref) <= FP32_TOL


# ---------------------------------------------------------------------------
# Packed weight layout: a permutation of the row-major codes, and packed GEMVs
# equal the row-major ones bit for bit.
# ---------------------------------------------------------------------------

PACK_FMTS = [(-1, 1.0, 16), (nq.NQ_W_Q8G64_F16S, 1.0, 16), (nq.NQ_W_MXFP8_G32, 1.0, 16),
             (nq.NQ_W_Q4G64_F16S, 0.5, 8), (nq.NQ_W_Q8G32_F16S, 1.0, 8), (nq.NQ_W_BF16, 2.0, 16)]


def _unpack_reference(packed, fmt, n, k):
    """Invert the documented layout with numpy: rows in blocks of 16; per chunk
    of KC columns, per row block, per piece q, the 64 lanes' pieces in lane
    order; lane 16 g + i holds row i of the block and piece q of lane group g
    (Q4: each 32-bit word also biased and reordered, see _q4_natural_words)."""
    kc = 256
    row_bytes = {0.5: k // 2, 1.0: k, 2.0: 2 * k}[dict((f, b) for f, b, _ in PACK_FMTS)[fmt]]
    pb = dict((f, p) for f, _, p in PACK_FMTS)[fmt]
    chunk_bytes = row_bytes * kc // k                       # bytes of one row per chunk
    np_ = chunk_bytes // (4 * pb)                           # pieces per lane per chunk
    nrb = -(-n // 16)
    out = np.zeros((nrb * 16, row_bytes), np.uint8)
    v = packed.reshape(k // kc, nrb, np_, 64, pb)
    for g in range(4):
        for q in range(np_):
            off = 64 * q + 16 * g if pb == 16 else 32 * q + 8 * g
            for c in range(k // kc):
                base = c * chunk_bytes + off
                out[:, base:base + pb] = v[c, :, q, 16 * g:16 * g + 16, :].reshape(nrb * 16, pb)
    if fmt == nq.NQ_W_Q4G64_F16S:
        out = _q4_natural_words(out)
    return out[:n]


def _q4_natural_words(b):
    """Packed Q4 words hold biased nibbles u = c ^ 8, code 2i at bits 4i and
    code 2i + 1 at bits 16 + 4i; return the row-major words (code j at bits 4j)."""
    o = b.view(np.uint32)
    w = np.zeros_like(o)
    for i in range(4):
        w |= ((o >> np.uint32(4 * i)) & np.uint32(0xF)) << np.uint32(8 * i)
        w |= ((o >> np.uint32(16 + 4 * i)) & np.uint32(0xF)) << np.uint32(8 * i + 4)
    return (w ^ np.uint32(0x88888888)).view(np.uint8)


@pytest.mark.parametrize("fmt,bpe,pb", PACK_FMTS)
@pytest.mark.parametrize("n,k", [(70, 512), (33, 768), (16, 256)])
def test_pack_is_the_documented_permutation(fmt, bpe, pb, n, k):
    nbytes = int(n * k * bpe)
    src = W.rng(110, n + k).integers(0, 256, nbytes, dtype=np.int16).astype(np.uint8)
    pk = empty((nq.nq_packed_weight_bytes(fmt, n, k),), np.uint8)
    nq.nq_pack_weights(fmt, dev(src), n, k, pk)
    back = _unpack_reference(host(pk, np.uint8), fmt, n, k)
    assert np.array_equal(back.reshape(-1), src)
    # padding rows of the last block are zero
    assert nq.nq_packed_weight_bytes(fmt, n, k) == -(-n // 16) * 16 * int(k * bpe)


# 16448 rows: one tile more than 256 CUs, so the row-FP8 kernels run the
# leftover tile on spread workgroups beside the whole tiles; at 3072 columns
# the grouped formats split K in three from 5 tokens on.  16384 rows: one
# tile per CU, where the grouped formats split K in two from 4 tokens on.
@pytest.mark.parametrize("name,fmt", [("fp8row", -1)] + GROUP_FMTS)
@pytest.mark.parametrize("n,k", [(1000, 1536), (200, 1280), (16448, 768), (16448, 3072), (16384, 1024)])
@pytest.mark.parametrize("t", [1, 16, 33])
def test_gemv_packed_equals_row_major(name, fmt, n, k, t):
    if name == "fp8row":
        w = W.bf16_normal(W.rng(111, n + k), (n, k), std=0.02)
        codes, scales = M.encode_fp8row_bf16(w)
        ref = M.gemv_fp8row(codes, scales, W.bf16_normal(W.rng(112, t + k), (t, k)))
    else:
        codes, scales = _grouped_inputs(name, n, k, n + k + t)
        ref = M.gemv_qgroup(name, codes, scales, W.bf16_normal(W.rng(112, t + k), (t, k)))
    x = W.bf16_normal(W.rng(112, t + k), (t, k))
    cd = dev(codes)
    sd = dev(scales) if scales is not None else None
    pk = empty((nq.nq_packed_weight_bytes(fmt, n, k),), np.uint8)
    nq.nq_pack_weights(fmt, cd, n, k, pk)
    wsp = nq.alloc_gemv_workspace(fmt, t, n, k, DEV)
    y_row, y_pk = empty((t, n), np.float32), empty((t, n), np.float32)
    if name == "fp8row":
        nq.nq_gemv_fp8row(cd, sd, dev(x), t, n, k, y_row, wsp)
        nq.nq_gemv_fp8row_packed(pk, sd, dev(x), t, n, k, y_pk, wsp)
    else:
        nq.nq_gemv_qgroup(fmt, cd, sd, dev(x), t, n, k, y_row, wsp)
        nq.nq_gemv_qgroup_packed(fmt, pk, sd, dev(x), t, n, k, y_pk, wsp)
    a, b = host(y_row, np.uint32), host(y_pk, np.uint32)
    assert np.array_equal(a, b)
    assert rel_fro(b.view(np.float32), ref) <= FP32_TOL


@pytest.mark.parametrize("t", [1, 33, 128, 129, 300])
def test_linear_route(t):
    n, k = 200, 640
    g = W.rng(108, t)
    x = W.bf16_normal(g, (t, k))
    w = W.int8_uniform(g, (n, k))
    ws = W.f16_log_uniform(g, (n, k // 64), -9, -5)
    xd, wd, wsd = dev(x), dev(w), dev(ws)
    y = empty((t, n), np.float32)
    aq, asc = empty((t, k), np.int8), empty((t, k // 64), np.float32)
    wsp = nq.alloc_gemv_workspace(nq.NQ_W_Q8G64_F16S, t, n, k, DEV)
    nq.nq_linear_q8g64(xd, t, wd, wsd, n, k, True, aq, asc, y, wsp)
    got = host(y, np.float32)
    ref = M.linear_w8g64(x, w, ws, True)
    assert rel_fro(got, ref) <= FP32_TOL
    direct = empty((t, n), np.float32)
    if t >= 129:
        nq.nq_gemm_w8a8_g64(aq, asc, wd, wsd, t, n, k, direct)
    else:
        nq.nq_gemv_qgroup(nq.NQ_W_Q8G64_F16S, wd, wsd, xd, t, n, k, direct, wsp)
    assert np.array_equal(host(direct, np.uint32), got.view(np.uint32))


@pytest.mark.parametrize("n,k", [(3, 128), (257, 1024), (130, 5120)])
def test_unpack_q4_to_int8(n, k):
    codes = W.q4_packed_uniform(W.rng(113, n + k), n, k)
    out = empty((n, k), np.int8)
    nq.nq_unpack_q4_to_int8(dev(codes), n, k, out)
    assert np.array_equal(host(out, np.int8).astype(np.int64), M.unpack_q4(codes, k))


@pytest.mark.parametrize("t", [1, 33, 128, 129, 300])
def test_linear_q4g64_route(t):
    n, k = 200, 1280
    d = W.grouped("q4g64", n, k, seed=t)
    x = W.bf16_normal(W.rng(114, t), (t, k))
    xd, wd, wsd = dev(x), dev(d["codes"]), dev(d["scales"])
    y = empty((t, n), np.float32)
    aq, asc, wi8 = empty((t, k), np.int8), empty((t, k // 64), np.float32), empty((n, k), np.int8)
    wsp = nq.alloc_gemv_workspace(nq.NQ_W_Q4G64_F16S, t, n, k, DEV)
    nq.nq_linear_q4g64(xd, t, wd, wsd, n, k, True, aq, asc, wi8, y, wsp)
    got = host(y, np.float32)
    assert rel_fro(got, M.linear_q4g64(x, d["codes"], d["scales"], True)) <= FP32_TOL
    direct = empty((t, n), np.float32)
    if t >= 129:
        assert np.array_equal(host(wi8, np.int8).astype(np.int64), M.unpack_q4(d["codes"], k))
        nq.nq_gemm_w8a8_g64(aq, asc, wi8, wsd, t, n, k, direct)
    else:
        nq.nq_gemv_qgroup(nq.NQ_W_Q4G64_F16S, wd, wsd, xd, t, n, k, direct, wsp)
    assert np.array_equal(host(direct, np.uint32), got.view(np.uint32))


@pytest.mark.slow
def test_linear_q4g64_prefill_full_size_sampled():
    """Q4 weights on the A8 route at the prefill chunk: 1792 x 17408 x 5120."""
    m, n, k = W.PREFILL_CHUNK, W.FFN, W.HIDDEN
    d = W.grouped("q4g64", n, k)
    x = W.w8a8_prefill()["x"]
    y = empty((m, n), np.float32)
    aq, asc, wi8 = empty((m, k), np.int8), empty((m, k // 64), np.float32), empty((n, k), np.int8)
    nq.nq_linear_q4g64(dev(x), m, dev(d["codes"]), dev(d["scales"]), n, k, True, aq, asc, wi8, y)
    assert np.array_equal(host(wi8, np.int8).astype(np.int64), M.unpack_q4(d["codes"], k))   # every code
    rows = _sampled_rows(m, 12, count=24)
    cols = _sampled_rows(n, 13, count=48)
    qa, sa = M.quantize_act_int8_g64(x[rows])
    ref = M.gemm_w8a8_g64(qa, sa, M.unpack_q4(d["codes"][cols], k), d["scales"][cols])
    assert rel_fro(host(y, np.float32)[np.ix_(rows, cols)], ref) <= FP32_TOL


# ---------------------------------------------------------------------------
# A8 decode GEMV (int8 activations at decode sizes, W8A8 arithmetic)
# ---------------------------------------------------------------------------

A8_FMTS = [("q8g64", nq.NQ_W_Q8G64_F16S), ("q4g64", nq.NQ_W_Q4G64_F16S)]


def _a8_weights(name, n, k, seed):
    d = W.grouped(name, n, k, seed)
    wq = d["codes"] if name == "q8g64" else M.unpack_q4(d["codes"], k).astype(np.int8)   # oracle's int codes
    return d["codes"], wq, d["scales"]


def _run_a8(fmt, codes_d, pk, ws_d, qa, sa, n, k, wmode, out="f32"):
    t = qa.shape[0]
    y = empty((t, n), np.float32 if out == "f32" else np.uint16)
    wsp = nq.alloc_gemv_a8_workspace(t, n, k, DEV) if wmode else None
    if pk is None:
        nq.nq_gemv_a8_g64(fmt, codes_d, ws_d, dev(qa), dev(sa), t, n, k, y, wsp)
    else:
        nq.nq_gemv_a8_g64_packed(fmt, pk, ws_d, dev(qa), dev(sa), t, n, k, y, wsp)
    got = host(y, np.float32 if out == "f32" else np.uint16)
    assert _counters_zero(wsp, n, 16)
    return got


@pytest.mark.parametrize("name,fmt", A8_FMTS)
@pytest.mark.parametrize("n,k", [(1000, 1536), (200, 1280), (70, 256), (16448, 768), (33, 5120)])
@pytest.mark.parametrize("t", [1, 3, 4, 5, 8, 9, 17, 33, 64, 65])
def test_gemv_a8(name, fmt, n, k, t):
    codes, wq, ws = _a8_weights(name, n, k, n + k + t)
    x = W.bf16_normal(W.rng(140, t + k), (t, k), outlier_p=0.01)
    qa, sa = M.quantize_act_int8_g64(x)
    ref = M.gemm_w8a8_g64(qa, sa, wq, ws)
    cd, sd = dev(codes), dev(ws)
    pk = _pack_dev(fmt, cd, n, k)
    outs = []
    for p in (None, pk):
        for wmode in (False, True):
            g32 = _run_a8(fmt, cd, p, sd, qa, sa, n, k, wmode)
            assert rel_fro(g32, ref) <= FP32_TOL, (p is None, wmode)
            outs.append(g32)
    g16 = _run_a8(fmt, cd, pk, sd, qa, sa, n, k, True, "bf16")
    assert np.array_equal(g16, bf16_of_f32_bits(outs[3]))
    assert np.array_equal(outs[0].view(np.uint32), outs[2].view(np.uint32))   # packed = row-major
    assert np.array_equal(outs[1].view(np.uint32), outs[3].view(np.uint32))


@pytest.mark.parametrize("name,fmt", A8_FMTS)
@pytest.mark.parametrize("t", [3, 7, 20])
def test_gemv_a8_group_sums_exact(name, fmt, t):
    """One nonzero group per token and power-of-two scales: every output is
    P * ws * as exactly, so the int32 group sums are checked bit for bit."""
    n, k = 130, 1024
    codes, wq, _ = _a8_weights(name, n, k, 5)
    g = W.rng(141, 0)
    qa = W.int8_uniform(g, (t, k))
    keep = g.integers(0, k // 64, t)
    for i in range(t):
        m = np.zeros(k, bool)
        m[64 * keep[i]:64 * keep[i] + 64] = True
        qa[i, ~m] = 0
    sa = np.exp2(g.integers(-8, -2, (t, k // 64))).astype(np.float32).view(np.uint32)
    ws = np.exp2(g.integers(-9, -5, (n, k // 64))).astype(np.float16).view(np.uint16)
    cd, sd = dev(codes), dev(ws)
    ref, sums = M.gemm_w8a8_g64(qa, sa, wq, ws, return_sums=True)
    for p in (None, _pack_dev(fmt, cd, n, k)):
        got = _run_a8(fmt, cd, p, sd, qa, sa, n, k, True)
        assert np.array_equal(got.astype(np.float64), ref)
    # the one nonzero group's sum, recovered exactly from the output
    ti, ni = np.arange(t)[:, None], np.arange(n)[None, :]
    denom = F.f16_decode(ws)[ni, keep[:, None]] * F.f32_decode(sa)[ti, keep[:, None]]
    assert np.array_equal(ref / denom, sums[ti, ni, keep[:, None]].astype(np.float64))


# The A8 decode rows bench.py times: 17408 x 5120 and 5120 x 17408, packed,
# T = 1, 8, 33, every row against the oracle.
@pytest.mark.slow
@pytest.mark.parametrize("name,fmt", A8_FMTS)
@pytest.mark.parametrize("n,k", [(W.FFN, W.HIDDEN), (W.HIDDEN, W.FFN)])
def test_gemv_a8_full_size(name, fmt, n, k):
    codes, wq, ws = _a8_weights(name, n, k, 0)
    cd, sd = dev(codes), dev(ws)
    pk = _pack_dev(fmt, cd, n, k)
    x33 = W.activations(33, k, workload=4, tensor=50)
    qa, sa = M.quantize_act_int8_g64(x33)
    ref33 = M.gemm_w8a8_g64(qa, sa, wq, ws)
    for t in (1, 8, 33):
        g32 = _run_a8(fmt, cd, pk, sd, qa[:t], sa[:t], n, k, True)
        assert rel_fro(g32, ref33[:t]) <= FP32_TOL, (name, t)
        gr = _run_a8(fmt, cd, None, sd, qa[:t], sa[:t], n, k, True)
        assert np.array_equal(g32.view(np.uint32), gr.view(np.uint32)), (name, t)


@pytest.mark.parametrize("t", [1, 33, 128, 129])
def test_linear_a8_decode_route(t):
    """Routed Q8 and Q4 group-64 projections with the A8 decode flag (and the
    prefill one): below 129 tokens the quantizer + A8 decode GEMV, from 129 on
    the W8A8 GEMM; bit-identical to the direct calls."""
    n, k = 200, 1280
    flags = nq.NQ_A8_PREFILL | nq.NQ_A8_DECODE
    assert nq.nq_route(t, flags) == (nq.NQ_ROUTE_A8 if t >= 129 else nq.NQ_ROUTE_A8_DECODE)
    x = W.bf16_normal(W.rng(142, t), (t, k))
    xd = dev(x)
    aq, asc = empty((t, k), np.int8), empty((t, k // 64), np.float32)
    for name, fmt in A8_FMTS:
        codes, wq, ws = _a8_weights(name, n, k, t + 1)
        cd, sd = dev(codes), dev(ws)
        y = empty((t, n), np.float32)
        wsp = nq.alloc_gemv_a8_workspace(t, n, k, DEV)
        if name == "q8g64":
            nq.nq_linear_q8g64(xd, t, cd, sd, n, k, flags, aq, asc, y, wsp)
            ref = M.linear_w8g64(x, codes, ws, True, True)
        else:
            wi8 = empty((n, k), np.int8)
            nq.nq_linear_q4g64(xd, t, cd, sd, n, k, flags, aq, asc, wi8, y, wsp)
            ref = M.linear_q4g64(x, codes, ws, True, True)
        got = host(y, np.float32)
        assert rel_fro(got, ref) <= FP32_TOL, name
        direct = empty((t, n), np.float32)
        if t >= 129:
            if name == "q8g64":
                nq.nq_gemm_w8a8_g64(aq, asc, cd, sd, t, n, k, direct)
            else:
                nq.nq_gemm_w8a8_g64(aq, asc, wi8, sd, t, n, k, direct)
        else:
            nq.nq_gemv_a8_g64(fmt, cd, sd, aq, asc, t, n, k, direct, wsp)
        assert np.array_equal(host(direct, np.uint32), got.view(np.uint32)), name


# ---------------------------------------------------------------------------
# Q3 / Q5 / Q6 group-64 (dense little-endian bit streams)
# ---------------------------------------------------------------------------

QB_FMTS = [("q3g64", nq.NQ_W_Q3G64_F16S, 3), ("q5g64", nq.NQ_W_Q5G64_F16S, 5), ("q6g64", nq.NQ_W_Q6G64_F16S, 6)]


def _qb_gemv(fmt, cd, pk, sd, x, n, k, wmode, out="f32"):
    t = x.shape[0]
    y = empty((t, n), np.float32 if out == "f32" else np.uint16)
    wsp = nq.alloc_gemv_workspace(fmt, t, n, k, DEV) if wmode else None
    if pk is None:
        nq.nq_gemv_qgroup(fmt, cd, sd, dev(x), t, n, k, y, wsp)
    else:
        nq.nq_gemv_qgroup_packed(fmt, pk, sd, dev(x), t, n, k, y, wsp)
    got = host(y, np.float32 if out == "f32" else np.uint16)
    assert _counters_zero(wsp, n, 16)
    return got


@pytest.mark.parametrize("name,fmt,bits", QB_FMTS)
@pytest.mark.parametrize("n,k", [(1000, 1536), (200, 1280), (70, 256), (16448, 768), (33, 5120)])
@pytest.mark.parametrize("t", [1, 2, 3, 4, 6, 8, 9, 16, 17, 24, 25, 33, 40, 41, 56, 65])
def test_gemv_qbits(name, fmt, bits, n, k, t):
    d = W.grouped(name, n, k, seed=n + t)
    x = W.bf16_normal(W.rng(150, t + k), (t, k))
    ref = M.gemv_qgroup(name, d["codes"], d["scales"], x)
    cd, sd = dev(d["codes"]), dev(d["scales"])
    pk = _pack_dev(fmt, cd, n, k)
    outs = []
    for p in (None, pk):
        for wmode in (False, True):
            g = _qb_gemv(fmt, cd, p, sd, x, n, k, wmode)
            assert rel_fro(g, ref) <= FP32_TOL, (p is None, wmode)
            outs.append(g)
    g16 = _qb_gemv(fmt, cd, pk, sd, x, n, k, True, "bf16")
    assert np.array_equal(g16, bf16_of_f32_bits(outs[3]))
    assert np.array_equal(outs[0].view(np.uint32), outs[2].view(np.uint32))      # packed = row-major
    assert np.array_equal(outs[1].view(np.uint32), outs[3].view(np.uint32))


@pytest.mark.parametrize("name,fmt,bits", QB_FMTS)
@pytest.mark.parametrize("t", [8, 40])
def test_gemv_qbits_every_code_large_offset(name, fmt, bits, t):
    """Every code value at every position of a group, against activations
    with a large common offset (30 + N(0, 1)): group sums of x dwarf those of
    x q, the hardest case for sums taken on codes shifted by 2^(b-1)."""
    n, k = 64, 1024
    q = (np.arange(n)[:, None] * 7 + np.arange(k)[None, :]) % (1 << bits) - (1 << (bits - 1))
    u = (q & ((1 << bits) - 1)).astype(np.uint8)
    stream = ((u[:, :, None] >> np.arange(bits, dtype=np.uint8)) & 1).reshape(n, k * bits)
    codes = np.packbits(stream, axis=1, bitorder="little")
    assert np.array_equal(M.unpack_qbits(codes, k, bits), q)     # the stream holds the intended codes
    scales = W.grouped(name, n, k, seed=11)["scales"]
    x32 = 30.0 + W.rng(151, t).standard_normal((t, k))
    x = W.to_bf16_bits(x32.astype(np.float32))
    ref = M.gemv_qgroup(name, codes, scales, x)
    cd, sd = dev(codes), dev(scales)
    pk = _pack_dev(fmt, cd, n, k)
    for p in (None, pk):
        g = _qb_gemv(fmt, cd, p, sd, x, n, k, True)
        assert rel_fro(g, ref) <= FP32_TOL, p is None


@pytest.mark.parametrize("name,fmt,bits", QB_FMTS)
def test_gemv_qbits_one_hot_is_exact(name, fmt, bits):
    """One-hot activations give the decoded codes times their scales, exactly."""
    n, k = 70, 512
    d = W.grouped(name, n, k, seed=3)
    cols = [0, 1, 15, 16, 63, 64, 200, 511]
    x = np.zeros((len(cols), k), np.float32)
    for i, c in enumerate(cols):
        x[i, c] = 1.0
    xb = W.to_bf16_bits(x)
    cd, sd = dev(d["codes"]), dev(d["scales"])
    ref = M.gemv_qgroup(name, d["codes"], d["scales"], xb)
    for p in (None, _pack_dev(fmt, cd, n, k)):
        assert np.array_equal(_qb_gemv(fmt, cd, p, sd, xb, n, k, True).astype(np.float64), ref)


def _unpack_qbits_packed_reference(packed, bits, n, k):
    """Invert the packed layout with numpy: per (chunk, row block), pieces of
    16 bytes (and an 8-byte tail) lane after lane; a lane's 8 b bytes are the
    2 b bytes of groups q = 0..3 of its row (lane 16 g + i: row i, codes
    64 q + 16 g + [0, 16))."""
    nrb, chunks, lb = -(-n // 16), k // 256, 8 * bits
    out = np.zeros((nrb * 16, k * bits // 8), np.uint8)
    blk = packed.reshape(chunks, nrb, 64 * lb)
    np16 = lb // 16
    for c in range(chunks):
        for rb in range(nrb):
            b = blk[c, rb]
            lanes = np.zeros((64, lb), np.uint8)
            for p in range(np16):
                lanes[:, 16 * p:16 * p + 16] = b[1024 * p:1024 * p + 1024].reshape(64, 16)
            if lb % 16:
                lanes[:, 16 * np16:] = b[1024 * np16:1024 * np16 + 512].reshape(64, 8)
            for lane in range(64):
                i, g = lane & 15, lane >> 4
                for q in range(4):
                    off = bits * (32 * c + 8 * q + 2 * g)
                    out[rb * 16 + i, off:off + 2 * bits] = lanes[lane, 2 * bits * q:2 * bits * (q + 1)]
    return out[:n]


@pytest.mark.parametrize("name,fmt,bits", QB_FMTS)
@pytest.mark.parametrize("n,k", [(70, 512), (16, 256)])
def test_pack_qbits_is_the_documented_permutation(name, fmt, bits, n, k):
    src = W.rng(151, n + bits).integers(0, 256, (n, k * bits // 8), dtype=np.int16).astype(np.uint8)
    pk = _pack_dev(fmt, dev(src), n, k)
    assert pk.numel() == -(-n // 16) * 16 * k * bits // 8
    assert np.array_equal(_unpack_qbits_packed_reference(host(pk, np.uint8), bits, n, k), src)


@pytest.mark.parametrize("name,fmt,bits", QB_FMTS)
@pytest.mark.parametrize("n,k", [(3, 64), (257, 1024), (130, 5120)])
def test_unpack_qbits_to_int8(name, fmt, bits, n, k):
    codes = W.grouped(name, n, k, seed=k)["codes"]
    out = empty((n, k), np.int8)
    nq.nq_unpack_qbits_to_int8(fmt, dev(codes), n, k, out)
    assert np.array_equal(host(out, np.int8).astype(np.int64), M.unpack_qbits(codes, k, bits))


@pytest.mark.parametrize("t", [1, 33, 129])
@pytest.mark.parametrize("name,fmt,bits", QB_FMTS)
def test_linear_qbits_route(name, fmt, bits, t):
    """Routed Q3/Q5/Q6 projections: BF16 GEMV, A8 decode (flag) and A8 prefill
    routes against the oracle, each bit-identical to its direct calls."""
    n, k = 200, 1280
    d = W.grouped(name, n, k, seed=t)
    x = W.bf16_normal(W.rng(152, t), (t, k))
    xd, cd, sd = dev(x), dev(d["codes"]), dev(d["scales"])
    for flags, a8d in ((nq.NQ_A8_PREFILL, False), (nq.NQ_A8_PREFILL | nq.NQ_A8_DECODE, True)):
        y = empty((t, n), np.float32)
        aq, asc, wi8 = empty((t, k), np.int8), empty((t, k // 64), np.float32), empty((n, k), np.int8)
        wsp = nq.alloc_gemv_workspace(fmt, t, n, k, DEV)
        wsa = nq.alloc_gemv_a8_workspace(t, n, k, DEV)
        ws_use = wsa if (a8d and t < 129) else wsp
        nq.nq_linear_qbits_g64(fmt, xd, t, cd, sd, n, k, flags, aq, asc, wi8, y, ws_use)
        got = host(y, np.float32)
        assert rel_fro(got, M.linear_qbits_g64(name, x, d["codes"], d["scales"], True, a8d)) <= FP32_TOL, flags
        direct = empty((t, n), np.float32)
        if t >= 129:
            assert np.array_equal(host(wi8, np.int8).astype(np.int64), M.unpack_qbits(d["codes"], k, bits))
            nq.nq_gemm_w8a8_g64(aq, asc, wi8, sd, t, n, k, direct)
        elif a8d:
            nq.nq_gemv_a8_g64(nq.NQ_W_Q8G64_F16S, wi8, sd, aq, asc, t, n, k, direct, wsa)
        else:
            nq.nq_gemv_qgroup(fmt, cd, sd, xd, t, n, k, direct, wsp)
        assert np.array_equal(host(direct, np.uint32), got.view(np.uint32)), flags


# The Q5 / Q3 rows bench.py times: 17408 x 5120 and 5120 x 17408, packed, T =
# 1, 8, 33, every row (the oracle runs in row bands).
@pytest.mark.slow
@pytest.mark.parametrize("name,fmt,bits", QB_FMTS[:2])
@pytest.mark.parametrize("n,k", [(W.FFN, W.HIDDEN), (W.HIDDEN, W.FFN)])
def test_gemv_qbits_full_size(name, fmt, bits, n, k):
    d = W.grouped(name, n, k)
    cd, sd = dev(d["codes"]), dev(d["scales"])
    pk = _pack_dev(fmt, cd, n, k)
    x33 = W.activations(33, k, workload=4, tensor=50)
    parts = _banded(lambda a, b: M.gemv_qgroup(name, d["codes"][a:b], d["scales"][a:b], x33), n)
    ref33 = np.concatenate(parts, axis=1)
    for t in (1, 8, 33):
        g32, g16, _ = _gemv_both_layouts(fmt, cd, pk, sd, x33[:t].copy(), n, k)
        assert rel_fro(g32, ref33[:t]) <= FP32_TOL, (name, t)
        assert rel_fro(F.bf16_decode(g16), ref33[:t]) <= BF16_TOL, (name, t)


@pytest.mark.slow
@pytest.mark.parametrize("name,fmt,bits", QB_FMTS[:2])
def test_linear_qbits_prefill_full_size_sampled(name, fmt, bits):
    """Q5 / Q3 weights on the A8 route at the prefill chunk: 1792 x 17408 x 5120."""
    m, n, k = W.PREFILL_CHUNK, W.FFN, W.HIDDEN
    d = W.grouped(name, n, k)
    x = W.w8a8_prefill(n=64)["x"]
    y = empty((m, n), np.float32)
    aq, asc, wi8 = empty((m, k), np.int8), empty((m, k // 64), np.float32), empty((n, k), np.int8)
    nq.nq_linear_qbits_g64(fmt, dev(x), m, dev(d["codes"]), dev(d["scales"]), n, k, nq.NQ_A8_PREFILL, aq, asc, wi8, y)
    rows = _sampled_rows(m, 14, count=24)
    cols = _sampled_rows(n, 15, count=48)
    assert np.array_equal(host(wi8, np.int8)[cols].astype(np.int64), M.unpack_qbits(d["codes"][cols], k, bits))
    qa, sa = M.quantize_act_int8_g64(x[rows])
    ref = M.gemm_w8a8_g64(qa, sa, M.unpack_qbits(d["codes"][cols], k, bits), d["scales"][cols])
    assert rel_fro(host(y, np.float32)[np.ix_(rows, cols)], ref) <= FP32_TOL
