"""Seeded synthetic inputs for the projection's workloads.

This module draws random numbers and lays them out in the storage formats the
library consumes; it holds none of the projection's arithmetic (no decoding,
no scaling, no quantization).  Both the tests (for the HIP library and for the
CPU oracle) and the benchmark take their inputs from here.

Every tensor gets its own independent stream: ``SeedSequence(seed,
spawn_key=(workload, tensor))``.  Normal draws are float32 and become BF16 by
torch's round-to-nearest-even cast; log-uniform scales are ``2**uniform(lo,
hi)`` cast to FP16 (numpy, round-to-nearest-even) or BF16.

Workload shapes follow the pages: hidden size 5120 and FFN width 17408, a
96-row gating projection kept in BF16, decode/verify steps of 1..33 tokens,
prefill chunks of 1792 tokens, a 152064-row output head.
"""

import numpy as np
import torch

# E4M3 byte values that are finite, non-NaN and nonzero: every code except
# +-0 (0x00, 0x80) and the two NaN codes (0x7F, 0xFF).  252 codes.
FINITE_NONZERO_E4M3 = np.array([c for c in range(256) if c not in (0x00, 0x80, 0x7F, 0xFF)],
                               dtype=np.uint8)

HIDDEN = 5120
FFN = 17408
GATE_ROWS = 96
PREFILL_CHUNK = 1792
HEAD_ROWS = 152064


def rng(workload, tensor, seed=0):
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(workload, tensor)))


def to_bf16_bits(x32):
    """float32 array -> BF16 bit patterns (uint16), round-to-nearest-even (torch)."""
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_normal(g, shape, std=1.0, outlier_p=0.0, outlier_mult=20.0):
    x = g.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if outlier_p > 0.0:
        mask = g.random(shape, dtype=np.float32) < outlier_p
        x[mask] *= np.float32(outlier_mult)
    return to_bf16_bits(x)


def e4m3_codes(g, shape):
    """Codes drawn uniformly from the 252 finite nonzero E4M3 values."""
    return FINITE_NONZERO_E4M3[g.integers(0, FINITE_NONZERO_E4M3.size, shape)]


def pack_bytes_to_words(b):
    """uint8 [N][K] -> uint32 [N][K/4], byte i of word j = element 4j+i (little-endian)."""
    b = np.ascontiguousarray(b, dtype=np.uint8)
    return b.view("<u4").reshape(b.shape[0], b.shape[1] // 4)


def f16_log_uniform(g, shape, lo, hi):
    return np.exp2(g.uniform(lo, hi, shape)).astype(np.float16).view(np.uint16)


def bf16_log_uniform_as_f32(g, shape, lo, hi):
    """log-uniform values rounded to BF16-representable float32 (block scales)."""
    b = to_bf16_bits(np.exp2(g.uniform(lo, hi, shape)).astype(np.float32))
    return (b.astype(np.uint32) << 16).view(np.float32)


def int8_uniform(g, shape, lo=-127, hi=127):
    return g.integers(lo, hi + 1, shape, dtype=np.int16).astype(np.int8)


def q4_packed_uniform(g, n, k):
    """Q4 codes uniform in [-8, 7], two per byte: uniform random bytes."""
    return g.integers(0, 256, (n, k // 2), dtype=np.int16).astype(np.uint8)


# ---------------------------------------------------------------------------
# The five workloads.
# ---------------------------------------------------------------------------


def mxfp8_gemv(n=256, k=512, t=1, seed=0):
    """MXFP8 GEMV: 252-code E4M3 weights, UE8M0 bytes uniform in [120, 130], x ~ N(0,1)."""
    words = pack_bytes_to_words(e4m3_codes(rng(1, 0, seed), (n, k)))
    e8 = rng(1, 1, seed).integers(120, 131, (n, k // 32)).astype(np.uint8)
    x = bf16_normal(rng(1, 2, seed), (t, k))
    return dict(words=words, e8m0=e8, x=x)


def fp8row_weights_bf16(n=FFN, k=HIDDEN, seed=0, workload=2):
    """BF16 weights ~ N(0, 0.02) (to be encoded with one scale per row)."""
    return bf16_normal(rng(workload, 0, seed), (n, k), std=0.02)


def activations(t, k, seed=0, workload=2, tensor=1, outlier_p=0.0):
    return bf16_normal(rng(workload, tensor, seed), (t, k), outlier_p=outlier_p)


def block128_codes(n=HIDDEN, k=FFN, seed=0):
    """Block-128x128 E4M3 codes and a weight_scale_inv grid log-uniform in [2^-10, 2^-4]."""
    codes = e4m3_codes(rng(3, 0, seed), (n, k))
    wsi = bf16_log_uniform_as_f32(rng(3, 1, seed), (-(-n // 128), -(-k // 128)), -10, -4)
    return dict(codes=codes, wsi=wsi)


def gate_bf16(n=GATE_ROWS, k=HIDDEN, seed=0):
    return bf16_normal(rng(3, 2, seed), (n, k), std=0.02)


QBITS = {"q3g64": 3, "q5g64": 5, "q6g64": 6}


def grouped(fmt, n, k, seed=0):
    """Q4 group-64 (codes in [-8,7]), Q8 group-32/64 (codes in [-127,127]) or
    Q3 / Q5 / Q6 group-64 (b-bit codes, uniform: uniform random bytes of the
    dense bit stream, K b / 8 bytes per row), FP16 scales log-uniform in
    [2^-9, 2^-5]."""
    gs = {"q4g64": 64, "q8g32": 32, "q8g64": 64, "q3g64": 64, "q5g64": 64, "q6g64": 64}[fmt]
    tag = {"q4g64": 0, "q8g32": 1, "q8g64": 2, "q3g64": 3, "q5g64": 4, "q6g64": 5}[fmt]
    if fmt == "q4g64":
        codes = q4_packed_uniform(rng(4, 10 * tag, seed), n, k)
    elif fmt in QBITS:
        codes = rng(4, 10 * tag, seed).integers(0, 256, (n, k * QBITS[fmt] // 8), dtype=np.int16).astype(np.uint8)
    else:
        codes = int8_uniform(rng(4, 10 * tag, seed), (n, k))
    scales = f16_log_uniform(rng(4, 10 * tag + 1, seed), (n, k // gs), -9, -5)
    return dict(codes=codes, scales=scales)


def mlx_affine_int8(n, k, seed=0):
    """MLX affine int8 weights (the draft layer's storage): uint8 codes uniform
    over 0..255, one FP16 scale per 128 codes log-uniform in [2^-12, 2^-6] and
    one FP16 bias per 128 codes, -scale * uniform(96, 160) (a group's minimum
    lies near -128 scales when its values centre on zero)."""
    g = rng(6, 0, seed)
    codes = g.integers(0, 256, (n, k), dtype=np.int16).astype(np.uint8)
    scales = f16_log_uniform(rng(6, 1, seed), (n, k // 128), -12, -6)
    s = scales.view(np.float16).astype(np.float64)
    biases = (-s * rng(6, 2, seed).uniform(96, 160, s.shape)).astype(np.float16).view(np.uint16)
    return dict(codes=codes, scales=scales, biases=biases)


def w8a8_prefill(m=PREFILL_CHUNK, n=FFN, k=HIDDEN, seed=0):
    """x ~ N(0,1) with 1% of elements x20; Q8 group-64 weights, FP16 scales."""
    x = bf16_normal(rng(5, 0, seed), (m, k), outlier_p=0.01)
    w = int8_uniform(rng(5, 1, seed), (n, k))
    ws = f16_log_uniform(rng(5, 2, seed), (n, k // 64), -9, -5)
    return dict(x=x, w=w, w_scale=ws)


def head_weights_bf16(n=HEAD_ROWS, k=HIDDEN, seed=0):
    return bf16_normal(rng(5, 3, seed), (n, k), std=0.02)
