"""The C ABI on the CPU: the library loads, exports every declared symbol, and
rejects invalid arguments with the documented status before any HIP call."""

import ctypes
import os
import re

import pytest

from quantized_weight_linear_amd import nq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nq.h")

A = 0x10000          # a 16-byte aligned fake device address (never dereferenced)
MIS = 0x10001        # a misaligned one


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(nq_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    return nq.lib()


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(L, n), n
        assert n in nq.SIGNATURES, n
    assert set(nq.SIGNATURES) == set(names)


def test_version_and_strings(L):
    assert L.nq_abi_version() == 1
    for s in range(7):
        assert L.nq_status_string(s)
    assert L.nq_status_string(99) == b"unknown status"


def test_route_rule(L):
    assert L.nq_route(128, 1) == nq.NQ_ROUTE_BF16
    assert L.nq_route(129, 1) == nq.NQ_ROUTE_A8
    assert L.nq_route(1792, 1) == nq.NQ_ROUTE_A8
    assert L.nq_route(1792, 0) == nq.NQ_ROUTE_BF16
    assert L.nq_route(0, 1) == nq.NQ_ROUTE_BF16


def test_decode_mxfp8_validation(L):
    f = L.nq_decode_mxfp8
    assert f(A, A, 4, 33, 0, A, None) == nq.NQ_ERR_SHAPE
    assert f(A, A, -1, 32, 0, A, None) == nq.NQ_ERR_SHAPE
    assert f(A, A, 4, 32, 7, A, None) == nq.NQ_ERR_FORMAT
    assert f(None, A, 4, 32, 0, A, None) == nq.NQ_ERR_NULL
    assert f(A, None, 4, 32, 0, A, None) == nq.NQ_ERR_NULL
    assert f(A, A, 4, 32, 0, None, None) == nq.NQ_ERR_NULL
    assert f(MIS, A, 4, 32, 0, A, None) == nq.NQ_ERR_ALIGN
    assert f(A, A, 4, 32, 1, MIS, None) == nq.NQ_ERR_ALIGN
    assert f(None, None, 0, 32, 0, None, None) == nq.NQ_OK      # empty: nothing to do


def test_decode_mlx_affine_int8_validation(L):
    f = L.nq_decode_mlx_affine_int8
    assert f(A, A, A, 4, 192, 0, A, None) == nq.NQ_ERR_SHAPE          # K % 128
    assert f(A, A, A, -1, 128, 0, A, None) == nq.NQ_ERR_SHAPE
    assert f(A, A, A, 4, 128, 5, A, None) == nq.NQ_ERR_FORMAT
    assert f(None, A, A, 4, 128, 0, A, None) == nq.NQ_ERR_NULL
    assert f(A, None, A, 4, 128, 0, A, None) == nq.NQ_ERR_NULL
    assert f(A, A, None, 4, 128, 0, A, None) == nq.NQ_ERR_NULL
    assert f(A, A, A, 4, 128, 1, None, None) == nq.NQ_ERR_NULL
    assert f(MIS, A, A, 4, 128, 0, A, None) == nq.NQ_ERR_ALIGN
    assert f(A, A, A, 4, 128, 1, MIS, None) == nq.NQ_ERR_ALIGN
    assert f(None, None, None, 0, 128, 0, None, None) == nq.NQ_OK    # empty: nothing to do


def test_reencode_validation(L):
    f = L.nq_reencode_block128_to_row
    assert f(A, A, 300, 520, 2, 5, 0, 300, A, A, None) == nq.NQ_ERR_SHAPE    # ceil(300/128) = 3
    assert f(A, A, 300, 520, 3, 4, 0, 300, A, A, None) == nq.NQ_ERR_SHAPE    # ceil(520/128) = 5
    assert f(A, A, 300, 520, 3, 5, 5, 5, A, A, None) == nq.NQ_ERR_RANGE
    assert f(A, A, 300, 520, 3, 5, -1, 5, A, A, None) == nq.NQ_ERR_RANGE
    assert f(A, A, 300, 520, 3, 5, 0, 301, A, A, None) == nq.NQ_ERR_RANGE
    assert f(None, A, 300, 520, 3, 5, 0, 300, A, A, None) == nq.NQ_ERR_NULL
    assert f(A, A, 300, 520, 3, 5, 0, 300, A, None, None) == nq.NQ_ERR_NULL
    assert f(A, MIS, 300, 520, 3, 5, 0, 300, A, A, None) == nq.NQ_ERR_ALIGN


def test_encode_and_quantize_validation(L):
    assert L.nq_encode_fp8row_bf16(A, -2, 8, A, A, None) == nq.NQ_ERR_SHAPE
    assert L.nq_encode_fp8row_bf16(A, 2, 8, None, A, None) == nq.NQ_ERR_NULL
    assert L.nq_encode_fp8row_bf16(A, 0, 8, None, None, None) == nq.NQ_OK
    q = L.nq_quantize_act_int8_g64
    assert q(A, 4, 65, A, A, None) == nq.NQ_ERR_SHAPE
    assert q(A, 4, 64, None, A, None) == nq.NQ_ERR_NULL
    assert q(A, 4, 64, A, MIS, None) == nq.NQ_ERR_ALIGN
    assert q(None, 0, 64, None, None, None) == nq.NQ_OK
    q8 = L.nq_quantize_act_fp8_row
    assert q8(A, -1, 64, A, A, None) == nq.NQ_ERR_SHAPE
    assert q8(A, 3, 64, A, None, None) == nq.NQ_ERR_NULL


def test_gemv_validation(L):
    g = L.nq_gemv_fp8row
    assert g(A, A, A, 4, 8, 64, 5, A, None, 0, None) == nq.NQ_ERR_FORMAT
    assert g(A, A, A, -4, 8, 64, 0, A, None, 0, None) == nq.NQ_ERR_SHAPE
    assert g(A, A, A, 4, 8, 64, 0, A, None, -1, None) == nq.NQ_ERR_SHAPE
    assert g(A, None, A, 4, 8, 64, 0, A, None, 0, None) == nq.NQ_ERR_NULL
    assert g(A, A, A, 4, 8, 64, 0, MIS, None, 0, None) == nq.NQ_ERR_ALIGN
    assert g(A, A, A, 4, 8, 64, 0, A, MIS, 1024, None) == nq.NQ_ERR_ALIGN
    assert g(A, A, None, 0, 8, 64, 0, None, None, 0, None) == nq.NQ_OK      # T = 0
    q = L.nq_gemv_qgroup
    assert q(9, A, A, A, 4, 8, 64, 0, A, None, 0, None) == nq.NQ_ERR_FORMAT
    assert q(nq.NQ_W_Q4G64_F16S, A, A, A, 4, 8, 96, 0, A, None, 0, None) == nq.NQ_ERR_SHAPE
    assert q(nq.NQ_W_Q8G32_F16S, A, A, A, 4, 8, 48, 0, A, None, 0, None) == nq.NQ_ERR_SHAPE
    assert q(nq.NQ_W_MXFP8_G32, A, A, A, 4, 8, 48, 0, A, None, 0, None) == nq.NQ_ERR_SHAPE
    assert q(nq.NQ_W_Q8G64_F16S, A, None, A, 4, 8, 64, 0, A, None, 0, None) == nq.NQ_ERR_NULL
    assert q(nq.NQ_W_Q8G64_F16S, A, A, A, 4, 8, 64, 2, A, None, 0, None) == nq.NQ_ERR_FORMAT
    assert q(nq.NQ_W_BF16, A, None, A, 0, 8, 64, 0, A, None, 0, None) == nq.NQ_OK    # BF16 needs no scales


# A pass addresses its tokens padded to whole blocks of 16 (the padding reads
# zero through out-of-range 32-bit buffer offsets): 17 tokens of 2^25 columns
# fit in 2 GiB, their 32 padded rows do not, so the call is refused.
def test_padded_token_rows_bound_the_shape(L):
    k = 1 << 25
    assert L.nq_gemv_qgroup(nq.NQ_W_Q5G64_F16S, A, A, A, 17, 1, k, 0, A, None, 0, None) == nq.NQ_ERR_SHAPE
    assert L.nq_gemv_a8_g64(nq.NQ_W_Q8G64_F16S, A, A, A, A, 17, 1, 2 * k, 0, A, None, 0, None) == nq.NQ_ERR_SHAPE
    assert L.nq_gemv_a8_g64(nq.NQ_W_Q8G64_F16S, A, A, A, A, 17, 1, 2 * k + 256, 0, A, None, 0, None) == nq.NQ_ERR_SHAPE


def test_gemm_validation(L):
    w = L.nq_gemm_w8a8_g64
    assert w(A, A, A, A, 4, 8, 96, 0, A, None, None) == nq.NQ_ERR_SHAPE
    assert w(A, A, A, None, 4, 8, 64, 0, A, None, None) == nq.NQ_ERR_NULL
    assert w(A, A, A, A, 4, 8, 64, 0, A, MIS, None) == nq.NQ_ERR_ALIGN
    assert w(A, A, A, A, 4, 8, 64, 3, A, None, None) == nq.NQ_ERR_FORMAT
    f = L.nq_gemm_fp8row
    assert f(A, A, A, 4, 8, 24, A, A, 0, A, None) == nq.NQ_ERR_SHAPE
    assert f(A, A, A, 4, 8, 32, None, A, 0, A, None) == nq.NQ_ERR_NULL
    assert f(A, A, A, 4, 8, 32, A, A, 0, MIS, None) == nq.NQ_ERR_ALIGN


def test_linear_validation(L):
    f = L.nq_linear_q8g64
    # the A8 route (T >= 129, allowed) needs the activation workspaces
    assert f(A, 129, A, A, 8, 64, 1, None, A, 0, A, None, 0, None) == nq.NQ_ERR_NULL
    assert f(A, 129, A, A, 8, 64, 1, A, None, 0, A, None, 0, None) == nq.NQ_ERR_NULL
    assert f(A, 129, A, A, 8, 96, 1, A, A, 0, A, None, 0, None) == nq.NQ_ERR_SHAPE
    assert f(A, 129, A, A, 8, 64, 1, MIS, A, 0, A, None, 0, None) == nq.NQ_ERR_ALIGN
    # the BF16 route does not look at them
    assert f(A, 0, A, A, 8, 64, 1, None, None, 0, None, None, 0, None) == nq.NQ_OK


def test_q4_a8_validation(L):
    u = L.nq_unpack_q4_to_int8
    assert u(A, 4, 96, A, None) == nq.NQ_ERR_SHAPE
    assert u(None, 4, 128, A, None) == nq.NQ_ERR_NULL
    assert u(A, 4, 128, None, None) == nq.NQ_ERR_NULL
    assert u(MIS, 4, 128, A, None) == nq.NQ_ERR_ALIGN
    assert u(None, 0, 128, None, None) == nq.NQ_OK
    f = L.nq_linear_q4g64
    assert f(A, 200, A, A, 8, 96, 1, A, A, A, 0, A, None, 0, None) == nq.NQ_ERR_SHAPE
    assert f(A, 200, A, A, 8, 128, 1, A, A, A, 3, A, None, 0, None) == nq.NQ_ERR_FORMAT
    assert f(A, 200, A, A, 8, 128, 1, A, A, None, 0, A, None, 0, None) == nq.NQ_ERR_NULL     # A8 route needs w_i8_ws
    assert f(A, 200, A, A, 8, 128, 1, A, A, MIS, 0, A, None, 0, None) == nq.NQ_ERR_ALIGN
    # the BF16 route does not need the A8 workspaces (nothing is launched: N = 0)
    assert f(A, 100, A, A, 0, 128, 1, None, None, None, 0, A, None, 0, None) == nq.NQ_OK


def test_packed_validation(L):
    # the packed layout exists for K % 256 == 0 only
    assert L.nq_pack_weights(-1, A, 8, 384, A, None) == nq.NQ_ERR_SHAPE
    assert L.nq_pack_weights(9, A, 8, 512, A, None) == nq.NQ_ERR_FORMAT
    assert L.nq_pack_weights(-1, None, 8, 512, A, None) == nq.NQ_ERR_NULL
    assert L.nq_gemv_fp8row_packed(A, A, A, 4, 8, 384, 0, A, None, 0, None) == nq.NQ_ERR_SHAPE
    assert L.nq_gemv_qgroup_packed(nq.NQ_W_Q8G32_F16S, A, A, A, 4, 8, 640, 0, A, None, 0, None) == nq.NQ_ERR_SHAPE
    assert L.nq_packed_weight_bytes(nq.NQ_W_Q4G64_F16S, 17, 512) == 32 * 256
    assert L.nq_packed_weight_bytes(nq.NQ_W_BF16, 16, 256) == 16 * 512


def test_workspace_query_is_host_only(L):
    assert L.nq_gemv_workspace_bytes(-1, -1, 8, 64) == 0
    assert L.nq_gemv_workspace_bytes(-1, 4, 8, 100) == 0       # fallback path needs none


# The GEMV plan, seen through the workspace it asks for (256 CUs: the count
# the library assumes without a device, and MI355X's).  Layout: a 4-byte
# counter per 64-row tile (padded to 256 bytes), then FP32 partials of 64
# rows x T tokens per split and tile, or per slot and leftover tile.
def test_gemv_plan_workspace(L):
    c272 = 1280                                  # 272 tiles x 4 bytes, padded to 256
    # row-FP8 17408 x 5120 (272 tiles, 20 chunks of 256): 16 leftover tiles,
    # 320 units, at most 2 beside a whole tile, so 160 spread workgroups of 2
    # units; a leftover tile meets at most 20 / 2 + 1 = 11 of them (slots).
    assert L.nq_gemv_workspace_bytes(-1, 1, 17408, 5120) == c272 + 16 * 11 * 1 * 64 * 4
    assert L.nq_gemv_workspace_bytes(-1, 33, 17408, 5120) == c272 + 16 * 11 * 33 * 64 * 4
    # 16384 rows: one whole tile per CU, nothing to exchange
    assert L.nq_gemv_workspace_bytes(-1, 1, 16384, 5120) == 0
    # The grouped formats at one token block take the same spread plan
    # (Q4 group-64 at 1 token, Q8 group-32 at 8)
    assert L.nq_gemv_workspace_bytes(nq.NQ_W_Q4G64_F16S, 1, 17408, 5120) == c272 + 16 * 11 * 1 * 64 * 4
    assert L.nq_gemv_workspace_bytes(nq.NQ_W_Q8G32_F16S, 8, 17408, 5120) == c272 + 16 * 11 * 8 * 64 * 4
    # ... and at 17 tokens (two token blocks) the streaming kernel with K in 3
    assert L.nq_gemv_workspace_bytes(nq.NQ_W_Q8G32_F16S, 17, 17408, 5120) == c272 + 3 * 17 * 272 * 64 * 4
    # Q4 group-64 at 16384 rows, one token: streaming kernel, whole tiles
    assert L.nq_gemv_workspace_bytes(nq.NQ_W_Q4G64_F16S, 1, 16384, 5120) == 0
    # 20480 rows (320 tiles, 64 leftover: too many to spread), 1 token: the
    # resident kernel, K split in 4 (ceil(320 x 4 / 256) x 5 = 25 chunks at most)
    assert L.nq_gemv_workspace_bytes(nq.NQ_W_Q4G64_F16S, 1, 20480, 5120) == 1280 + 4 * 1 * 320 * 64 * 4
    # row-FP8 5120 x 17408, 17 tokens (80 tiles, 68 chunks): streaming kernel
    # with the balanced split, 3 (ceil(80 x 3 / 256) x 23 = 23 chunks at most)
    assert L.nq_gemv_workspace_bytes(-1, 17, 5120, 17408) == 512 + 3 * 17 * 80 * 64 * 4
    # 24576 rows (384 tiles): two splits leave the busiest CU 3/2 of a tile,
    # three 5/3, so K is split in two
    assert L.nq_gemv_workspace_bytes(nq.NQ_W_Q8G32_F16S, 8, 24576, 5120) == 1536 + 2 * 8 * 384 * 64 * 4
    # Q8 group-32 at 16384 rows (one tile per CU), 8 tokens: streaming kernel,
    # K in two (two workgroups per CU)
    assert L.nq_gemv_workspace_bytes(nq.NQ_W_Q8G32_F16S, 8, 16384, 5120) == 1024 + 2 * 8 * 256 * 64 * 4


def test_binding_raises(L):
    with pytest.raises(nq.NQError) as e:
        nq._check(L.nq_gemm_w8a8_g64(A, A, A, A, 4, 8, 96, 0, A, None, None), "nq_gemm_w8a8_g64")
    assert e.value.status == nq.NQ_ERR_SHAPE and "invalid shape" in str(e.value)
