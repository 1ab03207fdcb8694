"""ctypes binding of libnq.so, with the C function names.

Argument marshalling only: each wrapper checks that tensors are contiguous,
passes their device pointers and sizes to the C entry point of the same name
on the current HIP stream, and raises NQError on a non-zero status.  Every
step of the computation runs in the library's HIP kernels; there is no
fallback.  BF16 / FP16 tensors may be passed as torch.bfloat16 / float16 or as
16-bit integer bit patterns.
"""

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnq.so")

NQ_OK, NQ_ERR_NULL, NQ_ERR_SHAPE, NQ_ERR_ALIGN, NQ_ERR_FORMAT, NQ_ERR_RANGE, NQ_ERR_HIP, NQ_ERR_SCRATCH = range(8)
NQ_GEMV_STATIC_SCRATCH_BYTES = 8 << 20
NQ_OUT_F32, NQ_OUT_BF16 = 0, 1
NQ_W_Q4G64_F16S, NQ_W_Q8G32_F16S, NQ_W_Q8G64_F16S, NQ_W_MXFP8_G32, NQ_W_BF16 = range(5)
NQ_W_Q3G64_F16S, NQ_W_Q5G64_F16S, NQ_W_Q6G64_F16S = 5, 6, 7
NQ_ROUTE_BF16, NQ_ROUTE_A8, NQ_ROUTE_A8_DECODE = 0, 1, 2
NQ_A8_PREFILL, NQ_A8_DECODE = 1, 2

# every entry point the header declares: name -> (restype, argtypes)
_P, _I64, _I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
SIGNATURES = {
    "nq_abi_version": (ctypes.c_int, []),
    "nq_status_string": (ctypes.c_char_p, [_I]),
    "nq_decode_mxfp8": (_I, [_P, _P, _I64, _I64, _I, _P, _P]),
    "nq_decode_mlx_affine_int8": (_I, [_P, _P, _P, _I64, _I64, _I, _P, _P]),
    "nq_reencode_block128_to_row": (_I, [_P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _P, _P, _P]),
    "nq_encode_fp8row_bf16": (_I, [_P, _I64, _I64, _P, _P, _P]),
    "nq_quantize_act_int8_g64": (_I, [_P, _I64, _I64, _P, _P, _P]),
    "nq_quantize_act_fp8_row": (_I, [_P, _I64, _I64, _P, _P, _P]),
    "nq_gemv_workspace_bytes": (_I64, [_I, _I64, _I64, _I64]),
    "nq_gemv_fp8row": (_I, [_P, _P, _P, _I64, _I64, _I64, _I, _P, _P, _I64, _P]),
    "nq_gemv_qgroup": (_I, [_I, _P, _P, _P, _I64, _I64, _I64, _I, _P, _P, _I64, _P]),
    "nq_gemm_w8a8_g64": (_I, [_P, _P, _P, _P, _I64, _I64, _I64, _I, _P, _P, _P]),
    "nq_gemm_fp8row": (_I, [_P, _P, _P, _I64, _I64, _I64, _P, _P, _I, _P, _P]),
    "nq_route": (_I, [_I64, _I]),
    "nq_packed_weight_bytes": (_I64, [_I, _I64, _I64]),
    "nq_pack_weights": (_I, [_I, _P, _I64, _I64, _P, _P]),
    "nq_gemv_fp8row_packed": (_I, [_P, _P, _P, _I64, _I64, _I64, _I, _P, _P, _I64, _P]),
    "nq_gemv_qgroup_packed": (_I, [_I, _P, _P, _P, _I64, _I64, _I64, _I, _P, _P, _I64, _P]),
    "nq_gemv_fp8row_packed_noalloc": (_I, [_P, _P, _P, _I64, _I64, _I64, _I, _P, _P]),
    "nq_stream_read_sink_words": (_I64, []),
    "nq_unpack_qbits_to_int8": (_I, [_I, _P, _I64, _I64, _P, _P]),
    "nq_linear_qbits_g64": (_I, [_I, _P, _I64, _P, _P, _I64, _I64, _I, _P, _P, _P, _I, _P, _P, _I64, _P]),
    "nq_gemv_a8_workspace_bytes": (_I64, [_I64, _I64, _I64]),
    "nq_gemv_a8_g64": (_I, [_I, _P, _P, _P, _P, _I64, _I64, _I64, _I, _P, _P, _I64, _P]),
    "nq_gemv_a8_g64_packed": (_I, [_I, _P, _P, _P, _P, _I64, _I64, _I64, _I, _P, _P, _I64, _P]),
    "nq_stream_read": (_I, [_P, _I64, _P, _P]),
    "nq_linear_q8g64": (_I, [_P, _I64, _P, _P, _I64, _I64, _I, _P, _P, _I, _P, _P, _I64, _P]),
    "nq_unpack_q4_to_int8": (_I, [_P, _I64, _I64, _P, _P]),
    "nq_linear_q4g64": (_I, [_P, _I64, _P, _P, _I64, _I64, _I, _P, _P, _P, _I, _P, _P, _I64, _P]),
}

_lib = None


class NQError(RuntimeError):
    def __init__(self, status, name):
        self.status = status
        msg = lib().nq_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{name} failed: {msg} (status {status})")


def lib():
    """Load libnq.so (once).  Raises ImportError when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is missing: build it with "
                              "`python -m quantized_weight_linear_amd.build`")
        l = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr() if t.numel() else None


def _size(t, nbytes, what):
    """Raise unless tensor t holds at least nbytes (the C ABI sees raw pointers only)."""
    have = 0 if t is None else t.numel() * t.element_size()
    if nbytes > 0 and have < nbytes:
        raise ValueError(f"{what}: {have} bytes given, {int(nbytes)} needed")


_CODE_BYTES = {NQ_W_Q4G64_F16S: 0.5, NQ_W_Q8G32_F16S: 1, NQ_W_Q8G64_F16S: 1, NQ_W_MXFP8_G32: 1, NQ_W_BF16: 2,
               NQ_W_Q3G64_F16S: 3 / 8, NQ_W_Q5G64_F16S: 5 / 8, NQ_W_Q6G64_F16S: 6 / 8}
_SCALE_BYTES = {NQ_W_Q4G64_F16S: 2 / 64, NQ_W_Q8G32_F16S: 2 / 32, NQ_W_Q8G64_F16S: 2 / 64,
                NQ_W_MXFP8_G32: 1 / 32, NQ_W_BF16: 0, NQ_W_Q3G64_F16S: 2 / 64, NQ_W_Q5G64_F16S: 2 / 64,
                NQ_W_Q6G64_F16S: 2 / 64}


def _stream(*tensors):
    for t in tensors:
        if t is not None and t.is_cuda:
            return torch.cuda.current_stream(t.device).cuda_stream
    return None


def _check(status, name):
    if status != NQ_OK:
        raise NQError(status, name)


def _out_dt(y):
    return NQ_OUT_BF16 if y.element_size() == 2 else NQ_OUT_F32


def nq_abi_version():
    return lib().nq_abi_version()


def _a8_flags(a8):
    """True / False (prefill A8 allowed or not) or an int of NQ_A8_* flags."""
    if isinstance(a8, bool):
        return NQ_A8_PREFILL if a8 else 0
    return int(a8)


def nq_route(T, a8):
    return lib().nq_route(T, _a8_flags(a8))


def nq_gemv_workspace_bytes(fmt, T, N, K):
    return lib().nq_gemv_workspace_bytes(fmt, T, N, K)


def alloc_gemv_workspace(fmt, T, N, K, device):
    """A zero-filled workspace big enough for nq_gemv_* at (fmt, T, N, K), or None."""
    n = nq_gemv_workspace_bytes(fmt, T, N, K)
    return torch.zeros(n, dtype=torch.uint8, device=device) if n > 0 else None


def nq_decode_mxfp8(words, e8m0, N, K, w_out):
    _size(words, N * K, "words"); _size(e8m0, N * K // 32, "e8m0")
    _size(w_out, N * K * w_out.element_size(), "w_out")
    _check(lib().nq_decode_mxfp8(_ptr(words), _ptr(e8m0), N, K, _out_dt(w_out), _ptr(w_out),
                                 _stream(words, w_out)), "nq_decode_mxfp8")


def nq_decode_mlx_affine_int8(codes, scales, biases, N, K, w_out):
    _size(codes, N * K, "codes"); _size(scales, N * (K // 128) * 2, "scales"); _size(biases, N * (K // 128) * 2, "biases")
    _size(w_out, N * K * w_out.element_size(), "w_out")
    _check(lib().nq_decode_mlx_affine_int8(_ptr(codes), _ptr(scales), _ptr(biases), N, K, _out_dt(w_out), _ptr(w_out),
                                           _stream(codes, w_out)), "nq_decode_mlx_affine_int8")


def nq_reencode_block128_to_row(codes, wsi, N, K, row_begin, row_end, out_codes, out_scale):
    gr, gc = wsi.shape
    _size(codes, N * K, "codes"); _size(wsi, 4 * gr * gc, "wsi")
    _size(out_codes, (row_end - row_begin) * K, "out_codes"); _size(out_scale, 2 * (row_end - row_begin), "out_scale")
    _check(lib().nq_reencode_block128_to_row(_ptr(codes), _ptr(wsi), N, K, gr, gc, row_begin, row_end,
                                             _ptr(out_codes), _ptr(out_scale), _stream(codes)),
           "nq_reencode_block128_to_row")


def nq_encode_fp8row_bf16(w, N, K, out_codes, out_scale):
    _size(w, 2 * N * K, "w"); _size(out_codes, N * K, "out_codes"); _size(out_scale, 2 * N, "out_scale")
    _check(lib().nq_encode_fp8row_bf16(_ptr(w), N, K, _ptr(out_codes), _ptr(out_scale), _stream(w)),
           "nq_encode_fp8row_bf16")


def nq_quantize_act_int8_g64(x, T, K, q, scale):
    _size(x, 2 * T * K, "x"); _size(q, T * K, "q"); _size(scale, 4 * T * (K // 64), "scale")
    _check(lib().nq_quantize_act_int8_g64(_ptr(x), T, K, _ptr(q), _ptr(scale), _stream(x)),
           "nq_quantize_act_int8_g64")


def nq_quantize_act_fp8_row(x, M, K, codes, scale):
    _size(x, 2 * M * K, "x"); _size(codes, M * K, "codes"); _size(scale, 4 * M, "scale")
    _check(lib().nq_quantize_act_fp8_row(_ptr(x), M, K, _ptr(codes), _ptr(scale), _stream(x)),
           "nq_quantize_act_fp8_row")


def _ws(workspace):
    return (_ptr(workspace), workspace.numel()) if workspace is not None else (None, 0)


def nq_gemv_fp8row(w, w_scale, x, T, N, K, y, workspace=None):
    _size(w, N * K, "w"); _size(w_scale, 2 * N, "w_scale"); _size(x, 2 * T * K, "x")
    _size(y, T * N * y.element_size(), "y")
    wp, wb = _ws(workspace)
    _check(lib().nq_gemv_fp8row(_ptr(w), _ptr(w_scale), _ptr(x), T, N, K, _out_dt(y), _ptr(y), wp, wb,
                                _stream(w, x)), "nq_gemv_fp8row")


def nq_gemv_qgroup(fmt, w_codes, w_scales, x, T, N, K, y, workspace=None):
    if fmt in _CODE_BYTES:
        _size(w_codes, N * K * _CODE_BYTES[fmt], "w_codes")
        _size(w_scales, N * K * _SCALE_BYTES[fmt], "w_scales")
    _size(x, 2 * T * K, "x"); _size(y, T * N * y.element_size(), "y")
    wp, wb = _ws(workspace)
    _check(lib().nq_gemv_qgroup(fmt, _ptr(w_codes), _ptr(w_scales), _ptr(x), T, N, K, _out_dt(y), _ptr(y),
                                wp, wb, _stream(w_codes, x)), "nq_gemv_qgroup")


def nq_gemm_w8a8_g64(a_q, a_scale, w_q, w_scale, M, N, K, y, group_sums=None):
    _size(a_q, M * K, "a_q"); _size(a_scale, 4 * M * (K // 64), "a_scale"); _size(w_q, N * K, "w_q")
    _size(w_scale, 2 * N * (K // 64), "w_scale"); _size(y, M * N * y.element_size(), "y")
    if group_sums is not None:
        _size(group_sums, 4 * M * N * (K // 64), "group_sums")
    _check(lib().nq_gemm_w8a8_g64(_ptr(a_q), _ptr(a_scale), _ptr(w_q), _ptr(w_scale), M, N, K, _out_dt(y),
                                  _ptr(y), _ptr(group_sums), _stream(a_q, w_q)), "nq_gemm_w8a8_g64")


def nq_gemm_fp8row(x, w, w_scale, M, N, K, a_codes, a_scale, y):
    _size(x, 2 * M * K, "x"); _size(w, N * K, "w"); _size(w_scale, 2 * N, "w_scale")
    _size(a_codes, M * K, "a_codes"); _size(a_scale, 4 * M, "a_scale"); _size(y, M * N * y.element_size(), "y")
    _check(lib().nq_gemm_fp8row(_ptr(x), _ptr(w), _ptr(w_scale), M, N, K, _ptr(a_codes), _ptr(a_scale),
                                _out_dt(y), _ptr(y), _stream(x, w)), "nq_gemm_fp8row")


def nq_linear_q8g64(x, T, w_q, w_scale, N, K, allow_a8, a_q_ws, a_scale_ws, y, workspace=None):
    _size(x, 2 * T * K, "x"); _size(w_q, N * K, "w_q"); _size(w_scale, 2 * N * (K // 64), "w_scale")
    _size(y, T * N * y.element_size(), "y")
    if nq_route(T, allow_a8) != NQ_ROUTE_BF16:
        _size(a_q_ws, T * K, "a_q_ws"); _size(a_scale_ws, 4 * T * (K // 64), "a_scale_ws")
    wp, wb = _ws(workspace)
    _check(lib().nq_linear_q8g64(_ptr(x), T, _ptr(w_q), _ptr(w_scale), N, K, _a8_flags(allow_a8),
                                 _ptr(a_q_ws), _ptr(a_scale_ws), _out_dt(y), _ptr(y), wp, wb,
                                 _stream(x, w_q)), "nq_linear_q8g64")


def nq_unpack_q4_to_int8(codes, N, K, out):
    _size(codes, N * K // 2, "codes"); _size(out, N * K, "out")
    _check(lib().nq_unpack_q4_to_int8(_ptr(codes), N, K, _ptr(out), _stream(codes, out)), "nq_unpack_q4_to_int8")


def nq_linear_q4g64(x, T, w_codes, w_scale, N, K, allow_a8, a_q_ws, a_scale_ws, w_i8_ws, y, workspace=None):
    _size(x, 2 * T * K, "x"); _size(w_codes, N * K // 2, "w_codes"); _size(w_scale, 2 * N * (K // 64), "w_scale")
    _size(y, T * N * y.element_size(), "y")
    route = nq_route(T, allow_a8)
    if route != NQ_ROUTE_BF16:
        _size(a_q_ws, T * K, "a_q_ws"); _size(a_scale_ws, 4 * T * (K // 64), "a_scale_ws")
    if route == NQ_ROUTE_A8:
        _size(w_i8_ws, N * K, "w_i8_ws")
    wp, wb = _ws(workspace)
    _check(lib().nq_linear_q4g64(_ptr(x), T, _ptr(w_codes), _ptr(w_scale), N, K, _a8_flags(allow_a8),
                                 _ptr(a_q_ws), _ptr(a_scale_ws), _ptr(w_i8_ws), _out_dt(y), _ptr(y), wp, wb,
                                 _stream(x, w_codes)), "nq_linear_q4g64")


def nq_gemv_a8_workspace_bytes(T, N, K):
    return lib().nq_gemv_a8_workspace_bytes(T, N, K)


def alloc_gemv_a8_workspace(T, N, K, device):
    """A zero-filled workspace big enough for nq_gemv_a8_* at (T, N, K), or None."""
    n = nq_gemv_a8_workspace_bytes(T, N, K)
    return torch.zeros(n, dtype=torch.uint8, device=device) if n > 0 else None


def _gemv_a8(name, fmt, w, w_scale, a_q, a_scale, T, N, K, y, workspace, packed):
    wbytes = nq_packed_weight_bytes(fmt, N, K) if packed else N * K * _CODE_BYTES.get(fmt, 1)
    _size(w, wbytes, "w"); _size(w_scale, 2 * N * (K // 64), "w_scale")
    _size(a_q, T * K, "a_q"); _size(a_scale, 4 * T * (K // 64), "a_scale"); _size(y, T * N * y.element_size(), "y")
    wp, wb = _ws(workspace)
    _check(getattr(lib(), name)(fmt, _ptr(w), _ptr(w_scale), _ptr(a_q), _ptr(a_scale), T, N, K, _out_dt(y), _ptr(y),
                                wp, wb, _stream(w, a_q)), name)


def nq_gemv_a8_g64(fmt, w_codes, w_scale, a_q, a_scale, T, N, K, y, workspace=None):
    _gemv_a8("nq_gemv_a8_g64", fmt, w_codes, w_scale, a_q, a_scale, T, N, K, y, workspace, False)


def nq_gemv_a8_g64_packed(fmt, w_packed, w_scale, a_q, a_scale, T, N, K, y, workspace=None):
    _gemv_a8("nq_gemv_a8_g64_packed", fmt, w_packed, w_scale, a_q, a_scale, T, N, K, y, workspace, True)


def nq_stream_read(src, sink):
    """Read all of src (a device tensor, 16-byte multiple) once; sink is an
    int32 device tensor of at least nq_stream_read_sink_words() elements."""
    nbytes = src.numel() * src.element_size()
    _size(sink, 4 * lib().nq_stream_read_sink_words(), "sink")
    _check(lib().nq_stream_read(_ptr(src), nbytes, _ptr(sink), _stream(src)), "nq_stream_read")


NQ_FMT_FP8ROW = -1     # the format code the packing calls use for row-scaled FP8


def nq_packed_weight_bytes(fmt, N, K):
    return lib().nq_packed_weight_bytes(fmt, N, K)


def nq_pack_weights(fmt, w, N, K, w_packed):
    code_bytes = 1 if fmt == NQ_FMT_FP8ROW else _CODE_BYTES.get(fmt, 1)
    _size(w, N * K * code_bytes, "w")
    _size(w_packed, nq_packed_weight_bytes(fmt, N, K), "w_packed")
    _check(lib().nq_pack_weights(fmt, _ptr(w), N, K, _ptr(w_packed), _stream(w)), "nq_pack_weights")


def nq_gemv_fp8row_packed(w_packed, w_scale, x, T, N, K, y, workspace=None):
    _size(w_packed, nq_packed_weight_bytes(NQ_FMT_FP8ROW, N, K), "w_packed")
    _size(w_scale, 2 * N, "w_scale"); _size(x, 2 * T * K, "x"); _size(y, T * N * y.element_size(), "y")
    wp, wb = _ws(workspace)
    _check(lib().nq_gemv_fp8row_packed(_ptr(w_packed), _ptr(w_scale), _ptr(x), T, N, K, _out_dt(y), _ptr(y),
                                       wp, wb, _stream(w_packed, x)), "nq_gemv_fp8row_packed")


def nq_gemv_qgroup_packed(fmt, w_packed, w_scales, x, T, N, K, y, workspace=None):
    if fmt in _CODE_BYTES:
        _size(w_packed, nq_packed_weight_bytes(fmt, N, K), "w_packed")
        _size(w_scales, N * K * _SCALE_BYTES[fmt], "w_scales")
    _size(x, 2 * T * K, "x"); _size(y, T * N * y.element_size(), "y")
    wp, wb = _ws(workspace)
    _check(lib().nq_gemv_qgroup_packed(fmt, _ptr(w_packed), _ptr(w_scales), _ptr(x), T, N, K, _out_dt(y),
                                       _ptr(y), wp, wb, _stream(w_packed, x)), "nq_gemv_qgroup_packed")


def nq_gemv_fp8row_packed_noalloc(w_packed, w_scale, x, T, N, K, y):
    _size(w_packed, nq_packed_weight_bytes(NQ_FMT_FP8ROW, N, K), "w_packed")
    _size(w_scale, 2 * N, "w_scale"); _size(x, 2 * T * K, "x"); _size(y, T * N * y.element_size(), "y")
    _check(lib().nq_gemv_fp8row_packed_noalloc(_ptr(w_packed), _ptr(w_scale), _ptr(x), T, N, K, _out_dt(y), _ptr(y),
                                               _stream(w_packed, x)), "nq_gemv_fp8row_packed_noalloc")


def nq_unpack_qbits_to_int8(fmt, codes, N, K, out):
    _size(codes, N * K * _CODE_BYTES[fmt], "codes"); _size(out, N * K, "out")
    _check(lib().nq_unpack_qbits_to_int8(fmt, _ptr(codes), N, K, _ptr(out), _stream(codes, out)),
           "nq_unpack_qbits_to_int8")


def nq_linear_qbits_g64(fmt, x, T, w_codes, w_scale, N, K, a8, a_q_ws, a_scale_ws, w_i8_ws, y, workspace=None):
    _size(x, 2 * T * K, "x"); _size(w_codes, N * K * _CODE_BYTES[fmt], "w_codes")
    _size(w_scale, 2 * N * (K // 64), "w_scale"); _size(y, T * N * y.element_size(), "y")
    if nq_route(T, a8) != NQ_ROUTE_BF16:
        _size(a_q_ws, T * K, "a_q_ws"); _size(a_scale_ws, 4 * T * (K // 64), "a_scale_ws")
        _size(w_i8_ws, N * K, "w_i8_ws")
    wp, wb = _ws(workspace)
    _check(lib().nq_linear_qbits_g64(fmt, _ptr(x), T, _ptr(w_codes), _ptr(w_scale), N, K, _a8_flags(a8),
                                     _ptr(a_q_ws), _ptr(a_scale_ws), _ptr(w_i8_ws), _out_dt(y), _ptr(y), wp, wb,
                                     _stream(x, w_codes)), "nq_linear_qbits_g64")
