"""Benchmark of the quantized-weight linear projection on one MI355X.

One step runs every row of the hot path on its workload, `--burst` launches
of a row back to back (default 8), inputs already resident in HBM, in this
order (prefill and conversions before decode, as in an engine step):
  quant_int8     1792x5120 per-token-per-64 int8 quantization
  gemm_w8a8      W8A8 GEMM M=1792, N=17408, K=5120
  gemm_fp8       per-token E4M3 quantization + FP8 GEMM, same shape
  q4_a8          Q4 group-64 weights on the A8 route, same shape: widening to
                 int8, and the routed projection (quantize + widen + GEMM)
  q5g64_a8 / q3g64_a8   the same for Q5 / Q3 group-64 weights
  reencode       block-128 E4M3 -> per-row FP8, 5120x17408
  gemv_down      re-encoded 5120x17408, T = 1, 33; BF16 gate 96x5120, T = 1, 33
  decode_mxfp8   MXFP8 256x512 decode (FP32 out)            + MXFP8 GEMV T=1
  decode_mlx     MLX affine int8 17408x5120 -> BF16 (the draft layer's storage)
  head           row-FP8 152064x5120, T = 1..64
  head_q8        the same head as Q8 group-32, T = 1..64 (FP8-versus-Q8 crossover)
  gemv_q4g64 / gemv_q8g32 / gemv_q5g64 / gemv_q3g64   at 17408x5120 and
                 5120x17408, T = 1, 8, 33
  a8_decode      A8 decode GEMV (int8 activations) on Q8 / Q4 group-64 weights
                 at both shapes, T = 1, 8, 33: the kernel, the routed step
                 (quantize + GEMV), and the BF16-activation Q8 GEMV beside it
  gemv_fp8row    row-FP8 17408x5120, T = 1, 4, 16, 33 (BF16 out)   <- headline
  hbm_read       a plain streaming read of 89 MB (rotating over > 512 MB) and
                 of 1 GiB: the measured HBM read ceiling
Weights of the decode GEMVs rotate over copies totalling more than 512 MB so
that the 256 MB last-level cache cannot serve them.  Every burst is bracketed
by HIP events on the stream it runs on (per-launch time = burst time / burst;
no event packet sits between two launches of a burst); per-row averages come
from those.

`value` is the headline: decode GEMV HBM GB/s on row-FP8 17408x5120 over
T = 1, 4, 16, 33 (algorithmic bytes / kernel time).  The prefill GEMMs are
reported in `prefill` and `roofline_prefill` (TOPS and fraction of the MFMA
peak), the measured HBM read ceiling (a plain streaming read, rows
hbm_read_*) beside the headline roofline, weight-bytes/s and tokens/s of every
decode row in `decode_per_shape`, and the oracle per (config, T) in
`cpu_baseline`.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# HBM traffic of the headline GEMV launches (packed row-FP8 17408x5120), from
# `rocprofv3 --pmc FETCH_SIZE` and `--pmc WRITE_SIZE` runs of
# `bench.py --rows gemv_fp8row,gemv_q4g64,gemv_q8g32`, in KiB per dispatch
# (the headline rows' launches after the warm-up step), scaled by the same
# counters on `bench.py --calibrate-copy` (a 256 MiB copy reads FETCH_SIZE
# 131083.5 KiB and writes WRITE_SIZE 262144 KiB: factors 1.99982 and 1.0).
# Summaries: profiles/gemv_fp8row_17408x5120_hbm_traffic.md.  Valid only for
# the GEMV code they were taken on (gemv_source_hash over GEMV_SOURCES).
GEMV_TRAFFIC = {
    "source_sha256_16": "b606c2413e711ba0",
    "fetch_factor": 262144.0 / 131083.5,
    "write_factor": 1.0,
    "fetch_kib": {"gemv_fp8row_T1": 43819.3, "gemv_fp8row_T4": 44009.3, "gemv_fp8row_T16": 44768.8,
                  "gemv_fp8row_T33": 45918.0},
    "write_kib": {"gemv_fp8row_T1": 79.5, "gemv_fp8row_T4": 301.5, "gemv_fp8row_T16": 1189.5,
                  "gemv_fp8row_T33": 2447.5},
}

GEMV_SOURCES = ("nq_launch.h", "nq_gemv_kernels.h", "nq_gemv.hip", "nq_gemv_fp8row.hip")

HBM_PEAK_GBS = 8000.0
INT8_PEAK_TOPS = 5000.0
FP8_PEAK_TFLOPS = 5000.0
ROTATE_BYTES = 512 << 20
DEV = "cuda:0"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=5)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--rows", default="all", help="comma list of row groups to run (default: all)")
    p.add_argument("--burst", type=int, default=8,
                   help="launches per row back to back between one pair of HIP events (default 8)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--rows-json", default=None, help="also write per-row results to this file")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain 256 MiB device copy 4 times: the reference for scaling the "
                        "FETCH_SIZE / WRITE_SIZE counters to bytes")
    return p.parse_args()


def calibrate_copy():
    """A copy of known size for the HBM traffic counters: each launch reads and
    writes exactly 256 MiB (torch's copy kernel, buffers far larger than L2)."""
    torch = _torch()
    src = torch.empty(256 << 20, dtype=torch.uint8, device=DEV).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": 256 << 20, "launches": 4}), flush=True)


class Row:
    """One timed launch: `work` is its algorithmic bytes (GB/s rows) or ops;
    decode GEMV rows also carry their weight bytes and token count, for the
    weight-bytes/s and tokens/s per layer shape."""

    def __init__(self, name, kernel, unit, work, fn, wbytes=None, tokens=None):
        self.name, self.kernel, self.unit, self.work, self.fn = name, kernel, unit, work, fn
        self.wbytes, self.tokens = wbytes, tokens
        self.ms = []


def _torch():
    import torch
    return torch


def to_dev(a):
    torch = _torch()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    elif a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).to(DEV)


def rotation(*tensors):
    """Copies of a weight set (first tensor sets the count) totalling > ROTATE_BYTES;
    returns a function that hands out the next copy on every call."""
    first = tensors[0]
    n = max(1, -(-ROTATE_BYTES // (first.numel() * first.element_size())))
    sets = [tuple(tensors)] + [tuple(t.clone() for t in tensors) for _ in range(n - 1)]
    state = [0]

    def nxt():
        v = sets[state[0] % len(sets)]
        state[0] += 1
        return v
    return nxt


def empty(shape, dtype):
    return _torch().empty(shape, dtype=dtype, device=DEV)


# Each section builds its rows in its own scope: the launch closures capture
# only names that are never rebound.

def rows_mxfp8(nq, W):
    torch = _torch()
    d = W.mxfp8_gemv()
    words, e8, x = to_dev(d["words"]), to_dev(d["e8m0"]), to_dev(d["x"])
    n, k = 256, 512
    out = empty((n, k), torch.float32)
    y = empty((1, n), torch.float32)
    return [Row("decode_mxfp8", "decode_mxfp8", "GB/s", n * k + n * k // 32 + 4 * n * k,
                lambda: nq.nq_decode_mxfp8(words, e8, n, k, out)),
            Row("gemv_mxfp8_T1", "gemv_mxfp8", "GB/s", n * k + n * k // 32 + 2 * k + 4 * n,
                lambda: nq.nq_gemv_qgroup(nq.NQ_W_MXFP8_G32, words, e8, x, 1, n, k, y))]


def rows_mlx(nq, W):
    """MLX affine int8 -> BF16 decode on a 17408x5120 projection (the draft
    layer's storage, decoded by the converter)."""
    torch = _torch()
    n, k = W.FFN, W.HIDDEN
    d = W.mlx_affine_int8(n, k)
    c, s, b = to_dev(d["codes"]), to_dev(d["scales"]), to_dev(d["biases"])
    out = empty((n, k), torch.int16)
    return [Row("decode_mlx_int8", "decode_mlx_int8", "GB/s", n * k + 4 * n * (k // 128) + 2 * n * k,
                lambda: nq.nq_decode_mlx_affine_int8(c, s, b, n, k, out))]


def rows_hbm_read(nq):
    """The measured HBM read ceiling: a plain streaming read (nq_stream_read)
    of 89,128,960 bytes (the headline weight's size) rotating over copies
    totalling more than 512 MB, and of one 1 GiB buffer."""
    torch = _torch()
    sink = empty((nq.lib().nq_stream_read_sink_words(),), torch.int32)
    b89 = empty((89128960,), torch.uint8).fill_(1)
    nxt = rotation(b89)
    big = empty((1 << 30,), torch.uint8).fill_(1)
    return [Row("hbm_read_89MB", "stream_read", "GB/s", 89128960, lambda: nq.nq_stream_read(nxt()[0], sink)),
            Row("hbm_read_1GiB", "stream_read", "GB/s", 1 << 30, lambda: nq.nq_stream_read(big, sink))]


def pack(nq, fmt, codes, n, k):
    """One-time weight packing (setup, not timed)."""
    torch = _torch()
    pk = empty((nq.nq_packed_weight_bytes(fmt, n, k),), torch.uint8)
    nq.nq_pack_weights(fmt, codes, n, k, pk)
    return pk


def _fp8row_gemv_rows(nq, prefix, kernel, q, s, xs, ts, rotate=True, packed=True):
    torch = _torch()
    n, k = q.shape
    if packed:
        q = pack(nq, -1, q, n, k)
    gemv = nq.nq_gemv_fp8row_packed if packed else nq.nq_gemv_fp8row
    nxt = rotation(q, s) if rotate else (lambda: (q, s))
    rows = []
    for t, xt in zip(ts, xs):
        y = empty((t, n), torch.int16)
        ws = nq.alloc_gemv_workspace(-1, t, n, k, DEV)

        def fn(t=t, xt=xt, y=y, ws=ws):
            qq, ss = nxt()
            gemv(qq, ss, xt, t, n, k, y, ws)
        rows.append(Row(f"{prefix}_T{t}", kernel, "GB/s", n * k + 2 * n + 2 * t * k + 2 * t * n, fn,
                        wbytes=n * k + 2 * n, tokens=t))
    return rows


def _encode_bf16_on_gpu(nq, w_bf16):
    torch = _torch()
    n, k = w_bf16.shape
    wb = to_dev(w_bf16)
    q, s = empty((n, k), torch.uint8), empty((n,), torch.int16)
    nq.nq_encode_fp8row_bf16(wb, n, k, q, s)
    del wb
    return q, s


def rows_gemv_fp8row(nq, W):
    n, k = W.FFN, W.HIDDEN
    q, s = _encode_bf16_on_gpu(nq, W.fp8row_weights_bf16(n, k))
    x33 = to_dev(W.activations(33, k))
    ts = (1, 4, 16, 33)
    xs = [x33[:t].contiguous() for t in ts]
    return (_fp8row_gemv_rows(nq, "gemv_fp8row", "gemv_fp8row", q, s, xs, ts) +
            _fp8row_gemv_rows(nq, "gemv_fp8row_rowmajor", "gemv_fp8row_rowmajor", q, s, xs, ts, packed=False))


def rows_reencode_and_down(nq, W, want_reencode, want_down):
    torch = _torch()
    d = W.block128_codes()
    n, k = d["codes"].shape
    codes, wsi = to_dev(d["codes"]), to_dev(d["wsi"])
    gr, gc = d["wsi"].shape
    q, s = empty((n, k), torch.uint8), empty((n,), torch.int16)
    nq.nq_reencode_block128_to_row(codes, wsi, n, k, 0, n, q, s)
    rows = []
    if want_reencode:
        rows.append(Row("reencode", "reencode", "GB/s", 2 * n * k + 4 * gr * gc + 2 * n,
                        lambda: nq.nq_reencode_block128_to_row(codes, wsi, n, k, 0, n, q, s)))
    if want_down:
        ts = (1, 33)
        xs = [to_dev(W.activations(t, k, workload=3, tensor=3)) for t in ts]
        rows += _fp8row_gemv_rows(nq, "gemv_down", "gemv_fp8row", q, s, xs, ts)
        rows += rows_gate(nq, W)
    return rows


def rows_gate(nq, W):
    torch = _torch()
    gate = to_dev(W.gate_bf16())
    n, k = W.GATE_ROWS, W.HIDDEN
    rows = []
    gate_pk = pack(nq, nq.NQ_W_BF16, gate, n, k)
    for t in (1, 33):
        xg = to_dev(W.activations(t, k, workload=3, tensor=4))
        yg = empty((t, n), torch.int16)
        wg = nq.alloc_gemv_workspace(nq.NQ_W_BF16, t, n, k, DEV)
        rows.append(Row(f"gemv_gate_T{t}", "gemv_bf16", "GB/s", 2 * n * k + 2 * t * k + 2 * t * n,
                        lambda t=t, xg=xg, yg=yg, wg=wg: nq.nq_gemv_qgroup_packed(nq.NQ_W_BF16, gate_pk, None, xg,
                                                                                  t, n, k, yg, wg),
                        wbytes=2 * n * k, tokens=t))
    return rows


def rows_grouped(nq, W, name):
    torch = _torch()
    fmt = {"q4g64": nq.NQ_W_Q4G64_F16S, "q8g32": nq.NQ_W_Q8G32_F16S, "q5g64": nq.NQ_W_Q5G64_F16S,
           "q3g64": nq.NQ_W_Q3G64_F16S}[name]
    gs = 32 if name == "q8g32" else 64
    rows = []
    for (n, k) in ((W.FFN, W.HIDDEN), (W.HIDDEN, W.FFN)):
        rows += _grouped_shape_rows(nq, W, name, fmt, gs, n, k, torch)
    return rows


def _grouped_shape_rows(nq, W, name, fmt, gs, n, k, torch):
    dd = W.grouped(name, n, k)
    cd, sd = to_dev(dd["codes"]), to_dev(dd["scales"])
    cbytes = cd.numel()
    nxt = rotation(pack(nq, fmt, cd, n, k), sd)
    rows = []
    for t in (1, 8, 33):
        y = empty((t, n), torch.int16)
        xt = to_dev(W.activations(t, k, workload=4, tensor=50))
        ws = nq.alloc_gemv_workspace(fmt, t, n, k, DEV)

        def fn(t=t, xt=xt, y=y, ws=ws):
            cc, ss = nxt()
            nq.nq_gemv_qgroup_packed(fmt, cc, ss, xt, t, n, k, y, ws)
        rows.append(Row(f"gemv_{name}_{n}x{k}_T{t}", f"gemv_{name}", "GB/s",
                        cbytes + 2 * n * (k // gs) + 2 * t * k + 2 * t * n, fn,
                        wbytes=cbytes + 2 * n * (k // gs), tokens=t))
    return rows


def rows_a8_decode(nq, W):
    """A8 decode (int8 activations at decode sizes) beside the BF16-activation
    GEMV on the same packed weights: Q8 group-64 and Q4 group-64 at
    17408x5120 and 5120x17408, T = 1, 8, 33.  gemv_a8_*: the A8 GEMV on
    activations already quantized; linear_a8d_*: the routed decode step
    (quantization + A8 GEMV, row-major weights as the routed call takes
    them); gemv_bf16act_q8g64_*: the BF16-activation GEMV on the same Q8
    weights (the Q4 one is the gemv_q4g64 rows)."""
    torch = _torch()
    rows = []
    for name, fmt, bpw in (("q8g64", nq.NQ_W_Q8G64_F16S, 1.0), ("q4g64", nq.NQ_W_Q4G64_F16S, 0.5)):
        for (n, k) in ((W.FFN, W.HIDDEN), (W.HIDDEN, W.FFN)):
            dd = W.grouped(name, n, k)
            cd, sd = to_dev(dd["codes"]), to_dev(dd["scales"])
            wbytes = int(n * k * bpw) + 2 * n * (k // 64)
            nxt = rotation(pack(nq, fmt, cd, n, k), sd)
            nxt_rm = rotation(cd, sd)
            for t in (1, 8, 33):
                x = to_dev(W.activations(t, k, workload=4, tensor=50))
                qa, sa = empty((t, k), torch.int8), empty((t, k // 64), torch.float32)
                nq.nq_quantize_act_int8_g64(x, t, k, qa, sa)
                y = empty((t, n), torch.int16)
                wsa = nq.alloc_gemv_a8_workspace(t, n, k, DEV)
                abytes = t * k + 4 * t * (k // 64) + 2 * t * n

                def fa(t=t, qa=qa, sa=sa, y=y, wsa=wsa, n=n, k=k, fmt=fmt, nxt=nxt):
                    cc, ss = nxt()
                    nq.nq_gemv_a8_g64_packed(fmt, cc, ss, qa, sa, t, n, k, y, wsa)

                def fr(t=t, x=x, qa=qa, sa=sa, y=y, wsa=wsa, n=n, k=k, fmt=fmt, nxt_rm=nxt_rm):
                    cc, ss = nxt_rm()
                    if fmt == nq.NQ_W_Q8G64_F16S:
                        nq.nq_linear_q8g64(x, t, cc, ss, n, k, nq.NQ_A8_DECODE, qa, sa, y, wsa)
                    else:   # the decode route needs no widened copy of the Q4 codes
                        nq.nq_linear_q4g64(x, t, cc, ss, n, k, nq.NQ_A8_DECODE, qa, sa, None, y, wsa)
                rows.append(Row(f"gemv_a8_{name}_{n}x{k}_T{t}", "gemv_a8", "GB/s", wbytes + abytes, fa,
                                wbytes=wbytes, tokens=t))
                rows.append(Row(f"linear_a8d_{name}_{n}x{k}_T{t}", "quant_int8+gemv_a8", "GB/s",
                                wbytes + 2 * t * k + 2 * t * n, fr, wbytes=wbytes, tokens=t))
                if name == "q8g64":
                    wsb = nq.alloc_gemv_workspace(fmt, t, n, k, DEV)

                    def fb(t=t, x=x, y=y, wsb=wsb, n=n, k=k, fmt=fmt, nxt=nxt):
                        cc, ss = nxt()
                        nq.nq_gemv_qgroup_packed(fmt, cc, ss, x, t, n, k, y, wsb)
                    rows.append(Row(f"gemv_bf16act_{name}_{n}x{k}_T{t}", "gemv_q8g64", "GB/s",
                                    wbytes + 2 * t * k + 2 * t * n, fb, wbytes=wbytes, tokens=t))
    return rows


def rows_head(nq, W):
    n, k = W.HEAD_ROWS, W.HIDDEN
    q, s = _encode_bf16_on_gpu(nq, W.head_weights_bf16())
    x64 = to_dev(W.activations(64, k, workload=5, tensor=4))
    ts = list(range(1, 65))
    return _fp8row_gemv_rows(nq, "head", "gemv_head", q, s, [x64[:t].contiguous() for t in ts], ts,
                             rotate=False)


def rows_head_q8(nq, W):
    """The output head stored as Q8 group-32 instead of row-FP8 (same shape,
    packed, T = 1..64), for the FP8-versus-Q8 crossover: synthetic Q8G32
    codes and FP16 scales of the head's shape (the GEMV's time does not depend
    on the code values)."""
    torch = _torch()
    n, k = W.HEAD_ROWS, W.HIDDEN
    dd = W.grouped("q8g32", n, k, seed=7)
    fmt = nq.NQ_W_Q8G32_F16S
    cd, sd = to_dev(dd["codes"]), to_dev(dd["scales"])
    pk = pack(nq, fmt, cd, n, k)
    del cd
    x64 = to_dev(W.activations(64, k, workload=5, tensor=4))
    rows = []
    for t in range(1, 65):
        xt = x64[:t].contiguous()
        y = empty((t, n), torch.int16)
        ws = nq.alloc_gemv_workspace(fmt, t, n, k, DEV)
        rows.append(Row(f"head_q8g32_T{t}", "gemv_head_q8g32", "GB/s",
                        n * k + 2 * n * (k // 32) + 2 * t * k + 2 * t * n,
                        lambda t=t, xt=xt, y=y, ws=ws: nq.nq_gemv_qgroup_packed(fmt, pk, sd, xt, t, n, k, y, ws),
                        wbytes=n * k + 2 * n * (k // 32), tokens=t))
    return rows


def rows_prefill(nq, W, want_quant, want_w8a8, want_fp8):
    torch = _torch()
    d = W.w8a8_prefill()
    m, k = d["x"].shape
    n = d["w"].shape[0]
    x = to_dev(d["x"])
    qa, sa = empty((m, k), torch.int8), empty((m, k // 64), torch.float32)
    nq.nq_quantize_act_int8_g64(x, m, k, qa, sa)
    rows = []
    if want_quant:
        rows.append(Row("quant_int8", "quant_int8", "GB/s", 2 * m * k + m * k + 4 * m * (k // 64),
                        lambda: nq.nq_quantize_act_int8_g64(x, m, k, qa, sa)))
    if want_w8a8:
        w, ws = to_dev(d["w"]), to_dev(d["w_scale"])
        y = empty((m, n), torch.float32)
        rows.append(Row("gemm_w8a8", "gemm_w8a8", "TOPS", 2 * m * n * k,
                        lambda: nq.nq_gemm_w8a8_g64(qa, sa, w, ws, m, n, k, y)))
    if want_fp8:
        rows.append(_fp8_gemm_row(nq, W, m, n, k))
    return rows


def rows_q4_a8(nq, W):
    """Q4 group-64 weights on the A8 route at the prefill chunk (1792 x 17408 x
    5120): the codes widened to int8, and the routed projection (activation
    quantization + widening + W8A8 GEMM)."""
    torch = _torch()
    d = W.grouped("q4g64", W.FFN, W.HIDDEN)
    n, k = W.FFN, W.HIDDEN
    m = W.PREFILL_CHUNK
    wc, ws = to_dev(d["codes"]), to_dev(d["scales"])
    x = to_dev(W.w8a8_prefill()["x"])
    aq, asc = empty((m, k), torch.int8), empty((m, k // 64), torch.float32)
    wi8 = empty((n, k), torch.int8)
    y = empty((m, n), torch.float32)
    return [Row("unpack_q4", "unpack_q4", "GB/s", n * k // 2 + n * k,
                lambda: nq.nq_unpack_q4_to_int8(wc, n, k, wi8)),
            Row("linear_q4g64_a8", "linear_q4g64_a8", "TOPS", 2 * m * n * k,
                lambda: nq.nq_linear_q4g64(x, m, wc, ws, n, k, True, aq, asc, wi8, y))]


def rows_qbits_a8(nq, W, name):
    """Q5 / Q3 group-64 weights on the A8 route at the prefill chunk (1792 x
    17408 x 5120): the codes widened to int8, and the routed projection
    (quantize + widen + W8A8 GEMM)."""
    torch = _torch()
    fmt, bits = {"q5g64": (nq.NQ_W_Q5G64_F16S, 5), "q3g64": (nq.NQ_W_Q3G64_F16S, 3)}[name]
    n, k, m = W.FFN, W.HIDDEN, W.PREFILL_CHUNK
    d = W.grouped(name, n, k)
    wc, ws = to_dev(d["codes"]), to_dev(d["scales"])
    x = to_dev(W.w8a8_prefill(n=64)["x"])
    aq, asc = empty((m, k), torch.int8), empty((m, k // 64), torch.float32)
    wi8 = empty((n, k), torch.int8)
    y = empty((m, n), torch.float32)
    return [Row(f"unpack_{name}", f"unpack_{name}", "GB/s", n * k * bits // 8 + n * k,
                lambda: nq.nq_unpack_qbits_to_int8(fmt, wc, n, k, wi8)),
            Row(f"linear_{name}_a8", f"linear_{name}_a8", "TOPS", 2 * m * n * k,
                lambda: nq.nq_linear_qbits_g64(fmt, x, m, wc, ws, n, k, nq.NQ_A8_PREFILL, aq, asc, wi8, y))]


def _fp8_gemm_row(nq, W, m, n, k):
    torch = _torch()
    q, s = _encode_bf16_on_gpu(nq, W.fp8row_weights_bf16(n, k))
    xf = to_dev(W.activations(m, k, workload=5, tensor=6))
    ac, asc = empty((m, k), torch.uint8), empty((m,), torch.float32)
    yf = empty((m, n), torch.float32)
    return Row("gemm_fp8", "gemm_fp8", "TFLOP/s", 2 * m * n * k,
               lambda: nq.nq_gemm_fp8row(xf, q, s, m, n, k, ac, asc, yf))


def build_rows(selected):
    from quantized_weight_linear_amd import nq
    from quantized_weight_linear_amd import workloads as W

    groups = None if selected == "all" else set(selected.split(","))

    def want(name):
        return groups is None or name in groups

    # Order within a step: prefill and conversion work first, decode work
    # after it, as in an engine step.  Kernels that write large outputs (the
    # GEMMs' 125 MB, the re-encode's 89 MB) leave dirty lines in the
    # memory-side cache, and the next kernel pays for writing them back
    # (a decode GEMV measured right after a 256 MiB fill runs ~16 us slower),
    # so the decode rows follow other decode rows, whose outputs are small.
    rows = []
    if want("quant_int8") or want("gemm_w8a8") or want("gemm_fp8"):
        rows += rows_prefill(nq, W, want("quant_int8"), want("gemm_w8a8"), want("gemm_fp8"))
    if want("q4_a8"):
        rows += rows_q4_a8(nq, W)
    for name in ("q5g64", "q3g64"):
        if want(f"{name}_a8"):
            rows += rows_qbits_a8(nq, W, name)
    if want("reencode") or want("gemv_down"):
        rows += rows_reencode_and_down(nq, W, want("reencode"), want("gemv_down"))
    if want("decode_mxfp8"):
        rows += rows_mxfp8(nq, W)
    if want("decode_mlx"):
        rows += rows_mlx(nq, W)
    if want("head"):
        rows += rows_head(nq, W)
    if want("head_q8"):
        rows += rows_head_q8(nq, W)
    for name in ("q4g64", "q8g32", "q5g64", "q3g64"):
        if want(f"gemv_{name}"):
            rows += rows_grouped(nq, W, name)
    if want("a8_decode"):
        rows += rows_a8_decode(nq, W)
    if want("gemv_fp8row"):
        rows += rows_gemv_fp8row(nq, W)
    if want("hbm_read"):
        rows += rows_hbm_read(nq)
    _torch().cuda.synchronize()
    return rows


def _blas_threads():
    try:
        import threadpoolctl
        return max((p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()), default=1)
    except Exception:
        return None


def cpu_baseline():
    """The oracle (as it stands) timed on the host cores, once per (config, T):
    the headline row-FP8 GEMV on the full 17408x5120 weight (`value`), and the
    other configs on bounded row samples (stated per entry), as weight-bytes/s
    (GB/s), tokens/s or ops/s.  Weight encoding and input generation are not
    timed.  Elementwise numpy runs on one core, float64 matmuls on the BLAS
    threads."""
    from oracle import method as M
    from quantized_weight_linear_amd import workloads as W

    out = {}

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    def gemv_entry(key, sec, wbytes, t, xy_bytes):
        out[f"{key}_GBps"] = round((wbytes + xy_bytes) / sec / 1e9, 4)
        out[f"{key}_weight_GBps"] = round(wbytes / sec / 1e9, 4)
        out[f"{key}_tok_s"] = round(t / sec, 2)

    # config 2 (the headline): full weight, T = 1, 4, 16, 33 (the weight's
    # encode is setup: run on row bands in threads, not timed)
    n, k = W.FFN, W.HIDDEN
    w2 = W.fp8row_weights_bf16(n, k)
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(min(16, len(os.sched_getaffinity(0)))) as ex:
        parts = list(ex.map(lambda r0: M.encode_fp8row_bf16(w2[r0:r0 + 512]), range(0, n, 512)))
    wq, ws = np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])
    del w2, parts
    x33 = W.activations(33, k)
    total_bytes, total_s = 0, 0.0
    for t in (1, 4, 16, 33):
        sec = timed(lambda: M.gemv_fp8row(wq, ws, x33[:t]))
        total_s += sec
        total_bytes += n * k + 2 * n + 2 * t * k + 2 * t * n
        gemv_entry(f"cfg2_fp8row_17408x5120_T{t}", sec, n * k + 2 * n, t, 2 * t * k + 2 * t * n)
    del wq, ws
    # config 1: MXFP8 256x512, T = 1
    d1 = W.mxfp8_gemv()
    out["cfg1_mxfp8_gemv_256x512_us"] = round(timed(lambda: M.gemv_qgroup("mxfp8", d1["words"], d1["e8m0"],
                                                                            d1["x"])) * 1e6, 1)
    # config 3: re-encode and down projection on 512 of the 5120 rows; the gate whole
    d3 = W.block128_codes()
    r3 = 512
    c3, w3 = d3["codes"][:r3], d3["wsi"][:r3 // 128]
    k3 = c3.shape[1]
    res = {}
    sec = timed(lambda: res.update(q=M.reencode_block128_to_row(c3, w3)))
    out["cfg3_reencode_512x17408_GBps"] = round((2 * r3 * k3 + 4 * w3.size + 2 * r3) / sec / 1e9, 4)
    q3, s3 = res["q"]
    for t in (1, 33):
        x = W.activations(t, k3, workload=3, tensor=3)
        sec = timed(lambda: M.gemv_fp8row(q3, s3, x))
        gemv_entry(f"cfg3_down_512x17408_T{t}", sec, r3 * k3 + 2 * r3, t, 2 * t * k3 + 2 * t * r3)
    gate = W.gate_bf16()
    for t in (1, 33):
        x = W.activations(t, W.HIDDEN, workload=3, tensor=4)
        sec = timed(lambda: M.gemv_qgroup("bf16", gate, None, x))
        gemv_entry(f"cfg3_gate_96x5120_T{t}", sec, 2 * gate.size, t, 2 * t * W.HIDDEN + 2 * t * 96)
    # config 4: Q4 group-64 / Q8 group-32 on 1024-row samples of both shapes
    for name, gs, bpw in (("q4g64", 64, 0.5), ("q8g32", 32, 1.0)):
        for (n4, k4) in ((W.FFN, W.HIDDEN), (W.HIDDEN, W.FFN)):
            r4 = 1024
            d4 = W.grouped(name, r4, k4)             # the first 1024 rows of the n4 x k4 matrix
            c4, s4 = d4["codes"], d4["scales"]
            wbytes = int(r4 * k4 * bpw) + 2 * r4 * (k4 // gs)
            for t in (1, 8, 33):
                x = W.activations(t, k4, workload=4, tensor=50)
                sec = timed(lambda: M.gemv_qgroup(name, c4, s4, x))
                gemv_entry(f"cfg4_{name}_{r4}of{n4}x{k4}_T{t}", sec, wbytes, t, 2 * t * k4 + 2 * t * r4)
    # config 5: int8 quantization of the whole chunk; W8A8 and FP8 GEMMs on
    # 1024 and 512 output columns of the chunk; the head at T = 1 on 4096 rows
    c5 = 1024
    d5 = W.w8a8_prefill(n=c5)                      # the whole chunk; the first 1024 weight rows
    m5, k5 = d5["x"].shape
    res = {}
    sec = timed(lambda: res.update(q=M.quantize_act_int8_g64(d5["x"])))
    out["cfg5_quant_int8_1792x5120_GBps"] = round((2 * m5 * k5 + m5 * k5 + 4 * m5 * (k5 // 64)) / sec / 1e9, 4)
    qa, sa = res["q"]
    sec = timed(lambda: M.gemm_w8a8_g64(qa, sa, d5["w"], d5["w_scale"]))
    out["cfg5_w8a8_1792x1024x5120_GOPS"] = round(2 * m5 * c5 * k5 / sec / 1e9, 3)
    wf = W.fp8row_weights_bf16(512, k5)
    wfq, wfs = M.encode_fp8row_bf16(wf)
    xf = W.activations(m5, k5, workload=5, tensor=6)
    sec = timed(lambda: M.gemm_fp8row(xf, wfq, wfs))
    out["cfg5_fp8_gemm_1792x512x5120_GFLOPS"] = round(2 * m5 * 512 * k5 / sec / 1e9, 3)
    hw = W.head_weights_bf16(n=4096)               # the first 4096 rows of the head
    hq, hs = M.encode_fp8row_bf16(hw)
    xh = W.activations(1, k5, workload=5, tensor=4)
    sec = timed(lambda: M.gemv_fp8row(hq, hs, xh))
    gemv_entry("cfg5_head_4096of152064x5120_T1", sec, 4096 * k5 + 2 * 4096, 1, 2 * k5 + 2 * 4096)

    line = {"value": round(total_bytes / total_s / 1e9, 3), "unit": "GB/s",
            "cores": len(os.sched_getaffinity(0)), "blas_threads": _blas_threads(), "kind": "oracle",
            "sample": "value: oracle decode GEMV (numpy float64) on the full row-FP8 17408x5120 weight, "
                      "T = 1, 4, 16, 33 once each (encode not timed); other keys: per (config, T) on the "
                      "row / column samples their names give"}
    line.update(out)
    return line


def gemv_source_hash():
    """sha256 prefix of the GEMV sources' code: comments and whitespace are
    dropped first, so that only a change of code invalidates the counters."""
    import hashlib
    import re
    h = hashlib.sha256()
    for name in GEMV_SOURCES:
        with open(os.path.join(ROOT, "quantized_weight_linear_amd", "csrc", name)) as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def gemv_traffic(names):
    """Measured HBM bytes per launch of the headline GEMV, or None when the
    kernel source changed since the counters were taken."""
    sha = gemv_source_hash()
    t = GEMV_TRAFFIC
    if sha != t["source_sha256_16"] or any(n not in t["fetch_kib"] for n in names):
        return None
    return {n: round(1024 * (t["fetch_kib"][n] * t["fetch_factor"] + t["write_kib"][n] * t["write_factor"]))
            for n in names}


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU; --gpus must be 1 (the path would shard "
                                   "along the output rows, with an all-gather of the outputs)"}))
        sys.exit(2)
    torch = _torch()
    from quantized_weight_linear_amd import nq
    nq.lib()
    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    t_setup = time.perf_counter()
    rows = build_rows(args.rows)
    log(f"setup {time.perf_counter() - t_setup:.1f}s, {len(rows)} launches per step")

    stream = torch.cuda.current_stream()
    enqueue_s = 0.0
    for i in range(max(1, args.warmup)):
        t0 = time.perf_counter()
        for r in rows:
            for _ in range(args.burst):
                r.fn()
        enqueue_s = max(enqueue_s, time.perf_counter() - t0)
        torch.cuda.synchronize()
        log(f"warmup step {i + 1}/{args.warmup} done (host enqueue {enqueue_s * 1e3:.1f} ms)")

    # The host needs longer to enqueue a launch than short kernels take to run,
    # so a spin kernel first holds the stream while the whole timed region is
    # enqueued; the events then see back-to-back kernels, not host latency.
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    torch.cuda._sleep(1 << 20)
    b.record(stream)
    torch.cuda.synchronize()
    cycles_per_ms = (1 << 20) / max(a.elapsed_time(b), 1e-3)
    hold_ms = 1.5 * enqueue_s * 1e3 * args.steps + 20.0

    events, steps_ev = [], []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    torch.cuda._sleep(int(hold_ms * cycles_per_ms))
    for _ in range(args.steps):
        s0 = torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        for r in rows:
            # a burst of launches between one pair of events: no event packet
            # sits between two launches, so the per-launch time is the
            # kernel's own duration plus the dispatch gap, as in a model's
            # back-to-back layers
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(args.burst):
                r.fn()
            b.record(stream)
            events.append((r, a, b))
        s1 = torch.cuda.Event(enable_timing=True)
        s1.record(stream)
        steps_ev.append((s0, s1))
    enq = time.perf_counter() - t0
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for r, a, b in events:
        r.ms.append(a.elapsed_time(b) / args.burst)
    gpu_step_ms = float(np.mean([s0.elapsed_time(s1) for s0, s1 in steps_ev]))
    log(f"timed {args.steps} steps: GPU {gpu_step_ms:.3f} ms/step, wall {wall:.3f}s "
        f"(enqueue {enq * 1e3:.1f} ms, hold {hold_ms:.1f} ms)")

    results = {}
    for r in rows:
        ms = float(np.mean(r.ms))
        if r.unit == "GB/s":
            rate = r.work / (ms * 1e-3) / 1e9
            frac = rate / HBM_PEAK_GBS
        else:
            rate = r.work / (ms * 1e-3) / 1e12
            frac = rate / (INT8_PEAK_TOPS if r.unit == "TOPS" else FP8_PEAK_TFLOPS)
        results[r.name] = {"kernel": r.kernel, "us": round(ms * 1e3, 3), "rate": round(rate, 2),
                           "unit": r.unit, "frac": round(frac, 4), "work": r.work}

    head = [r for r in rows if r.name.startswith("gemv_fp8row_T")]
    line = {"metric": "decode GEMV HBM GB/s (% peak) at T=1..33; prefill GEMM TOPS (% MFMA peak) at T=1792",
            "value": None, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(gpu_step_ms, 3), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "fp8(e4m3) weights x bf16 activations, fp32 accumulate",
            "data": "synthetic",
            "config": {"workload": "row-FP8 decode GEMV 17408x5120 (FFN up/gate), T=1,4,16,33, BF16 out; "
                                   "one step = every hot-path row once",
                       "T": "1,4,16,33", "N": 17408, "K": 5120}}
    if head:
        byt = sum(r.work * len(r.ms) for r in head)
        sec = sum(sum(r.ms) * 1e-3 for r in head)
        gbs = byt / sec / 1e9
        line["value"] = round(gbs, 2)
        per_launch = gemv_traffic([r.name for r in head])
        traffic = None
        if per_launch is not None:
            # whole-job HBM bytes per launch, averaged like `achieved`
            traffic = round(sum(per_launch[r.name] * len(r.ms) for r in head) / sum(len(r.ms) for r in head))
        roof = {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "gemv_mfma_kernel (one token block at T=1,4,16, three at T=33), packed row-FP8 17408x5120"}
        for r in head:
            roof[f"us_{r.name.split('_')[-1]}"] = results[r.name]["us"]
            roof[f"bytes_{r.name.split('_')[-1]}"] = r.work
            if per_launch is not None:
                roof[f"traffic_{r.name.split('_')[-1]}"] = per_launch[r.name]
        if "hbm_read_89MB" in results:
            ceil = results["hbm_read_89MB"]["rate"]
            roof["hbm_read_ceiling_89MB_GBps"] = ceil
            roof["frac_of_read_ceiling"] = round(gbs / ceil, 4)
        if "hbm_read_1GiB" in results:
            roof["hbm_read_ceiling_1GiB_GBps"] = results["hbm_read_1GiB"]["rate"]
        line["roofline"] = roof
    # prefill GEMMs (flat, so record parsers keep every figure)
    pre = {}
    for name, key, peak_name in (("gemm_w8a8", "w8a8", "int8"), ("gemm_fp8", "fp8", "fp8"),
                                 ("linear_q4g64_a8", "q4_a8_routed", "int8"),
                                 ("linear_q5g64_a8", "q5_a8_routed", "int8"),
                                 ("linear_q3g64_a8", "q3_a8_routed", "int8")):
        if name in results:
            v = results[name]
            pre[f"{key}_us"] = v["us"]
            pre[f"{key}_{'TFLOPS' if name == 'gemm_fp8' else 'TOPS'}"] = v["rate"]
            pre[f"{key}_frac_{peak_name}_peak"] = v["frac"]
    if "gemm_fp8" in results:
        pre["fp8_frac_bf16_peak"] = round(results["gemm_fp8"]["rate"] / (FP8_PEAK_TFLOPS / 2), 4)
    if pre:
        pre.update({"M": 1792, "N": 17408, "K": 5120})
        line["prefill"] = pre
    if "gemm_w8a8" in results:
        v = results["gemm_w8a8"]
        line["roofline_prefill"] = {"bound": "mfma", "achieved": v["rate"], "peak": INT8_PEAK_TOPS, "unit": "TOP/s",
                                    "frac": v["frac"], "us": v["us"],
                                    "kernel": "gemm_kernel<W8A8> (v_mfma_i32_32x32x32_i8, FP32 per-group rescale), "
                                              "M=1792 N=17408 K=5120"}
    cross = [t for t in range(1, 65) if f"head_T{t}" in results and f"head_q8g32_T{t}" in results]
    if cross:
        q8_faster = [t for t in cross if results[f"head_q8g32_T{t}"]["us"] < results[f"head_T{t}"]["us"]]
        line["head_fp8_vs_q8"] = {
            "shape": "152064x5120", "T": [cross[0], cross[-1]],
            "q8g32_faster_at_T": q8_faster,
            "fp8_us": [results[f"head_T{t}"]["us"] for t in cross],
            "q8g32_us": [results[f"head_q8g32_T{t}"]["us"] for t in cross]}
    a8 = {}
    for name in ("q8g64", "q4g64"):
        for shape in ("17408x5120", "5120x17408"):
            for t in (1, 8, 33):
                ka, kb = f"linear_a8d_{name}_{shape}_T{t}", (f"gemv_bf16act_{name}_{shape}_T{t}" if name == "q8g64"
                                                             else f"gemv_{name}_{shape}_T{t}")
                if ka in results and kb in results:
                    a8[f"{name}_{shape}_T{t}_a8_us"] = results[ka]["us"]
                    a8[f"{name}_{shape}_T{t}_bf16act_us"] = results[kb]["us"]
    if a8:
        line["a8_decode_vs_bf16act"] = a8
    # every row: [us, rate, fraction of its peak]; decode rows also
    # [weight GB/s, tokens/s] per layer shape
    line["rows"] = {k: [v["us"], v["rate"], v["frac"]] for k, v in results.items()}
    line["decode_per_shape"] = {r.name: [round(r.wbytes / (results[r.name]["us"] * 1e-6) / 1e9, 1),
                                         round(r.tokens / (results[r.name]["us"] * 1e-6), 1)]
                                for r in rows if r.wbytes is not None}
    line["timing"] = {"ms_per_step_gpu_events": round(gpu_step_ms, 3), "wall_s_timed_region": round(wall, 3),
                      "note": "timed region starts with a spin kernel that holds the stream while the host "
                              "enqueues all launches; per-launch times are HIP events on that stream"}
    if not args.no_cpu_baseline and head:
        log("cpu baseline (oracle) ...")
        line["cpu_baseline"] = cpu_baseline()
    if args.rows_json:
        with open(args.rows_json, "w") as f:
            json.dump(results, f, indent=1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
