"""The GEMV entry point that allocates nothing (static per-GPU scratch) against
the same call with a caller workspace, through the C ABI."""

import numpy as np
import pytest
import torch

from oracle import method as M
from quantized_weight_linear_amd import nq
from quantized_weight_linear_amd import workloads as W

DEV = "cuda"


def _dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def _packed_weights(n, k, seed):
    w = W.fp8row_weights_bf16(n, k, seed=seed)
    q = torch.empty((n, k), dtype=torch.uint8, device=DEV)
    s = torch.empty((n,), dtype=torch.int16, device=DEV)
    nq.nq_encode_fp8row_bf16(_dev(w), n, k, q, s)
    pk = torch.empty((nq.nq_packed_weight_bytes(-1, n, k),), dtype=torch.uint8, device=DEV)
    nq.nq_pack_weights(-1, q, n, k, pk)
    return w, pk, s


@pytest.mark.gpu
def test_noalloc_equals_workspace_call_twice():
    """Two calls in a row, the second smaller: 17408 x 5120 at T = 33 (spread
    workgroups exchange partials in the scratch), then 4096 x 4096 at T = 16
    (K split over workgroups, fewer counters), each bit-identical to
    nq_gemv_fp8row_packed with a zero-filled workspace, in FP32 and BF16, and
    within 1e-5 of the oracle on sampled rows."""
    for (n, k, t, seed) in [(W.FFN, W.HIDDEN, 33, 40), (4096, 4096, 16, 41)]:
        print(f"[gpu] noalloc n={n} k={k} t={t}", flush=True)
        assert 0 < nq.nq_gemv_workspace_bytes(-1, t, n, k) <= nq.NQ_GEMV_STATIC_SCRATCH_BYTES
        w, pk, s = _packed_weights(n, k, seed)
        x = W.activations(t, k, seed=seed)
        xd = _dev(x)
        for dt in (torch.float32, torch.int16):
            y_ref = torch.empty((t, n), dtype=dt, device=DEV)
            y_na = torch.full((t, n), -1, dtype=dt, device=DEV)
            nq.nq_gemv_fp8row_packed(pk, s, xd, t, n, k, y_ref, nq.alloc_gemv_workspace(-1, t, n, k, DEV))
            nq.nq_gemv_fp8row_packed_noalloc(pk, s, xd, t, n, k, y_na)
            torch.cuda.synchronize()
            assert torch.equal(y_ref, y_na), (n, k, t, dt)
        rows = np.unique(np.concatenate([[0, n - 1], np.arange(max(0, n - 1024), n, 7),
                                         W.rng(130, seed).integers(0, n, 64)]))
        qo, so = M.encode_fp8row_bf16(w[rows])
        ref = M.gemv_fp8row(qo, so, x)
        y32 = torch.empty((t, n), dtype=torch.float32, device=DEV)
        nq.nq_gemv_fp8row_packed_noalloc(pk, s, xd, t, n, k, y32)
        got = y32.cpu().numpy()[:, rows].astype(np.float64)
        err = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        assert err <= 1e-5, err


def test_noalloc_rejects_plans_beyond_the_scratch():
    """A call whose plan needs more than the static array is rejected before
    anything is enqueued (host-side check: no GPU needed)."""
    L = nq.lib()
    t, n, k = 64, 15360, 16384
    assert nq.nq_gemv_workspace_bytes(-1, t, n, k) > nq.NQ_GEMV_STATIC_SCRATCH_BYTES
    a = 0x10000
    assert L.nq_gemv_fp8row_packed_noalloc(a, a, a, t, n, k, 0, a, None) == nq.NQ_ERR_SCRATCH
    assert L.nq_status_string(nq.NQ_ERR_SCRATCH) != b"unknown status"
    assert L.nq_gemv_fp8row_packed_noalloc(a, a, a, 1, 64, 200, 0, a, None) == nq.NQ_ERR_SHAPE   # K % 256
    assert L.nq_gemv_fp8row_packed_noalloc(None, a, a, 1, 64, 256, 0, a, None) == nq.NQ_ERR_NULL
    assert L.nq_gemv_fp8row_packed_noalloc(a, a, a, 1, 64, 256, 0, 0x10001, None) == nq.NQ_ERR_ALIGN
