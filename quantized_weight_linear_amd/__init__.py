"""Quantized-weight linear projection for AMD MI355X (gfx950).

The product is libnq.so, a C-ABI library of HIP kernels (headers in
``include/nq.h``); ``quantized_weight_linear_amd.nq`` is its ctypes binding
and ``quantized_weight_linear_amd.workloads`` draws seeded synthetic inputs.
Build with ``python -m quantized_weight_linear_amd.build``.
"""
