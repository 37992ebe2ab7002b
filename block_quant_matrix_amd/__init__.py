"""Block-quantized (GGML Q8_0 / Q4_0) decode-path kernels for AMD MI355X (gfx950).

The compute lives in ``libzq.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/zq.h``).  ``block_quant_matrix_amd.zq`` is the thin
ctypes binding; ``block_quant_matrix_amd.inputs`` draws the seeded inputs.
"""
