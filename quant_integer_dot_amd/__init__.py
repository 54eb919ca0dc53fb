"""qdot: integer-dot block-quantized matmul for AMD MI355X (gfx950).

The compute runs in hand-written HIP kernels behind a C ABI (``libqdot.so``,
declared in ``include/qdot.h``).  ``binding`` is a thin ctypes layer with the
same names; the library is loaded on first use and its absence is an error.
"""
from .binding import (  # noqa: F401
    QDOT_Q4_K, QDOT_Q6_K, QDOT_IQ4_XS,
    QDOT_OK, QDOT_E_ARG, QDOT_E_ALIGN, QDOT_E_HIP,
    QdotError, library_path, load,
    qdot_block_bytes, qdot_weight_bytes, qdot_q8_1_bytes, qdot_isum_count,
    qdot_quantize_q8_1, qdot_qmatmul, qdot_qmatmul_dump_isums,
    qdot_status_str, qdot_kernel_name, qdot_build_id,
)
