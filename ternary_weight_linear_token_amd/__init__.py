"""MI355X (gfx950) BitNet b1.58 W2A8 BitLinear matmul.

A thin Python binding over the C ABI of libbitnet_w2a8.so (include/bitnet_w2a8.h):
argument checking and marshalling only.  Every step of the computation runs in the
library's HIP kernels; torch is used for device memory and the current stream.  There
is no CPU fallback: if the library cannot be loaded, or a call fails, an exception is
raised.
"""
from ._binding import (  # noqa: F401
    ALGO_AUTO,
    ALGO_SKINNY,
    ALGO_TILED,
    GEMV_MAX_M,
    MAX_GROUPS,
    OUT_BF16,
    OUT_F32,
    OUT_I32,
    SKINNY_MAX_M,
    BitnetError,
    a16_gemv,
    abi_version,
    bitlinear,
    gemm,
    gemm_grouped,
    gemm_noalloc,
    b3_row_bytes,
    pack_b3,
    quant_gemv_b3,
    gemm_plan,
    gemv,
    lib,
    library_path,
    pack_weights,
    quant_act,
    quant_act_per_tensor,
    quant_gemv,
    quant_gemv_grouped,
    quant_gemv_swiglu,
    status_str,
    unpack_weights,
    repack_codes,
    CODES_OFFSET,
    CODES_SIGN,
)
