"""MI355X (gfx950) per-token / per-group FP8 E4M3 / FP4 E2M1 activation cast.

The product path is the HIP library ``libtk_quant.so`` (C ABI in
``include/tk_quant.h``) and the thin ctypes binding in ``binding.py``.  Build
the library with ``python -m activation_quantization_token_amd.build``.
"""
from .binding import (  # noqa: F401
    GROUPS,
    QDTYPES,
    OUT_DTYPES,
    SCALE_FMTS,
    TkError,
    copy_stream,
    empty_outputs,
    load_library,
    per_block_cast,
    per_channel_cast,
    per_token_cast,
    per_token_cast_back,
    per_token_dequant,
    rmsnorm,
    rmsnorm_cast,
    silu32_bf16,
    stream_rw,
    swiglu_per_token_cast,
    tk_abi_version,
    tk_copy_stream,
    tk_per_block_cast,
    tk_per_channel_cast,
    tk_per_channel_workspace_bytes,
    tk_per_token_cast,
    tk_per_token_cast_f32,
    tk_per_token_cast_back,
    tk_per_token_dequant,
    tk_prepare_device,
    tk_rmsnorm,
    tk_rmsnorm_cast,
    tk_silu32_bf16,
    tk_stream_rw,
    tk_status_string,
    tk_swiglu_per_token_cast,
)
