"""MI355X-native Sketch Attention (SequenceO1) compression.

The computation lives in libsa.so (hand-written HIP for gfx950, C ABI in
include/sa.h); this package is its thin Python binding.
"""
from ._lib import (  # noqa: F401
    SA_BF16,
    SA_DEVICE_ERR_EXCHANGE,
    SA_DEVICE_ERR_OFFSETS,
    SA_DEVICE_ERR_RANGE,
    SA_DEVICE_ERR_SKETCH_ROW,
    SA_E_HIP,
    SA_E_INVALID,
    SA_E_UNSUPPORTED,
    SA_E_WORKSPACE,
    SA_F32,
    SA_FLAG_ONE_PASS,
    SA_FLAG_TWO_PASS,
    SA_OK,
    SaError,
    SketchCache,
    backward_workspace_size,
    compress,
    compress_backward,
    target_attention,
    target_attention_workspace_size,
    load,
    read_device_error,
    status_string,
    version,
    workspace_size,
)

__all__ = [
    "SketchCache",
    "compress", "compress_backward", "backward_workspace_size", "target_attention",
    "target_attention_workspace_size", "load", "read_device_error", "status_string", "version", "workspace_size",
    "SaError", "SA_OK", "SA_E_INVALID", "SA_E_UNSUPPORTED", "SA_E_WORKSPACE", "SA_E_HIP",
    "SA_BF16", "SA_F32", "SA_FLAG_ONE_PASS", "SA_FLAG_TWO_PASS", "SA_DEVICE_ERR_OFFSETS", "SA_DEVICE_ERR_RANGE", "SA_DEVICE_ERR_SKETCH_ROW",
    "SA_DEVICE_ERR_EXCHANGE",
]
