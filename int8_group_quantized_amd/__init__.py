"""MI355X-native weight-only group-quantized GEMM (W4A16 / W8A16, bf16 or
fp16 activations), the fixed-grid packer Q_s, dense dequantization, the
fixed-grid fake quantizer, and the drafter's sliding-window attention.

The computation lives in libqgemm.so (hand-written HIP for gfx950, C ABI in
include/qgemm.h); this package holds its sources, the build step and a thin
ctypes binding.
"""

from .binding import (  # noqa: F401
    QGError, lib, library_path, packed_bytes, workspace_bytes, rtn_scales,
    pack_to_grid, pack_to_grid_w4, pack_to_grid_w8, prepack, unpack, qgemm,
    qgemm_w4a16, qgemm_w8a16, dequant, fake_quant, FakeQuantSTE, qgemm_grouped,
    swa_attention, read_stream, READ_PROBE_MARK, prepack_scales, grouped_workspace_bytes,
    check_weight,
)
