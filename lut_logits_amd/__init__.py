"""lut_logits_amd -- residual product-quantized (RQ) LUT serving on MI355X (gfx950).

The compute lives in librq_lut.so (hand-written HIP kernels behind the C ABI
of include/rq_lut.h); `binding` marshals torch tensors into those calls.
`synth` draws seeded synthetic inputs; `formats` holds the storage
accounting.
"""
from . import formats, synth  # noqa: F401
from .binding import (RQ_BF16, RQ_CODES_BLOCKED, RQ_CODES_PACKED8, RQ_CODES_PACKED10, RQ_CODES_ROWS, RQ_F32, RQ_METHOD_MATRIX_CORES, RQ_METHOD_TABLE,
                      RQ_PRO_GELU_TANH_MUL,  # noqa: F401
                      RQ_PRO_NONE, DenseHead, DeviceMatrix, RQError, build_lut, logits, logits_method, logits_workspace, decode_rows, dense_logits, dense_logits_workspace, dense_tiled_bytes, pack_dense, stream_read, stream_read_configs, lds_gather, lib,
                      lut_bytes, lut_logits_plan, lut_logits_static, residual_norm,
                      lut_logits, lut_logits_workspace, lut_matvec, lut_matvec_workspace, lut_mlp, lut_mlp_workspace, pack_codes, pack_codes8, pack_codes10, packed8_codes_bytes, packed10_codes_bytes,
                      set_stage_events,
                      to_device, workspace)

__version__ = "0.1.0"
