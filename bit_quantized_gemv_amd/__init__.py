"""MI355X (gfx950) affine group-quantized matrix-vector product (qmv), with an
mxfp4 mode.

The compute path is the HIP library ``lib/libqmv.so`` (C ABI in
``include/qmv.h``); ``qmv.py`` only marshals torch tensors into it.
"""
from .qmv import (QmvError, affine, affine_ptr, kernel_info, status_string, library_path, lib,
                  stream_read_ptr, stream_read_ex_ptr, mxfp4, mxfp4_ptr, timeline, timeline_ptr,
                  shape_ptr, KernelInfo, TimelineInfo, STAMPS, DT_F32, DT_F16, DT_BF16, MAX_M)

__all__ = ["QmvError", "affine", "affine_ptr", "kernel_info", "status_string", "library_path", "lib",
           "stream_read_ptr", "stream_read_ex_ptr", "mxfp4", "mxfp4_ptr", "timeline", "timeline_ptr",
           "shape_ptr", "KernelInfo", "TimelineInfo", "STAMPS", "DT_F32", "DT_F16", "DT_BF16", "MAX_M"]
