"""MXFP4 MoE expert layer for MI355X (gfx950).

The layer itself is hand-written HIP in ``csrc/`` behind the C ABI of
``include/moe_mxfp4.h``, built into ``libmoe_mxfp4.so`` by ``build.py``.
``_lib`` is the ctypes binding (same names as the C ABI); ``layer`` builds a
device-resident synthetic layer for tests and benchmarks.
"""
from ._lib import (MOE_ACT_BF16, MOE_ACT_MXFP8, MOE_DT_BF16, MOE_DT_F32, MOE_DT_I32, MOE_DT_U8,
                   MOE_E_ALIGN, MOE_E_DTYPE, MOE_E_HIP, MOE_E_LIMIT,
                   MOE_E_NOT_INIT, MOE_E_NULL, MOE_E_OPTION, MOE_E_SHAPE, MOE_E_TOKENS, MOE_E_TOPK,
                   MOE_OK,
                   MOE_LAUNCH_AUTO, MOE_LAUNCH_FUSED, MOE_LAUNCH_QUEUE, MOE_LAUNCH_SELF_ROUTED,
                   MOE_LAUNCH_SPLIT,
                   MOE_LAYOUT_ROWS, MOE_LAYOUT_TILES, MOE_PATH_AUTO, MOE_PATH_GEMV,
                   MOE_PATH_MFMA, MoeError, lib, moe_mxfp4_prepack,
                   moe_mxfp4_finalize, moe_mxfp4_forward, moe_mxfp4_forward_ex,
                   moe_mxfp4_forward_noalloc, moe_mxfp4_forward_t, moe_mxfp4_init, moe_tensor,
                   moe_mxfp4_quantize, moe_mxfp4_status_string, moe_mxfp8_prepack,
                   moe_mxfp8_quantize, moe_probe_copy,
                   moe_probe_read_cached, moe_probe_sink_words, moe_probe_stream_read,
                   tensor_desc)

__all__ = [n for n in dir() if n.startswith(("moe_", "MOE_"))] + ["MoeError", "lib", "tensor_desc"]
