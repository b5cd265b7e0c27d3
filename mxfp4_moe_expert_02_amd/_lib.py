"""ctypes binding of libmoe_mxfp4.so, with the C ABI's own names.

Argument marshalling only: every step of the layer runs in the HIP library.
Tensors are torch device tensors (torch provides memory and streams); each
is checked for dtype, shape and contiguity here so that the pointer handed
to the library means what include/moe_mxfp4.h says it means.  There is no
fallback: if the library is not built this module raises on first use.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_MXFP4_LIB may name another build of the same library (e.g. a tuning variant)
LIB_PATH = os.environ.get("MOE_MXFP4_LIB") or os.path.join(HERE, "libmoe_mxfp4.so")

MOE_OK = 0
MOE_E_NULL = -1
MOE_E_SHAPE = -2
MOE_E_ALIGN = -3
MOE_E_TOPK = -4
MOE_E_TOKENS = -5
MOE_E_NOT_INIT = -6
MOE_E_HIP = -7
MOE_E_OPTION = -8
MOE_E_LIMIT = -9
MOE_E_DTYPE = -10

MOE_DT_BF16 = 1
MOE_DT_F32 = 2
MOE_DT_U8 = 3
MOE_DT_I32 = 4

MOE_ACT_BF16 = 0
MOE_ACT_MXFP8 = 1
MOE_PATH_AUTO = 0
MOE_PATH_GEMV = 1
MOE_PATH_MFMA = 2
MOE_LAYOUT_ROWS = 0
MOE_LAYOUT_TILES = 1
MOE_LAUNCH_AUTO = 0
MOE_LAUNCH_SPLIT = 1
MOE_LAUNCH_FUSED = 2
MOE_LAUNCH_SELF_ROUTED = 3
MOE_LAUNCH_QUEUE = 4

EXPORTED = ("moe_mxfp4_init", "moe_mxfp4_finalize", "moe_mxfp4_forward",
            "moe_mxfp4_forward_ex", "moe_mxfp4_quantize", "moe_mxfp4_status_string",
            "moe_mxfp4_prepack", "moe_mxfp8_quantize", "moe_mxfp8_prepack",
            "moe_probe_stream_read", "moe_probe_read_cached", "moe_probe_sink_words", "moe_probe_copy",
            "moe_mxfp4_forward_noalloc", "moe_mxfp4_forward_t")


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status}: {moe_mxfp4_status_string(status)}")


class moe_mxfp4_scales(ctypes.Structure):
    _fields_ = [("gate_up", ctypes.c_void_p), ("down", ctypes.c_void_p)]


class moe_tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("shape", ctypes.c_int64 * 4), ("ndim", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class moe_mxfp4_options(ctypes.Structure):
    _fields_ = [("act_format", ctypes.c_int32), ("gemm_path", ctypes.c_int32),
                ("ids", ctypes.c_void_p), ("weights", ctypes.c_void_p),
                ("counts", ctypes.c_void_p), ("offsets", ctypes.c_void_p),
                ("sorted", ctypes.c_void_p), ("x_codes", ctypes.c_void_p),
                ("x_scales", ctypes.c_void_p), ("events", ctypes.POINTER(ctypes.c_void_p)),
                ("num_events", ctypes.c_int32), ("weight_layout", ctypes.c_int32),
                ("launch", ctypes.c_int32), ("wait_error", ctypes.c_void_p),
                ("router_weight", ctypes.c_void_p), ("logits_out", ctypes.c_void_p),
                ("shared_gate_up", ctypes.c_void_p), ("shared_gate_up_scales", ctypes.c_void_p),
                ("shared_down", ctypes.c_void_p), ("shared_down_scales", ctypes.c_void_p),
                ("h_codes", ctypes.c_void_p), ("h_scales", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m mxfp4_moe_expert_02_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
        L.moe_mxfp4_init.restype = ctypes.c_int
        L.moe_mxfp4_init.argtypes = [i64, i64, i64, i64, i32]
        L.moe_mxfp4_finalize.restype = None
        L.moe_mxfp4_finalize.argtypes = []
        fwd = [vp, vp, i64, i32, vp, vp, ctypes.POINTER(moe_mxfp4_scales), vp, vp]
        L.moe_mxfp4_forward.restype = ctypes.c_int
        L.moe_mxfp4_forward.argtypes = fwd
        L.moe_mxfp4_forward_ex.restype = ctypes.c_int
        L.moe_mxfp4_forward_ex.argtypes = fwd + [ctypes.POINTER(moe_mxfp4_options)]
        L.moe_mxfp4_forward_t.restype = ctypes.c_int
        L.moe_mxfp4_forward_t.argtypes = [ctypes.POINTER(moe_tensor), ctypes.POINTER(moe_tensor), i32,
                                          ctypes.POINTER(moe_tensor), ctypes.POINTER(moe_tensor),
                                          ctypes.POINTER(moe_tensor), ctypes.POINTER(moe_tensor), vp,
                                          ctypes.POINTER(moe_mxfp4_options)]
        L.moe_mxfp4_forward_noalloc.restype = ctypes.c_int
        L.moe_mxfp4_forward_noalloc.argtypes = [vp, vp, i64, i32, i64, i64, i64, vp, vp,
                                                ctypes.POINTER(moe_mxfp4_scales), vp, vp]
        L.moe_mxfp4_quantize.restype = ctypes.c_int
        L.moe_mxfp4_quantize.argtypes = [vp, i64, i64, vp, vp, vp]
        L.moe_mxfp4_status_string.restype = ctypes.c_char_p
        L.moe_mxfp4_status_string.argtypes = [ctypes.c_int]
        L.moe_mxfp4_prepack.restype = ctypes.c_int
        L.moe_mxfp4_prepack.argtypes = [vp, vp, i64, i64, i64, i32, vp, vp, vp]
        L.moe_mxfp8_prepack.restype = ctypes.c_int
        L.moe_mxfp8_prepack.argtypes = [vp, vp, i64, i64, i64, i32, vp, vp, vp]
        L.moe_mxfp8_quantize.restype = ctypes.c_int
        L.moe_mxfp8_quantize.argtypes = [vp, i64, i64, vp, vp, vp]
        L.moe_probe_stream_read.restype = ctypes.c_int
        L.moe_probe_stream_read.argtypes = [vp, i64, vp, vp]
        L.moe_probe_read_cached.restype = ctypes.c_int
        L.moe_probe_read_cached.argtypes = [vp, i64, vp, vp]
        L.moe_probe_sink_words.restype = i64
        L.moe_probe_sink_words.argtypes = []
        L.moe_probe_copy.restype = ctypes.c_int
        L.moe_probe_copy.argtypes = [vp, vp, i64, vp]
        _lib = L
    return _lib


def moe_mxfp4_status_string(status: int) -> str:
    return lib().moe_mxfp4_status_string(int(status)).decode()


def _check(rc: int, where: str) -> int:
    if rc != MOE_OK:
        raise MoeError(rc, where)
    return rc


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def moe_mxfp4_init(max_tokens: int, num_experts: int, hidden: int, inter: int,
                   max_top_k: int, check: bool = True) -> int:
    rc = lib().moe_mxfp4_init(max_tokens, num_experts, hidden, inter, max_top_k)
    return _check(rc, "moe_mxfp4_init") if check else rc


def moe_mxfp4_finalize() -> None:
    lib().moe_mxfp4_finalize()


def _expect(t, dtype, shape, name):
    if t is None:
        return
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)}, got "
                         f"{t.dtype} {tuple(t.shape)} contiguous={t.is_contiguous()}")


def moe_mxfp4_forward_ex(x, router_logits, top_k: int, W_gate_up, W_down, scales, out,
                         stream=None, act_format: int = MOE_ACT_BF16,
                         gemm_path: int = MOE_PATH_AUTO, ids=None, weights=None,
                         counts=None, offsets=None, sorted=None, x_codes=None,
                         x_scales=None, events=None, weight_layout: int = MOE_LAYOUT_ROWS,
                         launch: int = MOE_LAUNCH_AUTO, wait_error=None,
                         router_weight=None, logits_out=None, shared=None,
                         h_codes=None, h_scales=None,
                         check: bool = True, validate: bool = True) -> int:
    """Enqueue one layer on ``stream`` (default: torch's current stream).

    x [T,H] bfloat16, router_logits [T,E] float32, W_gate_up [E,2I,H/2] uint8,
    W_down [E,H,I/2] uint8, scales = (gate_up [E,2I,H/32], down [E,H,I/32])
    uint8, out [T,H] bfloat16.  ``validate=False`` skips the Python-side
    shape checks so the library's own validation can be exercised.
    ``events``: up to 4 torch.cuda.Event (timing enabled) recorded by the
    library at its stage boundaries.  ``launch``: MOE_LAUNCH_*;
    ``wait_error``: optional int32 [1] device tensor (see the header).
    ``router_weight``: optional [E, H] bfloat16: the layer computes the
    logits itself (``router_logits`` may then be None); ``logits_out``:
    optional [T, E] float32 output of the logits routed on.  ``shared``:
    optional (gate_up tiles, gate_up tile scales, down tiles, down tile
    scales) of an MXFP8 shared expert (moe_mxfp8_prepack layout, uint8).
    ``h_codes`` [T*k, I] / ``h_scales`` [T*k, I/32] uint8: optional copies of
    h's MXFP8 encoding on the MXFP8 path, rows in expert-sorted order.
    """
    import torch
    if validate:
        T, H = x.shape
        E = router_weight.shape[0] if router_weight is not None else router_logits.shape[1]
        _expect(x, torch.bfloat16, (T, H), "x")
        if router_weight is not None:
            _expect(router_weight, torch.bfloat16, (E, H), "router_weight")
        else:
            _expect(router_logits, torch.float32, (T, E), "router_logits")
        if logits_out is not None:
            _expect(logits_out, torch.float32, (T, E), "logits_out")
        I2 = W_gate_up.numel() * 2 // (E * H)  # 2I from the byte count (both layouts)
        for t, n, name in ((W_gate_up, E * I2 * H // 2, "W_gate_up"), (W_down, E * H * I2 // 4, "W_down"),
                           (scales[0], E * I2 * H // 32, "scales[0]"),
                           (scales[1], E * H * I2 // 64, "scales[1]")):
            if t.dtype != torch.uint8 or t.numel() != n or not t.is_contiguous():
                raise ValueError(f"{name}: expected {n} contiguous uint8 bytes, got "
                                 f"{t.dtype} {tuple(t.shape)} contiguous={t.is_contiguous()}")
        _expect(out, torch.bfloat16, (T, H), "out")
        if h_codes is not None:
            _expect(h_codes, torch.uint8, (T * top_k, I2 // 2), "h_codes")
        if h_scales is not None:
            _expect(h_scales, torch.uint8, (T * top_k, I2 // 64), "h_scales")
        if shared is not None:
            I = I2 // 2
            for t, n, name in ((shared[0], 2 * I * H, "shared[0]"), (shared[1], 2 * I * H // 32, "shared[1]"),
                               (shared[2], H * I, "shared[2]"), (shared[3], H * I // 32, "shared[3]")):
                if t.dtype != torch.uint8 or t.numel() != n or not t.is_contiguous():
                    raise ValueError(f"{name}: expected {n} contiguous uint8 bytes, got "
                                     f"{t.dtype} {tuple(t.shape)} contiguous={t.is_contiguous()}")
    sh = [None] * 4 if shared is None else [_ptr(t) for t in shared]
    sc = moe_mxfp4_scales(_ptr(scales[0]), _ptr(scales[1])) if scales is not None else None
    ev_arr, n_ev = None, 0
    if events:
        handles = []
        for e in events:
            if not e.cuda_event:  # torch creates the event lazily at its first record
                e.record()
            handles.append(e.cuda_event)
        n_ev = len(handles)
        ev_arr = (ctypes.c_void_p * n_ev)(*handles)
    opt = moe_mxfp4_options(act_format, gemm_path, _ptr(ids), _ptr(weights), _ptr(counts),
                            _ptr(offsets), _ptr(sorted), _ptr(x_codes), _ptr(x_scales),
                            ctypes.cast(ev_arr, ctypes.POINTER(ctypes.c_void_p)) if ev_arr else None,
                            n_ev, weight_layout, launch, _ptr(wait_error), _ptr(router_weight),
                            _ptr(logits_out), *sh, _ptr(h_codes), _ptr(h_scales))
    T = x.shape[0] if x is not None else 0
    rc = lib().moe_mxfp4_forward_ex(_ptr(x), _ptr(router_logits), T, top_k, _ptr(W_gate_up),
                                    _ptr(W_down), ctypes.byref(sc) if sc is not None else None,
                                    _ptr(out), _stream(stream), ctypes.byref(opt))
    return _check(rc, "moe_mxfp4_forward_ex") if check else rc


def tensor_desc(t) -> moe_tensor:
    """The moe_tensor descriptor of a torch tensor (its own dtype, rank and
    shape: the library checks them, nothing is checked here)."""
    import torch
    codes = {torch.bfloat16: MOE_DT_BF16, torch.float32: MOE_DT_F32, torch.uint8: MOE_DT_U8,
             torch.int32: MOE_DT_I32}
    d = moe_tensor()
    d.data = t.data_ptr()
    d.ndim = t.dim()
    for i, n in enumerate(t.shape[:4]):
        d.shape[i] = n
    d.dtype = codes.get(t.dtype, 0)
    return d


def moe_mxfp4_forward_t(x, router_logits, top_k: int, W_gate_up, W_down, scales, out, stream=None,
                        weight_layout: int = MOE_LAYOUT_ROWS, gemm_path: int = MOE_PATH_AUTO,
                        launch: int = MOE_LAUNCH_AUTO, router_weight=None,
                        check: bool = True) -> int:
    """moe_mxfp4_forward_t: every tensor passed as a descriptor, the library
    checking element types, ranks and shapes (no checks in Python)."""
    sc = (moe_tensor * 2)(tensor_desc(scales[0]), tensor_desc(scales[1]))
    opt = moe_mxfp4_options()
    opt.weight_layout, opt.gemm_path, opt.launch = weight_layout, gemm_path, launch
    opt.router_weight = _ptr(router_weight)
    lg = None if router_logits is None else ctypes.byref(tensor_desc(router_logits))
    rc = lib().moe_mxfp4_forward_t(ctypes.byref(tensor_desc(x)), lg, top_k,
                                   ctypes.byref(tensor_desc(W_gate_up)), ctypes.byref(tensor_desc(W_down)),
                                   sc, ctypes.byref(tensor_desc(out)), _stream(stream),
                                   ctypes.byref(opt))
    return _check(rc, "moe_mxfp4_forward_t") if check else rc


def moe_mxfp4_forward(x, router_logits, top_k: int, W_gate_up, W_down, scales, out,
                      stream=None, check: bool = True) -> int:
    """The layer with bf16 activations (see moe_mxfp4_forward_ex for shapes)."""
    import torch
    T, H = x.shape
    E = router_logits.shape[1]
    I2 = W_gate_up.shape[1]
    _expect(x, torch.bfloat16, (T, H), "x")
    _expect(router_logits, torch.float32, (T, E), "router_logits")
    _expect(out, torch.bfloat16, (T, H), "out")
    sc = moe_mxfp4_scales(_ptr(scales[0]), _ptr(scales[1]))
    rc = lib().moe_mxfp4_forward(_ptr(x), _ptr(router_logits), T, top_k, _ptr(W_gate_up),
                                 _ptr(W_down), ctypes.byref(sc), _ptr(out), _stream(stream))
    return _check(rc, "moe_mxfp4_forward") if check else rc


def moe_mxfp4_forward_noalloc(x, router_logits, top_k: int, W_gate_up, W_down, scales, out,
                              num_experts: int, hidden: int, inter: int, stream=None,
                              check: bool = True) -> int:
    """The allocation-free layer (weights in the MFMA tile layout, at most 16
    tokens; see include/moe_mxfp4.h): x [T, H] bfloat16, router_logits
    [T, E] float32, out [T, H] bfloat16; W_gate_up / W_down / scales as
    written by moe_mxfp4_prepack."""
    import torch
    T = x.shape[0]
    _expect(x, torch.bfloat16, (T, hidden), "x")
    _expect(router_logits, torch.float32, (T, num_experts), "router_logits")
    _expect(out, torch.bfloat16, (T, hidden), "out")
    sc = moe_mxfp4_scales(_ptr(scales[0]), _ptr(scales[1]))
    rc = lib().moe_mxfp4_forward_noalloc(_ptr(x), _ptr(router_logits), T, top_k, num_experts, hidden,
                                         inter, _ptr(W_gate_up), _ptr(W_down), ctypes.byref(sc),
                                         _ptr(out), _stream(stream))
    return _check(rc, "moe_mxfp4_forward_noalloc") if check else rc


def moe_mxfp4_prepack(packed, scales, tiles, tile_scales, gate_up_pairs: bool,
                      stream=None, check: bool = True) -> int:
    """Rearrange row-major MXFP4 matrices packed [N, rows, cols/2] + scales
    [N, rows, cols/32] into the MFMA tile layout (same byte sizes)."""
    import torch
    N, rows, half = packed.shape
    cols = half * 2
    _expect(scales, torch.uint8, (N, rows, cols // 32), "scales")
    if tiles.numel() != packed.numel() or tile_scales.numel() != scales.numel():
        raise ValueError("moe_mxfp4_prepack: output sizes must equal input sizes")
    rc = lib().moe_mxfp4_prepack(_ptr(packed), _ptr(scales), N, rows, cols,
                                 1 if gate_up_pairs else 0, _ptr(tiles), _ptr(tile_scales),
                                 _stream(stream))
    return _check(rc, "moe_mxfp4_prepack") if check else rc


def moe_mxfp4_quantize(w, packed, scales, stream=None, check: bool = True) -> int:
    """Encode float32 w [rows, cols] to MXFP4 into packed [rows, cols/2] and
    scales [rows, cols/32] (uint8 device tensors)."""
    import torch
    rows, cols = w.shape
    _expect(w, torch.float32, (rows, cols), "w")
    _expect(packed, torch.uint8, (rows, cols // 2), "packed")
    _expect(scales, torch.uint8, (rows, cols // 32), "scales")
    rc = lib().moe_mxfp4_quantize(_ptr(w), rows, cols, _ptr(packed), _ptr(scales), _stream(stream))
    return _check(rc, "moe_mxfp4_quantize") if check else rc


def moe_mxfp8_prepack(codes, scales, tiles, tile_scales, gate_up_pairs: bool,
                      stream=None, check: bool = True) -> int:
    """Rearrange row-major MXFP8 matrices codes [N, rows, cols] + scales
    [N, rows, cols/32] into the MXFP8 tile layout (same byte sizes)."""
    import torch
    N, rows, cols = codes.shape
    _expect(scales, torch.uint8, (N, rows, cols // 32), "scales")
    if tiles.numel() != codes.numel() or tile_scales.numel() != scales.numel():
        raise ValueError("moe_mxfp8_prepack: output sizes must equal input sizes")
    rc = lib().moe_mxfp8_prepack(_ptr(codes), _ptr(scales), N, rows, cols,
                                 1 if gate_up_pairs else 0, _ptr(tiles), _ptr(tile_scales),
                                 _stream(stream))
    return _check(rc, "moe_mxfp8_prepack") if check else rc


def moe_mxfp8_quantize(w, codes, scales, stream=None, check: bool = True) -> int:
    """Encode float32 w [rows, cols] to MXFP8 into codes [rows, cols] and
    scales [rows, cols/32] (uint8 device tensors)."""
    import torch
    rows, cols = w.shape
    _expect(w, torch.float32, (rows, cols), "w")
    _expect(codes, torch.uint8, (rows, cols), "codes")
    _expect(scales, torch.uint8, (rows, cols // 32), "scales")
    rc = lib().moe_mxfp8_quantize(_ptr(w), rows, cols, _ptr(codes), _ptr(scales), _stream(stream))
    return _check(rc, "moe_mxfp8_quantize") if check else rc


def moe_probe_sink_words() -> int:
    return lib().moe_probe_sink_words()


def moe_probe_stream_read(src, sink, stream=None, check: bool = True) -> int:
    """Stream-read every byte of the device tensor ``src`` (128-bit loads)."""
    rc = lib().moe_probe_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                                     _stream(stream))
    return _check(rc, "moe_probe_stream_read") if check else rc


def moe_probe_read_cached(src, sink, stream=None, check: bool = True) -> int:
    """Read every byte of the device tensor ``src`` with cache-allocating loads."""
    rc = lib().moe_probe_read_cached(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                                     _stream(stream))
    return _check(rc, "moe_probe_read_cached") if check else rc


def moe_probe_copy(src, dst, stream=None, check: bool = True) -> int:
    """Copy the device tensor ``src`` into ``dst`` (same byte size)."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("moe_probe_copy: size mismatch")
    rc = lib().moe_probe_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream))
    return _check(rc, "moe_probe_copy") if check else rc
