"""ctypes binding of libuw.so: the same entry points as include/uw.h.

Argument marshalling only: torch tensors supply device memory and the HIP
stream; every computation runs in the library (host encoder, gfx950 kernels).
There is no fallback: if libuw.so is missing or fails to load, importing this
module raises.
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libuw.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "uw.h")

UW_OK = 0
UW_ERR_INVALID = -1
UW_ERR_FORMAT = -2
UW_ERR_NOSPACE = -3
UW_ERR_HIP = -4
UW_ERR_UNSUPPORTED = -5
UW_F32 = 0
UW_BF16 = 1
UW_VARIANT_AUTO = 0
UW_VARIANT_FUSED = 1
UW_VARIANT_DECOMPRESS_GEMM = 2
UW_VARIANT_FUSED_MFMA = 3
UW_VARIANT_PALETTE = 4
UW_VARIANT_COUNT = 5
UW_ENC_NO_PLAIN = 1
VARIANT_NAMES = {UW_VARIANT_AUTO: "auto", UW_VARIANT_FUSED: "fused", UW_VARIANT_DECOMPRESS_GEMM: "decompress_gemm",
                 UW_VARIANT_FUSED_MFMA: "fused_mfma", UW_VARIANT_PALETTE: "palette"}


class UwError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__(f"{where}: {message} (status {status})")
        self.status = status


class uw_encode_opts(ctypes.Structure):
    _fields_ = [("K", ctypes.c_int32), ("L", ctypes.c_int32), ("G", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class uw_info(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("K", ctypes.c_int32), ("L", ctypes.c_int32),
                ("G", ctypes.c_int32), ("plain", ctypes.c_int32), ("n_blocks", ctypes.c_int64),
                ("n_raw_groups", ctypes.c_int64), ("total_bytes", ctypes.c_uint64),
                ("max_segment_bytes", ctypes.c_uint32), ("palette", ctypes.c_uint8 * 32),
                ("code_len", ctypes.c_uint8 * 32), ("ratio", ctypes.c_double), ("bits_per_weight", ctypes.c_double)]


class uw_plan(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("variant", ctypes.c_int32), ("knob", ctypes.c_int32),
                ("time_us", ctypes.c_float), ("candidate_us", ctypes.c_float * UW_VARIANT_COUNT),
                ("candidate_knob", ctypes.c_int32 * UW_VARIANT_COUNT)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run python decode_gemv_canonical_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, I64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "uw_version": (I, []),
        "uw_status_string": (ctypes.c_char_p, [I]),
        "uw_last_error": (ctypes.c_char_p, []),
        "uw_encode": (I, [P, I64, I64, ctypes.POINTER(uw_encode_opts), P, ctypes.POINTER(SZ)]),
        "uw_blob_info": (I, [P, SZ, ctypes.POINTER(uw_info)]),
        "uw_matrix_device_bytes": (SZ, [P, SZ]),
        "uw_matrix_create": (I, [P, SZ, P, SZ, ctypes.POINTER(P)]),
        "uw_matrix_attach_palette": (I, [P, P]),
        "uw_matrix_destroy": (None, [P]),
        "uw_decompress": (I, [P, P, I64, P]),
        "uw_gemv_fused": (I, [P, P, I, P, I, P]),
        "uw_gemm_fused": (I, [P, P, I64, I64, I, P, I64, I, I, P, SZ, P]),
        "uw_gemm_with_plan": (I, [P, ctypes.POINTER(uw_plan), P, I64, I64, I, P, I64, I, P, SZ, P]),
        "uw_gemm_fused_static": (I, [P, P, I64, I64, I, P, I64, I, I, P]),
        "uw_plan_save": (I, [P, ctypes.c_char_p, ctypes.POINTER(SZ)]),
        "uw_plan_load": (I, [P, ctypes.c_char_p]),
        "uw_workspace_size": (SZ, [P, I64, I]),
        "uw_autotune": (I, [P, I64, P, SZ, P, ctypes.POINTER(uw_plan)]),
        "uw_autotune_scratch_size": (SZ, [P, I64]),
        "uw_get_plan": (I, [P, I64, ctypes.POINTER(uw_plan)]),
        "uw_set_plan": (I, [P, ctypes.POINTER(uw_plan)]),
        "uw_exponent_gemm": (I, [P, P, I64, I64, I, P, I64, I, P, SZ, P]),
        "uw_exponent_ws_size": (SZ, [P, I64]),
        "uw_bf16_gemm": (I, [P, I64, I64, I64, P, I64, I64, I, P, I64, I, P]),
        "uw_bf16_gemm_shaped": (I, [P, I64, I64, I64, P, I64, I64, P, I64, I, I, I, P]),
        "uw_bf16_gemm_shape_count": (I, []),
        "uw_read_probe": (I, [P, SZ, P, P]),
        "uw_read_probe_sink_size": (SZ, []),
        "uw_palette_encode": (I, [P, I64, I64, P, ctypes.POINTER(SZ)]),
        "uw_palette_info": (I, [P, SZ, ctypes.POINTER(I64), ctypes.POINTER(I64), ctypes.POINTER(I64)]),
        "uw_palette_create": (I, [P, SZ, P, ctypes.POINTER(P)]),
        "uw_palette_destroy": (None, [P]),
        "uw_palette_gemv": (I, [P, P, I, P, I, P]),
        "uw_palette_decompress": (I, [P, P, I64, P]),
        "uw_palette_gemm": (I, [P, P, I64, I64, I, P, I64, I, P]),
        "uw_palette_transcode_size": (SZ, [P]),
        "uw_palette_transcode": (I, [P, P, SZ, P]),
        "uw_palette_create_transcoded": (I, [P, P, ctypes.POINTER(P)]),
        "uw_sched_create": (I, [P, SZ, I, I, ctypes.POINTER(P)]),
        "uw_sched_destroy": (None, [P]),
        "uw_sched_decode_cus": (I, [P]),
        "uw_sched_prefetch": (I, [P, P, P, ctypes.POINTER(I)]),
        "uw_sched_gemm": (I, [P, I, P, I64, I64, I, P, I64, I, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def header_symbols() -> list[str]:
    """Entry points declared in include/uw.h."""
    text = open(HEADER_PATH).read()
    return sorted(set(re.findall(r"\b(uw_[a-z0-9_]+)\s*\(", text)))


def library() -> ctypes.CDLL:
    return _lib


def _check(rc: int, where: str) -> None:
    if rc != UW_OK:
        raise UwError(rc, where, (_lib.uw_last_error() or b"").decode())


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return UW_F32
    if t.dtype == torch.bfloat16:
        return UW_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


# Shapes of live handles (rows, cols, device index), so that the wrappers can
# check tensors before the library sees their pointers: the C side cannot
# know how large a buffer is, and an undersized or foreign one would be read
# or written out of bounds on the device.
_handles: dict[int, tuple[int, int, int]] = {}


def _register(handle: int, rows: int, cols: int, device_index: int) -> None:
    _handles[handle] = (rows, cols, device_index)


def _shape(handle: int) -> tuple[int, int, int]:
    if handle not in _handles:
        raise ValueError("unknown or closed handle")
    return _handles[handle]


def _on_device(t, dev: int, name: str) -> None:
    if not hasattr(t, "is_cuda") or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA tensor")
    if t.device.index != dev:
        raise ValueError(f"{name} is on cuda:{t.device.index}, the handle on cuda:{dev}")


def _check_vector(t, n: int, dev: int, name: str) -> None:
    if t.dim() != 1 or t.numel() != n or (n > 1 and t.stride(0) != 1):
        raise ValueError(f"{name} must be a contiguous vector of {n} elements, got shape {tuple(t.shape)}")
    _on_device(t, dev, name)


def _check_rows(t, batch: int | None, width: int, dev: int, name: str, exact: bool = True) -> None:
    """A [batch, >= width] (or == width) row-major tensor with unit inner stride."""
    if t.dim() != 2 or (batch is not None and t.shape[0] != batch):
        raise ValueError(f"{name} must be 2-D with {batch} rows, got shape {tuple(t.shape)}")
    if (t.shape[1] != width) if exact else (t.shape[1] < width):
        raise ValueError(f"{name} must have {'' if exact else 'at least '}{width} columns, got {t.shape[1]}")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have a unit inner stride")
    if t.shape[0] > 1 and t.stride(0) < t.shape[1]:
        raise ValueError(f"{name} rows overlap")
    _on_device(t, dev, name)


def _as_u16(w) -> np.ndarray:
    if hasattr(w, "numpy"):  # torch tensor on the CPU
        w = w.contiguous().view(dtype=__import__("torch").int16).numpy()
    a = np.ascontiguousarray(np.asarray(w))
    if a.dtype not in (np.uint16, np.int16):
        raise TypeError("weights must be 16-bit bf16 bit patterns")
    return a.view(np.uint16)


# -- entry points -----------------------------------------------------------

def uw_version() -> int:
    return _lib.uw_version()


def uw_status_string(status: int) -> str:
    return _lib.uw_status_string(status).decode()


def uw_last_error() -> str:
    return (_lib.uw_last_error() or b"").decode()


def uw_encode(w_bf16, K: int = 0, L: int = 0, G: int = 0, flags: int = 0) -> bytes:
    """bf16 bit patterns [rows, cols] (numpy uint16/int16 or a CPU torch tensor) -> blob bytes."""
    a = _as_u16(w_bf16)
    if a.ndim != 2:
        raise ValueError("need a 2-D matrix")
    opts = uw_encode_opts(K, L, G, flags)
    size = ctypes.c_size_t(0)
    _check(_lib.uw_encode(a.ctypes.data, a.shape[0], a.shape[1], ctypes.byref(opts), None, ctypes.byref(size)), "uw_encode")
    buf = np.empty(size.value, dtype=np.uint8)
    _check(_lib.uw_encode(a.ctypes.data, a.shape[0], a.shape[1], ctypes.byref(opts), buf.ctypes.data, ctypes.byref(size)),
           "uw_encode")
    return buf[: size.value].tobytes()


def uw_blob_info(blob: bytes) -> dict:
    info = uw_info()
    arr = np.frombuffer(blob, dtype=np.uint8)
    _check(_lib.uw_blob_info(arr.ctypes.data, arr.size, ctypes.byref(info)), "uw_blob_info")
    out = {f: getattr(info, f) for f, _ in uw_info._fields_}
    out["palette"] = list(info.palette)[: info.K]
    out["code_len"] = list(info.code_len)[: info.K]
    return out


def uw_matrix_device_bytes(host_blob: bytes) -> int:
    arr = np.frombuffer(host_blob, dtype=np.uint8)
    n = _lib.uw_matrix_device_bytes(arr.ctypes.data, arr.size)
    if n == 0:
        raise UwError(UW_ERR_FORMAT, "uw_matrix_device_bytes", uw_last_error())
    return n


def uw_matrix_create(host_blob: bytes, d_buf) -> int:
    """Handle for a blob already copied to the start of the CUDA uint8 tensor
    d_buf (256-byte aligned, at least uw_matrix_device_bytes(host_blob) bytes;
    the library writes its derived tables after the blob)."""
    arr = np.frombuffer(host_blob, dtype=np.uint8)
    if d_buf.dtype.itemsize != 1 or not d_buf.is_contiguous():
        raise ValueError("the device buffer must be a contiguous byte tensor")
    h = ctypes.c_void_p()
    _check(_lib.uw_matrix_create(arr.ctypes.data, arr.size, d_buf.data_ptr(), d_buf.numel(), ctypes.byref(h)),
           "uw_matrix_create")
    info = uw_blob_info(host_blob)
    _register(h.value, info["rows"], info["cols"], d_buf.device.index)
    return h.value


def uw_matrix_destroy(handle: int) -> None:
    _handles.pop(handle, None)
    _lib.uw_matrix_destroy(handle)


def uw_matrix_attach_palette(handle: int, palette_handle: int | None) -> None:
    _check(_lib.uw_matrix_attach_palette(handle, palette_handle), "uw_matrix_attach_palette")


def uw_decompress(handle: int, d_out, ld_out: int | None = None, stream=None) -> None:
    rows, cols, dev = _shape(handle)
    if d_out.element_size() != 2:
        raise ValueError("the output must hold 16-bit elements")
    _check_rows(d_out, rows, cols, dev, "out", exact=False)
    if ld_out is None:
        ld_out = d_out.stride(0)
    if ld_out != d_out.stride(0):
        raise ValueError("ld_out must be the output's row stride")
    _check(_lib.uw_decompress(handle, d_out.data_ptr(), ld_out, _stream(stream)), "uw_decompress")


def uw_gemv_fused(handle: int, x, y, stream=None) -> None:
    rows, cols, dev = _shape(handle)
    _check_vector(x, cols, dev, "x")
    _check_vector(y, rows, dev, "y")
    _check(_lib.uw_gemv_fused(handle, x.data_ptr(), _dtype_code(x), y.data_ptr(), _dtype_code(y), _stream(stream)),
           "uw_gemv_fused")


def _gemm_operands(handle: int, X, Y):
    rows, cols, dev = _shape(handle)
    _check_rows(X, None, cols, dev, "X")
    _check_rows(Y, X.shape[0], rows, dev, "Y", exact=False)
    return X.shape[0]


def _ws(ws, dev: int):
    if ws is None:
        return None, 0
    _on_device(ws, dev, "ws")
    if not ws.is_contiguous():
        raise ValueError("ws must be contiguous")
    return ws.data_ptr(), ws.numel() * ws.element_size()


def uw_gemm_fused(handle: int, X, Y, variant: int = UW_VARIANT_AUTO, ws=None, stream=None) -> None:
    batch = _gemm_operands(handle, X, Y)
    ws_ptr, ws_bytes = _ws(ws, _shape(handle)[2])
    _check(_lib.uw_gemm_fused(handle, X.data_ptr(), batch, X.stride(0), _dtype_code(X), Y.data_ptr(), Y.stride(0),
                              _dtype_code(Y), variant, ws_ptr, ws_bytes, _stream(stream)), "uw_gemm_fused")


def uw_gemm_fused_static(handle: int, X, Y, variant: int = UW_VARIANT_AUTO, stream=None) -> None:
    """uw_gemm_fused with no workspace: decompress + GEMM runs through the
    library's static scratch (nothing is allocated)."""
    batch = _gemm_operands(handle, X, Y)
    _check(_lib.uw_gemm_fused_static(handle, X.data_ptr(), batch, X.stride(0), _dtype_code(X), Y.data_ptr(),
                                     Y.stride(0), _dtype_code(Y), variant, _stream(stream)), "uw_gemm_fused_static")


def uw_gemm_with_plan(handle: int, variant: int, knob: int, X, Y, ws=None, stream=None) -> None:
    batch = _gemm_operands(handle, X, Y)
    ws_ptr, ws_bytes = _ws(ws, _shape(handle)[2])
    p = uw_plan()
    p.batch = batch
    p.variant = variant
    p.knob = knob
    _check(_lib.uw_gemm_with_plan(handle, ctypes.byref(p), X.data_ptr(), batch, X.stride(0), _dtype_code(X),
                                  Y.data_ptr(), Y.stride(0), _dtype_code(Y), ws_ptr, ws_bytes, _stream(stream)),
           "uw_gemm_with_plan")


def uw_plan_save(handle: int) -> str:
    size = ctypes.c_size_t(0)
    _check(_lib.uw_plan_save(handle, None, ctypes.byref(size)), "uw_plan_save")
    buf = ctypes.create_string_buffer(size.value)
    _check(_lib.uw_plan_save(handle, buf, ctypes.byref(size)), "uw_plan_save")
    return buf.value.decode()


def uw_plan_load(handle: int, text: str) -> None:
    _check(_lib.uw_plan_load(handle, text.encode()), "uw_plan_load")


def uw_workspace_size(handle: int, batch: int, variant: int = UW_VARIANT_AUTO) -> int:
    return _lib.uw_workspace_size(handle, batch, variant)


def uw_autotune_scratch_size(handle: int, batch: int) -> int:
    return _lib.uw_autotune_scratch_size(handle, batch)


def _plan_dict(p: uw_plan) -> dict:
    return {"batch": p.batch, "variant": p.variant, "variant_name": VARIANT_NAMES.get(p.variant, "?"),
            "knob": p.knob, "time_us": p.time_us,
            "candidate_us": {VARIANT_NAMES[v]: p.candidate_us[v]
                             for v in range(1, UW_VARIANT_COUNT) if p.candidate_us[v] >= 0},
            "candidate_knob": {VARIANT_NAMES[v]: p.candidate_knob[v]
                               for v in range(1, UW_VARIANT_COUNT) if p.candidate_us[v] >= 0}}


def uw_autotune(handle: int, batch: int, ws, stream=None) -> dict:
    _ws(ws, _shape(handle)[2])
    p = uw_plan()
    _check(_lib.uw_autotune(handle, batch, ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream),
                            ctypes.byref(p)), "uw_autotune")
    return _plan_dict(p)


def uw_get_plan(handle: int, batch: int) -> dict:
    p = uw_plan()
    _check(_lib.uw_get_plan(handle, batch, ctypes.byref(p)), "uw_get_plan")
    return _plan_dict(p)


def uw_exponent_ws_size(handle: int, batch: int) -> int:
    return _lib.uw_exponent_ws_size(handle, batch)


def uw_exponent_gemm(handle: int, X, Y, ws, stream=None) -> None:
    _gemm_operands(handle, X, Y)
    _ws(ws, _shape(handle)[2])
    _check(_lib.uw_exponent_gemm(handle, X.data_ptr(), X.shape[0], X.stride(0), _dtype_code(X), Y.data_ptr(),
                                 Y.stride(0), _dtype_code(Y), ws.data_ptr(), ws.numel() * ws.element_size(),
                                 _stream(stream)), "uw_exponent_gemm")


def uw_set_plan(handle: int, batch: int, variant: int, time_us: float = -1.0, knob: int = 0) -> None:
    p = uw_plan()
    p.batch = batch
    p.variant = variant
    p.knob = knob
    p.time_us = time_us
    for i in range(UW_VARIANT_COUNT):
        p.candidate_us[i] = -1.0
    _check(_lib.uw_set_plan(handle, ctypes.byref(p)), "uw_set_plan")


def _bf16_operands(W, X, Y):
    if W.dim() != 2 or W.element_size() != 2:
        raise ValueError("W must be a 2-D 16-bit tensor")
    rows, cols = W.shape
    dev = W.device.index if W.is_cuda else -1
    _check_rows(W, rows, cols, dev, "W")
    _check_rows(X, None, cols, dev, "X")
    _check_rows(Y, X.shape[0], rows, dev, "Y", exact=False)
    return rows, cols


def uw_bf16_gemm(W, X, Y, stream=None) -> None:
    rows, cols = _bf16_operands(W, X, Y)
    _check(_lib.uw_bf16_gemm(W.data_ptr(), rows, cols, W.stride(0), X.data_ptr(), X.shape[0], X.stride(0),
                             _dtype_code(X), Y.data_ptr(), Y.stride(0), _dtype_code(Y), _stream(stream)),
           "uw_bf16_gemm")


def uw_bf16_gemm_shaped(W, X, Y, shape: int, ks: int = 0, stream=None) -> None:
    rows, cols = _bf16_operands(W, X, Y)
    _check(_lib.uw_bf16_gemm_shaped(W.data_ptr(), rows, cols, W.stride(0), X.data_ptr(), X.shape[0], X.stride(0),
                                    Y.data_ptr(), Y.stride(0), _dtype_code(Y), shape, ks, _stream(stream)),
           "uw_bf16_gemm_shaped")


def uw_bf16_gemm_shape_count() -> int:
    return _lib.uw_bf16_gemm_shape_count()


def uw_read_probe_sink_size() -> int:
    return _lib.uw_read_probe_sink_size()


def uw_read_probe(src, sink, stream=None) -> None:
    _check(_lib.uw_read_probe(src.data_ptr(), src.numel() * src.element_size(), sink.data_ptr(), _stream(stream)),
           "uw_read_probe")


def uw_palette_encode(w_bf16) -> bytes:
    a = _as_u16(w_bf16)
    if a.ndim != 2:
        raise ValueError("weights must be a 2-D matrix")
    size = ctypes.c_size_t(0)
    _check(_lib.uw_palette_encode(a.ctypes.data, a.shape[0], a.shape[1], None, ctypes.byref(size)), "uw_palette_encode")
    buf = np.zeros(size.value, dtype=np.uint8)
    _check(_lib.uw_palette_encode(a.ctypes.data, a.shape[0], a.shape[1], buf.ctypes.data, ctypes.byref(size)),
           "uw_palette_encode")
    return buf.tobytes()


def uw_palette_info(blob: bytes) -> dict:
    arr = np.frombuffer(blob, dtype=np.uint8)
    rows, cols, n_raw = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(_lib.uw_palette_info(arr.ctypes.data, arr.size, ctypes.byref(rows), ctypes.byref(cols), ctypes.byref(n_raw)),
           "uw_palette_info")
    return {"rows": rows.value, "cols": cols.value, "n_raw": n_raw.value, "bytes": arr.size,
            "ratio": arr.size / (2 * rows.value * cols.value)}


def uw_palette_create(host_blob: bytes, d_blob) -> int:
    arr = np.frombuffer(host_blob, dtype=np.uint8)
    if d_blob.numel() != arr.size:
        raise ValueError("device blob size differs from the host blob")
    h = ctypes.c_void_p()
    _check(_lib.uw_palette_create(arr.ctypes.data, arr.size, d_blob.data_ptr(), ctypes.byref(h)), "uw_palette_create")
    info = uw_palette_info(host_blob)
    _register(h.value, info["rows"], info["cols"], d_blob.device.index)
    return h.value


def uw_palette_destroy(handle: int) -> None:
    _handles.pop(handle, None)
    _lib.uw_palette_destroy(handle)


def uw_palette_transcode_size(handle: int) -> int:
    return _lib.uw_palette_transcode_size(handle)


def uw_palette_transcode(handle: int, d_out, stream=None) -> None:
    _on_device(d_out, _shape(handle)[2], "out")
    if not d_out.is_contiguous():
        raise ValueError("out must be contiguous")
    _check(_lib.uw_palette_transcode(handle, d_out.data_ptr(), d_out.numel() * d_out.element_size(), _stream(stream)),
           "uw_palette_transcode")


def uw_palette_create_transcoded(handle: int, d_blob) -> int:
    rows, cols, dev = _shape(handle)
    _on_device(d_blob, dev, "d_blob")
    if d_blob.numel() * d_blob.element_size() < uw_palette_transcode_size(handle):
        raise ValueError("d_blob is smaller than the transcoded form")
    h = ctypes.c_void_p()
    _check(_lib.uw_palette_create_transcoded(handle, d_blob.data_ptr(), ctypes.byref(h)), "uw_palette_create_transcoded")
    _register(h.value, rows, cols, dev)
    return h.value


def uw_palette_gemv(handle: int, x, y, stream=None) -> None:
    rows, cols, dev = _shape(handle)
    _check_vector(x, cols, dev, "x")
    _check_vector(y, rows, dev, "y")
    _check(_lib.uw_palette_gemv(handle, x.data_ptr(), _dtype_code(x), y.data_ptr(), _dtype_code(y), _stream(stream)),
           "uw_palette_gemv")


def uw_palette_gemm(handle: int, X, Y, stream=None) -> None:
    batch = _gemm_operands(handle, X, Y)
    _check(_lib.uw_palette_gemm(handle, X.data_ptr(), batch, X.stride(0), _dtype_code(X), Y.data_ptr(), Y.stride(0),
                                _dtype_code(Y), _stream(stream)), "uw_palette_gemm")


def uw_palette_decompress(handle: int, d_out, ld_out: int | None = None, stream=None) -> None:
    rows, cols, dev = _shape(handle)
    if d_out.element_size() != 2:
        raise ValueError("the output must hold 16-bit elements")
    _check_rows(d_out, rows, cols, dev, "out", exact=False)
    if ld_out is None:
        ld_out = d_out.stride(0)
    if ld_out != d_out.stride(0):
        raise ValueError("ld_out must be the output's row stride")
    _check(_lib.uw_palette_decompress(handle, d_out.data_ptr(), ld_out, _stream(stream)), "uw_palette_decompress")


def uw_sched_create(d_slots, slot_bytes: int, n_slots: int, decode_cus: int = 0) -> int:
    if not d_slots.is_cuda or not d_slots.is_contiguous() or d_slots.numel() * d_slots.element_size() < slot_bytes * n_slots:
        raise ValueError("d_slots must be a contiguous CUDA buffer of n_slots * slot_bytes bytes")
    h = ctypes.c_void_p()
    _check(_lib.uw_sched_create(d_slots.data_ptr(), slot_bytes, n_slots, decode_cus, ctypes.byref(h)), "uw_sched_create")
    _register(h.value, 0, 0, d_slots.device.index)
    return h.value


def uw_sched_destroy(handle: int) -> None:
    _handles.pop(handle, None)
    _lib.uw_sched_destroy(handle)


def uw_sched_prefetch(sched: int, handle: int, stream=None) -> int:
    _shape(handle)
    slot = ctypes.c_int(-1)
    _check(_lib.uw_sched_prefetch(sched, handle, _stream(stream), ctypes.byref(slot)), "uw_sched_prefetch")
    return slot.value


def uw_sched_gemm(sched: int, slot: int, handle: int, X, Y, stream=None) -> None:
    """Y = X W^T from the slot uw_sched_prefetch filled with `handle`'s matrix
    (the handle is only used to check the operands' shapes)."""
    batch = _gemm_operands(handle, X, Y)
    _check(_lib.uw_sched_gemm(sched, slot, X.data_ptr(), batch, X.stride(0), _dtype_code(X), Y.data_ptr(), Y.stride(0),
                              _dtype_code(Y), _stream(stream)), "uw_sched_gemm")


class DecodeAhead:
    """A decode-ahead scheduler with its slots (uw_sched_*): prefetch(m)
    starts decompressing m on the side stream, gemm(slot, m, X, Y) multiplies
    from the slot on the caller's stream."""

    def __init__(self, slot_bytes: int, n_slots: int = 2, decode_cus: int = 0, device: str = "cuda"):
        import torch
        self.slot_bytes = (slot_bytes + 255) // 256 * 256
        self.d_slots = torch.empty(self.slot_bytes * n_slots, dtype=torch.uint8, device=device)
        self.handle = uw_sched_create(self.d_slots, self.slot_bytes, n_slots, decode_cus)
        self.decode_cus = _lib.uw_sched_decode_cus(self.handle)

    def prefetch(self, m: "CompressedMatrix", stream=None) -> int:
        return uw_sched_prefetch(self.handle, m.handle, stream)

    def gemm(self, slot: int, m: "CompressedMatrix", X, Y, stream=None) -> None:
        uw_sched_gemm(self.handle, slot, m.handle, X, Y, stream)

    def close(self) -> None:
        if getattr(self, "handle", None):
            uw_sched_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# -- convenience owner of a device blob + handle -----------------------------

class CompressedMatrix:
    """A blob copied to the current CUDA device plus its library handle."""

    def __init__(self, blob: bytes, device: str = "cuda"):
        import torch
        self.blob = blob
        self.info = uw_blob_info(blob)
        # the blob, then room for the tables the library derives from it
        self.d_buf = torch.empty(uw_matrix_device_bytes(blob), dtype=torch.uint8, device=device)
        if self.d_buf.data_ptr() % 256:
            raise RuntimeError("device buffer is not 256-byte aligned")
        self.d_buf[: len(blob)].copy_(torch.frombuffer(bytearray(blob), dtype=torch.uint8))
        self.d_blob = self.d_buf[: len(blob)]
        self.handle = uw_matrix_create(blob, self.d_buf)
        self.rows, self.cols = self.info["rows"], self.info["cols"]
        self.palette = None

    @classmethod
    def from_weights(cls, w_bf16, device: str = "cuda", **opts) -> "CompressedMatrix":
        return cls(uw_encode(w_bf16, **opts), device)

    def decompress(self, out=None, stream=None):
        import torch
        if out is None:
            out = torch.empty(self.rows, self.cols, dtype=torch.bfloat16, device=self.d_blob.device)
        uw_decompress(self.handle, out, out.stride(0), stream)
        return out

    def gemv(self, x, y=None, out_dtype=None, stream=None):
        import torch
        if y is None:
            y = torch.empty(self.rows, dtype=out_dtype or torch.float32, device=x.device)
        uw_gemv_fused(self.handle, x, y, stream)
        return y

    def gemm(self, X, Y=None, variant: int = UW_VARIANT_AUTO, ws=None, out_dtype=None, stream=None):
        import torch
        if Y is None:
            Y = torch.empty(X.shape[0], self.rows, dtype=out_dtype or torch.float32, device=X.device)
        uw_gemm_fused(self.handle, X, Y, variant, ws, stream)
        return Y

    def workspace(self, batch: int, variant: int = UW_VARIANT_AUTO, autotune: bool = False):
        import torch
        n = uw_workspace_size(self.handle, batch, variant)
        if autotune:
            n += uw_autotune_scratch_size(self.handle, batch)
        return torch.empty(max(n, 256), dtype=torch.uint8, device=self.d_blob.device)

    def autotune(self, batch: int, ws=None, stream=None) -> dict:
        if ws is None:
            ws = self.workspace(batch, autotune=True)
        return uw_autotune(self.handle, batch, ws, stream)

    def transcode_palette(self, attach: bool = True, stream=None) -> "PaletteMatrix":
        """The direct-palette form of the same weights, built on the device
        from this blob (uw_palette_transcode); attached as a candidate of
        this matrix unless attach is False."""
        import torch
        n = uw_palette_transcode_size(self.handle)
        if n == 0:
            raise UwError(UW_ERR_UNSUPPORTED, "uw_palette_transcode_size", "this matrix cannot be transcoded")
        d = torch.empty(n, dtype=torch.uint8, device=self.d_buf.device)
        uw_palette_transcode(self.handle, d, stream)
        p = PaletteMatrix.__new__(PaletteMatrix)
        p.blob = None
        p.d_blob = d
        p.handle = uw_palette_create_transcoded(self.handle, d)
        p.rows, p.cols = self.rows, self.cols
        p.info = {"rows": self.rows, "cols": self.cols, "n_raw": self.info["n_raw_groups"], "bytes": n,
                  "ratio": n / (2 * self.rows * self.cols)}
        if attach:
            self.attach_palette(p)
        return p

    def attach_palette(self, p: "PaletteMatrix | None") -> None:
        uw_matrix_attach_palette(self.handle, p.handle if p is not None else None)
        self.palette = p

    def save_plans(self) -> str:
        return uw_plan_save(self.handle)

    def load_plans(self, text: str) -> None:
        uw_plan_load(self.handle, text)

    def close(self) -> None:
        if getattr(self, "handle", None):
            uw_matrix_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class PaletteMatrix:
    """A UWP1 blob copied to the current CUDA device plus its library handle."""

    def __init__(self, blob: bytes, device: str = "cuda"):
        import torch
        self.blob = blob
        self.info = uw_palette_info(blob)
        self.d_blob = torch.frombuffer(bytearray(blob), dtype=torch.uint8).to(device)
        if self.d_blob.data_ptr() % 256:
            raise RuntimeError("device blob is not 256-byte aligned")
        self.handle = uw_palette_create(blob, self.d_blob)
        self.rows, self.cols = self.info["rows"], self.info["cols"]

    @classmethod
    def from_weights(cls, w_bf16, device: str = "cuda") -> "PaletteMatrix":
        return cls(uw_palette_encode(w_bf16), device)

    def decompress(self, out=None, stream=None):
        import torch
        if out is None:
            out = torch.empty(self.rows, self.cols, dtype=torch.bfloat16, device=self.d_blob.device)
        uw_palette_decompress(self.handle, out, out.stride(0), stream)
        return out

    def gemv(self, x, y=None, out_dtype=None, stream=None):
        import torch
        if y is None:
            y = torch.empty(self.rows, dtype=out_dtype or torch.float32, device=x.device)
        uw_palette_gemv(self.handle, x, y, stream)
        return y

    def gemm(self, X, Y=None, out_dtype=None, stream=None):
        import torch
        if Y is None:
            Y = torch.empty(X.shape[0], self.rows, dtype=out_dtype or torch.float32, device=X.device)
        uw_palette_gemm(self.handle, X, Y, stream)
        return Y

    def close(self) -> None:
        if getattr(self, "handle", None):
            uw_palette_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
