"""ctypes binding of libmmq (include/mmq.h): argument marshalling only.

Every function keeps the C name and argument order.  Buffer arguments accept a
torch tensor (its data pointer is passed; dtype, contiguity and device are
checked) or a plain integer address (used by host-only dry-run contexts).
``stream`` defaults to torch's current stream on the context's device.
Failures raise :class:`MmqError` carrying the status and mmq_last_error().

The library must be built (``quantized_matmul_rmsnorm_amd.build.build()``);
importing this module without it raises -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmmq.so")

MMQ_OK = 0
MMQ_E_ARG = -1
MMQ_E_SHAPE = -2
MMQ_E_TYPE = -3
MMQ_E_OOM = -4
MMQ_E_DEAD_WRITE = -5
MMQ_E_HIP = -6
MMQ_E_DEVICE = -7
STATUS_NAMES = {0: "MMQ_OK", -1: "MMQ_E_ARG", -2: "MMQ_E_SHAPE", -3: "MMQ_E_TYPE",
                -4: "MMQ_E_OOM", -5: "MMQ_E_DEAD_WRITE", -6: "MMQ_E_HIP", -7: "MMQ_E_DEVICE"}

MMQ_Q4_K = 12
MMQ_Q5_K = 13
MMQ_Q6_K = 14
MMQ_CTX_SYNC_CHECK = 1
MMQ_CTX_DRYRUN = 2
MMQ_USE_GEMM = 1
MMQ_USE_GEMM_PACKED = 4
MMQ_USE_GEMV = 2
MMQ_PLANE_ROWS = 32
MMQ_WRITE_AUTO = -1
MMQ_FOREIGN_F32 = 1
MMQ_FOREIGN_QUANT = 2
MMQ_NOALLOC_MAX_COLS = 32768

# Every symbol include/mmq.h declares (checked by the CPU tests).
EXPORTS = [
    "mmq_create", "mmq_destroy", "mmq_last_error", "mmq_set_scratch_cap", "mmq_plane_rows",
    "mmq_register_weight", "mmq_weight_free", "mmq_weight_bytes",
    "mmq_quant_rms", "mmq_quant_swiglu", "mmq_quant_f32",
    "mmq_gemm_q4k", "mmq_gemm_q6k", "mmvq_q6k", "mmvq_q6k_noalloc", "mmvq_q4k", "mmvq_q5k",
    "mmq_gemv_q6k_f32", "mmq_decode_q6k",
    "mmq_register_foreign_consumer", "mmq_plane_only",
    "mmq_cache_clear", "mmq_cache_invalidate", "mmq_plane_export", "mmq_stats",
]


class MmqError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class mmq_stats_t(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int64) for name in (
        "launches_quant_rms", "launches_quant_swiglu", "launches_quant_f32",
        "launches_gemm_q4k", "launches_gemm_q6k", "launches_mmvq_q6k",
        "cache_hits", "cache_misses", "cache_refusals", "cache_entries",
        "plane_bytes", "weight_bytes", "launches_mmvq_q4k", "degraded_writes",
        "unfused_fallbacks", "small_n_gemv", "launches_mmvq_q5k", "launches_gemv_f32")]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


def _load():
    # One HIP runtime per process: torch ships its own libamdhip64.so.7 (same
    # SONAME as the system one libmmq.so links against).  Loading torch first
    # makes libmmq bind to torch's runtime, so tensors torch allocates and the
    # kernels libmmq launches live in one runtime; the reverse order leaves
    # torch on a runtime it was not built for ("No HIP GPUs are available").
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libmmq.so is not built ({LIB_PATH}); run "
                          "quantized_matmul_rmsnorm_amd.build.build() -- there is no fallback")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, I64, U, F = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint,
                       ctypes.c_float)
    sig = {
        "mmq_create": (I, [I, U, ctypes.POINTER(P)]),
        "mmq_destroy": (None, [P]),
        "mmq_last_error": (ctypes.c_char_p, []),
        "mmq_set_scratch_cap": (I, [P, I64]),
        "mmq_plane_rows": (I64, [I64]),
        "mmq_register_weight": (I, [P, I, I64, I64, P, U, ctypes.POINTER(P)]),
        "mmq_weight_free": (None, [P]),
        "mmq_weight_bytes": (I64, [P]),
        "mmq_quant_rms": (I, [P, P, P, P, I64, I64, F, I, P]),
        "mmq_quant_swiglu": (I, [P, P, P, P, I64, I64, I, P]),
        "mmq_quant_f32": (I, [P, P, I64, I64, P]),
        "mmq_gemm_q4k": (I, [P, P, P, I64, P, P]),
        "mmq_gemm_q6k": (I, [P, P, P, I64, P, P]),
        "mmvq_q6k": (I, [P, P, P, P, P]),
        "mmvq_q6k_noalloc": (I, [P, P, P, P, P]),
        "mmvq_q4k": (I, [P, P, P, P, P]),
        "mmvq_q5k": (I, [P, P, P, P, P]),
        "mmq_gemv_q6k_f32": (I, [P, P, P, P, P]),
        "mmq_decode_q6k": (I, [P, P, P, P, P]),
        "mmq_register_foreign_consumer": (I, [P, I]),
        "mmq_plane_only": (I, [P]),
        "mmq_cache_clear": (None, [P]),
        "mmq_cache_invalidate": (I, [P, P]),
        "mmq_plane_export": (I, [P, P, I64, I64, I, P, P, P, P]),
        "mmq_stats": (I, [P, ctypes.POINTER(mmq_stats_t)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def last_error() -> str:
    return lib.mmq_last_error().decode()


def _check(rc: int) -> int:
    if rc != MMQ_OK:
        raise MmqError(rc, last_error())
    return rc


def _ptr(buf, dtype=None):
    """Address of a torch tensor (checked) or a plain integer address."""
    if buf is None:
        return None
    if isinstance(buf, int):
        return buf
    import torch
    if not isinstance(buf, torch.Tensor):
        raise TypeError(f"expected a torch tensor or an int address, got {type(buf)}")
    if dtype is not None and buf.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {buf.dtype}")
    if not buf.is_contiguous():
        raise ValueError("tensor must be contiguous")
    if not buf.is_cuda:
        raise ValueError("tensor must be on the GPU")
    return buf.data_ptr()


def _f32():
    import torch
    return torch.float32


def _stream(stream):
    if stream is None:
        import torch
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ---- thin wrappers with the C names ----

def mmq_create(device: int = 0, flags: int = 0):
    out = ctypes.c_void_p()
    _check(lib.mmq_create(device, flags, ctypes.byref(out)))
    return out.value


def mmq_destroy(ctx) -> None:
    lib.mmq_destroy(ctx)


def mmq_set_scratch_cap(ctx, nbytes: int) -> None:
    _check(lib.mmq_set_scratch_cap(ctx, nbytes))


def mmq_plane_rows(n: int) -> int:
    return lib.mmq_plane_rows(n)


def mmq_register_weight(ctx, wtype: int, rows: int, cols: int, raw_host, uses: int = 0):
    """raw_host: a C-contiguous numpy uint8 array (or bytes) of the raw superblocks."""
    import numpy as np
    if isinstance(raw_host, (bytes, bytearray, memoryview)):
        arr = np.frombuffer(raw_host, dtype=np.uint8)
    else:
        arr = np.ascontiguousarray(raw_host, dtype=np.uint8)
    bpb = {MMQ_Q4_K: 144, MMQ_Q5_K: 176, MMQ_Q6_K: 210}.get(wtype)
    if bpb is not None and rows >= 1 and cols >= 256 and cols % 256 == 0 and \
            arr.size != rows * (cols // 256) * bpb:
        # the C call reads exactly that many bytes from the pointer it is given
        raise ValueError(f"raw_host holds {arr.size} bytes; {rows} x {cols} of type {wtype} "
                         f"needs {rows * (cols // 256) * bpb}")
    out = ctypes.c_void_p()
    _check(lib.mmq_register_weight(ctx, wtype, rows, cols, arr.ctypes.data_as(ctypes.c_void_p),
                                   uses, ctypes.byref(out)))
    return out.value


def mmq_weight_free(w) -> None:
    lib.mmq_weight_free(w)


def mmq_weight_bytes(w) -> int:
    return lib.mmq_weight_bytes(w)


def mmq_quant_rms(ctx, x, w, y, n: int, d: int, eps: float, write_y: int, stream=None):
    f = _f32() if not isinstance(x, int) else None
    return _check(lib.mmq_quant_rms(ctx, _ptr(x, f), _ptr(w, f), _ptr(y, f), n, d, eps,
                                    int(write_y), _stream(stream)))


def mmq_quant_swiglu(ctx, gate, up, y, n: int, d: int, write_y: int, stream=None):
    f = _f32() if not isinstance(gate, int) else None
    return _check(lib.mmq_quant_swiglu(ctx, _ptr(gate, f), _ptr(up, f), _ptr(y, f), n, d,
                                       int(write_y), _stream(stream)))


def mmq_quant_f32(ctx, x, n: int, d: int, stream=None):
    f = _f32() if not isinstance(x, int) else None
    return _check(lib.mmq_quant_f32(ctx, _ptr(x, f), n, d, _stream(stream)))


def mmq_gemm_q4k(ctx, w, a, n: int, out, stream=None):
    f = _f32() if not isinstance(a, int) else None
    return _check(lib.mmq_gemm_q4k(ctx, w, _ptr(a, f), n, _ptr(out, f), _stream(stream)))


def mmq_gemm_q6k(ctx, w, a, n: int, out, stream=None):
    f = _f32() if not isinstance(a, int) else None
    return _check(lib.mmq_gemm_q6k(ctx, w, _ptr(a, f), n, _ptr(out, f), _stream(stream)))


def mmvq_q6k(ctx, w, a, out, stream=None):
    f = _f32() if not isinstance(a, int) else None
    return _check(lib.mmvq_q6k(ctx, w, _ptr(a, f), _ptr(out, f), _stream(stream)))


def mmvq_q6k_noalloc(ctx, w, a, out, stream=None):
    f = _f32() if not isinstance(a, int) else None
    return _check(lib.mmvq_q6k_noalloc(ctx, w, _ptr(a, f), _ptr(out, f), _stream(stream)))


def mmvq_q4k(ctx, w, a, out, stream=None):
    f = _f32() if not isinstance(a, int) else None
    return _check(lib.mmvq_q4k(ctx, w, _ptr(a, f), _ptr(out, f), _stream(stream)))


def mmq_gemv_q6k_f32(ctx, w, x, out, stream=None):
    f = _f32() if not isinstance(x, int) else None
    return _check(lib.mmq_gemv_q6k_f32(ctx, w, _ptr(x, f), _ptr(out, f), _stream(stream)))


def mmq_decode_q6k(ctx, w, x, out, stream=None):
    f = _f32() if not isinstance(x, int) else None
    return _check(lib.mmq_decode_q6k(ctx, w, _ptr(x, f), _ptr(out, f), _stream(stream)))


MMQ_DECODE_F32_GATE = 16_000_000


def mmvq_q5k(ctx, w, a, out, stream=None):
    f = _f32() if not isinstance(a, int) else None
    return _check(lib.mmvq_q5k(ctx, w, _ptr(a, f), _ptr(out, f), _stream(stream)))


def mmq_register_foreign_consumer(ctx, kind: int) -> None:
    _check(lib.mmq_register_foreign_consumer(ctx, kind))


def mmq_plane_only(ctx) -> bool:
    return bool(lib.mmq_plane_only(ctx))


def mmq_cache_clear(ctx) -> None:
    lib.mmq_cache_clear(ctx)


def mmq_cache_invalidate(ctx, key) -> None:
    _check(lib.mmq_cache_invalidate(ctx, _ptr(key)))


def mmq_plane_export(ctx, key, n: int, d: int, include_pad: int, q, dq, s, stream=None):
    import torch
    return _check(lib.mmq_plane_export(ctx, _ptr(key), n, d, int(include_pad),
                                       _ptr(q, torch.int8), _ptr(dq, torch.float32),
                                       _ptr(s, torch.int32), _stream(stream)))


def mmq_stats(ctx) -> dict:
    st = mmq_stats_t()
    _check(lib.mmq_stats(ctx, ctypes.byref(st)))
    return st.as_dict()
