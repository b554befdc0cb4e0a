"""ctypes binding of libfft_amd.so (the C ABI declared in include/fft.h).

The functions carry the C names and only marshal arguments: device pointers
and the HIP stream are taken from torch tensors and torch's current stream.
Every transform step runs in the HIP kernels of the library; there is no CPU
fallback.  Loading fails loudly if the library has not been built.

    plan = fft_plan_create(4096, 16384, FFT_C2C, FFT_FORWARD)
    fft_exec(plan, x, y)          # x, y: torch.complex64 tensors on the GPU
    fft_plan_destroy(plan)
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfft_amd.so")

FFT_C2C, FFT_R2C, FFT_C2R, FFT_R2C_DIRECT, FFT_C2R_DIRECT = 0, 1, 2, 3, 4
FFT_FORWARD, FFT_INVERSE = -1, 1
FFT_OK, FFT_EINVAL, FFT_ENOTSUP, FFT_ENOMEM, FFT_EHIP, FFT_ESTATE = 0, -1, -2, -3, -4, -5
FFT_OPT_SHIFT, FFT_OPT_MMAX, FFT_OPT_SPEC_LAYOUT, FFT_OPT_REAL_PAIRS = 1, 2, 3, 4

_NAMES = {0: "FFT_OK", -1: "FFT_EINVAL", -2: "FFT_ENOTSUP", -3: "FFT_ENOMEM",
          -4: "FFT_EHIP", -5: "FFT_ESTATE"}

# every symbol include/fft.h declares
EXPORTS = ("fft_plan_create", "fft_plan_create_2d", "fft_plan_set", "fft_plan_get_sizes",
           "fft_exec", "fft_plan_destroy", "fft_last_error", "fft_max_single_pass_length",
           "fft_exec_noalloc")
FFT_NOALLOC_MAX_SCRATCH_BYTES = 256 << 20


class FFTError(RuntimeError):
    """A library call returned an error; `.code` is the fft_status value."""

    def __init__(self, code, msg):
        super().__init__(f"{_NAMES.get(code, code)}: {msg}")
        self.code = code


_lib = None


def load_library(path):
    """Open one build of the library (the default one, or the LDS-poison
    debug build) with the argument types of include/fft.h."""
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m fourier_transform_amd.build`")
    L = ctypes.CDLL(path)
    i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    L.fft_plan_create.argtypes = [i64, i64, ci, ci]
    L.fft_plan_create.restype = vp
    L.fft_plan_create_2d.argtypes = [i64, i64, i64, ci, ci]
    L.fft_plan_create_2d.restype = vp
    L.fft_plan_set.argtypes = [vp, ci, i64]
    L.fft_plan_set.restype = ci
    L.fft_plan_get_sizes.argtypes = [vp, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    L.fft_plan_get_sizes.restype = ci
    L.fft_exec.argtypes = [vp, vp, vp, vp]
    L.fft_exec.restype = ci
    L.fft_exec_noalloc.argtypes = [vp, vp, vp, vp]
    L.fft_exec_noalloc.restype = ci
    L.fft_plan_destroy.argtypes = [vp]
    L.fft_plan_destroy.restype = None
    L.fft_last_error.argtypes = [ctypes.POINTER(ctypes.c_char_p)]
    L.fft_last_error.restype = ci
    L.fft_max_single_pass_length.argtypes = []
    L.fft_max_single_pass_length.restype = i64
    return L


def lib():
    """Load libfft_amd.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        _lib = load_library(LIB_PATH)
    return _lib


def fft_last_error():
    """(code, message) of the last call on this thread."""
    msg = ctypes.c_char_p()
    code = lib().fft_last_error(ctypes.byref(msg))
    return code, (msg.value or b"").decode()


def _raise_last():
    code, msg = fft_last_error()
    raise FFTError(code, msg)


def _check(rc):
    if rc != FFT_OK:
        _raise_last()
    return rc


def fft_plan_create(n, batch, kind=FFT_C2C, sign=FFT_FORWARD):
    """Plan `batch` transforms of length n; returns an opaque handle (int)."""
    p = lib().fft_plan_create(int(n), int(batch), int(kind), int(sign))
    if not p:
        _raise_last()
    return p


def fft_plan_create_2d(ny, nx, batch=1, kind=FFT_C2C, sign=FFT_FORWARD):
    """Plan `batch` 2D transforms of ny x nx; returns an opaque handle (int)."""
    p = lib().fft_plan_create_2d(int(ny), int(nx), int(batch), int(kind), int(sign))
    if not p:
        _raise_last()
    return p


# (in_bytes, out_bytes) per plan handle, for the size checks of fft_exec
# without a library call per exec; dropped when an option changes or the plan
# is destroyed
_sizes = {}


def fft_plan_set(plan, option, value):
    _sizes.pop(plan, None)
    return _check(lib().fft_plan_set(plan, int(option), int(value)))


def fft_plan_get_sizes(plan):
    """(in_bytes, out_bytes) the plan reads and writes."""
    a, b = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().fft_plan_get_sizes(plan, ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def _ptr_and_bytes(t):
    if isinstance(t, int):
        return t, None
    if not t.is_cuda:
        raise ValueError("fft_exec needs device tensors")
    if not t.is_contiguous():
        raise ValueError("fft_exec needs contiguous tensors")
    return t.data_ptr(), t.numel() * t.element_size()


def fft_exec(plan, x, y, stream=None):
    """Enqueue the plan on `stream` (default: torch's current stream).

    x, y: contiguous device tensors (or raw device pointers as ints).  Tensor
    sizes are checked against fft_plan_get_sizes before the call.
    """
    px, py, stream = _exec_args(plan, x, y, stream)
    return _check(lib().fft_exec(plan, px, py, stream))


def _exec_args(plan, x, y, stream):
    px, bx = _ptr_and_bytes(x)
    py, by = _ptr_and_bytes(y)
    sizes = _sizes.get(plan)
    if sizes is None:
        sizes = _sizes[plan] = fft_plan_get_sizes(plan)
    need_in, need_out = sizes
    if bx is not None and bx < need_in:
        raise ValueError(f"input holds {bx} bytes, plan reads {need_in}")
    if by is not None and by < need_out:
        raise ValueError(f"output holds {by} bytes, plan writes {need_out}")
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    elif not isinstance(stream, int):
        stream = stream.cuda_stream
    return px, py, stream


def fft_exec_noalloc(plan, x, y, stream=None):
    """fft_exec with the library's static per-device scratch instead of the
    plan's (include/fft.h): no device allocation; calls on one device that
    overlap in time race on that buffer."""
    px, py, stream = _exec_args(plan, x, y, stream)
    return _check(lib().fft_exec_noalloc(plan, px, py, stream))


def fft_plan_destroy(plan):
    _sizes.pop(plan, None)
    lib().fft_plan_destroy(plan)


def fft_max_single_pass_length():
    return int(lib().fft_max_single_pass_length())
