"""Double-precision CPU oracle for the FFT hot path (numpy front end of oracle.c).

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
benchmark's cpu_baseline leg may import this package.  It shares no code with
the HIP library in ``fourier_transform_amd`` and neither imports the other.

Every function takes the same values the GPU receives (complex64 / float32
arrays), widens them to float64 and returns float64 / complex128 results.
The arithmetic lives in ``oracle.c`` (recursive radix-2 decimation in time,
"High Performance Fourier Transforms on GPUs with GLSL", section 2.3.1,
Equation 9); this module only marshals arrays and arranges layouts.

Conventions (same sources as oracle.c):
  sign = -1 forward  X_k = sum_j x_j e^{-2 pi i jk/N}
  sign = +1 inverse  same sum with e^{+...}, NOT divided by N.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None
_I64 = ctypes.c_int64
_PTR = ctypes.c_void_p


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        lib.oracle_dft_brute.argtypes = [_PTR, _PTR, _I64, ctypes.c_int]
        lib.oracle_dft_brute.restype = None
        lib.oracle_fft.argtypes = [_PTR, _PTR, _I64, _I64, ctypes.c_int, ctypes.c_int]
        lib.oracle_fft_2d.argtypes = [_PTR, _PTR, _I64, _I64, _I64, ctypes.c_int,
                                      ctypes.c_int]
        lib.oracle_r2c.argtypes = [_PTR, _PTR, _I64, _I64, _I64, ctypes.c_int]
        lib.oracle_c2r.argtypes = [_PTR, _PTR, _I64, _I64, _I64, ctypes.c_int]
        lib.oracle_dft_synth_direct.argtypes = [_PTR, _PTR, _I64, _I64, _I64]
        lib.oracle_dft_synth_direct.restype = None
        lib.oracle_dft_analys_direct.argtypes = [_PTR, _PTR, _I64, _I64, _I64]
        lib.oracle_dft_analys_direct.restype = None
        lib.oracle_fftshift_index.argtypes = [_I64, _PTR]
        lib.oracle_ifftshift_index.argtypes = [_I64, _PTR]
        lib.oracle_fftshift_2d.argtypes = [_PTR, _PTR, _I64, _I64, _I64]
        lib.oracle_threads.argtypes = [ctypes.c_int]
        lib.oracle_dft.argtypes = [_PTR, _PTR, _I64, _I64, ctypes.c_int, ctypes.c_int]
        lib.oracle_dft_bins.argtypes = [_PTR, _I64, _PTR, _I64, _PTR, ctypes.c_int, ctypes.c_int]
        lib.oracle_dft2_bins.argtypes = [_PTR, _I64, _I64, _PTR, _PTR, _I64, _PTR, ctypes.c_int,
                                         ctypes.c_int]
        _LIB = lib
    return _LIB


def _c128(a):
    return np.ascontiguousarray(np.asarray(a), dtype=np.complex128)


def _f64(a):
    return np.ascontiguousarray(np.asarray(a), dtype=np.float64)


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments (rc={rc})")


def threads(requested: int = 0) -> int:
    """Number of threads the oracle uses for `requested` (<= 0: all online cores)."""
    return int(_lib().oracle_threads(requested))


def dft_brute(x, sign: int = -1):
    """The DFT written out, O(N^2), one row (Mota, section 2.2, Equation 5)."""
    x = _c128(x).reshape(-1)
    y = np.empty_like(x)
    _lib().oracle_dft_brute(_p(x), _p(y), x.size, sign)
    return y


def dft(x, sign: int = -1, nthreads: int = 0):
    """Batched DFT of any length over the last axis, by the definition
    (Mota, section 2.2, Equation 5), O(n^2) per row."""
    x = _c128(x)
    n = x.shape[-1]
    y = np.empty_like(x)
    _check(_lib().oracle_dft(_p(x), _p(y), n, x.size // max(n, 1), sign, nthreads), "dft")
    return y


def dft_bins(x, bins, sign: int = -1, nthreads: int = 0):
    """Selected outputs of the DFT of one row by the definition (O(n) per bin)."""
    x = _c128(x).reshape(-1)
    b = np.ascontiguousarray(np.asarray(bins, dtype=np.int64).reshape(-1))
    y = np.empty(b.size, np.complex128)
    _check(_lib().oracle_dft_bins(_p(x), x.size, _p(b), b.size, _p(y), sign, nthreads), "dft_bins")
    return y


def dft2_bins(x, k1, k2, sign: int = -1, nthreads: int = 0):
    """Selected outputs (k1[q], k2[q]) of the 2D DFT of one image by the definition."""
    x = _c128(x)
    ny, nx = x.shape
    a = np.ascontiguousarray(np.asarray(k1, dtype=np.int64).reshape(-1))
    b = np.ascontiguousarray(np.asarray(k2, dtype=np.int64).reshape(-1))
    y = np.empty(a.size, np.complex128)
    _check(_lib().oracle_dft2_bins(_p(x), ny, nx, _p(a), _p(b), a.size, _p(y), sign, nthreads),
           "dft2_bins")
    return y


def c2c(x, sign: int = -1, nthreads: int = 0):
    """Batched 1D transform over the last axis (recursive radix-2 DIT)."""
    x = _c128(x)
    n = x.shape[-1]
    y = np.empty_like(x)
    _check(_lib().oracle_fft(_p(x), _p(y), n, x.size // max(n, 1), sign, nthreads), "c2c")
    return y


def c2c_2d(x, sign: int = -1, nthreads: int = 0):
    """2D transform over the last two axes: rows, then columns (Equation 19);
    any sizes (the definition per axis when it is not a power of two)."""
    x = _c128(x)
    ny, nx = x.shape[-2], x.shape[-1]
    y = np.empty_like(x)
    _check(_lib().oracle_fft_2d(_p(x), _p(y), ny, nx, x.size // (ny * nx), sign,
                                nthreads), "c2c_2d")
    return y


def r2c(x, mmax: int = None, nthreads: int = 0):
    """Real analysis: forward transform of each real row, bins m = 0..mmax.

    Returns complex128 [batch..., mmax+1] (row-major).  mmax defaults to n/2.
    """
    x = _f64(x)
    n = x.shape[-1]
    if mmax is None:
        mmax = n // 2
    lead = x.shape[:-1]
    F = np.empty(lead + (mmax + 1,), np.complex128)
    _check(_lib().oracle_r2c(_p(x), _p(F), n, x.size // n, mmax, nthreads), "r2c")
    return F


def c2r(F, n: int, mmax: int = None, nthreads: int = 0):
    """Real synthesis from the Hermitian half spectrum F[..., 0..mmax] -> real rows of n.

    Im F_0 (and Im F_{n/2} when mmax = n/2) are ignored.  Unnormalised.
    """
    F = _c128(F)
    if mmax is None:
        mmax = F.shape[-1] - 1
    if F.shape[-1] != mmax + 1:
        raise ValueError("F must hold mmax+1 bins per row")
    lead = F.shape[:-1]
    x = np.empty(lead + (n,), np.float64)
    _check(_lib().oracle_c2r(_p(F), _p(x), n, F.size // (mmax + 1), mmax, nthreads),
           "c2r")
    return x


def dft_synth_direct(F, n: int, mmax: int):
    """Band-limited direct synthesis (fourier.ts dftSynthWGSL), f64, any n."""
    F = _c128(F)
    lead = F.shape[:-1]
    x = np.empty(lead + (n,), np.float64)
    _lib().oracle_dft_synth_direct(_p(F), _p(x), n, F.size // (mmax + 1), mmax)
    return x


def dft_analys_direct(x, mmax: int):
    """Band-limited direct analysis (fourier.ts dftAnalysWGSL), f64, any n."""
    x = _f64(x)
    n = x.shape[-1]
    lead = x.shape[:-1]
    F = np.empty(lead + (mmax + 1,), np.complex128)
    _lib().oracle_dft_analys_direct(_p(x), _p(F), n, x.size // n, mmax)
    return F


def fftshift_index(n: int):
    """Integer index map of the shift: out[i] = Y[idx[i]], idx[i] = (i - n//2) mod n
    (bin 0 moves to index n//2; for even n this is (i + n/2) mod n)."""
    idx = np.empty(n, np.int64)
    _check(_lib().oracle_fftshift_index(n, _p(idx)), "fftshift_index")
    return idx


def ifftshift_index(n: int):
    """Index map of the inverse rotation: out[i] = Y[idx[i]], idx[i] = (i + n//2) mod n."""
    idx = np.empty(n, np.int64)
    _check(_lib().oracle_ifftshift_index(n, _p(idx)), "ifftshift_index")
    return idx


def fftshift_2d(y):
    """Shift both of the last two axes: bin 0 to index floor(n/2) (numpy's fftshift)."""
    y = _c128(y)
    ny, nx = y.shape[-2], y.shape[-1]
    out = np.empty_like(y)
    _check(_lib().oracle_fftshift_2d(_p(y), _p(out), ny, nx, y.size // (ny * nx)),
           "fftshift_2d")
    return out
