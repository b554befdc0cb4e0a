"""Seeded synthetic inputs for the five transform workloads.

This module only draws random numbers and arranges them into arrays; it holds
none of the transform's arithmetic.  Both the GPU path (tests, bench) and the
double-precision oracle receive exactly the arrays built here.

Recipe (numpy ``default_rng(1000 + workload)``; values drawn in float64, then
rounded to float32):
  1  [8][1024] complex64, re and im i.i.d. U[-1, 1]            (forward C2C)
  2  [16384][4096] complex64, re and im i.i.d. U[-1, 1]        (forward + inverse)
  3  [32][2^22] complex64, re and im i.i.d. N(0, 1)            (forward, four-step)
  4  spectrum F, m-major [mmax+1][nlat] complex64 with nlat = 1024, nphi = 2048,
     mmax = 682: re and im i.i.d. N(0, 1), Im F_0 = 0          (C2R synthesis;
     the analysis input is that spectrum's synthesis, built by the caller)
  5  [8192][8192] complex64 image: sum of 16 complex sinusoids with integer
     frequencies (ky, kx) uniform in [0, 8192), unit amplitude and phase
     uniform in [0, 2 pi), plus complex noise with re and im i.i.d.
     N(0, 0.1^2)                                                (2D forward with
     the chessboard shift fused into the load)
  6  [65536][1000] complex64, re and im i.i.d. U[-1, 1]         (forward + inverse
     of a length that is not a power of two: the batched shape of workload 2,
     about 512 MiB, at n = 1000)

Random values are drawn with re and im interleaved (shape [..., 2]).
"""
import numpy as np

SEED_BASE = 1000

# full sizes of each workload
W1 = dict(n=1024, batch=8)
W2 = dict(n=4096, batch=16384)
W3 = dict(n=1 << 22, batch=32)
W4 = dict(nphi=2048, nlat=1024, mmax=682)
W5 = dict(ny=8192, nx=8192, tones=16, noise=0.1)
W6 = dict(n=1000, batch=65536)


def rng(workload: int, salt: int = 0):
    """Generator for a workload; `salt` gives independent streams for reduced sizes."""
    return np.random.default_rng(SEED_BASE + workload + 1000 * salt)


def _as_c64(pairs):
    return np.ascontiguousarray(pairs.astype(np.float32)).view(np.complex64)[..., 0]


def uniform_c64(shape, gen):
    """Complex64 array with re, im i.i.d. U[-1, 1]."""
    return _as_c64(gen.uniform(-1.0, 1.0, size=tuple(shape) + (2,)))


def normal_c64(shape, gen, sigma: float = 1.0):
    """Complex64 array with re, im i.i.d. N(0, sigma^2)."""
    return _as_c64(gen.normal(0.0, sigma, size=tuple(shape) + (2,)))


def workload1(n=W1["n"], batch=W1["batch"], salt=0):
    return uniform_c64((batch, n), rng(1, salt))


def workload2(n=W2["n"], batch=W2["batch"], salt=0):
    return uniform_c64((batch, n), rng(2, salt))


def workload3(n=W3["n"], batch=W3["batch"], salt=0):
    return normal_c64((batch, n), rng(3, salt))


def workload6(n=W6["n"], batch=W6["batch"], salt=0):
    return uniform_c64((batch, n), rng(6, salt))


def workload4_spectrum(nlat=W4["nlat"], mmax=W4["mmax"], salt=0):
    """m-major spectrum [mmax+1][nlat] complex64, Im F_0 = 0."""
    F = normal_c64((mmax + 1, nlat), rng(4, salt))
    F[0] = F[0].real
    return F


def workload5_params(tones=W5["tones"], n=W5["ny"], salt=0):
    """(ky, kx, phase) of the sinusoids, then the generator for the noise."""
    g = rng(5, salt)
    ky = g.integers(0, n, size=tones)
    kx = g.integers(0, n, size=tones)
    phase = g.uniform(0.0, 2.0 * np.pi, size=tones)
    return ky, kx, phase, g


def workload5(ny=W5["ny"], nx=W5["nx"], tones=W5["tones"], noise=W5["noise"], salt=0):
    """Sum of on-grid complex sinusoids plus complex normal noise, complex64 [ny][nx].

    Each tone is exp(i (2 pi (ky*i/ny + kx*j/nx) + phase)); the integer products
    are reduced modulo the length before scaling so the angles are exact in f64.
    """
    ky, kx, phase, g = workload5_params(tones, max(ny, nx), salt)
    ky = ky % ny
    kx = kx % nx
    img = np.zeros((ny, nx), np.complex128)
    iy = np.arange(ny, dtype=np.int64)
    ix = np.arange(nx, dtype=np.int64)
    for s in range(tones):
        a = np.exp(1j * (2.0 * np.pi * ((ky[s] * iy) % ny) / ny + phase[s]))
        b = np.exp(1j * (2.0 * np.pi * ((kx[s] * ix) % nx) / nx))
        img += np.outer(a, b)
    nz = g.normal(0.0, noise, size=(ny, nx, 2))
    img.real += nz[..., 0]
    img.imag += nz[..., 1]
    return img.astype(np.complex64)
