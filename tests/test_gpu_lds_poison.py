"""The LDS-poison debug build against the oracle.

libfft_amd_poison.so is the library compiled with FFTAMD_LDS_POISON=1: every
kernel first fills its LDS arrays with NaNs.  A kernel that reads LDS nothing
in the workgroup has written (a missing barrier, a wrong index, a pad element)
then puts NaNs in its output, which fails the comparison with the oracle.
One case of every kernel family runs here, in both directions where that
selects another kernel, and each is run twice and compared bit for bit.
"""
import os

import numpy as np
import pytest

import oracle
from fourier_transform_amd import build as B
from fourier_transform_amd import fft as F
from fourier_transform_amd import workloads as W

from gpu_helpers import c2c, c2c_2d, c2r, direct_analysis, direct_synthesis, r2c, rel_l2, say

pytestmark = pytest.mark.gpu
TOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _poison_library():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    if not os.path.exists(B.POISON_LIB):
        pytest.fail(f"{B.POISON_LIB} is missing: python -m fourier_transform_amd.build --variant all")
    saved = F._lib
    F._lib = F.load_library(B.POISON_LIB)
    try:
        yield
    finally:
        torch.cuda.synchronize()
        F._lib = saved


def _twice(fn):
    a, b = fn(), fn()
    assert np.array_equal(np.asarray(a).view(np.uint32), np.asarray(b).view(np.uint32))
    return a


C2C_CASES = [
    # single-pass rows (complex and split exchanges, wave-local and workgroup lines, rows
    # of 4-32 points staged through LDS)
    (2, 3), (16, 5), (8, 300), (32, 200), (64, 7), (1024, 8), (4096, 33), (8192, 3), (16384, 2),
    # four-step
    (1 << 15, 3), (1 << 20, 2),
    # mixed radix (one butterfly of <= 16, two of <= 8, two of <= 16 above 8192), Rader,
    # chirp (one kernel on a power of two up to 16384 and at 32768, one on a mixed-radix
    # length, three passes); the stage twiddles in LDS: rows of 3+ and 4 lines per
    # workgroup (360, 1000), Rader (1009), chirp on a mixed length (34), the four-step's
    # 8-column tiles (20000) and 16-column tiles with the two-level table in LDS (24576)
    (1000, 9), (360, 11), (12, 700), (6000, 3), (7776, 3), (12000, 2), (15360, 3), (1009, 5), (9001, 2), (97, 13), (17, 600), (1019, 4), (34, 300),
    (10001, 2), (1034, 3), (20011, 2), (20000, 2), (24576, 2),
]


@pytest.mark.parametrize("n,batch", C2C_CASES)
@pytest.mark.parametrize("sign", [-1, 1])
def test_poison_c2c(n, batch, sign):
    say(f"poison build: c2c n={n} batch={batch} sign={sign}")
    x = W.uniform_c64((batch, n), np.random.default_rng(n + batch))
    y = _twice(lambda: c2c(x, sign))
    assert rel_l2(y, oracle.dft(x, sign) if n & (n - 1) else oracle.c2c(x, sign)) <= TOL


@pytest.mark.parametrize("n,shift", [(4096, 1), (1 << 16, 1), (1001, 1), (1009, 2), (10001, 1)])
def test_poison_c2c_shift_in_place(n, shift):
    say(f"poison build: c2c n={n} shift={shift} in place")
    x = W.uniform_c64((3, n), np.random.default_rng(n))
    y = _twice(lambda: c2c(x, -1, shift=shift, inplace=True))
    want = oracle.dft(x, -1) if n & (n - 1) else oracle.c2c(x, -1)
    idx = oracle.fftshift_index(n) if shift == 1 else oracle.ifftshift_index(n)
    assert rel_l2(y, want[:, idx]) <= TOL


# other sizes: mixed-radix columns with one (100) and two (7776) butterflies
# per thread, power-of-two columns of a non-power-of-two image (64 x 1000),
# and the transposing form (1009 rows: a Rader length)
@pytest.mark.parametrize("ny,nx,batch", [(256, 512, 2), (1024, 1024, 1), (8192, 2048, 1), (8192, 64, 1),
                                         (100, 60, 2), (7776, 6, 1), (64, 1000, 1), (1009, 30, 1),
                                         (4096, 512, 1)])
def test_poison_2d(ny, nx, batch):
    say(f"poison build: 2d {ny}x{nx} batch={batch}")
    x = W.normal_c64((batch, ny, nx), np.random.default_rng(ny + nx))
    y = _twice(lambda: c2c_2d(x, -1))
    assert rel_l2(y, oracle.c2c_2d(x, -1)) <= TOL


@pytest.mark.parametrize("n,mmax,pairs", [(32, 16, False), (8, 4, True), (64, 32, False), (2048, 682, False), (2048, 682, True), (1000, 300, False),
                                          (999, 499, False)])
def test_poison_real(n, mmax, pairs):
    say(f"poison build: real n={n} mmax={mmax} pairs={pairs}")
    batch = 6
    g = np.random.default_rng(n)
    Fs = (g.standard_normal((batch, mmax + 1)) + 1j * g.standard_normal((batch, mmax + 1))).astype(np.complex64)
    Fs[:, 0] = Fs[:, 0].real
    if mmax == n // 2 and n % 2 == 0:
        Fs[:, mmax] = Fs[:, mmax].real
    xr = _twice(lambda: c2r(Fs.T.copy(), n, batch, mmax=mmax, mmajor=True, pairs=pairs))
    assert rel_l2(xr, oracle.c2r(Fs, n, mmax)) <= TOL
    x = xr.astype(np.float32)
    Z = _twice(lambda: r2c(x, mmax=mmax, mmajor=True, pairs=pairs))
    assert rel_l2(Z.T, oracle.r2c(x, mmax)) <= TOL


@pytest.mark.parametrize("n,batch,mmax", [(100, 5, 40), (2048, 300, 682)])
def test_poison_direct(n, batch, mmax):
    say(f"poison build: direct sums n={n} batch={batch} mmax={mmax}")
    g = np.random.default_rng(n)
    x = g.uniform(-1, 1, (batch, n)).astype(np.float32)
    Fs = _twice(lambda: direct_analysis(x, mmax=mmax))
    assert rel_l2(Fs, oracle.dft_analys_direct(x, mmax)) <= TOL
    xs = _twice(lambda: direct_synthesis(Fs, n, batch, mmax=mmax))
    assert rel_l2(xs, oracle.dft_synth_direct(Fs, n, mmax)) <= TOL
