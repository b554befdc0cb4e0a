"""Pins for the double-precision oracle (CPU only).

Each test ties the oracle to something other than itself: the DFT written out
as a double sum, the worked example printed by the pages, closed forms,
invariants, and a third-party FFT (numpy's pocketfft).  They are chosen so
that a dropped term, a wrong sign or index, or a transposed operand anywhere
in the oracle fails at least one of them.
"""
import os

import numpy as np
import pytest

import oracle
from fourier_transform_amd import workloads

HERE = os.path.dirname(os.path.abspath(__file__))


def rel(a, b):
    a = np.asarray(a, np.complex128)
    b = np.asarray(b, np.complex128)
    return float(np.linalg.norm((a - b).ravel()) / max(np.linalg.norm(b.ravel()), 1e-300))


def crand(shape, seed):
    g = np.random.default_rng(seed)
    return g.normal(size=shape) + 1j * g.normal(size=shape)


# --------------------------------------------------------------------------
# the definition written out (Mota, section 2.2, Equation 5) -- independent of
# the oracle's C code: a numpy matrix built from integer exponents
# --------------------------------------------------------------------------
def dft_matrix(n, sign):
    jk = np.outer(np.arange(n), np.arange(n)) % n
    return np.exp(sign * 2j * np.pi * jk / n)


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64])
@pytest.mark.parametrize("sign", [-1, 1])
def test_brute_force_matches_definition(n, sign):
    x = crand(n, 10 + n)
    assert rel(oracle.dft_brute(x, sign), dft_matrix(n, sign) @ x) < 1e-13


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64])
@pytest.mark.parametrize("sign", [-1, 1])
def test_fft_matches_brute_force(n, sign):
    x = crand((3, n), 20 + n)
    y = oracle.c2c(x, sign)
    for r in range(3):
        assert rel(y[r], oracle.dft_brute(x[r], sign)) < 1e-12
        assert rel(y[r], dft_matrix(n, sign) @ x[r]) < 1e-12


@pytest.mark.parametrize("n", [1, 7, 64, 1000])
@pytest.mark.parametrize("sign", [-1, 1])
def test_selected_bins_match_definition(n, sign):
    x = crand(n, 30 + n)
    bins = np.unique(np.array([0, 1, n // 2, n - 1, (5 * n) // 7]) % n)
    assert rel(oracle.dft_bins(x, bins, sign), (dft_matrix(n, sign) @ x)[bins]) < 1e-12
    assert rel(oracle.dft_bins(x, bins, sign, nthreads=1), oracle.dft_bins(x, bins, sign, nthreads=3)) < 1e-13


@pytest.mark.parametrize("ny,nx", [(1, 1), (4, 8), (16, 2), (32, 32)])
@pytest.mark.parametrize("sign", [-1, 1])
def test_selected_2d_bins_match_double_sum(ny, nx, sign):
    x = crand((ny, nx), ny + 5 * nx)
    want = dft_matrix(ny, sign) @ x @ dft_matrix(nx, sign)
    k1 = np.array([0, ny - 1, ny // 2, 1 % ny])
    k2 = np.array([0, nx // 3, nx - 1, nx // 2])
    assert rel(oracle.dft2_bins(x, k1, k2, sign), want[k1, k2]) < 1e-12


def test_printed_n8_example():
    """Mota, section 2.2 EXAMPLE (after Equation 6): one cosine period, N = 8."""
    rows = np.loadtxt(os.path.join(HERE, "golden", "mota_dft_n8_example.txt"))
    x_printed = rows[:, 1]
    X_printed = rows[:, 2] + 1j * rows[:, 3]
    # with the printed 3-decimal samples the page's integer outputs are the
    # rounded transform (X_1 = X_7 = 2 + 2.828 * 0.707 = 3.9997)
    X = oracle.c2c(x_printed.astype(np.complex128), -1)
    assert np.array_equal(np.round(X.real), X_printed.real)
    assert np.max(np.abs(X.imag)) < 1e-12
    assert abs(X[1] - (2 + 4 * 0.707 * np.sqrt(0.5))) < 1e-12
    # with exact cosine samples the transform is exactly [0, 4, 0, ..., 0, 4]
    xe = np.cos(2 * np.pi * np.arange(8) / 8)
    assert np.max(np.abs(oracle.c2c(xe.astype(np.complex128), -1) - X_printed)) < 1e-12


def test_dft4_equation7():
    """Mota, section 2.3, Equation 7: the four outputs of a length-4 forward DFT."""
    x = crand(4, 4)
    x0, x1, x2, x3 = x
    want = np.array([x0 + x1 + x2 + x3,
                     x0 - 1j * x1 - x2 + 1j * x3,
                     x0 - x1 + x2 - x3,
                     x0 + 1j * x1 - x2 - 1j * x3])
    assert rel(oracle.c2c(x, -1), want) < 1e-15
    # the inverse has the opposite sign on the odd terms
    want_inv = np.array([x0 + x1 + x2 + x3,
                         x0 + 1j * x1 - x2 - 1j * x3,
                         x0 - x1 + x2 - x3,
                         x0 - 1j * x1 - x2 + 1j * x3])
    assert rel(oracle.c2c(x, +1), want_inv) < 1e-15


@pytest.mark.parametrize("n", [16, 1024, 1 << 14])
@pytest.mark.parametrize("sign", [-1, 1])
def test_impulse_closed_form(n, sign):
    for n0 in (0, 1, 3, n // 2 + 1, n - 1):
        x = np.zeros(n, np.complex128)
        x[n0] = 1.0
        k = np.arange(n)
        want = np.exp(sign * 2j * np.pi * ((k * n0) % n) / n)
        assert np.max(np.abs(oracle.c2c(x, sign) - want)) < 1e-12


@pytest.mark.parametrize("n", [8, 4096])
def test_pure_tone_closed_form(n):
    for k0 in (0, 1, 5, n - 1):
        j = np.arange(n)
        x = np.exp(2j * np.pi * ((k0 * j) % n) / n)
        want = np.zeros(n, np.complex128)
        want[k0] = n
        assert np.max(np.abs(oracle.c2c(x, -1) - want)) < 1e-9 * n
        # and the inverse of a tone at -k0 is the same spike
        assert np.max(np.abs(oracle.c2c(np.conj(x), +1) - want)) < 1e-9 * n


@pytest.mark.parametrize("n", [2, 256, 1 << 16])
def test_parseval_linearity_roundtrip(n):
    x = crand((2, n), n)
    z = crand((2, n), n + 1)
    X = oracle.c2c(x, -1)
    assert abs(np.sum(np.abs(X) ** 2) - n * np.sum(np.abs(x) ** 2)) < 1e-10 * n * np.sum(
        np.abs(x) ** 2)
    a, b = 0.3 - 1.7j, -2.1 + 0.4j
    assert rel(oracle.c2c(a * x + b * z, -1), a * X + b * oracle.c2c(z, -1)) < 1e-13
    assert rel(oracle.c2c(X, +1) / n, x) < 1e-13


@pytest.mark.parametrize("n", [2, 8, 1024])
def test_shift_theorem(n):
    """Chessboard page: multiplying x_n by (-1)^n rotates the spectrum by N/2."""
    x = crand(n, 7 * n)
    chk = x * (-1.0) ** np.arange(n)
    assert rel(oracle.c2c(chk, -1), np.roll(oracle.c2c(x, -1), n // 2)) < 1e-13
    idx = oracle.fftshift_index(n)
    assert rel(oracle.c2c(chk, -1), oracle.c2c(x, -1)[idx]) < 1e-13


@pytest.mark.parametrize("n", [2, 4, 6, 8, 1024, 4096])
def test_fftshift_index_matches_numpy_exactly(n):
    a = np.arange(n)
    assert np.array_equal(oracle.fftshift_index(n), np.fft.fftshift(a))
    assert np.array_equal(oracle.fftshift_index(n), np.fft.ifftshift(a))


@pytest.mark.parametrize("n", [1, 3, 5, 7, 9, 15, 1001])
def test_fftshift_index_odd_matches_numpy_exactly(n):
    """Odd lengths: bin 0 moves to index (n-1)/2, as numpy's fftshift does
    (and unlike its ifftshift, which differs for odd n)."""
    a = np.arange(n)
    assert np.array_equal(oracle.fftshift_index(n), np.fft.fftshift(a))
    assert oracle.fftshift_index(n)[(n - 1) // 2] == 0


def test_fftshift_2d_matches_numpy_exactly():
    y = crand((2, 6, 8), 3)
    assert np.array_equal(oracle.fftshift_2d(y), np.fft.fftshift(y, axes=(-2, -1)))


def test_hermitian_symmetry_of_real_input():
    n = 512
    x = np.random.default_rng(5).normal(size=n)
    X = oracle.c2c(x.astype(np.complex128), -1)
    k = np.arange(1, n)
    assert np.max(np.abs(X[n - k] - np.conj(X[k]))) < 1e-11
    assert abs(X[0].imag) < 1e-12 and abs(X[n // 2].imag) < 1e-11


@pytest.mark.parametrize("n", [4, 64, 2048])
def test_r2c_is_forward_of_real_row(n):
    x = np.random.default_rng(n).normal(size=(3, n))
    F = oracle.r2c(x)
    assert F.shape == (3, n // 2 + 1)
    for r in range(3):
        assert rel(F[r], (dft_matrix(n, -1) @ x[r])[: n // 2 + 1]) < 1e-12
    F5 = oracle.r2c(x, mmax=1)
    assert F5.shape == (3, 2) and rel(F5, F[:, :2]) < 1e-15


@pytest.mark.parametrize("n,mmax", [(8, 4), (16, 3), (64, 20), (2048, 682)])
def test_c2r_band_limited_round_trip(n, mmax):
    """R2C(C2R(F))_m = N F_m for m <= mmax < N/2 (fourier.ts conventions)."""
    g = np.random.default_rng(n + mmax)
    F = g.normal(size=(4, mmax + 1)) + 1j * g.normal(size=(4, mmax + 1))
    if 2 * mmax < n:
        F[:, 0] = F[:, 0].real
        x = oracle.c2r(F, n, mmax)
        assert rel(oracle.r2c(x, mmax), n * F) < 1e-12
    else:  # mmax = n/2: bins 0 and n/2 are real
        F[:, 0] = F[:, 0].real
        F[:, -1] = F[:, -1].real
        x = oracle.c2r(F, n, mmax)
        assert rel(oracle.r2c(x, mmax), n * F) < 1e-12


def test_c2r_matches_explicit_hermitian_inverse():
    n, mmax = 32, 10
    g = np.random.default_rng(9)
    F = g.normal(size=mmax + 1) + 1j * g.normal(size=mmax + 1)
    X = np.zeros(n, np.complex128)
    X[0] = F[0].real                      # Im F_0 is ignored
    X[1:mmax + 1] = F[1:]
    X[n - np.arange(1, mmax + 1)] = np.conj(F[1:])
    want = (dft_matrix(n, +1) @ X).real
    assert np.max(np.abs(oracle.c2r(F, n, mmax) - want)) < 1e-12


@pytest.mark.parametrize("n,mmax", [(16, 5), (64, 31), (48, 20), (30, 7)])
def test_direct_band_limited_sums_match(n, mmax):
    """fourier.ts dft path: direct sums equal the FFT path (power-of-two n) and
    invert each other up to the factor n for any n."""
    g = np.random.default_rng(n * mmax)
    F = g.normal(size=(2, mmax + 1)) + 1j * g.normal(size=(2, mmax + 1))
    F[:, 0] = F[:, 0].real
    x = oracle.dft_synth_direct(F, n, mmax)
    assert rel(oracle.dft_analys_direct(x, mmax), n * F) < 1e-12
    if n & (n - 1) == 0:
        assert np.max(np.abs(x - oracle.c2r(F, n, mmax))) < 1e-11
        assert rel(oracle.dft_analys_direct(x, mmax), oracle.r2c(x, mmax)) < 1e-12


@pytest.mark.parametrize("ny,nx", [(2, 2), (8, 8), (16, 4), (4, 32)])
@pytest.mark.parametrize("sign", [-1, 1])
def test_2d_matches_double_sum(ny, nx, sign):
    """Mota, section 2.7, Equation 19 written out as a double sum."""
    x = crand((2, ny, nx), ny * nx)
    want = np.einsum("rm,bmn,cn->brc", dft_matrix(ny, sign), x, dft_matrix(nx, sign))
    assert rel(oracle.c2c_2d(x, sign), want) < 1e-12


def test_2d_separability():
    n = 64
    u, v = crand(n, 1), crand(n, 2)
    got = oracle.c2c_2d(np.outer(u, v), -1)
    assert rel(got, np.outer(oracle.c2c(u, -1), oracle.c2c(v, -1))) < 1e-13


@pytest.mark.parametrize("n", [2, 16, 512, 1 << 15])
def test_third_party_numpy_agreement(n):
    """Cross-check against numpy's pocketfft (a third-party library, not a dependency)."""
    x = crand((2, n), 3 * n)
    assert rel(oracle.c2c(x, -1), np.fft.fft(x, axis=-1)) < 1e-13
    assert rel(oracle.c2c(x, +1), n * np.fft.ifft(x, axis=-1)) < 1e-13


def test_rejects_invalid_sizes():
    with pytest.raises(ValueError):
        oracle.c2c(np.zeros(6, np.complex128))
    with pytest.raises(ValueError):
        oracle.fftshift_index(0)
    with pytest.raises(ValueError):
        oracle.r2c(np.zeros(8), mmax=5)


def test_threads_do_not_change_results():
    x = crand((7, 256), 11)
    assert np.array_equal(oracle.c2c(x, -1, nthreads=1), oracle.c2c(x, -1, nthreads=3))
    x2 = crand((2, 32, 16), 12)
    assert np.array_equal(oracle.c2c_2d(x2, -1, nthreads=1), oracle.c2c_2d(x2, -1, nthreads=5))


# --------------------------------------------------------------------------
# closed forms at workload shapes (reduced sizes so the CPU suite stays fast)
# --------------------------------------------------------------------------
def test_workload5_peaks_closed_form():
    """A 2D image of on-grid tones transforms to spikes of height ny*nx*e^{i phase};
    after the shift the spike for (ky, kx) sits at ((ky + ny/2) % ny, (kx + nx/2) % nx)."""
    ny = nx = 64
    img = workloads.workload5(ny=ny, nx=nx, tones=4, noise=0.0, salt=1)
    ky, kx, phase, _ = workloads.workload5_params(tones=4, n=ny, salt=1)
    Y = oracle.fftshift_2d(oracle.c2c_2d(img, -1))
    want = np.zeros((ny, nx), np.complex128)
    for s in range(4):
        want[(ky[s] % ny + ny // 2) % ny, (kx[s] % nx + nx // 2) % nx] += ny * nx * np.exp(
            1j * phase[s])
    # the image was rounded to complex64 (about 6e-8 relative per sample)
    assert rel(Y, want) < 1e-6


def test_workload_generators_are_deterministic():
    a = workloads.workload1()
    b = workloads.workload1()
    assert a.dtype == np.complex64 and a.shape == (8, 1024)
    assert np.array_equal(a, b)
    assert np.max(np.abs(a.real)) <= 1 and np.max(np.abs(a.imag)) <= 1
    F = workloads.workload4_spectrum()
    assert F.shape == (683, 1024) and np.all(F[0].imag == 0)


# --------------------------------------------------------------------------
# lengths that are not powers of two: the definition with tabulated factors
# --------------------------------------------------------------------------
GENERAL_N = [1, 2, 3, 5, 6, 7, 9, 12, 15, 30, 63, 100, 127, 1000, 1001]


@pytest.mark.parametrize("n", [n for n in GENERAL_N if n <= 64])
@pytest.mark.parametrize("sign", [-1, 1])
def test_dft_any_length_matches_brute_force(n, sign):
    """Against the double sum that evaluates every factor anew (oracle_dft_brute)."""
    x = crand((3, n), 31 * n)
    want = np.stack([oracle.dft_brute(r, sign) for r in x])
    assert rel(oracle.dft(x, sign), want) < 1e-13


@pytest.mark.parametrize("n", GENERAL_N)
def test_dft_any_length_third_party(n):
    """numpy's pocketfft (mixed radix / Bluestein inside) as a third-party check."""
    x = crand((2, n), 5 * n + 1)
    assert rel(oracle.dft(x, -1), np.fft.fft(x, axis=-1)) < 1e-12
    assert rel(oracle.dft(x, +1), n * np.fft.ifft(x, axis=-1)) < 1e-12


@pytest.mark.parametrize("n", [3, 7, 100, 1001])
def test_dft_any_length_closed_forms(n):
    """Impulse at j0 -> e^{sign 2 pi i k j0/n}; tone e^{2 pi i k0 j/n} -> n at bin k0
    (forward); Parseval."""
    j0, k0 = n // 3, (2 * n) // 5
    imp = np.zeros(n, np.complex128)
    imp[j0] = 1.0
    k = np.arange(n)
    for sign in (-1, 1):
        assert rel(oracle.dft(imp, sign), np.exp(sign * 2j * np.pi * ((k * j0) % n) / n)) < 1e-13
    tone = np.exp(2j * np.pi * ((k0 * k) % n) / n)
    want = np.zeros(n, np.complex128)
    want[k0] = n
    assert np.max(np.abs(oracle.dft(tone, -1) - want)) < 1e-9 * n
    x = crand(n, n)
    assert abs(np.sum(np.abs(oracle.dft(x, -1)) ** 2) - n * np.sum(np.abs(x) ** 2)) < 1e-9 * n * n


@pytest.mark.parametrize("n", [2, 8, 64, 1024])
def test_dft_any_length_agrees_with_radix2(n):
    """Two independent algorithms of the oracle agree at powers of two."""
    x = crand((2, n), 17 * n)
    for sign in (-1, 1):
        assert rel(oracle.dft(x, sign), oracle.c2c(x, sign)) < 1e-12


@pytest.mark.parametrize("n", [3, 5, 9, 101, 1001])
def test_shift_theorem_odd(n):
    """Chessboard page, odd case: multiplying x_j by e^{-sign 2 pi i M j/n},
    M = (n-1)/2, moves bin 0 to index M -- the index map of the oracle."""
    x = crand(n, 3 * n)
    m = (n - 1) // 2
    j = np.arange(n)
    idx = oracle.fftshift_index(n)
    for sign in (-1, 1):
        ramp = np.exp(-sign * 2j * np.pi * ((m * j) % n) / n)
        assert rel(oracle.dft(x * ramp, sign), oracle.dft(x, sign)[idx]) < 1e-12


@pytest.mark.parametrize("n", [1, 2, 3, 6, 7, 9, 1001, 1024])
def test_ifftshift_index_matches_numpy_exactly(n):
    a = np.arange(n)
    assert np.array_equal(oracle.ifftshift_index(n), np.fft.ifftshift(a))
    # it undoes the shift
    assert np.array_equal(np.arange(n)[oracle.fftshift_index(n)][oracle.ifftshift_index(n)], a)


@pytest.mark.parametrize("n", [3, 5, 101, 1001])
def test_ishift_theorem_odd(n):
    """Multiplying x_j by e^{+sign 2 pi i M j/n}, M = floor(n/2), rotates the
    spectrum the other way: the ifftshift index map."""
    x = crand(n, 5 * n)
    m = n // 2
    j = np.arange(n)
    idx = oracle.ifftshift_index(n)
    for sign in (-1, 1):
        ramp = np.exp(sign * 2j * np.pi * ((m * j) % n) / n)
        assert rel(oracle.dft(x * ramp, sign), oracle.dft(x, sign)[idx]) < 1e-12


# --------------------------------------------------------------------------
# real transforms at lengths that are not powers of two (the definition)
# --------------------------------------------------------------------------
REAL_ANY_N = [3, 6, 7, 10, 15, 100, 999, 1000]


@pytest.mark.parametrize("n", REAL_ANY_N)
def test_r2c_any_length(n):
    """Against numpy's rfft (third party) and the band-limited direct analysis
    (the oracle's separate fourier.ts sums)."""
    x = np.random.default_rng(n).normal(size=(3, n))
    assert rel(oracle.r2c(x), np.fft.rfft(x, axis=-1)) < 1e-12
    m = (n - 1) // 2
    assert rel(oracle.r2c(x, m), oracle.dft_analys_direct(x, m)) < 1e-12


@pytest.mark.parametrize("n", REAL_ANY_N)
def test_c2r_any_length(n):
    """Against the direct synthesis sums, numpy's irfft for the full half
    spectrum, and the band-limited round trip R2C(C2R(F)) = n F."""
    g = np.random.default_rng(n + 1)
    m = (n - 1) // 2
    F = g.normal(size=(3, m + 1)) + 1j * g.normal(size=(3, m + 1))
    F[:, 0] = F[:, 0].real
    x = oracle.c2r(F, n, m)
    assert rel(x, oracle.dft_synth_direct(F, n, m)) < 1e-12
    assert rel(oracle.r2c(x, m), n * F) < 1e-12
    H = g.normal(size=(2, n // 2 + 1)) + 1j * g.normal(size=(2, n // 2 + 1))
    H[:, 0] = H[:, 0].real
    if n % 2 == 0:
        H[:, -1] = H[:, -1].real
    assert rel(oracle.c2r(H, n), n * np.fft.irfft(H, n, axis=-1)) < 1e-12



@pytest.mark.parametrize("ny,nx", [(3, 5), (6, 8), (8, 6), (15, 12), (100, 64), (7, 1)])
def test_2d_any_size(ny, nx):
    """2D at sizes that are not powers of two: numpy's fft2 (third party), the
    written-out double sum on a few bins, and separability."""
    x = crand((2, ny, nx), ny * 100 + nx)
    y = oracle.c2c_2d(x, -1)
    assert rel(y, np.fft.fft2(x, axes=(-2, -1))) < 1e-12
    k1, k2 = np.array([0, ny - 1, ny // 2]), np.array([0, nx // 3, nx - 1])
    assert rel(y[0][k1, k2], oracle.dft2_bins(x[0], k1, k2, -1)) < 1e-12
    u, v = crand(ny, 1), crand(nx, 2)
    assert rel(oracle.c2c_2d(np.outer(u, v), +1), np.outer(oracle.dft(u, +1), oracle.dft(v, +1))) < 1e-12


@pytest.mark.parametrize("ny,nx", [(3, 5), (7, 7), (6, 9)])
def test_fftshift_2d_odd_matches_numpy(ny, nx):
    y = crand((2, ny, nx), 4)
    assert np.array_equal(oracle.fftshift_2d(y), np.fft.fftshift(y, axes=(-2, -1)))
