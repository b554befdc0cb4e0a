"""GPU parity for C2C lengths that are not powers of two, against the
oracle's DFT by the definition: mixed-radix Stockham stages (radices 2..8,
10..16) for the lengths up to 16384 with no prime factor above 13 and a
schedule, the four-step over two such lengths for the other lengths with no
prime factor above 13, Rader's convolution of length p - 1 on those stages
for primes p up to 16385 whose p - 1 has a schedule, Bluestein's chirp
transform for the rest (on a mixed-radix convolution length where that is
much shorter than the power of two).

Tolerance: relative L2 error <= 1e-5 over the whole output of a case.
"""
import numpy as np
import pytest

import oracle
from fourier_transform_amd import fft as F
from fourier_transform_amd import workloads as W

from gpu_helpers import c2c, c2c_2d, c2r, dev, empty, host, r2c, rel_l2, say

pytestmark = pytest.mark.gpu
TOL = 1e-5

# radix schedules of some mixed lengths: radices up to 16, one butterfly per
# thread: 18: 6 3; 42: 7 6; 150: 15 10; 360: 10 6 6; 720: 12 10 6;
# 840: 12 10 7; 1000: 10 10 10; 1296: 6 6 6 6; 2000: 10 8 5 5;
# 3000: 10 10 6 5; 4000: 10 10 8 5; 6000: 10 10 10 6; 1001: 13 11 7;
# 1331: 11 11 11; 2197: 13 13 13; 2002: 14 13 11; 5005: 13 11 7 5.  Radices
# up to 8, two per thread: 7776: 6 6 6 6 6.
SMALL = [3, 5, 6, 7, 9, 11, 12, 13, 14, 15, 17, 18, 21, 31, 35, 42, 48, 49, 96, 100, 121, 127, 143, 150,
         169, 255, 257, 360, 384, 720, 840]
LARGE = [1000, 1001, 1029, 1296, 1331, 1536, 2000, 2002, 2047, 2197, 2401, 3000, 3072, 4000, 4095,
         4097, 5000, 5005, 6000, 6144, 6250, 6561, 7168, 7776, 8000, 8191]


# primes by Rader's algorithm (the schedule of p - 1): 17: 16; 19: 6 3;
# 23: 11 2; 97: 12 8; 127: 7 6 3; 257: 16 16; 331: 11 6 5; 1009: 12 12 7;
# 2003: 14 13 11; 4001: 10 10 8 5; 7001: 10 10 10 7.  Primes whose p - 1
# has no schedule take the chirp transform: 509, 1019, 8191.
RADER = [17, 19, 23, 29, 37, 41, 97, 101, 127, 193, 257, 331, 641, 1009, 1201, 2003, 2017, 3001, 4001, 7001]


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    F.lib()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("n", SMALL + LARGE)
@pytest.mark.parametrize("sign", [-1, 1])
def test_any_length_sweep(n, sign):
    for batch in ((1, 3, 37) if n < 1000 else (1, 5)):
        say(f"any-length c2c n={n} batch={batch} sign={sign}")
        x = W.uniform_c64((batch, n), np.random.default_rng(n * 10 + batch))
        y = c2c(x, sign)
        assert rel_l2(y, oracle.dft(x, sign)) <= TOL, (n, batch)


@pytest.mark.parametrize("n", RADER + [509, 1019])
@pytest.mark.parametrize("sign", [-1, 1])
def test_primes(n, sign):
    """Primes: Rader's convolution where p - 1 has a schedule, else the chirp
    transform; batches that leave the last workgroup's lines partly empty."""
    for batch in (1, 7, 65):
        say(f"prime c2c n={n} batch={batch} sign={sign}")
        x = W.uniform_c64((batch, n), np.random.default_rng(n * 13 + batch))
        assert rel_l2(c2c(x, sign), oracle.dft(x, sign)) <= TOL, (n, batch)


# primes above 8193 by Rader's algorithm with two butterflies of up to 16
# values per thread (p - 1 above 8192): 8233: 14 14 7 6; 9001: 15 15 8 5;
# 12289: 16 16 8 6; 15361: 16 15 8 8; 14401: 15 15 8 8
RADER_WIDE = [8233, 9001, 12289, 14401, 15361]


@pytest.mark.parametrize("n", RADER_WIDE)
@pytest.mark.parametrize("sign", [-1, 1])
def test_primes_two_butterflies(n, sign):
    for batch in (1, 3):
        say(f"prime c2c (Rader, two butterflies) n={n} batch={batch} sign={sign}")
        x = W.uniform_c64((batch, n), np.random.default_rng(n * 19 + batch))
        assert rel_l2(c2c(x, sign), oracle.dft(x, sign)) <= TOL, (n, batch)


@pytest.mark.parametrize("n,shift", [(9001, 1), (12289, 2)])
def test_primes_two_butterflies_shift_in_place(n, shift):
    say(f"prime c2c (Rader, two butterflies) shift={shift} n={n}, in place")
    x = W.uniform_c64((2, n), np.random.default_rng(n + shift + 3))
    idx = oracle.fftshift_index(n) if shift == 1 else oracle.ifftshift_index(n)
    want = oracle.dft(x, 1)[:, idx]
    assert rel_l2(c2c(x, 1, shift=shift, inplace=True), want) <= TOL


# the chirp transform on a convolution length with a mixed-radix schedule
# (used where it is at least 1.3 times shorter than the power of two):
# 34: 70 = 10 7; 47: 96 = 16 6; 83: 165 = 15 11; 263: 525 = 15 7 5;
# 1034: 2080 = 16 13 10; 2053: 4116 = 12 7 7 7; 2111: 4224 = 11 8 8 6;
# 59 and 107 keep the power of two (128, 256)
CHIRP_MIXED = [34, 47, 59, 83, 107, 263, 1031, 1034, 1049, 2053, 2063, 2111]


@pytest.mark.parametrize("n", CHIRP_MIXED)
@pytest.mark.parametrize("sign", [-1, 1])
def test_chirp_mixed_length(n, sign):
    for batch in (1, 7, 65):
        say(f"chirp (mixed-radix m) c2c n={n} batch={batch} sign={sign}")
        x = W.uniform_c64((batch, n), np.random.default_rng(n * 17 + batch))
        assert rel_l2(c2c(x, sign), oracle.dft(x, sign)) <= TOL, (n, batch)


@pytest.mark.parametrize("n,shift", [(34, 1), (83, 2), (1034, 1), (1034, 2), (2053, 1), (2111, 2)])
def test_chirp_mixed_length_shift_and_in_place(n, shift):
    say(f"chirp (mixed-radix m) shift={shift} n={n}, in place")
    x = W.uniform_c64((3, n), np.random.default_rng(n + shift + 5))
    idx = oracle.fftshift_index(n) if shift == 1 else oracle.ifftshift_index(n)
    want = oracle.dft(x, -1)[:, idx]
    assert rel_l2(c2c(x, -1, shift=shift, inplace=True), want) <= TOL


@pytest.mark.parametrize("n", [3, 12, 15, 100, 360, 5, 17, 97, 257, 34, 83])
def test_short_lines_several_workgroups(n):
    """Lines of fewer than 128 threads (mixed radix, Rader, the chirp on a
    mixed-radix length) read and write their workgroup's rows as one block
    through LDS: many workgroups and a ragged last one, in place, and the
    shift (the sign flip of even n, the ramp of odd n)."""
    batch = 2000 + n % 7
    say(f"short lines n={n} batch={batch}")
    x = W.uniform_c64((batch, n), np.random.default_rng(n + 31))
    assert rel_l2(c2c(x, -1), oracle.dft(x, -1)) <= TOL
    assert rel_l2(c2c(x, 1, inplace=True), oracle.dft(x, 1)) <= TOL
    want = oracle.dft(x, -1)[:, oracle.fftshift_index(n)]
    assert rel_l2(c2c(x, -1, shift=1), want) <= TOL


@pytest.mark.parametrize("n", [7, 1000, 1009, 4097])
def test_any_length_in_place(n):
    say(f"any-length c2c in place n={n}")
    x = W.uniform_c64((4, n), np.random.default_rng(n + 1))
    assert rel_l2(c2c(x, -1, inplace=True), oracle.dft(x, -1)) <= TOL


@pytest.mark.parametrize("n", [3, 7, 12, 101, 255, 1001, 1009, 4095, 6000])
@pytest.mark.parametrize("sign", [-1, 1])
def test_any_length_shift(n, sign):
    """Fused shift (even and odd n): bin 0 lands at index floor(n/2), the
    oracle's index map applied to its own transform."""
    say(f"any-length shift n={n} sign={sign}")
    x = W.uniform_c64((3, n), np.random.default_rng(n + 7))
    want = oracle.dft(x, sign)[:, oracle.fftshift_index(n)]
    assert rel_l2(c2c(x, sign, shift=1), want) <= TOL


@pytest.mark.parametrize("n", [3, 7, 12, 257, 1001, 4095])
@pytest.mark.parametrize("sign", [-1, 1])
def test_any_length_inverse_shift(n, sign):
    """Shift option 2: index floor(n/2) moves to 0 (numpy's ifftshift of the
    output), for odd n one place away from option 1."""
    say(f"any-length inverse shift n={n} sign={sign}")
    x = W.uniform_c64((3, n), np.random.default_rng(n + 11))
    want = oracle.dft(x, sign)[:, oracle.ifftshift_index(n)]
    assert rel_l2(c2c(x, sign, shift=2), want) <= TOL


@pytest.mark.parametrize("n", [5, 1000, 2017, 8191])
def test_any_length_round_trip(n):
    say(f"any-length round trip n={n}")
    x = W.uniform_c64((6, n), np.random.default_rng(n + 3))
    z = c2c(c2c(x, -1), +1) / n
    assert rel_l2(z, x) <= TOL


def test_any_length_large_batch_sampled_rows():
    """n = 1000, 16384 rows (the batched shape of the 4096-point workload):
    every row against a property, sampled rows against the oracle."""
    import torch
    n, batch = 1000, 16384
    say(f"any-length c2c n={n} batch={batch}")
    x = W.uniform_c64((batch, n), np.random.default_rng(99))
    pf = F.fft_plan_create(n, batch, F.FFT_C2C, F.FFT_FORWARD)
    pi = F.fft_plan_create(n, batch, F.FFT_C2C, F.FFT_INVERSE)
    try:
        xd = dev(x)
        yd = torch.empty_like(xd)
        zd = torch.empty_like(xd)
        F.fft_exec(pf, xd, yd)
        F.fft_exec(pi, yd, zd)
        y, z = host(yd), host(zd)
    finally:
        F.fft_plan_destroy(pf)
        F.fft_plan_destroy(pi)
    rows = np.random.default_rng(5).choice(batch, 24, replace=False)
    assert rel_l2(y[rows], oracle.dft(x[rows], -1)) <= TOL
    assert rel_l2(y[-1:], oracle.dft(x[-1:], -1)) <= TOL     # the ragged last workgroup
    assert rel_l2(z / n, x) <= TOL                            # round trip over every row
    # Parseval over every row
    e = np.abs(np.sum(np.abs(y.astype(np.complex128)) ** 2, axis=1) /
               (n * np.sum(np.abs(x.astype(np.complex128)) ** 2, axis=1)) - 1)
    assert e.max() <= 1e-5


def test_any_length_deterministic():
    say("any-length determinism n=3000 batch=64")
    x = W.uniform_c64((64, 3000), np.random.default_rng(4))
    a, b = c2c(x, -1), c2c(x, -1)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_any_length_shift_option_and_sizes():
    """Shift is accepted for odd lengths on this path; sizes are n, not the
    internal transform length."""
    plan = F.fft_plan_create(1001, 3, F.FFT_C2C, F.FFT_FORWARD)
    try:
        F.fft_plan_set(plan, F.FFT_OPT_SHIFT, 1)
        assert F.fft_plan_get_sizes(plan) == (3 * 1001 * 8, 3 * 1001 * 8)
    finally:
        F.fft_plan_destroy(plan)


# --------------------------------------------------------------------------
# lengths above 8192 with a prime factor above 13: the chirp transform over
# m >= 2n - 1 points, in one kernel up to n = 16384 (m = 32768), above in
# three passes (the hooked four-step column pass, the fused row pass, the
# inverse column pass).  10007 and 12281 are primes whose p - 1 has no
# schedule.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("n", [8193, 10007, 12281, 16383, 16385, 20000, 30001])
@pytest.mark.parametrize("sign", [-1, 1])
def test_any_length_large_full(n, sign):
    say(f"any-length (chirp, {'one kernel' if n <= 16384 else 'three passes'}) n={n} sign={sign}")
    x = W.uniform_c64((3, n), np.random.default_rng(n + 21))
    assert rel_l2(c2c(x, sign), oracle.dft(x, sign)) <= TOL


@pytest.mark.parametrize("n", [65537, 100000, 1000003, (1 << 22) - 1])
def test_any_length_large_sampled_bins(n):
    """Longer rows: 64 sampled bins of every row by the definition, the round
    trip and Parseval over every value."""
    batch = 2
    say(f"any-length (four-step chirp) n={n} batch={batch}")
    x = W.uniform_c64((batch, n), np.random.default_rng(n % 1000 + 5))
    y = c2c(x, -1)
    bins = np.unique(np.concatenate([[0, 1, n // 2, n - 1],
                                     np.random.default_rng(7).integers(0, n, 60)]))
    for r in range(batch):
        assert rel_l2(y[r, bins], oracle.dft_bins(x[r], bins, -1)) <= TOL
    z = c2c(y, +1) / n
    assert rel_l2(z, x) <= TOL
    e = np.abs(np.sum(np.abs(y.astype(np.complex128)) ** 2) /
               (n * np.sum(np.abs(x.astype(np.complex128)) ** 2)) - 1)
    assert e <= 1e-5


# --------------------------------------------------------------------------
# lengths with no prime factor above 13 that no one-kernel schedule takes
# (above 16384, and 6561 = 3^8, 15625 = 5^6): the four-step n = n1 * n2,
# n2 <= 1024 closest to sqrt(n): mixed-radix column tiles times the
# twiddle, then row tiles of n1 stored transposed (n1 up to about 2540), or
# else the row plan of n1 and a transpose (3 * 2^20 = 3072 x 1024); the
# shift is a rotation of the output index in the last pass
# --------------------------------------------------------------------------
FOURSTEP_ANY = [6561, 15625, 16896, 20000, 24576, 30000]


@pytest.mark.parametrize("n", FOURSTEP_ANY)
@pytest.mark.parametrize("sign", [-1, 1])
def test_fourstep_any_full(n, sign):
    for batch in (1, 2):
        say(f"four-step (mixed radix) c2c n={n} batch={batch} sign={sign}")
        x = W.uniform_c64((batch, n), np.random.default_rng(n * 7 + batch))
        assert rel_l2(c2c(x, sign), oracle.dft(x, sign)) <= TOL, (n, batch)


@pytest.mark.parametrize("n,shift", [(6561, 1), (6561, 2), (20000, 1), (24576, 2), (15625, 1)])
def test_fourstep_any_shift_and_in_place(n, shift):
    say(f"four-step (mixed radix) shift={shift} n={n}, in place")
    x = W.uniform_c64((2, n), np.random.default_rng(n + shift + 11))
    idx = oracle.fftshift_index(n) if shift == 1 else oracle.ifftshift_index(n)
    want = oracle.dft(x, -1)[:, idx]
    assert rel_l2(c2c(x, -1, shift=shift, inplace=True), want) <= TOL


@pytest.mark.parametrize("n", [49152, 1000000, 3 << 20])
def test_fourstep_any_large_sampled_bins(n):
    """Longer smooth rows: 64 sampled bins of every row by the definition,
    the round trip and Parseval over every value."""
    batch = 2
    say(f"four-step (mixed radix) n={n} batch={batch}")
    x = W.uniform_c64((batch, n), np.random.default_rng(n % 1000 + 9))
    y = c2c(x, -1)
    bins = np.unique(np.concatenate([[0, 1, n // 2, n - 1],
                                     np.random.default_rng(8).integers(0, n, 60)]))
    for r in range(batch):
        assert rel_l2(y[r, bins], oracle.dft_bins(x[r], bins, -1)) <= TOL
    assert rel_l2(c2c(y, +1) / n, x) <= TOL
    e = np.abs(np.sum(np.abs(y.astype(np.complex128)) ** 2) /
               (n * np.sum(np.abs(x.astype(np.complex128)) ** 2)) - 1)
    assert e <= 1e-5


@pytest.mark.parametrize("n,shift", [(10001, 1), (10001, 2), (16000, 1), (20011, 1), (20011, 2)])
def test_any_length_large_shift_and_in_place(n, shift):
    say(f"any-length (chirp) shift={shift} n={n}, in place")
    x = W.uniform_c64((2, n), np.random.default_rng(n + shift))
    idx = oracle.fftshift_index(n) if shift == 1 else oracle.ifftshift_index(n)
    want = oracle.dft(x, -1)[:, idx]
    assert rel_l2(c2c(x, -1, shift=shift, inplace=True), want) <= TOL


# --------------------------------------------------------------------------
# R2C / C2R at lengths that are not powers of two: an any-length complex
# transform of n/2 (even n) or n (odd n) with the packing kernels around it
# --------------------------------------------------------------------------
REAL_N = [3, 5, 6, 7, 10, 12, 15, 100, 101, 360, 999, 1000, 1440, 2001, 2018, 4002, 10000, 20002]


@pytest.mark.parametrize("n", REAL_N)
def test_real_any_length_sweep(n):
    g = np.random.default_rng(n + 33)
    for batch, mmax, mmajor in ((1, None, False), (5, n // 3, True), (19, n // 2, False), (6, 0, True)):
        if n > 4096 and batch > 5:
            batch = 3
        m = n // 2 if mmax is None else mmax
        say(f"any-length r2c/c2r n={n} batch={batch} mmax={m} mmajor={mmajor}")
        x = g.uniform(-1, 1, size=(batch, n)).astype(np.float32)
        Fg = r2c(x, m, mmajor)
        assert rel_l2(Fg.T if mmajor else Fg, oracle.r2c(x, m)) <= TOL, (n, batch, m)
        S = (g.normal(size=(batch, m + 1)) + 1j * g.normal(size=(batch, m + 1))).astype(np.complex64)
        Sin = np.ascontiguousarray(S.T) if mmajor else S
        xg = c2r(Sin, n, batch, m, mmajor)
        assert rel_l2(xg, oracle.c2r(S, n, m)) <= TOL, (n, batch, m)


@pytest.mark.parametrize("n", [1 << 16, 1 << 20, 1 << 22])
def test_real_pow2_four_step(n):
    """Real rows of a power of two above one kernel's reach (32768): the
    four-step transform of n/2 complex values between the same pack/unpack
    kernels; full and cut band, both spectrum layouts, both directions."""
    g = np.random.default_rng(n % 1000 + 3)
    for batch, mmax, mmajor in ((2, n // 2, False), (3, n // 5, True)):
        say(f"pow2 r2c/c2r (four-step) n={n} batch={batch} mmax={mmax} mmajor={mmajor}")
        x = g.uniform(-1, 1, size=(batch, n)).astype(np.float32)
        Fg = r2c(x, mmax, mmajor)
        assert rel_l2(Fg.T if mmajor else Fg, oracle.r2c(x, mmax)) <= TOL, (n, batch, mmax)
        S = (g.normal(size=(batch, mmax + 1)) + 1j * g.normal(size=(batch, mmax + 1))).astype(np.complex64)
        Sin = np.ascontiguousarray(S.T) if mmajor else S
        assert rel_l2(c2r(Sin, n, batch, mmax, mmajor), oracle.c2r(S, n, mmax)) <= TOL, (n, batch, mmax)


def test_real_any_length_options():
    """Two-for-one packing needs a power-of-two length; sizes follow n."""
    plan = F.fft_plan_create(1000, 4, F.FFT_R2C, F.FFT_FORWARD)
    try:
        with pytest.raises(F.FFTError) as e:
            F.fft_plan_set(plan, F.FFT_OPT_REAL_PAIRS, 1)
        assert e.value.code == F.FFT_ENOTSUP
        F.fft_plan_set(plan, F.FFT_OPT_MMAX, 100)
        assert F.fft_plan_get_sizes(plan) == (4 * 1000 * 4, 4 * 101 * 8)
    finally:
        F.fft_plan_destroy(plan)


# --------------------------------------------------------------------------
# 2D plans with an axis that is not a power of two: the row plan, then the
# columns in place (power-of-two ny: the column kernel; a mixed-radix ny: its
# stages on column tiles in LDS) where a tile holds 8 or more columns, else
# rows, transpose, rows, transpose back; the shift is the shift of each axis
# --------------------------------------------------------------------------
SIZES_2D = [(3, 5, 2), (6, 10, 3), (100, 64, 2), (64, 100, 2), (360, 180, 1), (1000, 999, 1), (17, 1024, 2),
            (97, 331, 1), (10001, 6, 1),
            # column pass in place: power-of-two ny (16 and 8 columns per tile), mixed-radix ny (16 and 8,
            # one and two butterflies per thread, odd), then the transposing fallback (8192, 6000)
            (1024, 100, 2), (2048, 60, 1), (4096, 12, 1), (1000, 64, 1), (2000, 30, 1), (7776, 7, 1),
            (105, 64, 2), (64, 1000, 3), (8192, 20, 1), (6000, 20, 1),
            # an axis on the four-step of smooth lengths (rows of 20000; columns of 20000 through
            # the transposes)
            (6, 20000, 1), (20000, 6, 1)]


@pytest.mark.parametrize("ny,nx,batch", SIZES_2D)
@pytest.mark.parametrize("sign", [-1, 1])
def test_2d_any_size(ny, nx, batch, sign):
    say(f"2D any size {ny}x{nx} batch={batch} sign={sign}")
    x = W.uniform_c64((batch, ny, nx), np.random.default_rng(ny * 7 + nx))
    assert rel_l2(c2c_2d(x, sign), oracle.c2c_2d(x, sign)) <= TOL


@pytest.mark.parametrize("ny,nx", [(3, 5), (7, 8), (100, 99), (64, 100), (1024, 30), (1000, 64), (105, 60),
                                   (2000, 30), (6, 20000)])
@pytest.mark.parametrize("shift", [1, 2])
def test_2d_any_size_shift_and_in_place(ny, nx, shift):
    say(f"2D any size {ny}x{nx} shift={shift}, in place")
    x = W.uniform_c64((2, ny, nx), np.random.default_rng(ny + nx + shift))
    iy = oracle.fftshift_index(ny) if shift == 1 else oracle.ifftshift_index(ny)
    ix = oracle.fftshift_index(nx) if shift == 1 else oracle.ifftshift_index(nx)
    want = oracle.c2c_2d(x, -1)[:, iy][:, :, ix]
    assert rel_l2(c2c_2d(x, -1, shift=shift, inplace=True), want) <= TOL


# --------------------------------------------------------------------------
# buffers beyond 2^31 elements (64-bit row offsets): the seeded block tiled
# on the device, sampled rows at the start, the middle and the ragged end
# --------------------------------------------------------------------------
@pytest.mark.parametrize("n,batch", [(4096, (1 << 19) + 3), (1000, (1 << 21) + 5), (1009, (1 << 21) + 7),
                                     (1019, (1 << 21) + 9)])
def test_beyond_2p31_elements(n, batch):
    import torch
    say(f"c2c n={n} batch={batch} ({batch * n * 8 / 2**30:.1f} GiB per buffer)")
    block = W.uniform_c64((64, n), np.random.default_rng(n + 77))
    xd = dev(block).repeat((batch + 63) // 64, 1)[:batch].contiguous()
    plan = F.fft_plan_create(n, batch, F.FFT_C2C, F.FFT_FORWARD)
    try:
        yd = torch.empty_like(xd)
        F.fft_exec(plan, xd, yd)
        torch.cuda.synchronize()
        rows = np.array([0, 1, 63, batch // 2, batch - 65, batch - 2, batch - 1])
        y = yd[torch.from_numpy(rows).cuda()].cpu().numpy()
    finally:
        F.fft_plan_destroy(plan)
        del xd
        torch.cuda.empty_cache()
    want = oracle.dft(block[rows % 64], -1) if n & (n - 1) else oracle.c2c(block[rows % 64], -1)
    assert rel_l2(y, want) <= TOL


# --------------------------------------------------------------------------
# p x 2^k (p in 3, 5, 7, 9, 15, 25) and other smooth lengths above 8192: the
# mixed-radix kernel, with two butterflies of up to 16 values per thread above
# 8192 points (15625 = 5^6 has no such schedule: the chirp transform)
# --------------------------------------------------------------------------
PQ_N = [48, 80, 240, 400, 576, 960, 1792, 2304, 2560, 3840, 4608, 6400, 9216, 10240, 12288, 12800,
        14336, 15360, 9000, 10000, 12000, 16000, 15625]


@pytest.mark.parametrize("n", PQ_N)
@pytest.mark.parametrize("sign", [-1, 1])
def test_smooth_length_sweep(n, sign):
    for batch in (1, 7):
        say(f"smooth length c2c n={n} batch={batch} sign={sign}")
        x = W.uniform_c64((batch, n), np.random.default_rng(n * 3 + batch))
        assert rel_l2(c2c(x, sign), oracle.dft(x, sign)) <= TOL, (n, batch)


@pytest.mark.parametrize("n", [6, 48, 1000, 1536, 2002, 15360])
def test_even_shift_bit_exact_and_in_place(n):
    """The shift is the exact sign flip of (-1)^j (n even): bitwise the
    transform of the negated input; and the rotation of the oracle's.  The
    mixed-radix kernel, 15360 with two butterflies of up to 16 values per
    thread."""
    from gpu_helpers import negate_odd
    x = W.uniform_c64((3, n), np.random.default_rng(n + 9))
    ys = c2c(x, -1, shift=1)
    xn = negate_odd(x, np.broadcast_to(np.arange(n), x.shape))
    assert np.array_equal(ys.view(np.uint32), c2c(xn, -1).view(np.uint32))
    assert rel_l2(ys, oracle.dft(x, -1)[:, oracle.fftshift_index(n)]) <= TOL
    assert rel_l2(c2c(x, +1, inplace=True), oracle.dft(x, +1)) <= TOL
