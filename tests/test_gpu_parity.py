"""GPU parity: the HIP path (through the C ABI) against the f64 oracle.

Tolerance: relative L2 error <= 1e-5 over the whole output of a case, for every
length (single-pass, four-step, real and 2D).  Shift index work is checked
bit for bit.
"""
import numpy as np
import pytest

import oracle
from fourier_transform_amd import fft as F
from fourier_transform_amd import workloads as W

from gpu_helpers import (c2c, c2c_2d, c2r, dev, direct_analysis, direct_synthesis, empty, host,
                         negate_odd, r2c, rel_l2, say)

pytestmark = pytest.mark.gpu
TOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    F.lib()
    yield
    torch.cuda.synchronize()


# --------------------------------------------------------------------------
# workload 1: N = 1024, batch 8, forward; oracle and brute force
# --------------------------------------------------------------------------
def test_w1_forward_vs_oracle_and_brute_force():
    say("w1 n=1024 batch=8 forward")
    x = W.workload1()
    y = c2c(x, -1)
    assert rel_l2(y, oracle.c2c(x, -1)) <= TOL
    for r in range(x.shape[0]):
        assert rel_l2(y[r], oracle.dft_brute(x[r], -1)) <= TOL


# --------------------------------------------------------------------------
# every single-pass length, both directions, ragged batches
# --------------------------------------------------------------------------
@pytest.mark.parametrize("logn", range(1, 15))
@pytest.mark.parametrize("sign", [-1, 1])
def test_c2c_single_pass_sweep(logn, sign):
    n = 1 << logn
    for batch in (1, 3, 37):
        say(f"c2c n={n} batch={batch} sign={sign}")
        x = W.uniform_c64((batch, n), np.random.default_rng(logn * 100 + batch))
        y = c2c(x, sign)
        assert rel_l2(y, oracle.c2c(x, sign)) <= TOL, (n, batch)


@pytest.mark.parametrize("n", [2, 4, 8, 16, 32, 64])
def test_c2c_short_rows_several_workgroups(n):
    """Short rows: 4 to 32 points are read and written through LDS in the
    workgroup's order (256 or 128 rows per workgroup).  Several workgroups and
    a ragged last one, in place, and the shift, bitwise the transform of the
    negated input."""
    batch = 3 * 256 + 37
    say(f"c2c short rows n={n} batch={batch}")
    x = W.uniform_c64((batch, n), np.random.default_rng(n + 500))
    assert rel_l2(c2c(x, -1), oracle.c2c(x, -1)) <= TOL
    assert rel_l2(c2c(x, 1, inplace=True), oracle.c2c(x, 1)) <= TOL
    ys = c2c(x, -1, shift=1)
    xn = negate_odd(x, np.broadcast_to(np.arange(n), x.shape))
    assert np.array_equal(ys.view(np.uint32), c2c(xn, -1).view(np.uint32))


@pytest.mark.parametrize("n", [2, 64, 4096])
def test_c2c_in_place(n):
    say(f"c2c in place n={n}")
    x = W.uniform_c64((5, n), np.random.default_rng(n))
    assert rel_l2(c2c(x, -1, inplace=True), oracle.c2c(x, -1)) <= TOL


# --------------------------------------------------------------------------
# workload 2: N = 4096, batch 16384, forward then inverse (full size)
# --------------------------------------------------------------------------
def test_w2_forward_inverse_full():
    import torch
    say("w2 n=4096 batch=16384 forward+inverse")
    x = W.workload2()
    n, batch = W.W2["n"], W.W2["batch"]
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
    e_fwd = rel_l2(y, oracle.c2c(x, -1))
    e_inv = rel_l2(z, oracle.c2c(y, +1))
    e_rt = rel_l2(z / n, x)
    say(f"w2 rel_l2 forward={e_fwd:.3e} inverse={e_inv:.3e} round_trip={e_rt:.3e}")
    assert e_fwd <= TOL and e_inv <= TOL and e_rt <= TOL


def test_deterministic_repeat():
    say("determinism n=4096 batch=512")
    x = W.uniform_c64((512, 4096), np.random.default_rng(3))
    a, b = c2c(x, -1), c2c(x, -1)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


# --------------------------------------------------------------------------
# four-step (lengths beyond one workgroup)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("logn", [15, 16, 17, 20, 21, 22])
@pytest.mark.parametrize("sign", [-1, 1])
def test_fourstep_sweep(logn, sign):
    n = 1 << logn
    batch = 3 if logn < 20 else 2
    say(f"four-step n=2^{logn} batch={batch} sign={sign}")
    x = W.normal_c64((batch, n), np.random.default_rng(logn))
    assert rel_l2(c2c(x, sign), oracle.c2c(x, sign)) <= TOL


def test_fourstep_in_place():
    say("four-step in place n=2^16")
    x = W.normal_c64((2, 1 << 16), np.random.default_rng(7))
    assert rel_l2(c2c(x, -1, inplace=True), oracle.c2c(x, -1)) <= TOL


def _sampled_rel(got, want, rms):
    """Relative L2 error estimated on sampled outputs: the sample's error norm
    over what the full output's norm (rms * sqrt(count)) gives that many bins."""
    got = np.asarray(got, np.complex128)
    return float(np.linalg.norm(got - want) / (np.sqrt(got.size) * rms))


def test_fourstep_max_length_sampled_bins():
    """The longest supported length, 2^28 (2 GiB per buffer): sampled bins
    against the definition, plus Parseval over the whole output."""
    n = 1 << 28
    say("four-step n=2^28 batch=1 forward (maximum length)")
    x = np.random.default_rng(28).standard_normal(2 * n, dtype=np.float32).view(np.complex64)
    y = c2c(x.reshape(1, n), -1)[0]
    bins = np.array([0, 1, 12345, n // 2, n - 1, (1 << 27) + 3, 987654321 % n])
    px = float(np.sum(np.abs(x.astype(np.complex128)) ** 2))
    rms = np.sqrt(px)  # rms of the output bins: sqrt(n * px / n)
    e = _sampled_rel(y[bins], oracle.dft_bins(x, bins, -1), rms)
    say(f"2^28 sampled rel_l2 {e:.3e}")
    assert e <= TOL
    py = float(np.sum(np.abs(y.astype(np.complex128)) ** 2))
    assert abs(py / (n * px) - 1) < 1e-5


def test_2d_max_size_sampled_bins():
    """The largest 2D image, 16384 x 16384 (tall path), with the shift fused:
    sampled outputs against the 2D definition at the rotated indices."""
    ny = nx = 16384
    say("2d 16384x16384 shift (maximum size)")
    x = np.random.default_rng(14).standard_normal(2 * ny * nx, dtype=np.float32).view(
        np.complex64).reshape(ny, nx)
    y = c2c_2d(x.reshape(1, ny, nx), -1, shift=1)[0]
    i = np.array([0, 1, ny // 2, ny - 1, 777, 12000])
    j = np.array([0, nx - 1, nx // 2, 3, 9001, 5])
    want = oracle.dft2_bins(x, (i + ny // 2) % ny, (j + nx // 2) % nx, -1)
    rms = np.sqrt(float(np.sum(np.abs(x.astype(np.complex128)) ** 2)))
    e = _sampled_rel(y[i, j], want, rms)
    say(f"16384^2 sampled rel_l2 {e:.3e}")
    assert e <= TOL


def test_deterministic_fourstep_and_tall_2d():
    say("determinism four-step 2^20 and 2d 8192x64")
    x = W.normal_c64((2, 1 << 20), np.random.default_rng(20))
    a, b = c2c(x, -1), c2c(x, -1)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    x2 = W.normal_c64((1, 8192, 64), np.random.default_rng(21))
    a, b = c2c_2d(x2, -1, 1), c2c_2d(x2, -1, 1)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_w3_full_size_all_rows():
    """Workload 3 at full size (32 x 2^22), compared with the oracle element
    by element over the whole output: the oracle runs on chunks of 4 rows and
    the squared error and reference norms are summed over all 32."""
    say("w3 n=2^22 batch=32 forward, whole output")
    x = W.workload3()
    y = c2c(x, -1)
    err2 = ref2 = 0.0
    worst = 0.0
    for r0 in range(0, x.shape[0], 4):
        want = oracle.c2c(x[r0:r0 + 4], -1)
        d = y[r0:r0 + 4].astype(np.complex128) - want
        e2 = np.sum(np.abs(d) ** 2, axis=1)
        w2 = np.sum(np.abs(want) ** 2, axis=1)
        err2 += float(e2.sum())
        ref2 += float(w2.sum())
        worst = max(worst, float(np.sqrt(np.max(e2 / w2))))
    e = float(np.sqrt(err2 / ref2))
    say(f"w3 rel_l2 over all 32 rows: {e:.3e} (worst row {worst:.3e})")
    assert e <= TOL and worst <= TOL


# --------------------------------------------------------------------------
# real transforms
# --------------------------------------------------------------------------
@pytest.mark.parametrize("logn", range(2, 16))
def test_real_sweep(logn):
    n = 1 << logn
    g = np.random.default_rng(logn)
    for batch, mmax, mmajor in ((1, None, False), (5, n // 2 - 1, True), (19, max(0, n // 3), False),
                                (6, 0, True)):
        m = n // 2 if mmax is None else mmax
        say(f"r2c/c2r n={n} batch={batch} mmax={m} mmajor={mmajor}")
        x = g.uniform(-1, 1, size=(batch, n)).astype(np.float32)
        Fg = r2c(x, m, mmajor)
        Fo = oracle.r2c(x, m)
        assert rel_l2(Fg.T if mmajor else Fg, Fo) <= TOL, (n, batch, m)
        S = (g.normal(size=(batch, m + 1)) + 1j * g.normal(size=(batch, m + 1))).astype(np.complex64)
        Sin = np.ascontiguousarray(S.T) if mmajor else S
        xg = c2r(Sin, n, batch, m, mmajor)
        assert rel_l2(xg, oracle.c2r(S, n, m)) <= TOL, (n, batch, m)


@pytest.mark.parametrize("n", [8, 32, 64, 2048])
@pytest.mark.parametrize("pairs", [False, True])
def test_real_several_workgroups(n, pairs):
    """Batches of several workgroups with a ragged last one (the spectrum
    staging loop runs several rounds of loads per thread; rows of 32 reals
    are stored through LDS), both spectrum layouts, full and cut band."""
    g = np.random.default_rng(n + 77)
    batch = 602 if n < 2048 else 42
    for mmax, mmajor in ((n // 2, False), (n // 3, True)):
        say(f"r2c/c2r n={n} batch={batch} mmax={mmax} mmajor={mmajor} pairs={pairs}")
        x = g.uniform(-1, 1, size=(batch, n)).astype(np.float32)
        Fg = r2c(x, mmax, mmajor, pairs=pairs)
        assert rel_l2(Fg.T if mmajor else Fg, oracle.r2c(x, mmax)) <= TOL
        S = (g.normal(size=(batch, mmax + 1)) + 1j * g.normal(size=(batch, mmax + 1))).astype(np.complex64)
        Sin = np.ascontiguousarray(S.T) if mmajor else S
        assert rel_l2(c2r(Sin, n, batch, mmax, mmajor, pairs=pairs), oracle.c2r(S, n, mmax)) <= TOL


@pytest.mark.parametrize("logn", range(2, 15))
def test_real_pairs_sweep(logn):
    """Two real rows per complex transform (Mota, section 2.6, Eq. 17-18)."""
    n = 1 << logn
    g = np.random.default_rng(100 + logn)
    for batch, mmax, mmajor in ((2, None, False), (6, n // 2 - 1, True), (20, max(0, n // 3), False),
                                (4, 0, True)):
        m = n // 2 if mmax is None else mmax
        say(f"real pairs n={n} batch={batch} mmax={m} mmajor={mmajor}")
        x = g.uniform(-1, 1, size=(batch, n)).astype(np.float32)
        Fg = r2c(x, m, mmajor, pairs=True)
        assert rel_l2(Fg.T if mmajor else Fg, oracle.r2c(x, m)) <= TOL, (n, batch, m)
        S = (g.normal(size=(batch, m + 1)) + 1j * g.normal(size=(batch, m + 1))).astype(np.complex64)
        Sin = np.ascontiguousarray(S.T) if mmajor else S
        xg = c2r(Sin, n, batch, m, mmajor, pairs=True)
        assert rel_l2(xg, oracle.c2r(S, n, m)) <= TOL, (n, batch, m)


def test_real_pairs_options():
    plan = F.fft_plan_create(64, 3, F.FFT_R2C, F.FFT_FORWARD)
    try:
        with pytest.raises(F.FFTError) as e:
            F.fft_plan_set(plan, F.FFT_OPT_REAL_PAIRS, 1)      # odd batch
        assert e.value.code == F.FFT_EINVAL
    finally:
        F.fft_plan_destroy(plan)
    plan = F.fft_plan_create(32768, 2, F.FFT_C2R, F.FFT_INVERSE)
    try:
        with pytest.raises(F.FFTError) as e:
            F.fft_plan_set(plan, F.FFT_OPT_REAL_PAIRS, 1)      # beyond one workgroup
        assert e.value.code == F.FFT_ENOTSUP
    finally:
        F.fft_plan_destroy(plan)


def test_w4_synthesis_then_analysis():
    """Workload 4: nlat=1024 rows, nphi=2048, mmax=682, m-major spectrum."""
    p = W.W4
    n, nlat, mmax = p["nphi"], p["nlat"], p["mmax"]
    Fm = W.workload4_spectrum()                      # [683][1024] m-major
    say("w4 C2R synthesis")
    xg = c2r(Fm, n, nlat, mmax, mmajor=True)
    xo = oracle.c2r(Fm.T, n, mmax)
    e_syn = rel_l2(xg, xo)
    say("w4 R2C analysis")
    x32 = xo.astype(np.float32)                      # the oracle's rows, rounded
    Fg = r2c(x32, mmax, mmajor=True)
    e_ana = rel_l2(Fg.T, oracle.r2c(x32, mmax))
    e_closed = rel_l2(Fg / n, Fm)                    # R2C(C2R(F)) = n F
    say(f"w4 rel_l2 synthesis={e_syn:.3e} analysis={e_ana:.3e} closed_form={e_closed:.3e}")
    assert e_syn <= TOL and e_ana <= TOL and e_closed <= TOL


# --------------------------------------------------------------------------
# band-limited direct transforms (any length, matrix cores)
# --------------------------------------------------------------------------
def _spectrum(g, batch, m):
    return (g.normal(size=(batch, m + 1)) + 1j * g.normal(size=(batch, m + 1))).astype(np.complex64)


@pytest.mark.parametrize("n", [2, 3, 5, 30, 64, 100, 257, 1000, 2000, 4095])
def test_direct_sweep(n):
    """Direct analysis/synthesis against the oracle's direct sums (several
    64 x 64 tiles, ragged rows and columns, both spectrum layouts)."""
    g = np.random.default_rng(200 + n)
    half = (n - 1) // 2
    cases = [(1, half, False), (67, half, True), (130, n // 3 if 2 * (n // 3) < n else half, False),
             (5, 0, True)]
    for batch, m, mmajor in cases:
        if n >= 2000 and batch > 8:
            batch = 3                      # keep the O(batch n mmax) oracle fast
        say(f"direct n={n} batch={batch} mmax={m} mmajor={mmajor}")
        x = g.uniform(-1, 1, size=(batch, n)).astype(np.float32)
        Fg = direct_analysis(x, m, mmajor)
        assert rel_l2(Fg.T if mmajor else Fg, oracle.dft_analys_direct(x, m)) <= TOL, (n, batch, m)
        S = _spectrum(g, batch, m)
        Sin = np.ascontiguousarray(S.T) if mmajor else S
        xg = direct_synthesis(Sin, n, batch, m, mmajor)
        assert rel_l2(xg, oracle.dft_synth_direct(S, n, m)) <= TOL, (n, batch, m)


@pytest.mark.parametrize("n", [4096, 16384])
def test_direct_pow2_matches_fft_oracle(n):
    """Power-of-two lengths against the oracle's FFT-based real transforms
    (the same sums when 2 mmax < n), with more rows than one tile column."""
    g = np.random.default_rng(300 + n)
    batch, m = (130, n // 2 - 1) if n <= 4096 else (65, n // 2 - 1)
    say(f"direct pow2 n={n} batch={batch} mmax={m}")
    x = g.uniform(-1, 1, size=(batch, n)).astype(np.float32)
    assert rel_l2(direct_analysis(x, m), oracle.r2c(x, m)) <= TOL
    S = _spectrum(g, batch, m)
    assert rel_l2(direct_synthesis(np.ascontiguousarray(S.T), n, batch, m, True),
                  oracle.c2r(S, n, m)) <= TOL


def test_direct_max_length_odd_sampled_rows():
    """The longest odd length, 16383: every bin of sampled rows by the definition."""
    n, batch, m = 16383, 70, 8191
    g = np.random.default_rng(16383)
    x = g.uniform(-1, 1, size=(batch, n)).astype(np.float32)
    say(f"direct analysis n={n} batch={batch} mmax={m}")
    Fg = direct_analysis(x, m)
    for r in (0, 63, 69):
        assert rel_l2(Fg[r], oracle.dft_bins(x[r], np.arange(m + 1))) <= TOL, r
    S = _spectrum(g, batch, m)
    say(f"direct synthesis n={n} batch={batch} mmax={m}")
    xg = direct_synthesis(S, n, batch, m)
    for r in (1, 64):
        assert rel_l2(xg[r], oracle.dft_synth_direct(S[r:r + 1], n, m)[0]) <= TOL, r


def test_direct_w4_shape():
    """The w4 shape (nphi=2048, nlat=1024, mmax=682, m-major) through the
    direct kinds, against the oracle's real transforms and the closed form
    analysis(synthesis(F)) = n F."""
    p = W.W4
    n, nlat, mmax = p["nphi"], p["nlat"], p["mmax"]
    Fm = W.workload4_spectrum()
    say("w4 shape, direct synthesis")
    xg = direct_synthesis(Fm, n, nlat, mmax, mmajor=True)
    xo = oracle.c2r(Fm.T, n, mmax)
    say("w4 shape, direct analysis")
    x32 = xo.astype(np.float32)
    Fg = direct_analysis(x32, mmax, mmajor=True)
    e_syn, e_ana = rel_l2(xg, xo), rel_l2(Fg.T, oracle.r2c(x32, mmax))
    e_closed = rel_l2(Fg / n, Fm)
    say(f"direct w4 rel_l2 synthesis={e_syn:.3e} analysis={e_ana:.3e} closed_form={e_closed:.3e}")
    assert e_syn <= TOL and e_ana <= TOL and e_closed <= TOL


def test_direct_unaligned_buffers():
    """Buffers only 8-byte aligned take the narrow-load variants; same results."""
    import torch
    n, batch, m = 64, 70, 31
    g = np.random.default_rng(64)
    x = g.uniform(-1, 1, size=(batch, n)).astype(np.float32)
    S = _spectrum(g, batch, m + 1)[:, :m + 1]
    say("direct analysis/synthesis from 8-byte aligned buffers")
    for kind, sign, src, out_shape, want in (
            (F.FFT_R2C_DIRECT, -1, x, (batch, m + 1), oracle.dft_analys_direct(x, m)),
            (F.FFT_C2R_DIRECT, 1, S, (batch, n), oracle.dft_synth_direct(S, n, m))):
        plan = F.fft_plan_create(n, batch, kind, sign)
        try:
            F.fft_plan_set(plan, F.FFT_OPT_MMAX, m)
            flat = np.ascontiguousarray(src).view(np.float32).ravel()
            buf = torch.zeros(flat.size + 2, dtype=torch.float32, device="cuda")
            buf[2:] = torch.from_numpy(flat).cuda()
            dt = torch.complex64 if kind == F.FFT_R2C_DIRECT else torch.float32
            y = empty(out_shape, dt)
            F.fft_exec(plan, buf.data_ptr() + 8, y)
            assert rel_l2(host(y), want) <= TOL
        finally:
            F.fft_plan_destroy(plan)


def test_direct_options():
    plan = F.fft_plan_create(30, 2, F.FFT_R2C_DIRECT, F.FFT_FORWARD)
    try:
        assert F.fft_plan_get_sizes(plan) == (2 * 30 * 4, 2 * 15 * 8)   # default mmax 14
        for opt, val in ((F.FFT_OPT_MMAX, 15), (F.FFT_OPT_MMAX, -1), (F.FFT_OPT_SHIFT, 1),
                         (F.FFT_OPT_REAL_PAIRS, 1)):
            with pytest.raises(F.FFTError) as e:
                F.fft_plan_set(plan, opt, val)
            assert e.value.code == F.FFT_EINVAL, (opt, val)
    finally:
        F.fft_plan_destroy(plan)


# --------------------------------------------------------------------------
# 2D and the fused chessboard shift
# --------------------------------------------------------------------------
@pytest.mark.parametrize("ny,nx", [(2, 2), (4, 16), (16, 4), (32, 64), (256, 128), (128, 1024),
                                   (2048, 16), (16, 16384), (8192, 2), (8192, 16), (16384, 32)])
@pytest.mark.parametrize("shift", [0, 1])
def test_2d_sweep(ny, nx, shift):
    say(f"2d {ny}x{nx} shift={shift}")
    x = W.normal_c64((2, ny, nx), np.random.default_rng(ny * 7 + nx))
    y = c2c_2d(x, -1, shift)
    want = oracle.c2c_2d(x, -1)
    if shift:
        want = oracle.fftshift_2d(want)
    assert rel_l2(y, want) <= TOL
    yi = c2c_2d(x, +1, shift, inplace=True)
    want_i = oracle.c2c_2d(x, +1)
    if shift:
        want_i = oracle.fftshift_2d(want_i)
    assert rel_l2(yi, want_i) <= TOL


@pytest.mark.parametrize("ny,nx,batch", [(8192, 8192, 1), (8192, 2048, 2), (16384, 1024, 2), (16384, 4096, 1),
                                         (8192, 4096, 1), (16384, 2048, 1), (4096, 4096, 1), (4096, 1024, 2),
                                         (4096, 512, 3), (4096, 16384, 1), (8192, 1024, 1), (8192, 512, 2),
                                         (16384, 512, 1)])
def test_2d_tall(ny, nx, batch):
    """Images on the two-pass form (rows with the first column factor, then
    columns of 2048): 4096, 8192 and 16384 rows, 512 to 16384 columns.  Forward with the shift out of place, inverse in
    place, against the oracle; the shift bit for bit against the
    chessboard-negated input."""
    say(f"2d two-pass {ny}x{nx} batch={batch}")
    x = W.normal_c64((batch, ny, nx), np.random.default_rng(ny + nx))
    y = c2c_2d(x, -1, shift=1)
    assert rel_l2(y, oracle.fftshift_2d(oracle.c2c_2d(x, -1))) <= TOL
    ii, jj = np.meshgrid(np.arange(ny), np.arange(nx), indexing="ij")
    xn = negate_odd(x, np.broadcast_to(ii + jj, x.shape))
    del ii, jj
    assert np.array_equal(c2c_2d(xn, -1).view(np.uint32), y.view(np.uint32))
    del xn, y
    yi = c2c_2d(x, +1, inplace=True)
    assert rel_l2(yi, oracle.c2c_2d(x, +1)) <= TOL


def test_2d_tall_inverse_shift_is_the_same_map():
    """Even sizes: ifftshift is the same index map as fftshift, so SHIFT = 2
    gives the SHIFT = 1 output bit for bit on the two-pass tall path."""
    say("2d two-pass 8192x2048 shift=2 vs shift=1")
    x = W.normal_c64((1, 8192, 2048), np.random.default_rng(82))
    a, b = c2c_2d(x, +1, shift=1), c2c_2d(x, +1, shift=2)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_shift_bit_exact_1d():
    for n, batch in ((1024, 8), (4096, 3), (1 << 16, 2)):
        say(f"shift bit-exact 1d n={n}")
        x = W.uniform_c64((batch, n), np.random.default_rng(n))
        ys = c2c(x, -1, shift=1)
        xn = negate_odd(x, np.broadcast_to(np.arange(n), x.shape))
        yr = c2c(xn, -1, shift=0)
        assert np.array_equal(ys.view(np.uint32), yr.view(np.uint32))
        # and the shift is the index rotation of the plain transform
        assert rel_l2(ys, oracle.c2c(x, -1)[:, oracle.fftshift_index(n)]) <= TOL
        # the inverse rotation is the same map for even lengths, bit for bit
        assert np.array_equal(c2c(x, -1, shift=2).view(np.uint32), ys.view(np.uint32))


def test_shift_bit_exact_2d():
    say("shift bit-exact 2d 256x512")
    x = W.normal_c64((2, 256, 512), np.random.default_rng(11))
    ys = c2c_2d(x, -1, shift=1)
    ii, jj = np.meshgrid(np.arange(256), np.arange(512), indexing="ij")
    xn = negate_odd(x, np.broadcast_to(ii + jj, x.shape))
    yr = c2c_2d(xn, -1, shift=0)
    assert np.array_equal(ys.view(np.uint32), yr.view(np.uint32))


def test_w5_full_size():
    """Workload 5: 8192 x 8192 image, 2D forward with the shift fused."""
    p = W.W5
    say("w5 generate")
    x = W.workload5()
    say("w5 2d 8192x8192 shift")
    y = c2c_2d(x, -1, shift=1)
    want = oracle.fftshift_2d(oracle.c2c_2d(x, -1))
    e = rel_l2(y, want)
    say(f"w5 rel_l2={e:.3e}")
    assert e <= TOL
    # the tones land on their shifted bins with height ny*nx*e^{i phase}
    ky, kx, phase, _ = W.workload5_params()
    ny, nx = p["ny"], p["nx"]
    for s in range(p["tones"]):
        i, j = (ky[s] + ny // 2) % ny, (kx[s] + nx // 2) % nx
        want_peak = ny * nx * np.exp(1j * phase[s])
        # other tones on the same bin add up; only check isolated ones
        if np.sum((ky == ky[s]) & (kx == kx[s])) == 1:
            assert abs(y[i, j] - want_peak) / abs(want_peak) < 1e-4


@pytest.mark.parametrize("n", [512, 1024])
def test_2d_inverse_batched(n):
    """2D inverse transforms of 4 images per batch (the ocean-demo shape of the
    GLSL dissertation, Table 4, without the rendering)."""
    say(f"2d inverse {n}x{n} batch=4")
    x = W.normal_c64((4, n, n), np.random.default_rng(n + 4))
    assert rel_l2(c2c_2d(x, +1), oracle.c2c_2d(x, +1)) <= TOL


def test_graph_capture_replays():
    """fft_exec launches kernels only, so it can be captured in a HIP graph;
    every replay, with eager work in between, matches the eager result."""
    import torch
    say("graph capture: 1D n=4096, four-step 2^16 and 2^22 x 8, 2D 512x512 and 8192x8192, mixed radix 1000, "
        "Rader 1009, chirp 1019, 10001 (one kernel) and 20011 (three passes)")
    # 2^22 x 8 and 8192 x 8192 run the persistent passes with a staggered start
    cases = [(4096, 64, None), (1 << 16, 4, None), (1 << 22, 8, None), (512, 512, 2), (8192, 1, 8192),
             (1000, 16, None), (1009, 8, None), (1019, 8, None), (10001, 2, None), (20011, 2, None)]
    for n, b, ny in cases:
        if ny is None:
            plan = F.fft_plan_create(n, b, F.FFT_C2C, F.FFT_FORWARD)
            shape = (b, n)
        else:
            plan = F.fft_plan_create_2d(ny, n, b, F.FFT_C2C, F.FFT_FORWARD)
            F.fft_plan_set(plan, F.FFT_OPT_SHIFT, 1)
            shape = (b, ny, n)
        try:
            x = dev(W.normal_c64(shape, np.random.default_rng(n)))
            y_eager = torch.empty_like(x)
            y = torch.empty_like(x)
            F.fft_exec(plan, x, y_eager)
            torch.cuda.synchronize()
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):       # warm-up on the capture stream
                F.fft_exec(plan, x, y)
            torch.cuda.current_stream().wait_stream(s)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                F.fft_exec(plan, x, y)
            want = y_eager.cpu().numpy()
            for rep in range(3):
                y.zero_()
                torch.cuda.synchronize()
                g.replay()
                torch.cuda.synchronize()
                assert np.array_equal(y.cpu().numpy().view(np.uint32), want.view(np.uint32)), rep
                x.mul_(1.0)                   # eager work between replays
                torch.cuda.synchronize()
            del g
        finally:
            F.fft_plan_destroy(plan)


# --------------------------------------------------------------------------
# errors that need a live plan
# --------------------------------------------------------------------------
def test_exec_errors_and_state():
    import torch
    say("exec error paths")
    plan = F.fft_plan_create(64, 4, F.FFT_R2C, F.FFT_FORWARD)
    try:
        x = torch.zeros(4 * 64, dtype=torch.float32, device="cuda")
        lib = F.lib()
        assert lib.fft_exec(plan, x.data_ptr(), x.data_ptr(), None) == F.FFT_EINVAL
        assert lib.fft_exec(plan, x.data_ptr() + 4, x.data_ptr() + 1024, None) == F.FFT_EINVAL
        assert lib.fft_exec(plan, None, x.data_ptr(), None) == F.FFT_EINVAL
        with pytest.raises(F.FFTError) as e:
            F.fft_plan_set(plan, F.FFT_OPT_MMAX, 33)
        assert e.value.code == F.FFT_EINVAL
        with pytest.raises(F.FFTError):
            F.fft_plan_set(plan, F.FFT_OPT_SHIFT, 1)     # C2C only
        pc = F.fft_plan_create(12, 2, F.FFT_C2C, F.FFT_FORWARD)
        try:
            with pytest.raises(F.FFTError) as e:
                F.fft_plan_set(pc, F.FFT_OPT_SHIFT, 3)   # 0, 1 or 2
            assert e.value.code == F.FFT_EINVAL
        finally:
            F.fft_plan_destroy(pc)
        y = empty((4, 33), torch.complex64)
        F.fft_exec(plan, x, y)
        with pytest.raises(F.FFTError) as e:
            F.fft_plan_set(plan, F.FFT_OPT_MMAX, 3)
        assert e.value.code == F.FFT_ESTATE
        with pytest.raises(ValueError):
            F.fft_exec(plan, x[:10], y)                   # too small for the plan
        torch.cuda.synchronize()
    finally:
        F.fft_plan_destroy(plan)
    assert F.fft_plan_get_sizes is not None


def test_destroy_waits_for_its_own_work_only():
    """fft_plan_destroy waits for the plan's last exec (its event), not for
    the device: it returns while an unrelated stream still has queued work,
    and by then the plan's own transform has finished and is correct."""
    import time

    import torch
    say("destroy: own work done, unrelated stream still busy")
    n, batch = 4096, 2048
    x = W.uniform_c64((batch, n), np.random.default_rng(41))
    xd = dev(x)
    yd = torch.empty_like(xd)
    a = torch.randn(4096, 4096, device="cuda")
    b = torch.randn(4096, 4096, device="cuda")
    torch.mm(a, b)                                   # library start-up outside the timing
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(4):
        torch.mm(a, b)
    torch.cuda.synchronize()
    per_mm = (time.perf_counter() - t0) / 4
    reps = int(min(4000, max(8, 1.0 / max(per_mm, 1e-5))))  # about a second of queued work
    # Two created streams (work on the legacy null stream would wait for the
    # side stream by itself).  The transform is enqueued first: streams may
    # share a hardware queue, and then later side work cannot delay it; a
    # destroy that waited for the device would return only after the side
    # work, one that waits for the plan's own exec returns before.
    side, own = torch.cuda.Stream(), torch.cuda.Stream()
    plan = F.fft_plan_create(n, batch, F.FFT_C2C, F.FFT_FORWARD)
    destroyed = False
    try:
        F.fft_exec(plan, xd, yd, own)
        with torch.cuda.stream(side):
            for _ in range(reps):
                torch.mm(a, b)
        F.fft_plan_destroy(plan)
        destroyed = True
        side_busy = not side.query()
        own_done = own.query()
    finally:
        if not destroyed:
            F.fft_plan_destroy(plan)
    say(f"destroy returned with the side stream busy={side_busy} ({reps} products queued), own work done={own_done}")
    side.synchronize()
    assert side_busy
    assert own_done
    assert rel_l2(host(yd), oracle.c2c(x, -1)) <= TOL


def test_exec_on_two_streams_is_ordered():
    """Execs of one plan on two streams run one after the other (the second
    waits for the first's event), so a four-step plan, whose execs share the
    plan's scratch, gives both results correctly."""
    import torch
    say("one four-step plan on two streams")
    n, batch = 1 << 20, 4
    xs = [W.normal_c64((batch, n), np.random.default_rng(50 + i)) for i in range(2)]
    plan = F.fft_plan_create(n, batch, F.FFT_C2C, F.FFT_FORWARD)
    try:
        xd = [dev(x) for x in xs]
        yd = [torch.empty_like(v) for v in xd]
        s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
        torch.cuda.synchronize()
        F.fft_exec(plan, xd[0], yd[0], s1)
        F.fft_exec(plan, xd[1], yd[1], s2)
        torch.cuda.synchronize()
        for x, y in zip(xs, yd):
            assert rel_l2(host(y), oracle.c2c(x, -1)) <= TOL
    finally:
        F.fft_plan_destroy(plan)


def test_failed_exec_leaves_options_settable():
    """An exec that fails its checks does not lock the plan's options."""
    import torch
    say("failed exec keeps options settable")
    plan = F.fft_plan_create(64, 4, F.FFT_C2C, F.FFT_FORWARD)
    try:
        x = torch.zeros(4 * 64, dtype=torch.complex64, device="cuda")
        lib = F.lib()
        assert lib.fft_exec(plan, x.data_ptr() + 4, x.data_ptr(), None) == F.FFT_EINVAL
        F.fft_plan_set(plan, F.FFT_OPT_SHIFT, 1)          # still before the first successful exec
        F.fft_exec(plan, x, x)
        with pytest.raises(F.FFTError) as e:
            F.fft_plan_set(plan, F.FFT_OPT_SHIFT, 0)
        assert e.value.code == F.FFT_ESTATE
        torch.cuda.synchronize()
    finally:
        F.fft_plan_destroy(plan)


@pytest.mark.parametrize("sign", [-1, 1])
def test_lane_swap_exchange_lines(sign):
    """Lines of 64 and 32 threads whose second exchange is a lane swap
    (v_permlane32_swap / v_permlane16_swap instead of LDS): 512- and
    1024-point rows, the 2D row pass on 1024-point rows with the shift, real
    transforms with 512- and 1024-point halves and the chirp transform on a
    1024-point convolution."""
    g = np.random.default_rng(500 + sign)
    for n in (512, 1024):
        for batch in (1, 2, 5, 64):
            say(f"lane swap: c2c n={n} batch={batch} sign={sign}")
            x = W.uniform_c64((batch, n), g)
            assert rel_l2(c2c(x, sign), oracle.c2c(x, sign)) <= TOL, (n, batch)
    x = W.normal_c64((1, 64, 1024), g)
    say("lane swap: 2d 64x1024 shift")
    y = c2c_2d(x, sign, shift=1)
    assert rel_l2(y, oracle.fftshift_2d(oracle.c2c_2d(x, sign))) <= TOL
    for n in (500,):                       # chirp on m = 1024
        say(f"lane swap: c2c n={n} sign={sign}")
        x = W.uniform_c64((3, n), g)
        assert rel_l2(c2c(x, sign), oracle.dft(x, sign)) <= TOL, n
    if sign < 0:
        for n in (1024, 2048):
            say(f"lane swap: real n={n}")
            xr = g.uniform(-1, 1, (7, n)).astype(np.float32)
            Z = r2c(xr, n // 3, mmajor=True)
            assert rel_l2(Z.T, oracle.r2c(xr, n // 3)) <= TOL
            assert rel_l2(c2r(Z, n, 7, n // 3, mmajor=True), oracle.c2r(Z.T, n, n // 3)) <= TOL
