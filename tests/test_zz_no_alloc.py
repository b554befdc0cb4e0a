"""fft_exec_noalloc (the static-scratch variant of fft_exec) against fft_exec.

Two calls in a row on plans whose kernels use scratch, the second with a
smaller input, each compared with fft_exec on the same plan and input (the
same kernels, so the results agree to rounding; the bar is relative L2
<= 1e-5) and with the oracle.  Plans whose scratch exceeds the static buffer
are refused before any launch.
"""
import numpy as np
import pytest

import oracle
from fourier_transform_amd import fft as F
from fourier_transform_amd import workloads as W

from gpu_helpers import dev, host, rel_l2, say

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


def _both(plan, x, shape_out=None):
    """(fft_exec result, fft_exec_noalloc result) of one plan on one input."""
    import torch
    xd = dev(x)
    ya = torch.empty_like(xd)
    yb = torch.empty_like(xd)
    F.fft_exec(plan, xd, ya)
    lib = F.lib()
    rc = lib.fft_exec_noalloc(plan, xd.data_ptr(), yb.data_ptr(),
                              torch.cuda.current_stream().cuda_stream)
    assert rc == F.FFT_OK, F.fft_last_error()
    return host(ya), host(yb)


def test_noalloc_two_calls_second_smaller():
    # first call: a tall 2D image on the two-pass path (scratch of about 128 MiB)
    ny, nx = 8192, 2048
    say(f"noalloc call 1: 2d {ny}x{nx} shift (two-pass, scratch in the static buffer)")
    x1 = W.normal_c64((1, ny, nx), np.random.default_rng(81))
    p1 = F.fft_plan_create_2d(ny, nx, 1, F.FFT_C2C, F.FFT_FORWARD)
    try:
        F.fft_plan_set(p1, F.FFT_OPT_SHIFT, 1)
        a, b = _both(p1, x1)
    finally:
        F.fft_plan_destroy(p1)
    e = rel_l2(b, a)
    say(f"noalloc 2d vs fft_exec rel_l2 {e:.3e}")
    assert e <= TOL
    assert rel_l2(b, oracle.fftshift_2d(oracle.c2c_2d(x1, -1))) <= TOL

    # second call, smaller: a four-step plan (2^17 x 3, scratch 3 MiB)
    n, batch = 1 << 17, 3
    say(f"noalloc call 2: four-step n=2^17 batch={batch} inverse")
    x2 = W.normal_c64((batch, n), np.random.default_rng(82))
    p2 = F.fft_plan_create(n, batch, F.FFT_C2C, F.FFT_INVERSE)
    try:
        a, b = _both(p2, x2)
    finally:
        F.fft_plan_destroy(p2)
    e = rel_l2(b, a)
    say(f"noalloc four-step vs fft_exec rel_l2 {e:.3e}")
    assert e <= TOL
    assert rel_l2(b, oracle.c2c(x2, +1)) <= TOL


def test_noalloc_chirp_and_single_pass():
    """The three-pass chirp transform (two scratch buffers), the four-step of
    a smooth length (two passes through the scratch) and a plan without
    scratch, one after the other."""
    for n, batch in ((20011, 3), (20000, 3), (4096, 64)):
        say(f"noalloc: c2c n={n} batch={batch}")
        x = W.uniform_c64((batch, n), np.random.default_rng(n))
        p = F.fft_plan_create(n, batch, F.FFT_C2C, F.FFT_FORWARD)
        try:
            a, b = _both(p, x)
        finally:
            F.fft_plan_destroy(p)
        assert rel_l2(b, a) <= TOL
        assert rel_l2(b, oracle.dft(x, -1) if n & (n - 1) else oracle.c2c(x, -1)) <= TOL


def test_noalloc_smooth_three_pass():
    """The four-step of a smooth length whose row factor is too long for row
    tiles (3 * 2^20 = 3072 x 1024: the row plan of 3072 and a transpose),
    shifted: the static scratch against fft_exec, and sampled bins of the
    definition."""
    n, batch = 3 << 20, 2
    say(f"noalloc: smooth four-step n={n} batch={batch} shift")
    x = W.uniform_c64((batch, n), np.random.default_rng(n % 997))
    p = F.fft_plan_create(n, batch, F.FFT_C2C, F.FFT_FORWARD)
    try:
        F.fft_plan_set(p, F.FFT_OPT_SHIFT, 1)
        a, b = _both(p, x)
    finally:
        F.fft_plan_destroy(p)
    assert rel_l2(b, a) <= TOL
    bins = np.unique(np.random.default_rng(5).integers(0, n, 48))
    idx = oracle.fftshift_index(n)
    for r in range(batch):
        # output index i holds bin idx[i]
        assert rel_l2(b[r, bins], oracle.dft_bins(x[r], idx[bins], -1)) <= TOL


def test_noalloc_refuses_oversized_scratch():
    """A four-step plan whose scratch (batch*n*8 bytes) exceeds the static
    buffer is refused before any launch; fft_exec still runs it."""
    import torch
    n, batch = 1 << 22, 9          # 288 MiB of scratch
    assert batch * n * 8 > F.FFT_NOALLOC_MAX_SCRATCH_BYTES
    say(f"noalloc refusal: four-step n=2^22 batch={batch}")
    p = F.fft_plan_create(n, batch, F.FFT_C2C, F.FFT_FORWARD)
    try:
        x = torch.zeros((batch, n), dtype=torch.complex64, device="cuda")
        y = torch.full_like(x, 1.0)
        rc = F.lib().fft_exec_noalloc(p, x.data_ptr(), y.data_ptr(), torch.cuda.current_stream().cuda_stream)
        assert rc == F.FFT_ENOTSUP
        code, msg = F.fft_last_error()
        assert code == F.FFT_ENOTSUP and "static buffer" in msg, msg
        torch.cuda.synchronize()
        assert torch.all(y == 1.0)         # nothing ran
        F.fft_exec(p, x, y)
        torch.cuda.synchronize()
        assert torch.all(y == 0)
    finally:
        F.fft_plan_destroy(p)
