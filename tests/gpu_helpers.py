"""Helpers shared by the GPU tests: device transfers, plan execution, metrics."""
import sys

import numpy as np

from fourier_transform_amd import fft as F


def say(msg):
    """Name the GPU case about to run (flushed, so a crash still shows it)."""
    print(f"\n[gpu] {msg}", flush=True)
    sys.stdout.flush()


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def empty(shape, dtype):
    import torch
    return torch.empty(shape, dtype=dtype, device="cuda")


def rel_l2(got, want):
    got = np.asarray(got, np.complex128)
    want = np.asarray(want, np.complex128)
    return float(np.linalg.norm((got - want).ravel()) / np.linalg.norm(want.ravel()))


def c2c(x, sign, shift=0, inplace=False):
    """Run a 1D C2C plan over the rows of x (numpy complex64) and return the result."""
    import torch
    n = x.shape[-1]
    batch = x.size // n
    plan = F.fft_plan_create(n, batch, F.FFT_C2C, sign)
    try:
        if shift:
            F.fft_plan_set(plan, F.FFT_OPT_SHIFT, shift)
        xd = dev(x)
        yd = xd if inplace else torch.empty_like(xd)
        F.fft_exec(plan, xd, yd)
        return host(yd)
    finally:
        F.fft_plan_destroy(plan)


def c2c_2d(x, sign, shift=0, inplace=False):
    import torch
    ny, nx = x.shape[-2:]
    batch = x.size // (ny * nx)
    plan = F.fft_plan_create_2d(ny, nx, batch, F.FFT_C2C, sign)
    try:
        if shift:
            F.fft_plan_set(plan, F.FFT_OPT_SHIFT, shift)
        xd = dev(x)
        yd = xd if inplace else torch.empty_like(xd)
        F.fft_exec(plan, xd, yd)
        return host(yd)
    finally:
        F.fft_plan_destroy(plan)


def r2c(x, mmax=None, mmajor=False, pairs=False):
    """x: float32 [batch][n]; returns complex64 [batch][mmax+1] or [mmax+1][batch]."""
    import torch
    n = x.shape[-1]
    batch = x.size // n
    mmax = n // 2 if mmax is None else mmax
    plan = F.fft_plan_create(n, batch, F.FFT_R2C, F.FFT_FORWARD)
    try:
        F.fft_plan_set(plan, F.FFT_OPT_MMAX, mmax)
        F.fft_plan_set(plan, F.FFT_OPT_SPEC_LAYOUT, int(mmajor))
        F.fft_plan_set(plan, F.FFT_OPT_REAL_PAIRS, int(pairs))
        xd = dev(x)
        shape = (mmax + 1, batch) if mmajor else (batch, mmax + 1)
        yd = empty(shape, torch.complex64)
        F.fft_exec(plan, xd, yd)
        return host(yd)
    finally:
        F.fft_plan_destroy(plan)


def c2r(Fs, n, batch, mmax=None, mmajor=False, pairs=False):
    """Fs: complex64 spectrum in the given layout; returns float32 [batch][n]."""
    import torch
    mmax = n // 2 if mmax is None else mmax
    plan = F.fft_plan_create(n, batch, F.FFT_C2R, F.FFT_INVERSE)
    try:
        F.fft_plan_set(plan, F.FFT_OPT_MMAX, mmax)
        F.fft_plan_set(plan, F.FFT_OPT_SPEC_LAYOUT, int(mmajor))
        F.fft_plan_set(plan, F.FFT_OPT_REAL_PAIRS, int(pairs))
        xd = dev(Fs)
        yd = empty((batch, n), torch.float32)
        F.fft_exec(plan, xd, yd)
        return host(yd)
    finally:
        F.fft_plan_destroy(plan)


def negate_odd(x, axes_parity):
    """Flip the sign bits of re and im where the index parity (sum over the
    given parity arrays) is odd -- exact, bit for bit."""
    u = np.ascontiguousarray(x).view(np.uint32).reshape(x.shape + (2,)).copy()
    odd = (axes_parity & 1).astype(bool)
    u[odd] ^= np.uint32(0x80000000)
    return u.reshape(-1).view(np.complex64).reshape(x.shape)


def direct_analysis(x, mmax=None, mmajor=False):
    """FFT_R2C_DIRECT on x: float32 [batch][n] (any n); bins 0..mmax in the given layout."""
    import torch
    n = x.shape[-1]
    batch = x.size // n
    mmax = (n - 1) // 2 if mmax is None else mmax
    plan = F.fft_plan_create(n, batch, F.FFT_R2C_DIRECT, F.FFT_FORWARD)
    try:
        F.fft_plan_set(plan, F.FFT_OPT_MMAX, mmax)
        F.fft_plan_set(plan, F.FFT_OPT_SPEC_LAYOUT, int(mmajor))
        xd = dev(x)
        shape = (mmax + 1, batch) if mmajor else (batch, mmax + 1)
        yd = empty(shape, torch.complex64)
        F.fft_exec(plan, xd, yd)
        return host(yd)
    finally:
        F.fft_plan_destroy(plan)


def direct_synthesis(Fs, n, batch, mmax=None, mmajor=False):
    """FFT_C2R_DIRECT: spectrum (bins 0..mmax, given layout) -> float32 [batch][n]."""
    import torch
    mmax = (n - 1) // 2 if mmax is None else mmax
    plan = F.fft_plan_create(n, batch, F.FFT_C2R_DIRECT, F.FFT_INVERSE)
    try:
        F.fft_plan_set(plan, F.FFT_OPT_MMAX, mmax)
        F.fft_plan_set(plan, F.FFT_OPT_SPEC_LAYOUT, int(mmajor))
        xd = dev(Fs)
        yd = empty((batch, n), torch.float32)
        F.fft_exec(plan, xd, yd)
        return host(yd)
    finally:
        F.fft_plan_destroy(plan)
