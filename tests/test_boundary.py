"""The C-ABI boundary on the CPU: the library loads, exports every symbol
include/fft.h declares, and rejects bad arguments before any HIP call."""
import os
import re

import pytest

from fourier_transform_amd import fft as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "fft.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fft_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(F.LIB_PATH):
        from fourier_transform_amd import build
        build.build()
    return F.lib()


def test_header_and_binding_agree():
    assert declared_functions() == sorted(F.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_max_single_pass_length(lib):
    assert F.fft_max_single_pass_length() == 16384


def err_of(fn, *args):
    with pytest.raises(F.FFTError) as e:
        fn(*args)
    return e.value.code


@pytest.mark.parametrize("args,code", [
    ((0, 1, F.FFT_C2C, -1), F.FFT_EINVAL),          # n < 1
    ((8, 0, F.FFT_C2C, -1), F.FFT_EINVAL),          # batch < 1
    ((8, 1, 7, -1), F.FFT_EINVAL),                  # bad kind
    ((8, 1, F.FFT_C2C, 0), F.FFT_EINVAL),           # bad sign
    ((8, 1, F.FFT_R2C, +1), F.FFT_EINVAL),          # R2C is forward
    ((8, 1, F.FFT_C2R, -1), F.FFT_EINVAL),          # C2R is inverse
    (((1 << 22) + 1, 1, F.FFT_C2C, -1), F.FFT_ENOTSUP),  # not a power of two and above 2^22
    ((5000000, 4, F.FFT_C2C, 1), F.FFT_ENOTSUP),
    ((1, 1, F.FFT_C2C, -1), F.FFT_ENOTSUP),         # too short
    ((2, 1, F.FFT_R2C, -1), F.FFT_ENOTSUP),         # real transforms need n >= 4
    ((1 << 29, 1, F.FFT_C2C, -1), F.FFT_ENOTSUP),   # beyond the four-step range
    ((1 << 30, 1, F.FFT_R2C, -1), F.FFT_ENOTSUP),   # real powers of two end at 2^29
    ((1 << 40, 1 << 40, F.FFT_C2C, -1), F.FFT_EINVAL),  # size overflow
    (((1 << 22) + 2, 1, F.FFT_R2C, -1), F.FFT_ENOTSUP),  # R2C beyond 2^22 that is not a power of two
    ((1, 1, F.FFT_R2C_DIRECT, -1), F.FFT_ENOTSUP),  # direct kinds: 2 <= n <= 16384
    ((16385, 1, F.FFT_C2R_DIRECT, 1), F.FFT_ENOTSUP),
    ((30, 1, F.FFT_R2C_DIRECT, 1), F.FFT_EINVAL),   # analysis is forward
    ((30, 1, F.FFT_C2R_DIRECT, -1), F.FFT_EINVAL),  # synthesis is inverse
    ((30, 1, 5, -1), F.FFT_EINVAL),                 # no kind 5
])
def test_create_rejects(lib, args, code):
    assert err_of(F.fft_plan_create, *args) == code
    c, msg = F.fft_last_error()
    assert c == code and msg


@pytest.mark.parametrize("args,code", [
    ((0, 8, 1, F.FFT_C2C, -1), F.FFT_EINVAL),
    ((8, 8, 0, F.FFT_C2C, -1), F.FFT_EINVAL),
    ((8, 8, 1, F.FFT_R2C, -1), F.FFT_ENOTSUP),
    ((6, 8, 70000, F.FFT_C2C, -1), F.FFT_ENOTSUP),   # any sizes: at most 65535 images
    ((6, (1 << 22) + 1, 1, F.FFT_C2C, -1), F.FFT_ENOTSUP),
    ((8, 32768, 1, F.FFT_C2C, -1), F.FFT_ENOTSUP),
    ((1, 8, 1, F.FFT_C2C, -1), F.FFT_ENOTSUP),
    ((8, 8, 1, F.FFT_C2C, 3), F.FFT_EINVAL),
    ((8192, 2, 70000, F.FFT_C2C, -1), F.FFT_ENOTSUP),   # tall images: at most 65535
    ((8, 8, 1, F.FFT_R2C_DIRECT, -1), F.FFT_ENOTSUP),   # 2D plans are C2C only
])
def test_create_2d_rejects(lib, args, code):
    assert err_of(F.fft_plan_create_2d, *args) == code


def test_null_plan_calls(lib):
    assert lib.fft_plan_set(None, F.FFT_OPT_SHIFT, 1) == F.FFT_EINVAL
    assert lib.fft_exec(None, 8, 8, None) == F.FFT_EINVAL
    assert lib.fft_plan_get_sizes(None, None, None) == F.FFT_EINVAL
    lib.fft_plan_destroy(None)  # no-op
    assert F.fft_last_error()[0] == F.FFT_OK


def test_valid_create_without_device_reports_hip_error(lib):
    """With no GPU the checks pass and the first HIP call fails cleanly."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present")
    code = err_of(F.fft_plan_create, 1024, 8, F.FFT_C2C, -1)
    assert code in (F.FFT_EHIP, F.FFT_ENOMEM)


@pytest.mark.parametrize("n,kind,sign", [(2, F.FFT_R2C_DIRECT, -1), (1000, F.FFT_R2C_DIRECT, -1),
                                         (999, F.FFT_C2R_DIRECT, 1), (16384, F.FFT_C2R_DIRECT, 1)])
def test_direct_kinds_accept_any_length(lib, n, kind, sign):
    """Any 2 <= n <= 16384 passes the checks of the direct kinds (with no GPU
    the first HIP call then fails)."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present")
    assert err_of(F.fft_plan_create, n, 3, kind, sign) in (F.FFT_EHIP, F.FFT_ENOMEM)


@pytest.mark.parametrize("n", [3, 12, 1000, 1001, 8191, 8193, 100000, (1 << 22) - 1])
def test_c2c_any_length_up_to_2p22_passes_the_checks(lib, n):
    """C2C lengths that are not powers of two (mixed-radix or chirp paths) are
    accepted up to 2^22 (with no GPU the first HIP call then fails)."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present")
    assert err_of(F.fft_plan_create, n, 3, F.FFT_C2C, -1) in (F.FFT_EHIP, F.FFT_ENOMEM)
