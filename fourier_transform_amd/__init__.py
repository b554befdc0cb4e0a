"""MI355X-native batched fp32 FFT (natural-order Stockham, HIP for gfx950).

The transforms run in the HIP library ``libfft_amd.so`` behind the C ABI in
``include/fft.h``; ``fourier_transform_amd.fft`` is its thin ctypes binding.
Importing this package does not load the library; the binding loads it on
first use and raises if it has not been built.
"""
__all__ = ["fft", "workloads"]
