"""MI355X-native FP8 W8A8 quantized linear (gfx950 HIP kernels behind a C ABI).

The HIP library is loaded lazily on first use, so importing the package (for
example for ``synth``) works on machines without a GPU; every compute call goes
through ``libfp8w8a8.so`` and raises if that library is missing.
"""
