"""DFlash block-diffusion drafter forward for AMD MI355X (gfx950).

The compute lives in ``libdflash.so`` (C ABI: ``include/dflash.h``; HIP
kernels under ``csrc/``).  ``dflash`` is its ctypes binding.
"""
