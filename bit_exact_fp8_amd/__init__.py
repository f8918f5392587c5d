"""MI355X-native bit-exact emulated FP8 scaled GEMM.

``scaled_mm`` / ``accumulate`` call the HIP library ``libemu_fp8gemm.so``
through its C ABI (``include/emu_fp8gemm.h``).  Importing this package does
not load the library; the first call does, and fails loudly if it is missing.
"""
from .api import (EmuError, accumulate, abi_version, library_path, scaled_mm,  # noqa: F401
                  workspace_bytes)
