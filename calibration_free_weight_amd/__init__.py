"""MI355X-native HQQ (Half-Quadratic Quantization) weight quantizer.

The product is the HIP library ``libhqq.so`` (C ABI in ``include/hqq.h``); ``hqq`` is its
thin Python binding.
"""
from . import hqq  # noqa: F401
