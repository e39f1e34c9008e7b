"""MI355X-native speculative-sampling verify step.

``verify`` enqueues the HIP kernels of libsv.so (C ABI in include/sv.h) on the
current torch stream; ``sample`` draws one token per row with the same
truncation (the draft side's sampling step, or plain decoding).  ``workloads``
builds the seeded synthetic inputs.
"""
from ._lib import (SV_BF16, SV_F32, SV_MAX_TOP_K, load, params_tensor, sample, verify,
                   workspace_bytes)

__all__ = ["verify", "sample", "params_tensor", "workspace_bytes", "load", "SV_F32", "SV_BF16",
           "SV_MAX_TOP_K"]
