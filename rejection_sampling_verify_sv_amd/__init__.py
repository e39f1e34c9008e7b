"""MI355X-native speculative-sampling verify step.

``verify`` enqueues the HIP kernels of libsv.so (C ABI in include/sv.h) on the
current torch stream; ``verify_tree`` checks a tree of candidate tokens; ``sample`` draws one token per row with the same
truncation (the draft side's sampling step, or plain decoding);
``accept_stats`` gives per-row acceptance statistics of one draft position.
``workloads`` builds the seeded synthetic inputs.
"""
from ._lib import (SV_BF16, SV_F32, SV_MAX_TOP_K, accept_stats, load, params_tensor, sample,
                   stream_read, verify, verify_tree, workspace_bytes)

__all__ = ["verify", "verify_tree", "sample", "accept_stats", "params_tensor", "workspace_bytes", "load",
           "stream_read", "SV_F32", "SV_BF16", "SV_MAX_TOP_K"]
