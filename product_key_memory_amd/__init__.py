"""Product-key memory layer for AMD Instinct MI355X (gfx950).

The work is done by hand-written HIP kernels in ``libpkm.so`` behind the C ABI
of ``include/pkm.h``.  This package only marshals PyTorch tensors (device
memory and the current HIP stream) into those calls:

    q, z, mean, rstd = pkm_query_forward(x, W)      # optional: q = BN(x W^T) in the library
    y, idx, weights, scores = pkm_forward(q, keys, values, k)
    dq, dkeys, dvalues = pkm_backward(q, keys, values, idx, weights, dy)
    slot_start, order = pkm_slot_sort(idx, n)     # picks grouped by memory slot
    pkm_sparse_sgd(values, dvalues, slot_start, lr)  # update of the selected slots only
    dq, dkeys = pkm_backward_sgd(q, keys, values, idx, weights, dy, lr)  # both fused, in place
    counts, used = pkm_slot_usage(slot_start)     # slots in use
    y, idx, weights, scores = pkm_flat_forward(q, keys, values, k)   # the flat-key search

Shapes: q [T, H, d_k], keys [H, 2, n, d_k/2], values [n*n, d_v], dy [T, d_v];
float32 or bfloat16 (all the same dtype), contiguous, on one GPU.
"""
from .pkm import (PKMError, ProductKeyMemoryFunction, pkm_backward, pkm_backward_sgd, pkm_flat_forward,
                  pkm_forward,
                  pkm_query_backward, pkm_query_forward, pkm_slot_sort, pkm_slot_usage,
                  pkm_sparse_adam, pkm_sparse_sgd, pkm_status_string, pkm_workspace_bytes,
                  problem)

__all__ = ["PKMError", "ProductKeyMemoryFunction", "pkm_backward", "pkm_backward_sgd",
           "pkm_flat_forward", "pkm_forward",
           "pkm_query_backward", "pkm_query_forward", "pkm_slot_sort", "pkm_slot_usage",
           "pkm_sparse_adam", "pkm_sparse_sgd", "pkm_status_string", "pkm_workspace_bytes",
           "problem"]
