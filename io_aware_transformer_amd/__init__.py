"""Exact scaled-dot-product attention for AMD MI355X (gfx950).

The computation lives in hand-written HIP kernels behind the C ABI of
``include/fa.h`` (``libfa.so``); this package only marshals torch tensors
into that ABI.  ``fwd``/``bwd`` (with their local-attention and packed
variable-length forms, and the split key/value forward ``fwd_split`` with its
merge ``lse_merge``) raise ``LibraryNotBuilt`` when the library is missing --
there is no fallback path.
"""

from ._lib import FA_BF16, FA_FP32, FAError, LibraryNotBuilt, load as load_library
from .attention import (bwd, bwd_blocksparse, bwd_dropout, bwd_varlen, bwd_varlen_workspace_size, bwd_window,
                        bwd_workspace_size, fwd, fwd_blocksparse, fwd_dropout, fwd_split, fwd_split_parts,
                        fwd_split_workspace_size, fwd_varlen, fwd_window, lse_merge)

__all__ = ["fwd", "bwd", "bwd_workspace_size", "fwd_split", "fwd_split_parts", "fwd_split_workspace_size",
           "lse_merge", "fwd_window", "bwd_window", "fwd_blocksparse", "bwd_blocksparse",
           "fwd_dropout", "bwd_dropout", "fwd_varlen", "bwd_varlen", "bwd_varlen_workspace_size",
           "FAError", "LibraryNotBuilt", "load_library", "FA_BF16", "FA_FP32"]
