"""fp64 CPU oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, header,
helper or constant with the HIP library under ``io_aware_transformer_amd/``
and imports nothing from it.

The oracle is the plain definition of attention (materialise the score
matrix, stable row softmax, multiply by V) and the textbook analytic
backward, in float64, one (batch, query-head) unit at a time, plus
attention with queries and keys of different lengths, attention over a key
range, the merge of partial results over disjoint key ranges, local
(sliding-window) attention, batches of packed sequences of different
lengths, block-sparse attention and attention with dropout on the
probabilities (keep mask from Philox-4x32-10).  Every function cites the passage of the source pages it follows;
see ``oracle/attention.py``, ``oracle/splitkv.py``, ``oracle/window.py`` and
``oracle/varlen.py``, ``oracle/blocksparse.py`` and ``oracle/dropout.py``.
"""

from .dropout import (dropout_backward, dropout_forward, dropout_head_backward, dropout_head_forward,
                      dropout_threshold, keep_mask, philox4x32_10)
from .blocksparse import blocksparse_backward, blocksparse_forward, blocksparse_visible
from .attention import (
    attention_forward,
    attention_backward,
    attention_forward_rows,
    head_forward,
    head_backward,
    kv_head_of,
)
from .splitkv import cross_forward, merge_partials, partial_forward
from .varlen import varlen_backward, varlen_forward
from .window import window_backward, window_forward, window_visible

__all__ = [
    "attention_forward",
    "attention_backward",
    "attention_forward_rows",
    "head_forward",
    "head_backward",
    "kv_head_of",
    "cross_forward",
    "partial_forward",
    "merge_partials",
    "window_forward",
    "window_backward",
    "window_visible",
    "varlen_forward",
    "varlen_backward",
    "blocksparse_forward",
    "blocksparse_backward",
    "blocksparse_visible",
    "dropout_forward",
    "dropout_backward",
    "dropout_head_forward",
    "dropout_head_backward",
    "dropout_threshold",
    "keep_mask",
    "philox4x32_10",
]
