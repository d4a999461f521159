"""Plain CPU oracle for grouped-query attention over a KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code with the HIP library and imports
nothing from ``kv_cache_transformer_amd``.

Every function computes the plain definition of its operator in float64 with
numpy: dense score matrices, masks as booleans or additive terms, an explicit
softmax and an explicit product with V.  Results are rounded to the storage
type T (round-to-nearest-even) only where an operator materialises a T
tensor, i.e. the present key/value cache rows.  Attention outputs stay
float64.

The operators follow four ONNX-Runtime contrib operator pages:
``com.microsoft.GroupQueryAttention``, ``com.microsoft.DecoderMaskedMultiHeadAttention``,
``com.microsoft.SparseAttention`` and ``com.microsoft.PackedAttention``.
Each function cites the page and section it follows.  Where a page is silent
the reading taken is stated in the docstring.

``oracle.pool`` runs the GroupQueryAttention and SparseAttention oracles over
chunks of query rows of a named full-size workload in child processes (rows
are independent, so the chunks are the whole computation cut into pieces).

Parity pins (tests/test_oracle_*.py) check this oracle against pure-Python
brute force (``oracle.brute``), torch's float64 SDPA and rms_norm on the CPU,
closed forms and invariants.  No function here is "parity unpinned".
"""

from .common import (
    rms_norm,
    rotary,
    softcap,
    default_scale,
    round_to,
    attend,
)
from .gqa import gqa
from .dmmha import dmmha
from .sparse import sparse, csr_visible_blocks
from .packed import packed, packed_schedule

__all__ = [
    "rms_norm",
    "rotary",
    "softcap",
    "default_scale",
    "round_to",
    "attend",
    "gqa",
    "dmmha",
    "sparse",
    "csr_visible_blocks",
    "packed",
    "packed_schedule",
]
