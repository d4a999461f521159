"""MI355X (gfx950) grouped-query attention over a KV cache.

Thin Python binding of the C-ABI library ``libkvattn.so`` (declared in
``include/kvattn.h``).  Every function here only marshals torch tensors into
tensor descriptors and calls the library on the current torch stream; all of
the arithmetic runs in the library's HIP kernels.  torch supplies device
memory (inputs, outputs, workspace) and the stream.

If the library is missing or fails to load, every call raises RuntimeError:
there is no fallback implementation.

Operators (one per ONNX-Runtime contrib operator page):
  gqa_attention     com.microsoft.GroupQueryAttention
  decode_mha        com.microsoft.DecoderMaskedMultiHeadAttention
  sparse_attention  com.microsoft.SparseAttention
  packed_attention  com.microsoft.PackedAttention
"""

from ._binding import (  # noqa: F401
    KvattnError,
    decode_mha,
    gqa_attention,
    gqa_attention_noalloc,
    library,
    library_path,
    packed_attention,
    packed_schedule,
    set_decode_split,
    sparse_attention,
)

__all__ = [
    "KvattnError",
    "gqa_attention",
    "gqa_attention_noalloc",
    "decode_mha",
    "sparse_attention",
    "packed_attention",
    "packed_schedule",
    "set_decode_split",
    "library",
    "library_path",
]
