"""AuT audio-encoder forward pass for MI355X (hand-written HIP for gfx950).

``packed_windowed_attention_amd.aut`` binds the C ABI of ``libaut.so``
(declared in include/aut.h).  The library is loaded on first use; there is no
CPU fallback.
"""
from . import aut  # noqa: F401
