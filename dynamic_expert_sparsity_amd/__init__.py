"""BEAM masked-MoE layer forward on MI355X (gfx950): Python binding.

The compute lives in the HIP library libbeam_moe.so (C-ABI declared in
include/beam_moe.h).  This package only marshals torch tensors into that
library's calls; it has no CPU fallback and raises if the library is missing.
"""
