"""Paged FlashAttention over an FP8/fp16 block-paged KV cache, for MI355X (gfx950).

The computation lives in libpagedattn.so (hand-written HIP kernels behind the
C ABI in include/pagedattn.h). ``attention_paged_flashattention_amd.pagedattn``
is its thin Python binding; importing it fails if the library is not built.
``synth`` holds the seeded synthetic workloads.
"""

__all__ = ["pagedattn", "synth", "build"]
