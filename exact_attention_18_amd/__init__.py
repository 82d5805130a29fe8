"""MI355X-native fused exact-attention forward (gfx950 HIP kernels behind a C-ABI).

``exact_attention_18_amd.attn`` is the thin ctypes binding over ``libattn.so``
(argument marshalling only; every step of the forward runs in the HIP
kernels).  ``exact_attention_18_amd.inputs`` draws the seeded synthetic
workloads.  Importing the package loads nothing: the shared library is opened
on first use and a missing library is an error, never a fallback.
"""

__all__ = ["attn", "inputs"]
