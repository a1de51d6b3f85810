"""MI355X-native causal block-sparse attention (the SSA hot path).

Block summaries and scores, top-k block selection, block-sparse attention
forward, and the full-attention counterpart with per-row dropped mass, as
hand-written HIP kernels for gfx950 behind a C-ABI library (``libssa.so``).
The Python layer only marshals arguments; importing the binding fails loudly
when the library has not been built.
"""
__all__ = ["workloads"]
