"""GPT-2 training step on MI355X (gfx950): hand-written HIP kernels behind a
C-ABI library (``libgpt2_hip.so``), with a thin ctypes binding.

Importing this package loads nothing; ``gpt_transformer_lm_amd.lib`` loads the
shared library on first use and raises if it has not been built.
"""

__all__ = ["lib", "synthetic"]
