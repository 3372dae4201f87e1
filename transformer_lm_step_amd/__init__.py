"""GPT-2 training step (forward, backward, AdamW) on MI355X (gfx950).

The compute lives in ``libgpt2_hip.so`` (hand-written HIP kernels behind the C
ABI of ``include/gpt2.h`` and ``include/gpt2_ops.h``).  ``binding`` marshals
arguments to it and raises on import if the library has not been built;
``model.GPT2`` allocates the caller-owned device buffers with PyTorch.
``build`` compiles the library.
"""
