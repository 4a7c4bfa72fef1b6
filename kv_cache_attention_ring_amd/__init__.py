"""Write-time RoPE + FP8 ring KV cache, delta rebase and FP8 window attention
for one AMD MI355X (gfx950).

The compute path is a C-ABI shared library of hand-written HIP kernels
(``libkvring.so``, declared in ``include/kvring.h``); ``kvring`` is its thin
ctypes binding.  ``inputs`` holds the seeded synthetic input generators.
"""
__all__ = ["kvring", "inputs"]
