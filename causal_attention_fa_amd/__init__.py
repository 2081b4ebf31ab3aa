"""MI355X (gfx950) fused causal flash attention: forward, backward and RoPE.

Submodules:
    fa     -- ctypes binding of libfa.so (the C ABI in include/fa.h) and thin
              torch conveniences; importing it requires the built library.
    synth  -- seeded synthetic inputs and the workload table (no kernel
              arithmetic).
    build  -- builds libfa.so with hipcc for gfx950.

The package root imports nothing heavy so the input generators are usable
without a GPU or a built library.
"""
