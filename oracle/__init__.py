"""Slow, plain float64 CPU oracle for fused causal attention and RoPE.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only the test suite, the smoke check and the CPU
baseline leg of the benchmark use it.  It shares no code, header, table or
helper with the HIP kernels in ``causal_attention_fa_amd``; the two meet only
on seeded inputs drawn by ``causal_attention_fa_amd.synth``, which holds no
arithmetic of the method.

Sources (web pages; cited by title and section throughout):

* Forge commit "Add HF streaming data pipeline and three research reports",
  file ARCHITECTURES.md: the per-family table (Qwen 2.5 GQA 28H/4KV, Gemma 2
  local/global 1:1 with attention softcap 50 and head_dim 256, Gemma 3
  5 local : 1 global with window 1024) and the prioritised plan, wave 2:
  item 8 (sliding-window mask q-W < k <= q, out-of-window tiles skipped),
  item 9 (softcap cap*tanh(s/cap) on pre-softmax scores).
* Same commit, README diff: RoPE on interleaved pairs; GQA.
* Forge commit log for src/nn/attention.h: "Wave 1" (RoPE kernels read a
  host-precomputed inverse-frequency table), "Wave 2" (sliding_window with
  sliding_global_every, attn_softcap with the exact tanh' chain in backward).
* forge-studio RESEARCH.md, section 2 (config schema): defaults
  sliding_window(0), sliding_global_every(0), attn_softcap(0),
  n_kv_heads(=n_heads), rope_theta(10000); validations n_heads % n_kv_heads
  == 0 and even head_dim.
* Same commit, INFERENCE_RESEARCH.md, section 2 ("KV cache"): a cache
  preallocated at maximum length, [layer][head][seq][d], read by a
  dedicated single-query kernel split along the cache.

Modules:
    attention  -- attn_fwd / attn_bwd definitions (full score matrix, fp64),
                  row/column-restricted evaluators for sampled checks at
                  large T, layer_window.
    rope       -- inv_freq table (plain and llama3-rescaled), per-layer
                  RoPE base, rope / rope_bwd.
    decode     -- single-query decode over a KV cache, and the exact merge
                  of partial results over disjoint key sets.

Every function is pinned by tests in tests/test_oracle_*.py to closed
forms, invariants, library routines or brute force; see each function's
docstring for its pins.
"""
from . import attention, decode, rope  # noqa: F401
