"""CPU oracle for Gemma-4-style grouped-query attention over a KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path (``global_gqa_attention_window_amd``) and never reads that path's outputs.

Everything is float64 NumPy, rounded to bf16 only at the points the method
names (TensorFold PR #1183 "cuda gemma4: images on the 12B ...", squashed
commit bodies, the window_rows and attention_range notes: the checker holds
float64 values at the rounding points, with the spread fp32 arithmetic can
reach around them).

Modules
  bf16      float64 -> bf16 round-to-nearest-even, ordered bit keys
  contract  key-block sizes, P modes and the error radius constants
  attn_ref  key sets, decode (one pass and chunked), prefill, radius, check
  brute     loop-per-element reference for tiny shapes, written apart

Parity pins (see tests/test_oracle_*.py): the bf16 value printed on the pages,
exhaustive-style bf16 checks against integer rounding, brute force on tiny
inputs, closed forms (one key returns V, identical keys return the mean of V),
the merge identity, window-over-ring equals masked linear, and the two-halves
P bound.  Two parts are "parity unpinned" by the pages themselves: the
absolute output values (the pages print none) and the key-block size at which
P is rounded against the running max (a contract constant of this library).
"""
