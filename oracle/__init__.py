"""CPU oracle of the DFlash block-diffusion drafter forward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code with the
HIP path; its only common input is the seeded generator module ``synth``.

It is a plain, slow, float64 NumPy restatement of what the pages define:

* the session state machine of Ollama ``mlxrunner/dflash.go``
  (``committed``, ``flush``, ``takePending``, ``commitBlock``, ``propose``,
  ``selectBlock``), in ``oracle.session``;
* the context path (taps -> ``fc`` -> ``hidden_norm`` -> per-layer K/V, one
  cache entry per slot) and the block path (anchor + n mask rows attending over
  that cache, rows 1..n unembedded) described by the same file and by the
  mlxcel PR "feat(speculative): add the Laguna DFlash drafter" (context path,
  fused QKV, per-head gate, sliding window, drop-before-fc), in
  ``oracle.model``;
* the batched sampler (penalties from committed history only, temperature,
  softmax, Gumbel-max with Philox4x64-10), in ``oracle.sampler``;
* speculative verification of a drafted block against target logits (greedy
  per-position argmax; the speculative-sampling acceptance rule with the
  draft's proposal probabilities), in ``oracle.verify``.

With ``emulate_bf16=True`` it rounds to bf16 at the points where the GPU path
stores bf16 (every GEMM input operand, Q after norm and RoPE, every K/V cache
entry, the gated attention output); everything else stays float64.

Pins: every function is checked in ``tests/test_oracle_*.py`` against
something other than itself (transformers' Qwen3 attention and MLP, torch's
``rms_norm`` and ``scaled_dot_product_attention``, numpy's Philox, closed
forms and invariants the pages state; verification against the
rejection-sampling theorem it exists to satisfy).  The Laguna variant (aux
norms, context input norm, fused qkv, gate, window) is pinned against a
forward assembled from transformers' Qwen3 modules plus those steps written in
torch, with planted mistakes showing each pin discriminates; see the test
headers.
"""
