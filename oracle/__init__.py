"""CPU oracle for the Orthrus decode round -- TEST INFRASTRUCTURE.

A plain, slow, obviously correct NumPy statement (float64 by default) of what the decode
round computes: dual-view attention under the draft and verify masks, the decoder rows of
both views, the LM head and its argmax, the greedy consensus with KV rollback, the
temperature > 0 rejection-sampling accept and the Philox4x64-10 uniforms it draws.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package.  It shares no code with the HIP library (``orthrus_round_amd``) and
never imports it; the two meet only on inputs drawn by ``synth``.

Parity status per function (pins live in ``tests/test_oracle_*.py``):
* philox4x64 / uniforms ........ pinned to numpy.random.Philox words
* rmsnorm, rope ................ pinned to torch rms_norm, complex rotation, norm/relative-position invariants
* draft/verify attention ....... pinned to torch scaled_dot_product_attention (float64) + special cases
* grouped_attention ............ the same attention in matrix-product form: pinned to SDPA and to the
                                 row form
* ar_pass / decoder rows ....... pinned to transformers' Llama decoder (float64) with the same weights
* draft_pass ................... pinned to the same Llama with a block mask when both views share weights
* argmax ....................... ties -> lowest id, pinned by duplicated LM-head rows
* consensus .................... exhaustive first-mismatch closed form
* softmax_t ..................... scipy / torch softmax of z/T in float64, two-logit closed form
* gumbel_sample ................. chi-square against scipy's softmax(z/T) on seeded Philox draws,
                                 greedy in the T -> 0 limit
* rejection_accept / race ...... acceptance rate sum(min(p, q)) and output law p (p, q from scipy),
                                 greedy consensus in the T -> 0 limit
* generate / generate_ar, T > 0  first two committed tokens follow the AR law p(t1) p(t2 | t1)
                                 (chi-square over seeded runs on a one-layer, 8-token decoder)
* log_confidence ............... closed form on a two-logit row; exp sums to 1 over the vocabulary
* two_step_draft ............... n_fill = 0 is the one-pass draft; the filled slots keep pass-one
                                 tokens and are the n_fill most confident
* generate vs generate_ar ...... losslessness (identical greedy trajectories), forced full/zero
                                 acceptance, K = 1, poisoned dead cache slots
* token values on random weights: parity unpinned by the pages (no worked example exists);
  pinned only through the properties above.
"""
