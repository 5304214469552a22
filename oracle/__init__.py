"""CPU oracle for the draft-tree construction hot path -- TEST INFRASTRUCTURE ONLY.

A plain, slow, single-threaded (numpy, float64) statement of what the method
computes, written from the pages and shared with nothing on the GPU side. Only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it; the library under ``draft_tree_construction_amd``
never does, and fails loudly when its HIP build is missing.

Pages cited by title and section:

* "DARTree: Speculative Diffusion Decoding With Autoregressive Draft Trees"
  (papercache summary of arXiv 2608.13524): Algorithm 1, the depth-bonus score
  s_beta, Lemma 1 and its proof, and the background on speculative sampling and
  DDTree.
* "TALON: Confidence-Aware Speculative Decoding with Adaptive Token Trees"
  (papernotes, NeurIPS 2026): key designs 1-2 (root Top-K, gating against the
  per-depth anchor m_d, global budget N), and its research background (the static
  D x K grid expansion it compares against).
* Course notes "Sampling, speculative decoding and multi-token prediction"
  (unit 11): the accept / residual rule, the three-token worked example, the
  degenerate cases, the bonus token and the per-round yield.
* "GRAFT: adaptive DLM draft-tree construction with target-distilled edge scoring"
  (paper page): method sections on target-distilled edge scoring (the edge MLP),
  inference (best-first by summed edge scores) and state-aware budget allocation.
* "DDTree: from theory to practice" (CSDN blog): Top-B prefixes, the S_K
  restriction, the heap over rank descriptors, the debugging checklist.

Modules: ``rowsweep`` (log-softmax + top-K), ``marginal`` (DDTree Top-B), ``depthwise`` (DARTree Algorithm 1),
``gated`` (TALON), ``static`` (the static D x K grid), ``tdes`` (GRAFT edge scores, best-first, budget), ``treeout`` (parent array and mask), ``accept`` (greedy and
residual acceptance walks), ``philox`` (Philox4x32-10).
"""
