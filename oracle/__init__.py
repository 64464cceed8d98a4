"""fp64 CPU oracle for the speculative-decoding verification step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link anything in this package: only the tests, the graft entry's smoke check
and the benchmark's CPU-baseline leg use it.  It shares no code with the HIP
library; the two meet only in the seeded inputs of the `synth` module.

It is a plain, slow, obviously correct restatement of the method in NumPy
float64, written from these sources (cited by page title and section):

* CMU 15-779 lecture 17 notes ("LLM serving (2): speculative decoding"),
  sections 2.2-2.4 (greedy verification, speculative sampling, Algorithm 1),
  4.3 (the topology-aware causal mask and depth positions of tree-parallel
  decoding), 4.4 (VerifyGreedy on a token tree) and 4.5 (naive sampling and multi-step
  speculative sampling on a tree).
* "LLM speculative decoding close-reading notes 02: original speculative
  decoding", sections 4 (the full algorithm with uniforms r_i), 5.1 (residual
  normaliser), 10 (greedy special case) and 11.3 (per-request RNG streams).
* "Speculative decoding: draft, verify and payoff", chapter 2 section 2 (the
  four steps of one round).
* "LLM speculative decoding close-reading notes 02", section 5.4 (any
  decoding strategy applied alike to p and q keeps the method exact: the
  consistent top-k and top-p filters).

Every reading the pages leave open (which uniform feeds the final draw, the
inverse-CDF convention, tie-breaks, the empty residual, the tree contract) is
fixed in `specverify_oracle` where the step is taken.  All functions are
pinned by `tests/test_oracle_*.py`.
"""
from .specverify_oracle import (  # noqa: F401
    ChainResult, TreeResult, ProbsResult,
    logits_to_f64, softmax_t, accept_threshold, inverse_cdf_draw,
    chain_distributions, chain_decide_request, verify_chain, RaggedChainResult, verify_chain_ragged,
    topk_filter, topp_filter, verify_chain_topk, TOPK_MAX, TOPK_MAX_KEPT,
    topp_cut, FilteredChainResult, filtered_distributions, filter_params, verify_chain_filtered,
    verify_tree, probs_debug, tree_node_depths, TreeMaskResult, tree_attention_mask,
    mss_thresholds, mss_node, mss_proposals, tree_children, verify_tree_mss,
)
